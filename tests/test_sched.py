"""Host check of the kernels' workgroup order (exact_attention_24_amd/csrc/attn_sched.h),
compiled as plain C++: bijection, one XCD per head, grouped heads together, every
XCD holding heads of every sequence, heaviest causal tiles first."""
import pathlib
import shutil
import subprocess

import pytest

ROOT = pathlib.Path(__file__).resolve().parents[1]


def test_tile_order(tmp_path):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = tmp_path / "sched_check"
    subprocess.run([cxx, "-std=c++17", "-O1", f"-I{ROOT / 'exact_attention_24_amd' / 'csrc'}",
                    str(ROOT / "tests" / "sched_check.cpp"), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0 and out.stdout.strip() == "ok", out.stdout
