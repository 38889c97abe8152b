"""Build the gfx950 HIP library libattn.so in-tree with hipcc.

Every source is compiled for gfx950 only, with packed-fp32 instruction
selection switched off (-packed-fp32-ops), then linked into
exact_attention_24_amd/lib/libattn.so. Objects go to _build/ at the repo root.
"""
from __future__ import annotations

import concurrent.futures
import os
import pathlib
import shutil
import subprocess

PKG = pathlib.Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
LIB_DIR = PKG / "lib"
LIB_PATH = LIB_DIR / "libattn.so"
BUILD_DIR = ROOT / "_build"
SOURCES = ["attn_api.cpp", "attn_fwd.hip", "attn_fwd_f32.hip", "attn_fwd8.hip", "attn_bwd.hip", "attn_decode.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def compile_flags() -> list[str]:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
            "-Wno-unused-function", "-Wno-unused-variable",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            f"-I{ROOT / 'include'}", f"-I{CSRC}"]


def _compile(src: pathlib.Path, obj: pathlib.Path, verbose: bool) -> None:
    cmd = [hipcc(), *compile_flags(), "-x", "hip", "-c", str(src), "-o", str(obj)]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src.name}:\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False) -> pathlib.Path:
    """Compile every source and link libattn.so; always rebuilds."""
    BUILD_DIR.mkdir(exist_ok=True)
    LIB_DIR.mkdir(exist_ok=True)
    objs = [BUILD_DIR / (pathlib.Path(s).stem + ".o") for s in SOURCES]
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        list(ex.map(lambda so: _compile(CSRC / so[0], so[1], verbose), zip(SOURCES, objs)))
    tmp = LIB_PATH.with_suffix(".so.tmp")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-o", str(tmp), *map(str, objs)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}{res.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
