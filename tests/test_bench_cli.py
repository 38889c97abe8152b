"""CPU checks of the benchmark script's contract: the FLOP convention, the
distribution statistics, the refusal of more than one GPU, the oracle-based
CPU baseline and the traffic figure read from the committed profile."""
import math
import pathlib
import subprocess
import sys

import bench
from attn_inputs import WORKLOADS, make_workload_inputs

ROOT = pathlib.Path(__file__).resolve().parent.parent


def test_flop_convention():
    # 4*B*H*N^2*d, halved for the causal mask: 274.9 GFLOP for the headline workload
    assert bench.fwd_flops(2, 32, 4096, 128, True) == 4 * 2 * 32 * 4096 ** 2 * 128 / 2
    assert bench.fwd_flops(4, 16, 2048, 64, False) == 4 * 4 * 16 * 2048 ** 2 * 64
    assert math.isclose(bench.fwd_flops(2, 32, 4096, 128, True) / 1e9, 274.878, rel_tol=1e-5)


def test_median_and_p90_of_sorted_times():
    per = [float(i) for i in range(1, 51)]  # 50 sorted launch times
    med, p90 = bench.stats(per)
    assert med == 26.0 and p90 == 45.0
    assert bench.stats([3.0]) == (3.0, 3.0)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_cpu_baseline_runs_the_oracle():
    w = WORKLOADS["single_head_f32_n256_d64"]
    x = make_workload_inputs(w)
    r = bench.cpu_baseline(x, w, 0.01)
    assert r["kind"] == "oracle" and r["unit"] == "TFLOP/s"
    assert r["value"] > 0 and r["cores"] >= 1
    assert "1 of 1 (b,h) heads" in r["sample"]


def test_headline_traffic_matches_the_kernel_sources():
    """The roofline's traffic figure comes from the committed counter summary
    and is reported only while the forward kernel's sources hash to the value
    recorded there: a change to those sources must come with new counters."""
    t = bench.profiled_traffic()
    assert t is not None, ("forward kernel sources changed since "
                           f"{bench.PROFILE} was taken: re-take FETCH_SIZE/WRITE_SIZE")
    assert 0 < t < 10 * 2 ** 30
