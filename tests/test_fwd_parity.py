"""GPU parity of the attention forward (through the C ABI) against the fp64 oracle.

Pages cited (by title):
  [SafeSoftmax] "FlashAttention：从 Safe Softmax 到分块计算"
  [OpOpt]       "Attention 算子优化:从物化 N×N 矩阵到 FlashAttention 与 PagedAttention"
  [AIInfra]     the AIInfra FlashAttention note on dpshk.com
"""
import math

import numpy as np
import pytest
import torch

import exact_attention_24_amd as ea
import oracle
from attn_inputs import WORKLOADS, make_inputs, make_workload_inputs
from tests.parity import LSE_TOL, O_TOL, assert_close, dtype_name, lse_tol, oracle_fwd_threads, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def run_fwd(q, k, v, scale, causal=False, seqlens=None):
    dq, dk, dv = (t.to(DEV) for t in (q, k, v))
    sl = seqlens.to(DEV) if seqlens is not None else None
    o, lse = ea.attn_fwd(dq, dk, dv, scale=scale, causal=causal, seqlens=sl)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def check_full(x, scale, causal, tag):
    q, k, v, sl = x["q"], x["k"], x["v"], x["seqlens"]
    o, lse = run_fwd(q, k, v, scale, causal, sl)
    ro, rl = oracle.attn_ref_fwd(q, k, v, scale, causal, sl)
    dn = dtype_name(q)
    assert_close(o, ro, O_TOL[dn], f"{tag} O")
    assert_close(lse, rl, lse_tol(dn, q, k, scale), f"{tag} LSE")
    # padded rows exactly zero, LSE exactly -inf
    if sl is not None:
        for b, L in enumerate(sl.tolist()):
            assert torch.all(o[b, :, L:] == 0), f"{tag}: padded rows of O not zero"
            assert torch.all(torch.isneginf(lse[b, :, L:])), f"{tag}: padded LSE not -inf"


# ------------------------------------------------------------ pinned page cases

@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_hand_case(dtype, d, causal):
    """The hand-derived N=4, d=2 integer case ([AIInfra] §3.1), zero-padded to d:
    scores are unchanged, the extra output columns must be exactly 0."""
    Q = torch.tensor([[1, 0], [0, 1], [1, 1], [0, 0]], dtype=torch.float32)
    K = torch.tensor([[0, 0], [1, 0], [0, 1], [1, 1]], dtype=torch.float32)
    V = torch.tensor([[1, 2], [3, 4], [5, 6], [7, 8]], dtype=torch.float32)
    pad = lambda t: torch.nn.functional.pad(t, (0, d - 2))[None, None].to(dtype).contiguous()
    q, k, v = pad(Q), pad(K), pad(V)
    o, lse = run_fwd(q, k, v, 1.0, causal)
    ro, rl = oracle.attn_ref_fwd(q, k, v, 1.0, causal)
    # bf16: O is in [4, 8), where half a bf16 ulp is 2^-6 = 0.0156, plus P rounded to
    # bf16 before the P V product (relative 2^-9) times max|V| = 8: 0.0156.
    # fp16: half an ulp in [4, 8) is 2^-9, P's relative rounding 2^-11.
    tol = {torch.float32: 1e-5, torch.bfloat16: 2 ** -6 + 2 ** -9 * 8,
           torch.float16: 2 ** -9 + 2 ** -11 * 8}[dtype]
    assert_close(o, ro, tol, "hand O")
    # the inputs are small integers, exact in every format, and LSE never sees a
    # 16-bit rounding: fp32 statistics reach 1e-5 whatever the input format
    assert_close(lse, rl, 1e-5, "hand LSE")
    assert torch.all(o[..., 2:] == 0)
    if causal:
        assert torch.equal(o[0, 0, 0, :2], V[0].to(dtype)), "causal row 0 must be V_0 exactly"


def _one_hot_case(scores_by_key, values_by_key, N, d, dtype):
    """q = e_1, k_j = s_j e_1 at chosen key positions, all other keys k = -100 e_1
    (weight e^-103 relative, which underflows to 0 in fp32); V column 0 holds the values."""
    q = torch.zeros(1, 1, N, d)
    q[..., 0] = 1.0
    k = torch.zeros(1, 1, N, d)
    k[..., 0] = -100.0
    v = torch.zeros(1, 1, N, d)
    for j, s in scores_by_key.items():
        k[0, 0, j, 0] = s
    for j, val in values_by_key.items():
        v[0, 0, j, 0] = val
    return q.to(dtype), k.to(dtype), v.to(dtype)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
def test_two_block_example(dtype):
    """[OpOpt] §三: blocks [1,2] and [3,1] in two different KV tiles merge to
    l = 2e^-2 + e^-1 + 1 ~= 1.638 relative to the max 3, so LSE = 3 + ln l."""
    keys = {0: 1.0, 1: 2.0, 70: 3.0, 71: 1.0}
    vals = {0: 0.5, 1: 1.0, 70: 1.5, 71: 2.0}
    q, k, v = _one_hot_case(keys, vals, 128, 64, dtype)
    o, lse = run_fwd(q, k, v, 1.0)
    l = 2 * math.exp(-2) + math.exp(-1) + 1
    assert abs(math.exp(float(lse[0, 0, 0]) - 3.0) - 1.638) <= 1e-3  # the page's printed value
    assert abs(float(lse[0, 0, 0]) - (3 + math.log(l))) <= 1e-5  # exact inputs, fp32 statistics
    want = (0.5 * math.exp(-2) + 1.0 * math.exp(-1) + 1.5 + 2.0 * math.exp(-2)) / l
    # bf16: O ~ 1.35, half an ulp in [1, 2) is 2^-8, plus 2^-9 * max|V| = 2^-8;
    # fp16: 2^-11 + 2^-11 * max|V|
    tol = {torch.float32: 1e-5, torch.bfloat16: 2 ** -8 + 2 ** -9 * 2,
           torch.float16: 2 ** -11 + 2 ** -11 * 2}[dtype]
    assert abs(float(o[0, 0, 0, 0]) - want) <= tol


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_merge_example(dtype):
    """[SafeSoftmax] §3.3: scores [1,2] in one tile and [3] in the next, v = [10,20,30]
    (bf16: v = [1,2,3], the same example scaled by 1/10, to keep O within the bf16
    tolerance), o = u / l with l = e^-1 (e^-1 + 1) + 1 and u = e^-1 u1 + 30."""
    f = 1.0 if dtype == torch.float32 else 0.1
    q, k, v = _one_hot_case({0: 1.0, 1: 2.0, 64: 3.0}, {0: 10 * f, 1: 20 * f, 64: 30 * f},
                            128, 128, dtype)
    o, lse = run_fwd(q, k, v, 1.0)
    l = math.exp(-1) * (math.exp(-1) + 1) + 1
    u = math.exp(-1) * (10 * math.exp(-1) + 20) + 30
    tol = 1e-5 if dtype == torch.float32 else 2e-2
    assert abs(float(o[0, 0, 0, 0]) - f * u / l) <= tol
    assert abs(float(lse[0, 0, 0]) - (3 + math.log(l))) <= 1e-5  # exact inputs, fp32 statistics


# ----------------------------------------------- small shapes, full comparison

SMALL = [  # (B, H, N, d) spanning several tiles with ragged tails
    (1, 1, 1, 64), (2, 3, 17, 64), (1, 2, 64, 128), (2, 2, 129, 64), (2, 3, 300, 128),
    (1, 2, 517, 64), (3, 1, 700, 128),
]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32, torch.float16],
                         ids=["bf16", "f32", "f16"])
@pytest.mark.parametrize("causal", [False, True], ids=["dense", "causal"])
@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s)))
def test_small_full(shape, causal, dtype):
    B, H, N, d = shape
    x = make_inputs(B, H, N, d, dtype, seed=hash((shape, causal)) % 10000)
    check_full(x, 1 / math.sqrt(d), causal, f"small{shape}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32, torch.float16],
                         ids=["bf16", "f32", "f16"])
@pytest.mark.parametrize("causal", [False, True], ids=["dense", "causal"])
@pytest.mark.parametrize("d", [64, 128])
def test_small_varlen(d, causal, dtype):
    """Padded batch with lengths 0, 1, a ragged value, a tile multiple and N."""
    B, H, N = 6, 2, 333
    x = make_inputs(B, H, N, d, dtype, seed=77 + d)
    x["seqlens"] = torch.tensor([0, 1, 200, 128, N, 37], dtype=torch.int32)
    check_full(x, 1 / math.sqrt(d), causal, f"varlen d={d}")


@pytest.mark.parametrize("heads", [(8, 8), (16, 8)], ids=["mha", "gqa"])
@pytest.mark.parametrize("causal", [False, True], ids=["dense", "causal"])
def test_varlen_length_order(causal, heads):
    """A padded batch whose head count lets the kernel launch sequences in
    order of decreasing length (ties included: the order must still cover
    every (sequence, head, tile) exactly once); every row checked."""
    H, H_kv = heads
    B, N, d = 7, 300, 128
    x = make_inputs(B, H, N, d, torch.bfloat16, seed=79 + causal, H_kv=H_kv)
    x["seqlens"] = torch.tensor([37, 300, 0, 150, 300, 1, 150], dtype=torch.int32)
    check_full(x, 1 / math.sqrt(d), causal, "length-ordered varlen")


@pytest.mark.parametrize("causal", [False, True], ids=["dense", "causal"])
def test_varlen_many_sequences(causal):
    """More sequences than a wave has lanes (B = 70): the kernel launches them
    in batch order instead of by decreasing length; lengths include 0, 1, the
    tile edges and N; every row checked."""
    B, H, N, d = 70, 8, 150, 64
    x = make_inputs(B, H, N, d, torch.bfloat16, seed=83 + causal)
    g = torch.Generator().manual_seed(83)
    lens = torch.randint(0, N + 1, (B,), generator=g, dtype=torch.int64).to(torch.int32)
    lens[:6] = torch.tensor([0, 1, 63, 64, 128, N], dtype=torch.int32)
    x["seqlens"] = lens
    check_full(x, 1 / math.sqrt(d), causal, "varlen B=70")


# ------------------------------------------------ full workloads, every output

FWD_WORKLOADS = [n for n, w in WORKLOADS.items() if w.Nq is None]  # decode has its own test


@pytest.mark.parametrize("name", FWD_WORKLOADS)
def test_workload_full(name):
    """Each workload at its full size, in the launch configuration the benchmark
    times: every O and LSE entry of every head against the oracle ([AIInfra]
    §3.1's random comparison, whole tensors); padded rows exactly 0 / -inf."""
    w = WORKLOADS[name]
    x = make_workload_inputs(w)
    q, k, v, sl = x["q"], x["k"], x["v"], x["seqlens"]
    print(f"workload {name}: GPU forward", flush=True)
    o, lse = run_fwd(q, k, v, w.scale, w.causal, sl)
    assert torch.isfinite(o).all(), "non-finite output"
    print(f"workload {name}: oracle over {w.B * w.H} heads", flush=True)
    ro, rl = oracle_fwd_threads(q, k, v, w.scale, w.causal, sl)
    dn = dtype_name(q)
    assert_close(o, ro, O_TOL[dn], f"{name} O")
    assert_close(lse, rl, LSE_TOL[dn], f"{name} LSE")
    if sl is not None:
        for b, L in enumerate(sl.tolist()):
            assert torch.all(o[b, :, L:] == 0) and torch.all(torch.isneginf(lse[b, :, L:]))


@pytest.mark.parametrize("causal", [False, True], ids=["dense", "causal"])
def test_long_context_sampled_rows(causal):
    """N = 32768 (256 row tiles of 128, 512 key tiles of 64): sampled rows of
    every head against the oracle, including both ends and tile boundaries."""
    B, H, N, d = 1, 4, 32768, 128
    x = make_inputs(B, H, N, d, torch.bfloat16, seed=81 + causal)
    o, lse = run_fwd(x["q"], x["k"], x["v"], 1 / math.sqrt(d), causal)
    assert torch.isfinite(o).all()
    rng = np.random.default_rng(81)
    for h in range(H):
        rows = sorted({0, 1, 127, 128, 4095, 16384, N - 65, N - 64, N - 1} |
                      set(rng.integers(0, N, size=8).tolist()))
        ro, rl = oracle.attn_ref_rows(x["q"], x["k"], x["v"], 0, h, rows, 1 / math.sqrt(d), causal)
        assert_close(o[0, h, rows], ro, O_TOL["bf16"], f"N=32768 O (h={h})")
        assert_close(lse[0, h, rows], rl, LSE_TOL["bf16"], f"N=32768 LSE (h={h})")


# ------------------------------------------------------------- edge and stress

@pytest.mark.parametrize("d", [64, 128])
def test_f16_large_values(d):
    """fp16's range: Q, K scaled x8 (scores in the hundreds) and V x64 (|V| in
    the hundreds, far above bf16 tests' magnitudes but well inside fp16): the
    weights P stay <= 256 and O <= max|V|, so nothing overflows; compared with
    the tolerance scaled by max|V|."""
    x = make_inputs(1, 2, 300, d, torch.float16, seed=13)
    big = make_inputs(1, 2, 300, d, torch.float16, seed=13, std=8.0)
    x["q"], x["k"] = big["q"], big["k"]
    x["v"] = (x["v"].float() * 64).to(torch.float16)
    o, lse = run_fwd(x["q"], x["k"], x["v"], 1 / math.sqrt(d), True)
    ro, rl = oracle.attn_ref_fwd(x["q"], x["k"], x["v"], 1 / math.sqrt(d), True)
    assert_close(o, ro, O_TOL["f16"] * 64, "f16 large values O")
    assert_close(lse, rl, lse_tol("f16", x["q"], x["k"], 1 / math.sqrt(d)), "f16 large values LSE")


def rising_scores(B, H, N, d, dtype, step, seed):
    """Inputs whose scores rise along the keys: q . k_j = step * j plus small
    noise, so every key tile's scores lie far above the previous tiles' max and
    the online softmax has to move its reference max on every tile."""
    x = make_inputs(B, H, N, d, dtype, seed=seed, std=0.05)
    x["q"] = x["q"].float()
    x["k"] = x["k"].float()
    x["q"][..., 0] = 1.0
    x["k"][..., 0] = step * torch.arange(N, dtype=torch.float32)
    x["q"] = x["q"].to(dtype)
    x["k"] = x["k"].to(dtype)
    x["v"] = make_inputs(B, H, N, d, dtype, seed=seed + 1)["v"]
    return x


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True], ids=["dense", "causal"])
def test_rising_scores_move_the_reference(causal, dtype):
    """Scores grow by 16 per 64-key tile (23 in log2 units, above the 2^8
    weight bound), so every tile takes the rescaling path of the online
    softmax ([SafeSoftmax] §3.2): O and LSE must still match the oracle."""
    x = rising_scores(2, 2, 333, 128, dtype, 0.25, seed=91)
    o, lse = run_fwd(x["q"], x["k"], x["v"], 1.0, causal)
    ro, rl = oracle.attn_ref_fwd(x["q"], x["k"], x["v"], 1.0, causal)
    dn = dtype_name(x["q"])
    assert_close(o, ro, O_TOL[dn], "rising scores O")
    assert_close(lse, rl, lse_tol(dn, x["q"], x["k"], 1.0), "rising scores LSE")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("causal", [False, True], ids=["dense", "causal"])
def test_padding_contents_never_read(causal, dtype):
    """Padded positions (at or past a sequence's length) hold NaN in Q, K and V:
    valid rows must still match the oracle (which never looks at them) and
    padded rows must be exactly 0 / -inf."""
    B, H, N, d = 3, 2, 333, 128
    x = make_inputs(B, H, N, d, dtype, seed=78)
    x["seqlens"] = torch.tensor([100, 333, 0], dtype=torch.int32)
    clean = {k_: (v_.clone() if v_ is not None else None) for k_, v_ in x.items()}
    for b, L in enumerate(x["seqlens"].tolist()):
        for n in ("q", "k", "v"):
            x[n][b, :, L:] = float("nan")
    o, lse = run_fwd(x["q"], x["k"], x["v"], 1 / math.sqrt(d), causal, x["seqlens"])
    ro, rl = oracle.attn_ref_fwd(clean["q"], clean["k"], clean["v"], 1 / math.sqrt(d), causal,
                                 clean["seqlens"])
    dn = dtype_name(x["q"])
    assert_close(o, ro, O_TOL[dn], "NaN padding O")
    assert_close(lse, rl, LSE_TOL[dn], "NaN padding LSE")


def test_deterministic():
    x = make_inputs(2, 4, 1000, 128, torch.bfloat16, seed=5)
    a = run_fwd(x["q"], x["k"], x["v"], 0.088, True)
    b = run_fwd(x["q"], x["k"], x["v"], 0.088, True)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("d", [64, 128])
def test_stress_large_scores(d):
    """[AIInfra] §3.1: a large Q K^T range. Q and K are scaled x8 (scores reach the
    hundreds); V stays N(0,1), so O keeps the magnitude the bf16 tolerance is set for."""
    x = make_inputs(1, 2, 400, d, torch.bfloat16, seed=9)
    big = make_inputs(1, 2, 400, d, torch.bfloat16, seed=9, std=8.0)
    x["q"], x["k"] = big["q"], big["k"]
    check_full(x, 1 / math.sqrt(d), False, "large scores")
    check_full(x, 1 / math.sqrt(d), True, "large scores causal")


def test_stress_identical_and_similar_queries():
    """[AIInfra] §3.1: identical query vectors, and a query equal to every key."""
    x = make_inputs(1, 1, 300, 128, torch.bfloat16, seed=10)
    q = x["q"].clone()
    q[:] = q[0, 0, 0]
    o, _ = run_fwd(q, x["k"], x["v"], 0.088)
    assert torch.all(o == o[0, 0, 0]), "identical queries must give identical rows"
    k = q.clone()
    o2, lse2 = run_fwd(q, k, x["v"], 0.088)
    ro, rl = oracle.attn_ref_fwd(q, k, x["v"], 0.088)
    assert_close(o2, ro, O_TOL["bf16"], "query equal to every key")


def test_shift_invariance():
    """[SafeSoftmax] §2: K -> K + 1 c^T shifts each score row by a constant; O is unchanged."""
    x = make_inputs(1, 2, 500, 64, torch.float32, seed=11)
    c = torch.randn(64, generator=torch.Generator().manual_seed(3)) * 2
    o1, l1 = run_fwd(x["q"], x["k"], x["v"], 0.125, True)
    o2, l2 = run_fwd(x["q"], x["k"] + c, x["v"], 0.125, True)
    assert_close(o2, o1, 2e-5, "shift invariance")


def test_guard_band_untouched():
    """Outputs live inside a larger buffer: nothing past the tensor may be written."""
    B, H, N, d = 1, 2, 77, 128
    x = make_inputs(B, H, N, d, torch.bfloat16, seed=12)
    n = B * H * N * d
    buf = torch.full((n + 4096,), -7.0, dtype=torch.bfloat16, device=DEV)
    lbuf = torch.full((B * H * N + 256,), -7.0, dtype=torch.float32, device=DEV)
    o = buf[:n].view(B, H, N, d)
    lse = lbuf[: B * H * N].view(B, H, N)
    ea.attn_fwd(x["q"].to(DEV), x["k"].to(DEV), x["v"].to(DEV), out=o, lse=lse, causal=True)
    torch.cuda.synchronize()
    assert torch.all(buf[n:] == -7.0) and torch.all(lbuf[B * H * N:] == -7.0)
    ro, _ = oracle.attn_ref_fwd(x["q"], x["k"], x["v"], 1 / math.sqrt(d), True)
    assert_close(o.cpu(), ro, O_TOL["bf16"], "guard-band run")
