"""GPU parity of the FP8 forward (attn_fwd_fp8, through the C ABI) against the
fp64 oracle on the dequantised inputs.

The bar is derived, per output element, from the arithmetic the kernel does
(the pages fix no precision for an FP8 path; "FlashAttention：从 Safe Softmax
到分块计算" §9.2 names scaling, accumulation and error control as what it has
to handle, "Attention 算子优化..." §六 keeps softmax and accumulation in fp32):

  * weights rounded to E4M3 for the V product: an unnormalised weight w has
    error <= 2^-4 w (w >= 2^-6) or <= min(w, 2^-10) below; divided by the row
    sum l >= 1 (the reference never exceeds the row max) this is at most
    2^-4 p + min(p, 2^-10) per normalised weight p;
  * the FP8 matrix cores' sums: measured on the device with an in-bounds
    probe over 524,288 random 16x16x128 E4M3 products spanning the whole E4M3
    range, |error| <= 2^-12.4 * sum_k |a_k b_k|; the bar takes 2^-11. A score
    is off by at most delta_j = 2^-11 * scale * sum_c |q_c k_jc|, which moves
    each weight by a factor exp(delta) and l alike (<= 2 delta relative on
    O); each of the nt tile updates of O adds at most 2^-11 of the O
    accumulated so far (<= nt * 2^-11 * sum_j p_j |V_j| in all);
  * rounding O to bf16 (2^-8 relative) or fp16 (2^-11).
  bound[i, c] = sum_j (2^-4 p_ij + min(p_ij, 2^-10)) |V_jc|
              + (2 max_j delta_ij + nt * 2^-11) * sum_j p_ij |V_jc|
              + unit_out * |O_ic| + 1e-6
  The LSE uses the fp32 weights, so its error is the scores' error:
  |LSE_i - LSE_ref_i| <= max_j delta_ij + 1e-5.
"""
import math

import numpy as np
import pytest
import torch

import exact_attention_24_amd as ea
import oracle
from attn_inputs import fp8_cache, fp8_head, make_inputs
from tests.parity import log, metrics, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
ACC = 2.0 ** -11                      # matrix-core sum error per unit of sum |a b|
UNIT_OUT = {torch.bfloat16: 2.0 ** -8, torch.float16: 2.0 ** -11}


def fp8_case(B, H, N, seed, H_kv=None, seqlens=None, q=None, k=None, v=None):
    """Seeded N(0,1) inputs quantised as the kernel takes them: Q per token,
    K and V per (batch, K/V head); returns the bytes, the scales and the fp64
    dequantised tensors the oracle reads."""
    x = make_inputs(B, H, N, 128, torch.float32, seed=seed, H_kv=H_kv)
    q = x["q"] if q is None else q
    k = x["k"] if k is None else k
    v = x["v"] if v is None else v
    q8, qs = fp8_cache(q)
    k8, ks = fp8_head(k, seqlens)
    v8, vs = fp8_head(v, seqlens)
    Hk = k.shape[1]
    qd = oracle.dequant_fp8(q8, qs)
    kd = oracle.dequant_fp8(k8, ks[:, :, None].expand(B, Hk, N))
    vd = oracle.dequant_fp8(v8, vs[:, :, None].expand(B, Hk, N))
    return dict(q8=q8, k8=k8, v8=v8, qs=qs, ks=ks, vs=vs, qd=qd, kd=kd, vd=vd)


def run(c, scale, causal, seqlens=None, out_dtype=torch.bfloat16):
    t = {n: c[n].to(DEV) for n in ("q8", "k8", "v8", "qs", "ks", "vs")}
    sl = seqlens.to(DEV) if seqlens is not None else None
    o, lse = ea.attn_fwd_fp8(t["q8"], t["k8"], t["v8"], t["qs"], t["ks"], t["vs"], scale=scale,
                             causal=causal, seqlens=sl, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


def bars(qd, kd, vd, o_ref, p, rows, scale, causal, L, unit_out):
    """The per-element O bars and per-row LSE bars above for the query rows
    ``rows`` of one head, given the oracle's O and P for those rows."""
    N = kd.shape[0]
    j = np.arange(N)[None, :]
    visible = (j < L) & ((~np.bool_(causal)) | (j <= np.asarray(rows)[:, None]))
    delta = ACC * scale * (np.abs(qd[rows]) @ np.abs(kd).T)     # score error bars
    dmax = np.where(visible, delta, 0.0).max(axis=1)
    nt = max(1, -(-max(L, 1) // 128))
    absv = np.abs(vd)
    bound = ((2.0 ** -4 * p + np.minimum(p, 2.0 ** -10)) @ absv
             + (2 * dmax + nt * ACC)[:, None] * (p @ absv) + unit_out * np.abs(o_ref) + 1e-6)
    return bound, dmax + 1e-5


def head_ref_and_bound(qd, kd, vd, scale, causal, L, unit_out):
    """Oracle O, LSE of one head and its bars (fp64)."""
    rows = np.arange(qd.shape[0])
    o_ref, lse_ref, p = oracle.attn_ref_head(qd, kd, vd, scale, causal, L, return_p=True)
    bound, lse_bar = bars(qd, kd, vd, o_ref, p, rows, scale, causal, L, unit_out)
    return o_ref, lse_ref, bound, lse_bar


def check(c, o, lse, scale, causal, seqlens, out_dtype, what):
    B, H, N, _ = c["qd"].shape
    Hk = c["kd"].shape[1]
    worst_ratio, worst_lse = 0.0, 0.0
    for b in range(B):
        L = N if seqlens is None else int(min(max(int(seqlens[b]), 0), N))
        for h in range(H):
            g = oracle.kv_head(h, H, Hk)
            o_ref, lse_ref, bound, lse_bar = head_ref_and_bound(
                c["qd"][b, h], c["kd"][b, g], c["vd"][b, g], scale, causal, L, UNIT_OUT[out_dtype])
            got, gl = o[b, h], lse[b, h]
            assert np.isfinite(got).all(), f"{what}: non-finite O in head ({b}, {h})"
            err = np.abs(got - o_ref)
            ratio = float((err / bound).max())
            worst_ratio = max(worst_ratio, ratio)
            assert ratio <= 1.0, (f"{what}: head ({b},{h}) |O - O_ref| exceeds the derived bar by "
                                  f"x{ratio:.2f} (max err {err.max():.3e})")
            fin = np.isfinite(lse_ref)
            assert np.array_equal(np.isfinite(gl), fin), f"{what}: LSE finiteness differs ({b},{h})"
            assert np.all(gl[~fin] == -np.inf)
            if L < N:
                assert np.all(got[L:] == 0.0), f"{what}: padded O rows not zero ({b},{h})"
            lerr = np.abs(gl[fin] - lse_ref[fin])
            worst_lse = max(worst_lse, float((lerr / lse_bar[fin]).max()) if lerr.size else 0.0)
            assert np.all(lerr <= lse_bar[fin]), f"{what}: LSE error {lerr.max():.3e} ({b},{h})"
    log({"what": what, "kind": "fp8_bound_ratio", "o_ratio": worst_ratio, "lse_ratio": worst_lse,
         **{k: v for k, v in metrics(o, o).items() if k == "n"}})
    return worst_ratio


SHAPES = [(1, 2, 128), (2, 4, 200), (1, 2, 333), (1, 1, 1), (2, 2, 640)]


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True], ids=["dense", "causal"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_fwd8_small(shape, causal, out_dtype):
    """Several 128-key tiles with a ragged tail, one-row and one-tile cases."""
    B, H, N = shape
    c = fp8_case(B, H, N, seed=B * 100 + H * 10 + N + 3 * causal)
    scale = 1.0 / math.sqrt(128)
    o, lse = run(c, scale, causal, out_dtype=out_dtype)
    check(c, o, lse, scale, causal, None, out_dtype, f"fp8 fwd {shape} causal={causal}")


def test_fwd8_statistical_bar():
    """Beyond the worst case: on N(0,1) inputs the E4M3 roundings of the
    weights in the normal range are unbiased and independent, each within
    +-2^-4 of its weight (variance <= (2^-4)^2 / 3), so the error of O_ic has
    standard deviation sigma_ic <= 2^-4 / sqrt(3) * sqrt(sum_j p_ij^2 V_jc^2).
    Every element must lie within 7 sigma plus the deterministic terms of the
    worst-case bar (subnormal weights, matrix-core sums, rounding of O)."""
    B, H, N = 1, 4, 512
    c = fp8_case(B, H, N, seed=9)
    scale = 1.0 / math.sqrt(128)
    o, lse = run(c, scale, False)
    worst = 0.0
    for h in range(H):
        qd, kd, vd = c["qd"][0, h], c["kd"][0, h], c["vd"][0, h]
        o_ref, lse_ref, p = oracle.attn_ref_head(qd, kd, vd, scale, False, N, return_p=True)
        rows = np.arange(N)
        delta = ACC * scale * (np.abs(qd) @ np.abs(kd).T)
        dmax = delta.max(axis=1)
        absv = np.abs(vd)
        sigma = 2.0 ** -4 / math.sqrt(3.0) * np.sqrt((p * p) @ (vd * vd))
        det = (np.minimum(p, 2.0 ** -10) @ absv + (2 * dmax + (N // 128) * ACC)[:, None] * (p @ absv)
               + UNIT_OUT[torch.bfloat16] * np.abs(o_ref) + 1e-6)
        ratio = float((np.abs(o[0, h] - o_ref) / (7.0 * sigma + det)).max())
        worst = max(worst, ratio)
        assert ratio <= 1.0, f"head {h}: O error exceeds 7 sigma + deterministic terms (x{ratio:.2f})"
    log({"what": "fp8 fwd statistical bar", "kind": "fp8_bound_ratio", "o_ratio": worst})


@pytest.mark.parametrize("causal", [False, True], ids=["dense", "causal"])
def test_fwd8_grouped_heads(causal):
    """Eight query heads over two K/V heads (per-K/V-head scales shared by
    four query heads)."""
    c = fp8_case(2, 8, 300, seed=17 + causal, H_kv=2)
    scale = 1.0 / math.sqrt(128)
    o, lse = run(c, scale, causal)
    check(c, o, lse, scale, causal, None, torch.bfloat16, f"fp8 fwd gqa causal={causal}")


@pytest.mark.parametrize("causal", [False, True], ids=["dense", "causal"])
def test_fwd8_padded_batch(causal):
    """Per-sequence lengths (0, 1, ragged, full) with the padding bytes set to
    0x7F (E4M3 NaN): they are never read, padded O rows are 0 and their LSE
    -inf. Eight heads, so the launch takes the longest-sequence-first order."""
    B, H, N = 4, 8, 400
    lens = torch.tensor([0, 1, 257, 400], dtype=torch.int32)
    c = fp8_case(B, H, N, seed=23 + causal, seqlens=lens)
    for b in range(B):
        L = int(lens[b])
        for name in ("q8", "k8", "v8"):
            c[name][b, :, L:, :] = 0x7F
    o, lse = run(c, 1.0 / math.sqrt(128), causal, seqlens=lens)
    check(c, o, lse, 1.0 / math.sqrt(128), causal, lens, torch.bfloat16,
          f"fp8 fwd padded causal={causal}")


def test_fwd8_many_sequences():
    """More sequences than a wave has lanes (B = 70): the launch takes batch
    order instead of the longest-sequence-first order; lengths include 0, 1,
    a tile edge and N, padding bytes set to 0x7F (E4M3 NaN)."""
    B, H, N = 70, 8, 150
    g = torch.Generator().manual_seed(29)
    lens = torch.randint(0, N + 1, (B,), generator=g, dtype=torch.int64).to(torch.int32)
    lens[:5] = torch.tensor([0, 1, 128, 129, N], dtype=torch.int32)
    c = fp8_case(B, H, N, seed=29, seqlens=lens)
    for b in range(B):
        L = int(lens[b])
        for name in ("q8", "k8", "v8"):
            c[name][b, :, L:, :] = 0x7F
    o, lse = run(c, 1.0 / math.sqrt(128), True, seqlens=lens)
    check(c, o, lse, 1.0 / math.sqrt(128), True, lens, torch.bfloat16, "fp8 fwd B=70 padded")


def test_fwd8_rising_scores_rescale():
    """Scores that rise along the keys (key rows scaled by 1 .. 40 before
    quantisation): later tiles exceed the first tile's reference by far more
    than 8 / (scale log2 e), so the kernel's rescale path runs for most tiles;
    weights stay <= 2^8 and inside E4M3's range."""
    B, H, N = 1, 2, 700
    x = make_inputs(B, H, N, 128, torch.float32, seed=31)
    ramp = torch.linspace(1.0, 40.0, N)[None, None, :, None]
    q = x["q"].abs() * 0.5
    k = x["k"].abs() * ramp
    c = fp8_case(B, H, N, seed=31, q=q, k=k)
    scale = 1.0 / math.sqrt(128)
    for causal in (False, True):
        o, lse = run(c, scale, causal)
        check(c, o, lse, scale, causal, None, torch.bfloat16, f"fp8 fwd rising causal={causal}")


def test_fwd8_token_scales_span_decades():
    """Per-token Q scales over six decades (rows scaled by 10^-3 .. 10^3 before
    quantisation), so the per-query constant folds very different scales."""
    B, H, N = 1, 4, 256
    x = make_inputs(B, H, N, 128, torch.float32, seed=37)
    mag = torch.logspace(-3, 3, N)[None, None, :, None]
    c = fp8_case(B, H, N, seed=37, q=x["q"] * mag * 1e-3)
    scale = 1.0 / math.sqrt(128)
    o, lse = run(c, scale, True)
    check(c, o, lse, scale, True, None, torch.bfloat16, "fp8 fwd token scales")


def test_fwd8_guard_bands_untouched():
    """O and LSE written into the middle of larger buffers: the canaries around
    them keep their bytes."""
    B, H, N = 2, 2, 300
    c = fp8_case(B, H, N, seed=41)
    t = {n: c[n].to(DEV) for n in ("q8", "k8", "v8", "qs", "ks", "vs")}
    n_o, n_l = B * H * N * 128, B * H * N
    big_o = torch.full((n_o + 2048,), 7.0, dtype=torch.bfloat16, device=DEV)
    big_l = torch.full((n_l + 512,), 7.0, dtype=torch.float32, device=DEV)
    o = big_o[1024:1024 + n_o].view(B, H, N, 128)
    lse = big_l[256:256 + n_l].view(B, H, N)
    ea.attn_fwd_fp8(t["q8"], t["k8"], t["v8"], t["qs"], t["ks"], t["vs"], causal=True, out=o, lse=lse)
    torch.cuda.synchronize()
    bo, bl = big_o.float().cpu(), big_l.cpu()
    assert torch.all(bo[:1024] == 7.0) and torch.all(bo[1024 + n_o:] == 7.0)
    assert torch.all(bl[:256] == 7.0) and torch.all(bl[256 + n_l:] == 7.0)
    check(c, o.float().cpu().numpy(), lse.cpu().numpy(), 1.0 / math.sqrt(128), True, None,
          torch.bfloat16, "fp8 fwd guard")


def test_fwd8_workload_sampled_rows():
    """The FP8 benchmark workload at full size (B=2, H=32, N=4096, causal): rows
    sampled from every head (first, last, the 128-row tile edges and random
    ones), each against the oracle row by row with its own bar."""
    B, H, N = 2, 32, 4096
    c = fp8_case(B, H, N, seed=4242)
    scale = 1.0 / math.sqrt(128)
    o, lse = run(c, scale, True)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, 1, 127, 128, 2047, 2048, N - 129, N - 1],
                                     rng.integers(0, N, 8)]))
    worst = 0.0
    for b in range(B):
        for h in range(H):
            qd, kd, vd = c["qd"][b, h], c["kd"][b, h], c["vd"][b, h]
            o_ref, lse_ref, p = oracle.attn_ref_head(qd, kd, vd, scale, True, N, rows=rows,
                                                     return_p=True)
            bound, lse_bar = bars(qd, kd, vd, o_ref, p, rows, scale, True, N,
                                  UNIT_OUT[torch.bfloat16])
            ratio = float((np.abs(o[b, h, rows] - o_ref) / bound).max())
            worst = max(worst, ratio)
            assert ratio <= 1.0, f"workload head ({b},{h}): x{ratio:.2f} over the bar"
            assert np.all(np.abs(lse[b, h, rows] - lse_ref) <= lse_bar)
    log({"what": "fp8 fwd workload sampled", "kind": "fp8_bound_ratio", "o_ratio": worst})
