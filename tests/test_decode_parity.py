"""GPU parity of the split-KV decode (through the C ABI, attn_decode) against the
fp64 oracle's decode (the last Nq positions of each sequence; causal masking
is bottom-right aligned).

Tolerances are the forward's (tests/parity.py): the split kernel computes the
same products and softmax as the forward kernel and the merge is fp32.
Pages cited (by title):
  [SafeSoftmax] "FlashAttention：从 Safe Softmax 到分块计算" (§3.2 merge, §10 split K/V)
  [OpOpt]       "Attention 算子优化:从物化 N×N 矩阵到 FlashAttention 与 PagedAttention" (§五)
"""
import math

import numpy as np
import pytest
import torch

import exact_attention_24_amd as ea
import oracle
from attn_inputs import WORKLOADS, fp8_cache, make_inputs, make_workload_inputs
from tests.parity import LSE_TOL, O_TOL, assert_close, dtype_name, lse_tol

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

# (B, H, H_kv, Nq, Nk, d): one token against a ragged cache; 5 tokens, MHA;
# 4 tokens x group 4 = 16 columns; MQA with 16 heads x 4 tokens = 64 columns
# (two column blocks, one two-wave workgroup); 16 tokens over 129 keys; MQA
# with 32 heads x 4 tokens = 128 columns (two two-wave workgroups); 3 tokens x
# group 32 = 96 columns (three column blocks, one wave each); 44 heads x 4
# tokens = 176 columns (six blocks, the last half full: three two-wave
# workgroups)
SHAPES = [(2, 8, 2, 1, 300, 128), (1, 4, 4, 5, 700, 64), (3, 32, 8, 4, 1000, 128),
          (1, 16, 1, 4, 333, 128), (2, 2, 2, 16, 129, 64), (1, 32, 1, 4, 500, 128),
          (2, 64, 2, 3, 260, 64), (1, 44, 1, 4, 200, 64)]


def run_decode(x, scale, causal, kv_lens=None, num_splits=0):
    q, k, v = (x[n].to(DEV) for n in ("q", "k", "v"))
    kl = kv_lens.to(DEV) if kv_lens is not None else None
    o, lse = ea.attn_decode(q, k, v, scale=scale, causal=causal, kv_lens=kl, num_splits=num_splits)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


@pytest.mark.parametrize("splits", [0, 1, 3])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True], ids=["dense", "causal"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_decode_small(shape, causal, dtype, splits):
    B, H, H_kv, Nq, Nk, d = shape
    x = make_inputs(B, H, Nk, d, dtype, seed=sum(shape) + 7 * causal, H_kv=H_kv, Nq=Nq)
    o, lse = run_decode(x, 1 / math.sqrt(d), causal, num_splits=splits)
    ro, rl = oracle.attn_ref_decode(x["q"], x["k"], x["v"], 1 / math.sqrt(d), causal)
    dn = dtype_name(x["q"])
    assert_close(o, ro, O_TOL[dn], f"decode{shape} O")
    assert_close(lse, rl, LSE_TOL[dn], f"decode{shape} LSE")


@pytest.mark.parametrize("splits", [15, 16, 17, 40], ids=lambda s: f"splits{s}")
def test_decode_merge_blocks(splits):
    """The merge takes the splits in blocks of 16 (every load of a block issued
    before any is used, slots past the last split weighted zero): one block
    minus one slot, exactly one block, one block plus one split, and three
    blocks with the last half full, against the oracle. With per-sequence
    lengths some splits are empty (l = 0) inside a block, and sequence 0 has
    no keys at all."""
    B, H, H_kv, Nq, d = 3, 8, 2, 2, 128
    Nk = 64 * splits  # 64 keys per split, so the plan keeps exactly `splits`
    x = make_inputs(B, H, Nk, d, torch.bfloat16, seed=67 + splits, H_kv=H_kv, Nq=Nq)
    lens = torch.tensor([0, Nk // 2 - 5, Nk], dtype=torch.int32)
    o, lse = run_decode(x, 1 / math.sqrt(d), True, lens, num_splits=splits)
    ro, rl = oracle.attn_ref_decode(x["q"], x["k"], x["v"], 1 / math.sqrt(d), True, lens)
    assert_close(o, ro, O_TOL["bf16"], f"decode merge {splits} O")
    assert_close(lse, rl, LSE_TOL["bf16"], f"decode merge {splits} LSE")
    assert torch.all(o[0] == 0) and torch.all(torch.isneginf(lse[0]))


def test_decode_merge_very_negative_maxima():
    """Every score far below -1e30 (a huge scale on negative dot products):
    each split's running max is about -5.9e33 in log2 units, and the merge
    must still combine all of them (uniform weights: O is the mean of the
    visible V rows, LSE = S + ln L)."""
    B, H, H_kv, Nq, Nk, d = 1, 2, 1, 1, 200, 64
    x = make_inputs(B, H, Nk, d, torch.bfloat16, seed=71, H_kv=H_kv, Nq=Nq)
    x["q"] = torch.full_like(x["q"], 8.0)
    x["k"] = torch.full_like(x["k"], -8.0)
    scale = 1e30
    o, lse = run_decode(x, scale, False, num_splits=3)
    ro, rl = oracle.attn_ref_decode(x["q"], x["k"], x["v"], scale, False)
    assert torch.all(torch.isfinite(lse))
    assert_close(o, ro, O_TOL["bf16"], "very negative maxima O")
    # LSE = -4096e30 + ln 200 in fp32: compare relative to its magnitude
    assert float(((lse.double() - torch.as_tensor(rl)).abs() / torch.as_tensor(rl).abs()).max()) <= 1e-6


@pytest.mark.parametrize("heads", [(8, 2), (32, 2), (64, 2)],
                         ids=["one_wave", "two_waves", "two_workgroups"])
@pytest.mark.parametrize("causal", [False, True], ids=["dense", "causal"])
def test_decode_kv_lens(causal, heads):
    """Per-sequence cache lengths: empty, one key, fewer keys than queries (the
    earliest queries then see nothing under the causal mask), ragged, full.
    With 32 query heads over 2 K/V heads the 64 columns run as one two-wave
    workgroup; with 64 heads, 128 columns, as two."""
    H, H_kv = heads
    B, Nq, Nk, d = 6, 4, 500, 128
    x = make_inputs(B, H, Nk, d, torch.bfloat16, seed=61 + causal, H_kv=H_kv, Nq=Nq)
    lens = torch.tensor([0, 1, 3, 257, 500, 64], dtype=torch.int32)
    o, lse = run_decode(x, 1 / math.sqrt(d), causal, lens, num_splits=4)
    ro, rl = oracle.attn_ref_decode(x["q"], x["k"], x["v"], 1 / math.sqrt(d), causal, lens)
    assert_close(o, ro, O_TOL["bf16"], "decode kv_lens O")
    assert_close(lse, rl, LSE_TOL["bf16"], "decode kv_lens LSE")
    assert torch.all(o[0] == 0) and torch.all(torch.isneginf(lse[0]))


def test_decode_matches_forward_rows():
    """With Nq = Nk the decode is the causal forward; for Nq < Nk its rows are
    the forward's last Nq rows (same products; agreement within the bf16 O
    tolerance, the two kernels round differently)."""
    B, H, N, d = 2, 4, 256, 128
    x = make_inputs(B, H, N, d, torch.bfloat16, seed=62)
    o_f, l_f = ea.attn_fwd(x["q"].to(DEV), x["k"].to(DEV), x["v"].to(DEV), causal=True)
    qd = x["q"][:, :, N - 8:].contiguous()
    o_d, l_d = run_decode({"q": qd, "k": x["k"], "v": x["v"]}, 1 / math.sqrt(d), True)
    assert_close(o_d, o_f[:, :, N - 8:].cpu().double().numpy(), O_TOL["bf16"], "decode vs fwd O")
    assert_close(l_d, l_f[:, :, N - 8:].cpu().double().numpy(), LSE_TOL["bf16"], "decode vs fwd LSE")


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8kv"])
def test_decode_rising_scores(fp8):
    """Scores grow by 8 per 32-key chunk (11.5 in log2 units, above the 2^8
    weight bound), so every chunk of every split moves the reference max and
    rescales its partial state before the merge."""
    B, H, H_kv, Nq, Nk, d = 2, 8, 2, 3, 700, 128
    x = make_inputs(B, H, Nk, d, torch.bfloat16, seed=93, H_kv=H_kv, Nq=Nq, std=0.05)
    q, k = x["q"].float(), x["k"].float()
    q[..., 0] = 1.0
    k[..., 0] = 0.25 * torch.arange(Nk, dtype=torch.float32)
    x["q"], x["k"] = q.to(torch.bfloat16), k.to(torch.bfloat16)
    x["v"] = make_inputs(B, H, Nk, d, torch.bfloat16, seed=94, H_kv=H_kv, Nq=Nq)["v"]
    if fp8:
        k8, v8, ks, vs, kd, vd = _fp8_case(x)
        o, lse = run_decode_fp8(x["q"], k8, v8, ks, vs, 1.0, True, num_splits=3)
        ro, rl = oracle.attn_ref_decode(x["q"], kd, vd, 1.0, True)
        kk = torch.from_numpy(kd)
    else:
        o, lse = run_decode(x, 1.0, True, num_splits=3)
        ro, rl = oracle.attn_ref_decode(x["q"], x["k"], x["v"], 1.0, True)
        kk = x["k"]
    assert_close(o, ro, O_TOL["bf16"], "rising decode O")
    assert_close(lse, rl, lse_tol("bf16", x["q"], kk, 1.0), "rising decode LSE")


def test_decode_split_invariance():
    """The split count changes only the rounding of the merge."""
    x = make_inputs(2, 8, 3000, 128, torch.bfloat16, seed=63, H_kv=2, Nq=2)
    a = run_decode(x, 0.088, True, num_splits=1)
    b = run_decode(x, 0.088, True, num_splits=0)
    c = run_decode(x, 0.088, True, num_splits=40)
    for other in (b, c):
        assert float((a[0].float() - other[0].float()).abs().max()) <= 2 * 2 ** -8
        assert float((a[1] - other[1]).abs().max()) <= 1e-4


@pytest.mark.parametrize("name", [n for n, w in WORKLOADS.items() if w.Nq is not None and not w.kv_fp8])
def test_decode_workload_full(name):
    """The decode workloads at full size, as the benchmark runs them: every O
    and LSE entry of every (batch, head) against the oracle."""
    w = WORKLOADS[name]
    x = make_workload_inputs(w)
    o, lse = run_decode(x, w.scale, w.causal, x["seqlens"])
    assert torch.isfinite(o).all()
    ro, rl = oracle.attn_ref_decode(x["q"], x["k"], x["v"], w.scale, w.causal, x["seqlens"])
    assert_close(o, ro, O_TOL["bf16"], f"{name} O")
    assert_close(lse, rl, LSE_TOL["bf16"], f"{name} LSE")


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8kv"])
def test_decode_guard_band_untouched(fp8):
    """O and LSE live inside larger buffers filled with a sentinel: nothing
    outside them may be written, and the values are still right."""
    B, H, H_kv, Nq, Nk, d = 2, 16, 2, 3, 517, 128
    x = make_inputs(B, H, Nk, d, torch.bfloat16, seed=17 + fp8, H_kv=H_kv, Nq=Nq)
    n, nl = B * H * Nq * d, B * H * Nq
    obuf = torch.full((n + 8192,), -7.0, dtype=torch.bfloat16, device=DEV)
    lbuf = torch.full((nl + 512,), -7.0, dtype=torch.float32, device=DEV)
    o = obuf[4096:4096 + n].view(B, H, Nq, d)
    lse = lbuf[256:256 + nl].view(B, H, Nq)
    q = x["q"].to(DEV)
    if fp8:
        k8, v8, ks, vs, kd, vd = _fp8_case(x)
        ea.attn_decode_fp8kv(q, k8.to(DEV), v8.to(DEV), ks.to(DEV), vs.to(DEV), causal=True,
                             num_splits=3, out=o, lse=lse)
        ro, rl = oracle.attn_ref_decode(x["q"], kd, vd, 1 / math.sqrt(d), True)
    else:
        ea.attn_decode(q, x["k"].to(DEV), x["v"].to(DEV), causal=True, num_splits=3, out=o, lse=lse)
        ro, rl = oracle.attn_ref_decode(x["q"], x["k"], x["v"], 1 / math.sqrt(d), True)
    torch.cuda.synchronize()
    assert torch.all(obuf[:4096] == -7.0) and torch.all(obuf[4096 + n:] == -7.0), "O guard band written"
    assert torch.all(lbuf[:256] == -7.0) and torch.all(lbuf[256 + nl:] == -7.0), "LSE guard band written"
    assert_close(o.cpu(), ro, O_TOL["bf16"], "guard-band decode O")
    assert_close(lse.cpu(), rl, LSE_TOL["bf16"], "guard-band decode LSE")


# ------------------------------------------------------------- FP8 K/V cache

def run_decode_fp8(q, k8, v8, ks, vs, scale, causal, kv_lens=None, num_splits=0):
    t = [x.to(DEV) for x in (q, k8, v8, ks, vs)]
    kl = kv_lens.to(DEV) if kv_lens is not None else None
    o, lse = ea.attn_decode_fp8kv(*t, scale=scale, causal=causal, kv_lens=kl, num_splits=num_splits)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def _fp8_case(x):
    k8, ks = fp8_cache(x["k"])
    v8, vs = fp8_cache(x["v"])
    return k8, v8, ks, vs, oracle.dequant_fp8(k8, ks), oracle.dequant_fp8(v8, vs)


# (B, H, H_kv, Nq, Nk, d)
FP8_SHAPES = [(2, 8, 2, 1, 300, 128), (1, 16, 1, 4, 333, 128), (2, 4, 4, 3, 700, 128),
              (1, 8, 8, 16, 129, 128), (2, 8, 2, 1, 300, 64), (1, 16, 1, 4, 333, 64),
              (2, 4, 4, 3, 700, 64), (1, 32, 1, 4, 250, 128)]


@pytest.mark.parametrize("splits", [0, 3])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True], ids=["dense", "causal"])
@pytest.mark.parametrize("shape", FP8_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_decode_fp8kv_small(shape, causal, dtype, splits):
    """FP8 (E4M3, per-token scale) K/V: the oracle attends over the dequantised
    cache in fp64; the bar is the 16-bit path's (the FP8 values are exact on
    chip, the scales are applied in fp32)."""
    B, H, H_kv, Nq, Nk, d = shape
    x = make_inputs(B, H, Nk, d, dtype, seed=sum(shape) + 5 * causal, H_kv=H_kv, Nq=Nq)
    k8, v8, ks, vs, kd, vd = _fp8_case(x)
    o, lse = run_decode_fp8(x["q"], k8, v8, ks, vs, 1 / math.sqrt(d), causal, num_splits=splits)
    ro, rl = oracle.attn_ref_decode(x["q"], kd, vd, 1 / math.sqrt(d), causal)
    dn = dtype_name(x["q"])
    assert_close(o, ro, O_TOL[dn], f"fp8 decode{shape} O")
    assert_close(lse, rl, LSE_TOL[dn], f"fp8 decode{shape} LSE")


def test_decode_fp8kv_lens_and_scales():
    """Cache lengths 0..Nk and per-token scales spanning six orders of magnitude
    (rows scaled by 10^-3 .. 10^3 before quantisation)."""
    B, H, H_kv, Nq, Nk = 4, 8, 2, 2, 400
    x = make_inputs(B, H, Nk, 128, torch.bfloat16, seed=71, H_kv=H_kv, Nq=Nq)
    mag = torch.logspace(-3, 3, Nk)[None, None, :, None]
    x["k"] = (x["k"].float() * mag).to(torch.bfloat16)
    x["v"] = (x["v"].float() * mag.flip(2)).to(torch.bfloat16)
    k8, v8, ks, vs, kd, vd = _fp8_case(x)
    lens = torch.tensor([0, 1, 250, 400], dtype=torch.int32)
    q = (x["q"].float() * 1e-3).to(torch.bfloat16)  # keep scores O(1) against |K| up to 10^3
    o, lse = run_decode_fp8(q, k8, v8, ks, vs, 1 / math.sqrt(128), True, lens, num_splits=5)
    ro, rl = oracle.attn_ref_decode(q, kd, vd, 1 / math.sqrt(128), True, lens)
    scale_v = float(np.abs(vd).max())
    assert_close(o, ro, O_TOL["bf16"] * scale_v, "fp8 decode lens O")
    assert_close(lse, rl, LSE_TOL["bf16"], "fp8 decode lens LSE")


def test_decode_fp8kv_f16_large_value_scale():
    """fp16 queries over an FP8 cache whose value scale reaches ~450 (one V entry
    of 2e5 in one token, the rest small): the per-token scale multiplies the
    softmax weight before the weight is rounded to fp16, so the weight must
    stay <= 1 (exact running max) for weight * scale to stay finite. That
    token's key scores 5.3 above the rest (weight e^5.3 ~ 200 against ~700
    others of ~1), so it carries a weight fraction of about 0.22 and O stays
    inside fp16's range."""
    B, H, H_kv, Nq, Nk, d = 1, 8, 2, 1, 700, 128
    x = make_inputs(B, H, Nk, d, torch.float16, seed=73, H_kv=H_kv, Nq=Nq, std=0.05)
    q, k, v = x["q"].float(), x["k"].float(), x["v"].float()
    q[..., 0] = 1.0
    big = [400]
    k[:, :, big, 0] = 5.3
    v[:, :, big, 5] = 2.0e5
    # the cache is built from the fp32 values (2e5 is beyond fp16's range; the
    # cache format does not depend on the query format)
    x["q"], x["k"], x["v"] = q.to(torch.float16), k.to(torch.float16), v
    k8, v8, ks, vs, kd, vd = _fp8_case(x)
    assert float(vs.max()) > 256.0
    o, lse = run_decode_fp8(x["q"], k8, v8, ks, vs, 1.0, False, num_splits=2)
    ro, rl = oracle.attn_ref_decode(x["q"], kd, vd, 1.0, False)
    assert np.abs(ro).max() < 65504
    assert torch.isfinite(o).all(), "weight x value scale overflowed fp16"
    # absolute bar scaled by the largest |V| (the fp16 rounding of O and of the
    # weights is relative to it)
    assert_close(o, ro, O_TOL["f16"] * float(np.abs(vd).max()), "fp16 large v_scale O")
    assert_close(lse, rl, lse_tol("f16", x["q"], torch.from_numpy(kd), 1.0), "fp16 large v_scale LSE")


def test_decode_fp8kv_workload_full():
    """The FP8 decode workload at full size (B=8, 64 query heads over 8 K/V
    heads, 8192 cached positions, one new token), as the benchmark runs it:
    every O and LSE entry against the oracle over the dequantised cache."""
    w = WORKLOADS["decode_fp8kv_bf16_b8_h64_hkv8_nq1_nk8192_d128"]
    x = make_workload_inputs(w)
    k8, v8, ks, vs, kd, vd = _fp8_case(x)
    o, lse = run_decode_fp8(x["q"], k8, v8, ks, vs, w.scale, w.causal)
    assert torch.isfinite(o).all()
    ro, rl = oracle.attn_ref_decode(x["q"], kd, vd, w.scale, w.causal)
    assert_close(o, ro, O_TOL["bf16"], "fp8 workload O")
    assert_close(lse, rl, LSE_TOL["bf16"], "fp8 workload LSE")
