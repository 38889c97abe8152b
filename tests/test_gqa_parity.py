"""GPU parity of grouped- and multi-query attention (K/V with fewer heads than Q)
through the C ABI (attn_fwd_gqa, attn_bwd_gqa) against the fp64 oracle.

Query head h reads K/V head h // (H // H_kv); a K/V head's dK, dV sum the
gradients of its group. Tolerances are those of the plain-attention parity
tests (tests/parity.py).
Pages cited (by title):
  [OpOpt] "Attention 算子优化:从物化 N×N 矩阵到 FlashAttention 与 PagedAttention" (§五)
"""
import math

import numpy as np
import pytest
import torch

import exact_attention_24_amd as ea
import oracle
from attn_inputs import WORKLOADS, make_inputs, make_workload_inputs
from tests.parity import (GRAD_REL_FRO, GRAD_TOL, GRAD_ZERO_ABS, LSE_TOL, O_TOL, assert_close,
                          dtype_name, rel_fro, to_np)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

# (B, H, H_kv, N, d): group sizes 3, 4 (multi-query), 2 and 2, ragged lengths
SHAPES = [(2, 6, 2, 200, 128), (1, 4, 1, 130, 64), (2, 8, 4, 77, 64), (1, 2, 1, 333, 128)]


def _run(x, scale, causal, grad):
    q, k, v = (x[n].to(DEV) for n in ("q", "k", "v"))
    sl = x["seqlens"].to(DEV) if x["seqlens"] is not None else None
    o, lse = ea.attn_fwd(q, k, v, scale=scale, causal=causal, seqlens=sl)
    out = [o, lse]
    if grad:
        out += list(ea.attn_bwd(q, k, v, o, x["do"].to(DEV), lse, scale=scale, causal=causal,
                                seqlens=sl))
    torch.cuda.synchronize()
    return [t.cpu() for t in out]


def _check_grads(got, ref, tag, tol=GRAD_REL_FRO):
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        assert torch.isfinite(g).all(), f"{tag} {name}: non-finite gradient"
        if not np.any(to_np(r)):
            assert float(g.abs().max()) <= GRAD_ZERO_ABS, f"{tag} {name}: exact gradient is 0"
            continue
        e = rel_fro(g, r)
        assert e <= tol, f"{tag} {name}: rel Frobenius err {e:.3e} > {tol}"


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32, torch.float16],
                         ids=["bf16", "f32", "f16"])
@pytest.mark.parametrize("causal", [False, True], ids=["dense", "causal"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_gqa_forward(shape, causal, dtype):
    B, H, H_kv, N, d = shape
    x = make_inputs(B, H, N, d, dtype, seed=sum(shape) + causal, H_kv=H_kv)
    o, lse = _run(x, 1 / math.sqrt(d), causal, grad=False)
    ro, rl = oracle.attn_ref_fwd(x["q"], x["k"], x["v"], 1 / math.sqrt(d), causal)
    dn = dtype_name(x["q"])
    assert_close(o, ro, O_TOL[dn], f"GQA{shape} O")
    assert_close(lse, rl, LSE_TOL[dn], f"GQA{shape} LSE")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True], ids=["dense", "causal"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_gqa_backward(shape, causal, dtype):
    B, H, H_kv, N, d = shape
    x = make_inputs(B, H, N, d, dtype, seed=100 + sum(shape) + causal, with_grad=True,
                    H_kv=H_kv)
    got = _run(x, 1 / math.sqrt(d), causal, grad=True)[2:]
    assert got[1].shape == x["k"].shape and got[2].shape == x["v"].shape
    ref = oracle.attn_ref_bwd(x["q"], x["k"], x["v"], x["do"], 1 / math.sqrt(d), causal)
    _check_grads(got, ref, f"GQA{shape}", GRAD_TOL[dtype_name(x["q"])])


@pytest.mark.parametrize("causal", [False, True], ids=["dense", "causal"])
def test_gqa_varlen(causal):
    """Padded batch with grouped heads: lengths 0, 1, ragged, a tile multiple and N."""
    B, H, H_kv, N, d = 5, 4, 2, 290, 128
    x = make_inputs(B, H, N, d, torch.bfloat16, seed=90 + causal, with_grad=True, H_kv=H_kv)
    x["seqlens"] = torch.tensor([0, 1, 200, 128, N], dtype=torch.int32)
    o, lse, dq, dk, dv = _run(x, 1 / math.sqrt(d), causal, grad=True)
    ro, rl = oracle.attn_ref_fwd(x["q"], x["k"], x["v"], 1 / math.sqrt(d), causal, x["seqlens"])
    assert_close(o, ro, O_TOL["bf16"], "GQA varlen O")
    assert_close(lse, rl, LSE_TOL["bf16"], "GQA varlen LSE")
    ref = oracle.attn_ref_bwd(x["q"], x["k"], x["v"], x["do"], 1 / math.sqrt(d), causal,
                              x["seqlens"])
    _check_grads((dq, dk, dv), ref, "GQA varlen")
    for b, L in enumerate(x["seqlens"].tolist()):
        assert torch.all(dq[b, :, L:] == 0) and torch.all(dk[b, :, L:] == 0)
        assert torch.all(dv[b, :, L:] == 0)


def test_gqa_workload_sampled_kv_head():
    """The grouped-query workload at full size (B=2, H=32 over H_kv=8, N=4096,
    d=128, causal), forward and backward in one pass; the oracle recomputes the
    four query heads of one K/V head and that head's summed dK, dV."""
    w = WORKLOADS["gqa_causal_bf16_b2_h32_hkv8_n4096_d128"]
    x = make_workload_inputs(w)
    o, lse, dq, dk, dv = _run(x, w.scale, w.causal, grad=True)
    for t in (o, dq, dk, dv):
        assert torch.isfinite(t).all()
    b, g = 1, 5
    G = w.H // w.kv_heads
    rdk = np.zeros((w.N, w.d))
    rdv = np.zeros((w.N, w.d))
    for h in range(g * G, (g + 1) * G):
        rdq, dk_h, dv_h = oracle.attn_ref_bwd_head(x["q"][b, h], x["k"][b, g], x["v"][b, g],
                                                   x["do"][b, h], w.scale, w.causal)
        rdk += dk_h
        rdv += dv_h
        e = rel_fro(dq[b, h], rdq)
        assert e <= GRAD_REL_FRO, f"dQ head {h}: {e:.3e}"
    for name, got, ref in (("dK", dk[b, g], rdk), ("dV", dv[b, g], rdv)):
        e = rel_fro(got, ref)
        assert e <= GRAD_REL_FRO, f"{name} K/V head {g}: {e:.3e}"


def test_gqa_matches_repeated_heads():
    """Grouped K/V heads give the same forward bits as plain attention over K/V
    repeated per group (the same kernels read the same K/V rows), and the
    grouped dK, dV match the group sums of the plain backward within rounding
    of the sum order."""
    B, H, H_kv, N, d = 2, 8, 2, 300, 128
    x = make_inputs(B, H, N, d, torch.bfloat16, seed=95, with_grad=True, H_kv=H_kv)
    rep = dict(x)
    rep["k"] = x["k"].repeat_interleave(H // H_kv, dim=1).contiguous()
    rep["v"] = x["v"].repeat_interleave(H // H_kv, dim=1).contiguous()
    a = _run(x, 1 / math.sqrt(d), True, grad=True)
    r = _run(rep, 1 / math.sqrt(d), True, grad=True)
    assert torch.equal(a[0], r[0]) and torch.equal(a[1], r[1])
    assert torch.equal(a[2], r[2])  # dQ: same per-head computation
    for i in (3, 4):
        summed = r[i].double().view(B, H_kv, H // H_kv, N, d).sum(dim=2)
        e = rel_fro(a[i], summed)
        assert e <= 1e-2, f"grouped vs summed plain gradient: {e:.3e}"
