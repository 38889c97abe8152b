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
from tests.parity import (LSE_TOL, O_TOL, assert_close, check_grad, check_grads, dtype_name,
                          GRAD_BLOCK_TOL, GRAD_TOL, rel_fro, to_np)

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
    check_grads(got, ref, f"GQA{shape}")


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
    check_grads((dq, dk, dv), ref, "GQA varlen")
    for b, L in enumerate(x["seqlens"].tolist()):
        assert torch.all(dq[b, :, L:] == 0) and torch.all(dk[b, :, L:] == 0)
        assert torch.all(dv[b, :, L:] == 0)


def test_gqa_workload_kv_heads():
    """The grouped-query workload at full size (B=2, H=32 over H_kv=8, N=4096,
    d=128, causal), forward and backward in one pass: every O and LSE entry,
    and for eight K/V heads (one per XCD residue of the dK/dV kernel's head
    index) the summed dK, dV and the dQ of their four query heads, per tensor
    and per 64-row block."""
    import concurrent.futures
    from tests.parity import oracle_fwd_threads
    w = WORKLOADS["gqa_causal_bf16_b2_h32_hkv8_n4096_d128"]
    x = make_workload_inputs(w)
    o, lse, dq, dk, dv = _run(x, w.scale, w.causal, grad=True)
    for t in (o, dq, dk, dv):
        assert torch.isfinite(t).all()
    ro, rl = oracle_fwd_threads(x["q"], x["k"], x["v"], w.scale, w.causal)
    assert_close(o, ro, O_TOL["bf16"], "GQA workload O")
    assert_close(lse, rl, LSE_TOL["bf16"], "GQA workload LSE")
    G = w.H // w.kv_heads
    kv_heads = [divmod(bkv, w.kv_heads) for bkv in (0, 9, 2, 11, 4, 13, 6, 15)]
    assert len({(b * w.kv_heads + g) % 8 for b, g in kv_heads}) == 8
    q, k, v, do = (to_np(x[n]) for n in ("q", "k", "v", "do"))
    jobs = [(b, g, h) for b, g in kv_heads for h in range(g * G, (g + 1) * G)]

    def one(job):
        b, g, h = job
        return oracle.attn_ref_bwd_head(q[b, h], k[b, g], v[b, g], do[b, h], w.scale, w.causal)

    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        ref = dict(zip(jobs, ex.map(one, jobs)))
    for b, g in kv_heads:
        rdk = sum(ref[(b, g, h)][1] for h in range(g * G, (g + 1) * G))
        rdv = sum(ref[(b, g, h)][2] for h in range(g * G, (g + 1) * G))
        for h in range(g * G, (g + 1) * G):
            check_grad(dq[b, h], ref[(b, g, h)][0], GRAD_TOL["bf16"], GRAD_BLOCK_TOL["bf16"],
                       f"GQA workload dQ head ({b},{h})")
        check_grad(dk[b, g], rdk, GRAD_TOL["bf16"], GRAD_BLOCK_TOL["bf16"], f"GQA workload dK ({b},{g})")
        check_grad(dv[b, g], rdv, GRAD_TOL["bf16"], GRAD_BLOCK_TOL["bf16"], f"GQA workload dV ({b},{g})")


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
