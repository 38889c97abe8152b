"""GPU parity at sizes whose tensors hold more than 2^31 elements (bytes, for
FP8): every offset past the 32-bit range must reach its own element. Each
test runs one launch configuration of the benchmark shape scaled up in heads
(or batch), then checks heads on both sides of the 2^31-element mark against
the fp64 oracle: sampled rows for the forwards and the decode, whole heads
for the backward, with the bars of the other parity tests.

Inputs are drawn on the device (attn_inputs.make_inputs_device); the oracle
reads host copies of the heads it checks.
"""
import math

import numpy as np
import pytest
import torch

import exact_attention_24_amd as ea
import oracle
from attn_inputs import fp8_cache, fp8_head, make_inputs_device
from tests.parity import LSE_TOL, O_TOL, assert_close, check_grads
from tests.test_fwd8_parity import UNIT_OUT, bars

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

# 2 x 2080 heads of 4096 x 128: 2,181,038,080 elements per tensor. Head
# (b, h) starts at element (b * 2080 + h) * 4096 * 128, past 2^31 from
# (1, 2016) on.
B, H, N, D = 2, 2080, 4096, 128
HEADS = [(0, 0), (0, 1000), (1, 2016), (1, H - 1)]
ROWS = [0, 1, 127, 128, 2047, 2048, N - 129, N - 1]
SCALE = 1.0 / math.sqrt(D)


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _head(t, b, h):
    return t[b:b + 1, h:h + 1].cpu()


def test_sizes_cross_2g_elements():
    assert B * H * N * D > 2 ** 31
    assert (1 * H + 2016) * N * D >= 2 ** 31 > (1 * H + 2015) * N * D
    assert (8 * 63 + 5) * DNK * D >= 2 ** 31 > (8 * 63 + 4) * DNK * D


def test_fwd_beyond_2g_elements():
    x = make_inputs_device(B, H, N, D, torch.bfloat16, seed=9101, device=DEV)
    o, lse = ea.attn_fwd(x["q"], x["k"], x["v"], scale=SCALE, causal=True)
    torch.cuda.synchronize()
    for b, h in HEADS:
        print(f"fwd head ({b}, {h})", flush=True)
        q1, k1, v1 = (_head(x[n], b, h) for n in ("q", "k", "v"))
        ro, rl = oracle.attn_ref_rows(q1, k1, v1, 0, 0, ROWS, SCALE, True)
        assert_close(o[b, h, ROWS].cpu(), ro, O_TOL["bf16"], f">2^31 fwd O ({b},{h})")
        assert_close(lse[b, h, ROWS].cpu(), rl, LSE_TOL["bf16"], f">2^31 fwd LSE ({b},{h})")
    del x, o, lse
    _free()


def test_bwd_beyond_2g_elements():
    x = make_inputs_device(B, H, N, D, torch.bfloat16, seed=9102, device=DEV, with_grad=True)
    o, lse = ea.attn_fwd(x["q"], x["k"], x["v"], scale=SCALE, causal=True)
    dq, dk, dv = ea.attn_bwd(x["q"], x["k"], x["v"], o, x["do"], lse, scale=SCALE, causal=True)
    torch.cuda.synchronize()
    for b, h in [HEADS[0], HEADS[-1]]:
        print(f"bwd head ({b}, {h})", flush=True)
        q1, k1, v1, do1 = (_head(x[n], b, h)[0, 0] for n in ("q", "k", "v", "do"))
        ref = oracle.attn_ref_bwd_head(q1, k1, v1, do1, SCALE, True)
        got = tuple(_head(t, b, h)[0, 0] for t in (dq, dk, dv))
        check_grads(got, ref, f">2^31 bwd ({b},{h})", "bf16")
    del x, o, lse, dq, dk, dv
    _free()


def test_fwd_fp8_beyond_2g_bytes():
    x = make_inputs_device(B, H, N, D, torch.float32, seed=9103, device=DEV)
    q8, qs = fp8_cache(x["q"])
    k8, ks = fp8_head(x["k"])
    v8, vs = fp8_head(x["v"])
    del x
    _free()
    o, lse = ea.attn_fwd_fp8(q8, k8, v8, qs, ks, vs, scale=SCALE, causal=True,
                             out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    rows = np.asarray(ROWS)
    for b, h in HEADS:
        print(f"fp8 fwd head ({b}, {h})", flush=True)
        qd = oracle.dequant_fp8(q8[b, h].cpu(), qs[b, h].cpu())
        kd = oracle.dequant_fp8(k8[b, h].cpu(), ks[b, h].cpu().expand(N))
        vd = oracle.dequant_fp8(v8[b, h].cpu(), vs[b, h].cpu().expand(N))
        o_ref, lse_ref, p = oracle.attn_ref_head(qd, kd, vd, SCALE, True, N, rows=rows,
                                                 return_p=True)
        bound, lse_bar = bars(qd, kd, vd, o_ref, p, rows, SCALE, True, N,
                              UNIT_OUT[torch.bfloat16])
        got = o[b, h, ROWS].float().cpu().numpy()
        ratio = float((np.abs(got - o_ref) / bound).max())
        assert ratio <= 1.0, f">2^31 FP8 fwd head ({b},{h}): x{ratio:.2f} over the bar"
        assert np.all(np.abs(lse[b, h, ROWS].cpu().numpy() - lse_ref) <= lse_bar)
    del q8, k8, v8, qs, ks, vs, o, lse
    _free()


# Decode: 64 sequences, 8 K/V heads of 33000 cached positions: 2,162,688,000
# elements per cache tensor; sequence b's K/V head g starts at element
# (8 b + g) * 33000 * 128, past 2^31 from (63, 5) on (query heads 40-47).
DB, DH, DHKV, DNK = 64, 64, 8, 33000
DEC_HEADS = [(0, 0), (31, 17), (63, 40), (63, DH - 1)]


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8kv"])
def test_decode_beyond_2g_elements(fp8):
    assert DB * DHKV * DNK * D > 2 ** 31
    x = make_inputs_device(DB, DH, DNK, D, torch.bfloat16, seed=9104 + fp8, device=DEV,
                           H_kv=DHKV, Nq=1)
    if fp8:
        k8, ks = fp8_cache(x["k"])
        v8, vs = fp8_cache(x["v"])
        del x["k"], x["v"]
        _free()
        o, lse = ea.attn_decode_fp8kv(x["q"], k8, v8, ks, vs, scale=SCALE, causal=True)
    else:
        o, lse = ea.attn_decode(x["q"], x["k"], x["v"], scale=SCALE, causal=True)
    torch.cuda.synchronize()
    for b, h in DEC_HEADS:
        print(f"decode{'/fp8' if fp8 else ''} head ({b}, {h})", flush=True)
        g = oracle.kv_head(h, DH, DHKV)
        if fp8:
            kd = oracle.dequant_fp8(k8[b:b + 1, g:g + 1].cpu(), ks[b:b + 1, g:g + 1].cpu())
            vd = oracle.dequant_fp8(v8[b:b + 1, g:g + 1].cpu(), vs[b:b + 1, g:g + 1].cpu())
        else:
            kd, vd = _head(x["k"], b, g), _head(x["v"], b, g)
        ro, rl = oracle.attn_ref_decode(_head(x["q"], b, h), kd, vd, SCALE, True)
        assert_close(o[b, h].cpu(), ro[0, 0], O_TOL["bf16"], f">2^31 decode O ({b},{h})")
        assert_close(lse[b, h].cpu(), rl[0, 0], LSE_TOL["bf16"], f">2^31 decode LSE ({b},{h})")
    del x, o, lse
    if fp8:
        del k8, v8, ks, vs
    _free()
