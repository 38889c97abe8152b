"""GPU test of attn_bwd_noalloc, the backward entry point that allocates
nothing (its workspace is the library's static device scratch), called
through the C ABI and compared with attn_bwd_gqa, which takes a caller-
allocated workspace: two calls in a row, the second on a smaller input, must
give bit-identical gradients (the same kernels run on the same statistics)."""
import ctypes
import math

import pytest
import torch

import exact_attention_24_amd as ea
from attn_inputs import make_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

# (B, H, H_kv, N, d, causal, seqlens): the second case is smaller in every
# size, so it reads only scratch entries its own pre-pass wrote.
CASES = [(2, 8, 4, 700, 128, True, None),
         (1, 2, 2, 150, 64, False, [150])]


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr() if t is not None else 0)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
def test_noalloc_matches_workspace_entry(dtype):
    lib = ea.lib()
    code = ea.DTYPE_BF16 if dtype == torch.bfloat16 else ea.DTYPE_F16
    for i, (B, H, H_kv, N, d, causal, lens) in enumerate(CASES):
        print(f"noalloc case {i}: B={B} H={H} H_kv={H_kv} N={N} d={d} causal={causal}", flush=True)
        x = make_inputs(B, H, N, d, dtype, seed=600 + i, with_grad=True, H_kv=H_kv)
        q, k, v, do = (x[n].to(DEV) for n in ("q", "k", "v", "do"))
        sl = torch.tensor(lens, dtype=torch.int32, device=DEV) if lens is not None else None
        scale = 1 / math.sqrt(d)
        o, lse = ea.attn_fwd(q, k, v, scale=scale, causal=causal, seqlens=sl)
        want = ea.attn_bwd(q, k, v, o, do, lse, scale=scale, causal=causal, seqlens=sl)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        st = lib.attn_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse),
                                  _ptr(dq), _ptr(dk), _ptr(dv), B, H, H_kv, N, d, code,
                                  ctypes.c_float(scale), int(causal), _ptr(sl), stream)
        assert st == 0, (st, lib.attn_last_error())
        torch.cuda.synchronize()
        for name, a, b in zip(("dQ", "dK", "dV"), (dq, dk, dv), want):
            assert torch.isfinite(a).all(), f"case {i} {name}: non-finite"
            assert torch.equal(a, b), f"case {i} {name}: differs from attn_bwd_gqa"


def test_noalloc_rejects_oversize():
    """More query rows than the static scratch holds: rejected on the host with
    ATTN_ERR_UNSUPPORTED and a message naming the limit; nothing is launched
    (the pointers are never touched)."""
    lib = ea.lib()
    P = ctypes.c_void_p(0x10000)
    st = lib.attn_bwd_noalloc(P, P, P, P, P, P, P, P, P, 1, 64, 64, 32769, 128, ea.DTYPE_BF16,
                              ctypes.c_float(0.088), 1, None, None)
    assert st == 2
    assert b"limit" in lib.attn_last_error()
