"""The C-ABI calls under HIP graph capture (torch.cuda.CUDAGraph): they enqueue
kernels on the caller's stream only, allocate nothing and never synchronise, so a
captured forward, backward or decode replays like the eager call. Each graph is
replayed several times with new input contents copied into its static buffers
between replays (ordinary eager work in between), and every replay is compared
bit for bit with an eager call on the same data (same kernels, same inputs)."""
import math

import pytest
import torch

import exact_attention_24_amd as ea
from attn_inputs import fp8_cache, make_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _capture(fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # warm-up on the side stream, as torch recommends before capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def test_forward_backward_graph_replays():
    B, H, N, d = 2, 4, 333, 128
    scale = 1 / math.sqrt(d)
    x = make_inputs(B, H, N, d, torch.bfloat16, seed=201, with_grad=True)
    q, k, v, do = (x[n].to(DEV) for n in ("q", "k", "v", "do"))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=DEV)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(ea.attn_bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=DEV)

    def step():
        ea.attn_fwd(q, k, v, scale=scale, causal=True, out=o, lse=lse)
        ea.attn_bwd(q, k, v, o, do, lse, scale=scale, causal=True, dq=dq, dk=dk, dv=dv,
                    workspace=ws)

    g = _capture(step)
    for r in range(3):
        y = make_inputs(B, H, N, d, torch.bfloat16, seed=300 + r, with_grad=True)
        for dst, n in ((q, "q"), (k, "k"), (v, "v"), (do, "do")):
            dst.copy_(y[n].to(DEV))
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (o, lse, dq, dk, dv)]
        ro, rl = ea.attn_fwd(q, k, v, scale=scale, causal=True)
        rdq, rdk, rdv = ea.attn_bwd(q, k, v, ro, do, rl, scale=scale, causal=True)
        torch.cuda.synchronize()
        for name, a, b in zip(("O", "LSE", "dQ", "dK", "dV"), got, (ro, rl, rdq, rdk, rdv)):
            assert torch.equal(a, b), f"replay {r}: {name} differs from the eager call"


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8kv"])
def test_decode_graph_replays(fp8):
    B, H, H_kv, Nq, Nk, d = 4, 32, 2, 4, 1000, 128
    x = make_inputs(B, H, Nk, d, torch.bfloat16, seed=211, H_kv=H_kv, Nq=Nq)
    q = x["q"].to(DEV)
    lens = torch.tensor([1000, 1, 517, 0], dtype=torch.int32, device=DEV)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=DEV)
    ws = torch.empty(ea.attn_decode_workspace_bytes(B, H, H_kv, Nq, Nk, d), dtype=torch.uint8,
                     device=DEV)
    if fp8:
        k8, ks = (t.to(DEV) for t in fp8_cache(x["k"]))
        v8, vs = (t.to(DEV) for t in fp8_cache(x["v"]))
        call = lambda **kw: ea.attn_decode_fp8kv(q, k8, v8, ks, vs, causal=True, kv_lens=lens, **kw)
    else:
        k, v = x["k"].to(DEV), x["v"].to(DEV)
        call = lambda **kw: ea.attn_decode(q, k, v, causal=True, kv_lens=lens, **kw)

    g = _capture(lambda: call(out=o, lse=lse, workspace=ws))
    for r in range(3):
        y = make_inputs(B, H, Nk, d, torch.bfloat16, seed=400 + r, H_kv=H_kv, Nq=Nq)
        q.copy_(y["q"].to(DEV))
        if fp8:
            for dst, src in ((k8, fp8_cache(y["k"])), (v8, fp8_cache(y["v"]))):
                dst.copy_(src[0].to(DEV))
            ks.copy_(fp8_cache(y["k"])[1].to(DEV))
            vs.copy_(fp8_cache(y["v"])[1].to(DEV))
        else:
            k.copy_(y["k"].to(DEV))
            v.copy_(y["v"].to(DEV))
        g.replay()
        torch.cuda.synchronize()
        got = (o.clone(), lse.clone())
        ro, rl = call()
        torch.cuda.synchronize()
        assert torch.equal(got[0], ro) and torch.equal(got[1], rl), f"replay {r} differs"


def test_fp8_forward_graph_replays():
    B, H, N, d = 2, 8, 300, 128
    from attn_inputs import fp8_head

    def draw(seed):
        y = make_inputs(B, H, N, d, torch.float32, seed=seed)
        q8, qs = fp8_cache(y["q"])
        k8, ks = fp8_head(y["k"])
        v8, vs = fp8_head(y["v"])
        return [t.to(DEV) for t in (q8, k8, v8, qs, ks, vs)]

    bufs = draw(401)
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=DEV)
    g = _capture(lambda: ea.attn_fwd_fp8(*bufs, causal=True, out=o, lse=lse))
    for r in range(3):
        for dst, src in zip(bufs, draw(500 + r)):
            dst.copy_(src)
        g.replay()
        torch.cuda.synchronize()
        got = (o.clone(), lse.clone())
        ro, rl = ea.attn_fwd_fp8(*bufs, causal=True)
        torch.cuda.synchronize()
        assert torch.equal(got[0], ro) and torch.equal(got[1], rl), f"replay {r} differs"
