"""CPU checks of the C-ABI library: it loads, exports every function that
include/attn.h declares, and its host-side argument validation returns the
documented status codes. Nothing here launches a kernel: every call below is
rejected on the host before any HIP call is made."""
import ctypes
import pathlib
import re
import subprocess

import pytest

import exact_attention_24_amd as ea

ROOT = pathlib.Path(__file__).resolve().parents[1]
HEADER = ROOT / "include" / "attn.h"

OK, INVALID, UNSUPPORTED, HIP = 0, 1, 2, 3


def declared_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not ea.LIB_PATH.exists():
        pytest.fail(f"{ea.LIB_PATH} is missing: run __graft_entry__.build() first")
    return ea.lib()


def test_header_declares_the_binding_symbols():
    assert declared_functions() == sorted(ea.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", str(ea.LIB_PATH)], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\s[TW]\s+(\S+)$", out, flags=re.M))
    for name in declared_functions():
        assert name in exported, f"{name} is not a defined dynamic symbol (C linkage)"


def test_status_strings(L):
    assert ea.attn_status_string(OK) == "ATTN_OK"
    assert ea.attn_status_string(INVALID) == "ATTN_ERR_INVALID_ARG"
    assert ea.attn_status_string(UNSUPPORTED) == "ATTN_ERR_UNSUPPORTED"
    assert ea.attn_status_string(HIP) == "ATTN_ERR_HIP"
    assert ea.attn_status_string(77) == "ATTN_STATUS_UNKNOWN"
    assert L.attn_last_error() == b""


# Fake, 16-byte-aligned "device" addresses: never dereferenced, because every
# call below fails validation first. As a second guard these tests do not run
# where a GPU is visible (a call that passed validation by mistake would launch
# a kernel on them).
P = 0x10000


def _gpu_visible():
    import torch
    return torch.cuda.device_count() > 0


cpu_only = pytest.mark.skipif(_gpu_visible(), reason="fake device pointers: host-only checks")


def fwd(L, q=P, k=P, v=P, o=P, lse=P, B=1, H=1, N=64, d=64, dtype=1, scale=0.125, causal=0,
        seqlens=0):
    return L.attn_fwd(q, k, v, o, lse, B, H, N, d, dtype, scale, causal, seqlens, 0)


@pytest.mark.parametrize("kw,want", [
    (dict(q=0), INVALID), (dict(k=0), INVALID), (dict(v=0), INVALID), (dict(o=0), INVALID),
    (dict(B=0), INVALID), (dict(H=-1), INVALID), (dict(N=0), INVALID), (dict(d=0), INVALID),
    (dict(dtype=7), INVALID), (dict(d=96), UNSUPPORTED), (dict(d=256), UNSUPPORTED),
    (dict(d=32), UNSUPPORTED), (dict(scale=0.0), INVALID), (dict(scale=-1.0), INVALID),
    (dict(scale=float("nan")), INVALID), (dict(scale=float("inf")), INVALID),
    (dict(q=P + 8), INVALID), (dict(o=P + 4), INVALID), (dict(lse=P + 2), INVALID),
    (dict(seqlens=P + 1), INVALID), (dict(B=1 << 20, H=1 << 12, N=1 << 12), UNSUPPORTED),
])
@cpu_only
def test_fwd_rejects_bad_arguments(L, kw, want):
    # scale and null-pointer checks come after size checks; each case fails exactly one rule
    assert fwd(L, **kw) == want


def bwd(L, ws_bytes=None, **kw):
    a = dict(q=P, k=P, v=P, o=P, do=P, lse=P, dq=P, dk=P, dv=P, ws=P, B=1, H=1, N=64, d=64,
             dtype=1, scale=0.125, causal=0, seqlens=0)
    a.update(kw)
    if ws_bytes is None:
        ws_bytes = L.attn_bwd_workspace_bytes(a["B"], a["H"], a["N"], a["d"], a["dtype"])
    return L.attn_bwd(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"],
                      a["dv"], a["ws"], ws_bytes, a["B"], a["H"], a["N"], a["d"], a["dtype"],
                      a["scale"], a["causal"], a["seqlens"], 0)


@pytest.mark.parametrize("kw,want", [
    (dict(do=0), INVALID), (dict(lse=0), INVALID), (dict(dq=0), INVALID), (dict(ws=0), INVALID),
    (dict(dk=P + 8), INVALID), (dict(ws=P + 16), INVALID), (dict(d=80), UNSUPPORTED),
    (dict(ws_bytes=16), INVALID), (dict(scale=0.0), INVALID), (dict(dtype=0), UNSUPPORTED),
    (dict(N=-5), INVALID),
])
@cpu_only
def test_bwd_rejects_bad_arguments(L, kw, want):
    kw = dict(kw)
    ws_bytes = kw.pop("ws_bytes", None)
    assert bwd(L, ws_bytes, **kw) == want


def fwd_gqa(L, H=4, H_kv=2, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, N=64, d=64, dtype=1, scale=0.125, causal=0, seqlens=0)
    a.update(kw)
    return L.attn_fwd_gqa(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], H, H_kv, a["N"], a["d"],
                          a["dtype"], a["scale"], a["causal"], a["seqlens"], 0)


@pytest.mark.parametrize("H,H_kv", [(4, 0), (4, -1), (4, 3), (4, 8), (6, 4)])
@cpu_only
def test_gqa_rejects_bad_head_counts(L, H, H_kv):
    assert fwd_gqa(L, H, H_kv, q=0) == INVALID  # still rejected (null q) ...
    assert fwd_gqa(L, H, H_kv) == INVALID       # ... and for the head count alone


@cpu_only
def test_gqa_validates_like_fwd(L):
    assert fwd_gqa(L, 4, 2, d=96) == UNSUPPORTED
    assert fwd_gqa(L, 4, 2, scale=0.0) == INVALID
    ws = L.attn_bwd_workspace_bytes(1, 4, 64, 64, 1)
    assert L.attn_bwd_gqa(P, P, P, P, P, P, P, P, P, P, ws, 1, 4, 3, 64, 64, 1, 0.125, 0, 0,
                          0) == INVALID
    assert L.attn_bwd_gqa(P, P, P, P, P, P, P, P, P, 0, ws, 1, 4, 2, 64, 64, 1, 0.125, 0, 0,
                          0) == INVALID


def test_workspace_bytes(L):
    # two fp32 [B,H,N] sections (delta, log2-scaled LSE), each rounded up to 256 bytes
    assert L.attn_bwd_workspace_bytes(2, 16, 8192, 128, 1) == 2 * (2 * 16 * 8192 * 4)
    assert L.attn_bwd_workspace_bytes(1, 1, 3, 64, 1) == 2 * 256
    assert L.attn_bwd_workspace_bytes(1, 1, 0, 64, 1) == 0
    assert L.attn_bwd_workspace_bytes(1, 1, 8, 100, 1) == 0


def dec(L, fp8=False, ws_bytes=None, **kw):
    a = dict(q=P, k=P, v=P, ks=P, vs=P, o=P, lse=P, B=2, H=8, H_kv=2, Nq=1, Nk=300, d=128,
             dtype=1, scale=0.088, causal=1, kv_lens=0, splits=0, ws=P)
    a.update(kw)
    if ws_bytes is None:
        ws_bytes = L.attn_decode_workspace_bytes(a["B"], a["H"], a["H_kv"], a["Nq"], a["Nk"],
                                                 a["d"], a["dtype"], a["splits"])
    tail = (a["B"], a["H"], a["H_kv"], a["Nq"], a["Nk"], a["d"], a["dtype"], a["scale"],
            a["causal"], a["kv_lens"], a["splits"], a["ws"], ws_bytes, 0)
    if fp8:
        return L.attn_decode_fp8kv(a["q"], a["k"], a["v"], a["ks"], a["vs"], a["o"], a["lse"], *tail)
    return L.attn_decode(a["q"], a["k"], a["v"], a["o"], a["lse"], *tail)


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8kv"])
@pytest.mark.parametrize("kw,want", [
    (dict(q=0), INVALID), (dict(k=0), INVALID), (dict(o=0), INVALID), (dict(ws=0), INVALID),
    (dict(q=P + 8), INVALID), (dict(ws=P + 16), INVALID), (dict(lse=P + 2), INVALID),
    (dict(kv_lens=P + 1), INVALID), (dict(B=0), INVALID), (dict(Nq=0), INVALID),
    (dict(Nk=0), INVALID), (dict(H_kv=3), INVALID), (dict(H_kv=0), INVALID),
    (dict(H_kv=16), INVALID), (dict(splits=-1), INVALID), (dict(dtype=5), INVALID),
    (dict(dtype=0), UNSUPPORTED), (dict(d=96), UNSUPPORTED), (dict(scale=0.0), INVALID),
    (dict(scale=float("nan")), INVALID), (dict(ws_bytes=256), INVALID),
])
@cpu_only
def test_decode_rejects_bad_arguments(L, fp8, kw, want):
    kw = dict(kw)  # the parameter dict is shared by both formats
    ws_bytes = kw.pop("ws_bytes", None)
    assert dec(L, fp8, ws_bytes, **kw) == want


@cpu_only
def test_decode_fp8kv_specific_rules(L):
    assert dec(L, True, d=96) == UNSUPPORTED   # FP8 caches: d = 64 or 128
    assert dec(L, True, ks=0) == INVALID       # both scale arrays are required
    assert dec(L, True, vs=P + 2) == INVALID


def fwd8(L, q=P, k=P, v=P, qs=P, ks=P, vs=P, o=P, lse=P, B=1, H=2, H_kv=1, N=64, d=128,
         dtype=1, scale=0.088, causal=0, seqlens=0):
    return L.attn_fwd_fp8(q, k, v, qs, ks, vs, o, lse, B, H, H_kv, N, d, dtype, scale, causal,
                          seqlens, 0)


@pytest.mark.parametrize("kw,want", [
    (dict(q=0), INVALID), (dict(k=0), INVALID), (dict(v=0), INVALID), (dict(o=0), INVALID),
    (dict(qs=0), INVALID), (dict(ks=0), INVALID), (dict(vs=0), INVALID),
    (dict(q=P + 8), INVALID), (dict(o=P + 4), INVALID), (dict(qs=P + 2), INVALID),
    (dict(lse=P + 2), INVALID), (dict(seqlens=P + 1), INVALID),
    (dict(B=0), INVALID), (dict(N=0), INVALID), (dict(H_kv=3), INVALID), (dict(H_kv=0), INVALID),
    (dict(d=64), UNSUPPORTED), (dict(d=96), UNSUPPORTED), (dict(dtype=0), UNSUPPORTED),
    (dict(dtype=9), INVALID), (dict(scale=0.0), INVALID), (dict(scale=float("nan")), INVALID),
])
@cpu_only
def test_fwd_fp8_rejects_bad_arguments(L, kw, want):
    assert fwd8(L, **kw) == want


def test_decode_workspace_bytes(L):
    # One split: fp32 O [rows][1][d] and (m, l) [rows][1][2], each section rounded to 256 B.
    rows = 2 * 8 * 3
    up = lambda n: (n + 255) // 256 * 256
    assert L.attn_decode_workspace_bytes(2, 8, 2, 3, 300, 128, 1, 1) == up(rows * 128 * 4) + up(rows * 2 * 4)
    # More splits never need less; automatic (0) is a valid request; invalid sizes give 0.
    sizes = [L.attn_decode_workspace_bytes(8, 64, 8, 1, 8192, 128, 1, s) for s in (1, 4, 16, 0)]
    assert sizes[0] < sizes[1] < sizes[2] and sizes[3] > 0 and all(x % 256 == 0 for x in sizes)
    assert L.attn_decode_workspace_bytes(1, 4, 3, 1, 100, 128, 1, 0) == 0   # H_kv does not divide H
    assert L.attn_decode_workspace_bytes(1, 4, 2, 1, 100, 96, 1, 0) == 0    # unsupported d
    assert L.attn_decode_workspace_bytes(1, 4, 2, 1, 100, 128, 0, 0) == 0   # fp32


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        ea.attn_fwd(x, x, x)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(ea, "_lib", None)
    monkeypatch.setattr(ea, "LIB_PATH", tmp_path / "nope.so")
    with pytest.raises(RuntimeError, match="not found"):
        ea.lib()


def bwd_noalloc(L, **kw):
    a = dict(q=P, k=P, v=P, o=P, do=P, lse=P, dq=P, dk=P, dv=P, B=1, H=4, H_kv=2, N=64, d=64,
             dtype=1, scale=0.125, causal=0, seqlens=0)
    a.update(kw)
    return L.attn_bwd_noalloc(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"],
                              a["dv"], a["B"], a["H"], a["H_kv"], a["N"], a["d"], a["dtype"],
                              a["scale"], a["causal"], a["seqlens"], 0)


@pytest.mark.parametrize("kw,want", [
    (dict(q=0), INVALID), (dict(dv=0), INVALID), (dict(lse=0), INVALID), (dict(B=0), INVALID),
    (dict(H_kv=3), INVALID), (dict(d=96), UNSUPPORTED), (dict(scale=0.0), INVALID),
    (dict(dtype=0), UNSUPPORTED), (dict(dtype=9), INVALID),
    # 2^21 query rows is the static scratch's limit: one more row is refused
    (dict(B=1, H=64, H_kv=64, N=32769), UNSUPPORTED), (dict(B=2, H=32, H_kv=32, N=32769), UNSUPPORTED),
])
@cpu_only
def test_bwd_noalloc_rejects_bad_arguments(L, kw, want):
    assert bwd_noalloc(L, **kw) == want


@cpu_only
def test_bwd_noalloc_names_its_limit(L):
    assert bwd_noalloc(L, B=4, H=32, H_kv=32, N=16385) == UNSUPPORTED
    assert b"2097152" in L.attn_last_error()
