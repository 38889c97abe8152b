"""Plant plausible mistakes in the oracle (on the CPU) and check that the pin suite
catches every one of them: a dropped term, a wrong sign or index, a transposed
operand, an off-by-one mask. A pin that raises (for example on a shape error)
counts as catching the mistake."""
import types

import numpy as np
import pytest

import oracle.attention as A
from tests.oracle_pins import ALL_PINS, BWD_PINS, DECODE_PINS, FWD_PINS, GQA_PINS


def _run_pins(impl, pins):
    caught = []
    for pin in pins:
        try:
            with np.errstate(all="ignore"):
                pin(impl)
        except Exception:  # noqa: BLE001 - any failure means the pin saw the mutant
            caught.append(pin.__name__)
    return caught


# ---- forward mutants: each replaces one step of the oracle with a broken copy

def _no_scale(q, k, scale):
    return q @ k.T


def _transposed(q, k, scale):
    return scale * (k @ q.T)


def _negated(q, k, scale):
    return -scale * (q @ k.T)


def _mask_factory(kind):
    def mask(s, row_index, causal, valid_len):
        s = s.copy()
        key = np.arange(s.shape[1])[None, :]
        if kind == "padding_off_by_one":
            hidden = key > valid_len
        else:
            hidden = key >= valid_len
        if causal:
            if kind == "causal_diagonal_hidden":
                hidden = hidden | (key >= row_index[:, None])
            elif kind == "causal_reversed":
                hidden = hidden | (key < row_index[:, None])
            elif kind == "causal_ignored":
                pass
            else:
                hidden = hidden | (key > row_index[:, None])
        s[np.broadcast_to(hidden, s.shape)] = -np.inf
        return s
    return mask


def _softmax_factory(kind):
    def softmax(s):
        rows = s.shape[0]
        m = np.array([np.max(s[i]) if s.shape[1] else -np.inf for i in range(rows)])
        if kind == "no_max_subtraction":
            e = np.exp(s)
            l = e.sum(axis=1)
            p = e / l[:, None]
            return p, np.zeros(rows), l
        e = np.where(np.isfinite(m)[:, None], np.exp(s - np.where(np.isfinite(m), m, 0)[:, None]), 0)
        l = e.sum(axis=1)
        if kind == "wrong_row_normaliser":
            p = e / l[::-1][:, None]
        elif kind == "lse_without_max":
            p = np.where(l[:, None] > 0, e / np.where(l > 0, l, 1)[:, None], 0)
            return p, np.zeros(rows), l
        elif kind == "max_over_columns":
            mc = np.max(s, axis=0)
            e = np.exp(s - mc[None, :])
            l = e.sum(axis=1)
            p = e / l[:, None]
        else:
            p = np.where(l[:, None] > 0, e / np.where(l > 0, l, 1)[:, None], 0)
        return p, m, l
    return softmax


FWD_MUTANTS = {
    "no_scale": ("scores", _no_scale),
    "transposed_operand": ("scores", _transposed),
    "negated_scores": ("scores", _negated),
    "causal_diagonal_hidden": ("mask", _mask_factory("causal_diagonal_hidden")),
    "causal_reversed": ("mask", _mask_factory("causal_reversed")),
    "causal_ignored": ("mask", _mask_factory("causal_ignored")),
    "padding_off_by_one": ("mask", _mask_factory("padding_off_by_one")),
    "no_max_subtraction": ("softmax_three_pass", _softmax_factory("no_max_subtraction")),
    "wrong_row_normaliser": ("softmax_three_pass", _softmax_factory("wrong_row_normaliser")),
    "lse_without_max": ("softmax_three_pass", _softmax_factory("lse_without_max")),
    "max_over_columns": ("softmax_three_pass", _softmax_factory("max_over_columns")),
}


@pytest.mark.parametrize("name", sorted(FWD_MUTANTS))
def test_forward_mutant_is_caught(name, monkeypatch):
    attr, fn = FWD_MUTANTS[name]
    monkeypatch.setattr(A, attr, fn)
    impl = types.SimpleNamespace(head=A.attn_ref_head, bwd_head=A.attn_ref_bwd_head)
    caught = _run_pins(impl, FWD_PINS)
    assert caught, f"mutant {name} passed every forward pin"


# ---- backward mutants: the oracle's backward with one term broken

def _bwd_factory(kind):
    def bwd(q, k, v, do, scale, causal=False, valid_len=None):
        q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
        _, _, p = A.attn_ref_head(q, k, v, scale, causal, valid_len, return_p=True)
        dv = p.T @ do
        dp = do @ v.T
        D = np.sum(dp * p, axis=1)
        ds = p * (dp - D[:, None])
        dq = scale * (ds @ k)
        dk = scale * (ds.T @ q)
        if kind == "ds_sign":
            ds = p * (D[:, None] - dp)
            dq, dk = scale * (ds @ k), scale * (ds.T @ q)
        elif kind == "dq_missing_scale":
            dq = ds @ k
        elif kind == "dk_missing_scale":
            dk = ds.T @ q
        elif kind == "D_without_p":
            ds = p * (dp - dp.sum(axis=1)[:, None])
            dq, dk = scale * (ds @ k), scale * (ds.T @ q)
        elif kind == "dk_untransposed":
            dk = scale * (ds @ q)
        elif kind == "dv_untransposed":
            dv = p @ do
        elif kind == "dp_untransposed_v":
            dp = do @ v[::-1].T
            D = np.sum(dp * p, axis=1)
            ds = p * (dp - D[:, None])
            dq, dk = scale * (ds @ k), scale * (ds.T @ q)
        elif kind == "dropped_D":
            ds = p * dp
            dq, dk = scale * (ds @ k), scale * (ds.T @ q)
        return dq, dk, dv
    return bwd


BWD_MUTANTS = ["ds_sign", "dq_missing_scale", "dk_missing_scale", "D_without_p",
               "dk_untransposed", "dv_untransposed", "dp_untransposed_v", "dropped_D"]


@pytest.mark.parametrize("name", BWD_MUTANTS)
def test_backward_mutant_is_caught(name):
    impl = types.SimpleNamespace(head=A.attn_ref_head, bwd_head=_bwd_factory(name))
    caught = _run_pins(impl, BWD_PINS)
    assert caught, f"mutant {name} passed every backward pin"


def test_unmutated_backward_copy_passes():
    """The mutant factory with no mutation passes every pin (the harness is sound)."""
    impl = types.SimpleNamespace(head=A.attn_ref_head, bwd_head=_bwd_factory("none"),
                                 fwd=A.attn_ref_fwd, bwd=A.attn_ref_bwd, decode=A.attn_ref_decode,
                                 e4m3=A.e4m3_decode, dequant=A.dequant_fp8)
    assert _run_pins(impl, ALL_PINS) == []


# ---- grouped K/V head mutants

def _kv_interleaved(h, H, H_kv):
    return h % H_kv


def _gqa_bwd_overwrite(q, k, v, do, scale, causal=False, seqlens=None):
    """The batched backward with the group sum replaced by the last head's term."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    B, H, N, _ = q.shape
    H_kv = k.shape[1]
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(B):
        L = N if seqlens is None else int(seqlens[b])
        for h in range(H):
            g = h // (H // H_kv)
            dq[b, h], dk[b, g], dv[b, g] = A.attn_ref_bwd_head(q[b, h], k[b, g], v[b, g], do[b, h],
                                                               scale, causal, L)
    return dq, dk, dv


def test_gqa_interleaved_grouping_is_caught(monkeypatch):
    monkeypatch.setattr(A, "kv_head", _kv_interleaved)
    impl = types.SimpleNamespace(head=A.attn_ref_head, fwd=A.attn_ref_fwd, bwd=A.attn_ref_bwd)
    assert _run_pins(impl, GQA_PINS), "interleaved K/V grouping passed every grouped-head pin"


def test_gqa_missing_group_sum_is_caught():
    impl = types.SimpleNamespace(head=A.attn_ref_head, fwd=A.attn_ref_fwd, bwd=_gqa_bwd_overwrite)
    assert _run_pins(impl, GQA_PINS), "dropped group sum passed every grouped-head pin"


# ---- decode mutants: the decode with the query positions misplaced

def _decode_factory(offset_kind):
    def decode(q, k, v, scale, causal=False, kv_lens=None, heads=None):
        q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
        B, H, Nq, _ = q.shape
        H_kv, Nk = k.shape[1], k.shape[2]
        o = np.zeros(q.shape[:3] + (v.shape[-1],))
        lse = np.zeros(q.shape[:3])
        for b in range(B):
            L = Nk if kv_lens is None else int(np.clip(kv_lens[b], 0, Nk))
            pos = {"top_left": np.arange(Nq), "off_by_one": L - Nq + 1 + np.arange(Nq)}[offset_kind]
            for h in range(H):
                g = h // (H // H_kv)
                s = A.mask(A.scores(q[b, h], k[b, g], scale), pos, causal, L)
                p, m, l = A.softmax_three_pass(s)
                o[b, h] = p @ v[b, g]
                with np.errstate(divide="ignore"):
                    lse[b, h] = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
        return o, lse
    return decode


@pytest.mark.parametrize("kind", ["top_left", "off_by_one"])
def test_decode_position_mutant_is_caught(kind):
    impl = types.SimpleNamespace(head=A.attn_ref_head, fwd=A.attn_ref_fwd,
                                 decode=_decode_factory(kind), e4m3=A.e4m3_decode,
                                 dequant=A.dequant_fp8)
    assert _run_pins(impl, DECODE_PINS), f"decode mutant {kind} passed every decode pin"


def _e4m3_bias8(byte_values):
    """E4M3 with the exponent bias off by one (8 instead of 7)."""
    return A.e4m3_decode(byte_values) / 2.0


def _e4m3_no_subnormals(byte_values):
    """E4M3 with exponent field 0 read as a normal number."""
    u = np.asarray(byte_values, dtype=np.int64)
    v = A.e4m3_decode(byte_values)
    e, m = (u >> 3) & 15, (u & 7)
    fixed = np.where(u >> 7, -1.0, 1.0) * (1.0 + m / 8.0) * np.exp2(-7.0)
    return np.where(e == 0, fixed, v)


@pytest.mark.parametrize("fn", [_e4m3_bias8, _e4m3_no_subnormals], ids=["bias8", "no_subnormals"])
def test_e4m3_mutant_is_caught(fn):
    impl = types.SimpleNamespace(head=A.attn_ref_head, fwd=A.attn_ref_fwd, decode=A.attn_ref_decode,
                                 e4m3=fn, dequant=A.dequant_fp8)
    assert _run_pins(impl, DECODE_PINS), "E4M3 decoder mutant passed every pin"


# ---- FP8 dequantisation mutants: the per-token scale applied wrongly

def _dequant_divide(x8, scale):
    """Divides by the scale instead of multiplying."""
    return A.e4m3_decode(np.asarray(x8)) / np.asarray(scale, dtype=np.float64)[..., None]


def _dequant_column_axis(x8, scale):
    """Broadcasts the per-token scale along the columns instead of the tokens."""
    return A.e4m3_decode(np.asarray(x8)) * np.asarray(scale, dtype=np.float64)[..., None, :]


def _dequant_first_token(x8, scale):
    """Uses the first token's scale for every token of a head."""
    s = np.asarray(scale, dtype=np.float64)
    return A.e4m3_decode(np.asarray(x8)) * s[..., :1, None]


def _dequant_flat_scale(x8, scale):
    """Indexes the scales by token only, ignoring the head (head 0's scales everywhere)."""
    s = np.asarray(scale, dtype=np.float64)
    if s.ndim >= 2:
        s = np.broadcast_to(s[..., :1, :], s.shape)
    return A.e4m3_decode(np.asarray(x8)) * s[..., None]


@pytest.mark.parametrize("fn", [_dequant_divide, _dequant_column_axis, _dequant_first_token,
                                _dequant_flat_scale],
                         ids=["divide", "column_axis", "first_token", "flat_scale"])
def test_dequant_mutant_is_caught(fn):
    impl = types.SimpleNamespace(head=A.attn_ref_head, fwd=A.attn_ref_fwd, decode=A.attn_ref_decode,
                                 e4m3=A.e4m3_decode, dequant=fn)
    assert _run_pins(impl, DECODE_PINS), "dequantisation mutant passed every pin"
