"""Pins for the CPU oracle: checks against what the pages and the mathematics fix.

Each ``pin_*`` takes an implementation namespace ``impl`` with
    impl.head(q, k, v, scale, causal=False, valid_len=None, return_p=False)
        -> (O, LSE) or (O, LSE, P)                       (one head, fp64)
    impl.bwd_head(q, k, v, do, scale, causal=False, valid_len=None)
        -> (dQ, dK, dV)
and raises AssertionError when the implementation disagrees with the pin.
The oracle must pass every pin; deliberately broken copies of it (the mutant
tests) must each fail at least one, which shows the pins can see a dropped
term, a wrong sign or index, or a transposed operand.

Pages cited (by title):
  [SafeSoftmax]  "FlashAttention：从 Safe Softmax 到分块计算"
  [OpOpt]        "Attention 算子优化:从物化 N×N 矩阵到 FlashAttention 与 PagedAttention"
  [AIInfra]      the AIInfra FlashAttention note on dpshk.com
"""
from __future__ import annotations

import json
import math
import pathlib
import types

import numpy as np
import torch

GOLDEN = pathlib.Path(__file__).parent / "golden"
E = math.e


def golden(name: str) -> dict:
    return json.loads((GOLDEN / name).read_text(encoding="utf-8"))


def oracle_impl():
    import oracle.attention as A
    return types.SimpleNamespace(head=lambda *a, **kw: A.attn_ref_head(*a, **kw),
                                 bwd_head=lambda *a, **kw: A.attn_ref_bwd_head(*a, **kw),
                                 fwd=lambda *a, **kw: A.attn_ref_fwd(*a, **kw),
                                 bwd=lambda *a, **kw: A.attn_ref_bwd(*a, **kw),
                                 decode=lambda *a, **kw: A.attn_ref_decode(*a, **kw),
                                 e4m3=lambda *a, **kw: A.e4m3_decode(*a, **kw),
                                 dequant=lambda *a, **kw: A.dequant_fp8(*a, **kw))


def _rng(seed):
    return np.random.default_rng(seed)


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    fin = np.isfinite(b)
    assert np.array_equal(np.isfinite(a), fin), f"{what}: finiteness differs"
    assert np.array_equal(a[~fin], b[~fin]), f"{what}: non-finite entries differ"
    err = np.max(np.abs(a[fin] - b[fin])) if fin.any() else 0.0
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


# ---------------------------------------------------------------- page examples

def pin_two_block_example(impl):
    """[OpOpt] §三 worked example: blocks [1,2] and [3,1] merge to l ~= 1.638.

    Scores s_j = q.k_j with q = [1], k_j = [s_j], scale 1, so the oracle's LSE
    is ln(sum_j e^{s_j}); relative to the merged max 3 the page prints 1.638
    (sum of the rounded terms 0.135 + 0.368 + 1 + 0.135), and 1.368 for the
    first block on its own relative to its max 2.
    """
    g = golden("online_softmax_two_blocks.json")
    blocks = g["blocks"]
    row = blocks[0] + blocks[1]
    q = np.array([[1.0]])
    v = np.arange(1.0, len(row) + 1.0)[:, None]
    _, lse = impl.head(q, np.array(row)[:, None], v, 1.0)
    rel3 = math.exp(lse[0] - g["printed"]["merged_max"])
    assert abs(rel3 - g["printed"]["merged_sum_relative_to_merged_max"]) <= 1e-3
    assert abs(rel3 - g["printed"]["one_shot_sum_relative_to_3"]) <= 1e-3
    # exact closed form of the same sum
    assert abs(rel3 - (2 * math.exp(-2) + math.exp(-1) + 1)) <= 1e-14
    _, lse1 = impl.head(q, np.array(blocks[0])[:, None], v[:2], 1.0)
    rel2 = math.exp(lse1[0] - g["printed"]["first_block_max"])
    assert abs(rel2 - g["printed"]["first_block_sum_relative_to_its_max"]) <= 1e-3
    assert abs(rel2 - (math.exp(-1) + 1)) <= 1e-14


def pin_merge_example(impl):
    """[SafeSoftmax] §3.3: scores [1,2,3] with v = [10,20,30].

    The page's merged statistics: l = e^-1 (e^-1 + 1) + 1 and
    u = e^-1 u1 + 30 with u1 = 10 e^-1 + 20, and u / l is the one-shot result.
    The oracle's output must equal u / l; on the first block alone it must
    equal u1 / (e^-1 + 1).
    """
    g = golden("merge_rule_example.json")
    s = np.array(g["scores"])
    vv = np.array(g["values"])
    q = np.array([[1.0]])
    o, lse = impl.head(q, s[:, None], vv[:, None], 1.0)
    l = math.exp(-1) * (math.exp(-1) + 1) + 1
    u1 = 10 * math.exp(-1) + 20
    u = math.exp(-1) * u1 + 30
    assert abs(o[0, 0] - u / l) <= 1e-12, (o[0, 0], u / l)
    # coefficient form from the fixture
    l2 = sum(math.exp(e) for e in g["coefficients"]["merged_l_exponents"])
    u2 = sum(c * math.exp(e) for c, e in g["coefficients"]["merged_u_terms"])
    assert abs(l - l2) <= 1e-15 and abs(u - u2) <= 1e-13
    assert abs(lse[0] - (3 + math.log(l))) <= 1e-14
    o1, _ = impl.head(q, s[:2, None], vv[:2, None], 1.0)
    assert abs(o1[0, 0] - u1 / (math.exp(-1) + 1)) <= 1e-12
    # known probabilities of softmax([1,2,3]) to 7 digits
    _, _, p = impl.head(q, s[:, None], vv[:, None], 1.0, return_p=True)
    assert np.max(np.abs(p[0] - np.array([0.0900306, 0.2447285, 0.6652410]))) <= 1e-7


def pin_safe_softmax_example(impl):
    """[SafeSoftmax] §2.1: x = [1,2,3]; probabilities are [e^-2, e^-1, 1] / sum."""
    g = golden("safe_softmax_example.json")
    x = np.array(g["x"])
    q = np.array([[1.0]])
    _, _, p = impl.head(q, x[:, None], np.eye(3), 1.0, return_p=True)
    w = np.array([math.exp(e) for e in g["printed"]["exp_x_minus_m_exponents"]])
    _close(p[0], w / w.sum(), 1e-15, "safe softmax example")


# --------------------------------------------------------------- hand case N=4

def _hand():
    g = golden("hand_case_n4_d2.json")
    return (np.array(g["Q"], float), np.array(g["K"], float), np.array(g["V"], float))


def pin_hand_case_noncausal(impl):
    """Hand-derived N=4, d=2 integer case ([AIInfra] §3.1 asks for one).

    With scale 1, S = Q K^T = [[0,1,0,1],[0,0,1,1],[0,1,1,2],[0,0,0,0]], so
      row 0 = (V0 + V2 + e (V1 + V3)) / (2 + 2e)
      row 1 = (V0 + V1 + e (V2 + V3)) / (2 + 2e)
      row 2 = (V0 + e (V1 + V2) + e^2 V3) / (1 + e)^2
      row 3 = mean of V
    and LSE = [ln(2+2e), ln(2+2e), 2 ln(1+e), ln 4].
    """
    Q, K, V = _hand()
    o, lse = impl.head(Q, K, V, 1.0)
    want = np.array([
        (V[0] + V[2] + E * (V[1] + V[3])) / (2 + 2 * E),
        (V[0] + V[1] + E * (V[2] + V[3])) / (2 + 2 * E),
        (V[0] + E * (V[1] + V[2]) + E * E * V[3]) / (1 + E) ** 2,
        V.mean(axis=0),
    ])
    _close(o, want, 1e-13, "hand case O")
    _close(lse, [math.log(2 + 2 * E), math.log(2 + 2 * E), 2 * math.log(1 + E), math.log(4)],
           1e-13, "hand case LSE")
    # printed decimals of the derivation, as a second check on the closed forms
    _close(o[:, 0], [4.46211716, 4.92423431, 5.38635147, 4.0], 1e-8, "hand case O decimals")


def pin_hand_case_causal(impl):
    """Causal version of the hand case (top-left alignment: query i sees keys 0..i).

      row 0 = V0; row 1 = (V0 + V1) / 2 (both scores 0);
      row 2 = (V0 + e (V1 + V2)) / (1 + 2e); row 3 = mean of V
    and LSE = [0, ln 2, ln(1 + 2e), ln 4].
    """
    Q, K, V = _hand()
    o, lse = impl.head(Q, K, V, 1.0, causal=True)
    want = np.array([V[0], (V[0] + V[1]) / 2, (V[0] + E * (V[1] + V[2])) / (1 + 2 * E),
                     V.mean(axis=0)])
    _close(o, want, 1e-13, "hand causal O")
    _close(lse, [0.0, math.log(2), math.log(1 + 2 * E), math.log(4)], 1e-13, "hand causal LSE")


def pin_hand_case_scaled(impl):
    """Hand case with scale 1/sqrt(2): every exponent is divided by sqrt(2)."""
    Q, K, V = _hand()
    c = math.exp(1 / math.sqrt(2))
    o, lse = impl.head(Q, K, V, 1 / math.sqrt(2))
    want = np.array([
        (V[0] + V[2] + c * (V[1] + V[3])) / (2 + 2 * c),
        (V[0] + V[1] + c * (V[2] + V[3])) / (2 + 2 * c),
        (V[0] + c * (V[1] + V[2]) + c * c * V[3]) / (1 + c) ** 2,
        V.mean(axis=0),
    ])
    _close(o, want, 1e-13, "hand scaled O")
    _close(o[:3, 0], [4.3395231, 4.6790462, 5.0185693], 1e-7, "hand scaled decimals")
    _close(lse[:2], [math.log(2 + 2 * c)] * 2, 1e-13, "hand scaled LSE")


# ------------------------------------------------------------------ invariants

def _rand_head(seed, n=13, d=5, scale_mag=1.0):
    r = _rng(seed)
    return (r.standard_normal((n, d)) * scale_mag, r.standard_normal((n, d)) * scale_mag,
            r.standard_normal((n, d)))


def pin_rows_sum_to_one(impl):
    """Each row of P is a probability distribution over the visible keys."""
    for causal in (False, True):
        for L in (None, 9):
            q, k, v = _rand_head(1)
            _, _, p = impl.head(q, k, v, 0.4, causal, L, return_p=True)
            rows = np.arange(q.shape[0]) < (L if L is not None else q.shape[0])
            _close(p[rows].sum(axis=1), np.ones(rows.sum()), 1e-14, "row sums")
            assert np.all(p >= 0.0)
            if L is not None:
                assert np.all(p[:, L:] == 0.0), "padded keys must get zero probability"
            if causal:
                assert np.all(np.triu(p, 1) == 0.0), "future keys must get zero probability"


def pin_shift_invariance(impl):
    """[SafeSoftmax] §2: adding a constant to a score row leaves the softmax unchanged.

    K -> K + 1 c^T adds scale * q_i . c to every score of row i.
    """
    for causal in (False, True):
        q, k, v = _rand_head(2)
        c = _rng(3).standard_normal(k.shape[1]) * 3.0
        o1, lse1 = impl.head(q, k, v, 0.5, causal)
        o2, lse2 = impl.head(q, k + c[None, :], v, 0.5, causal)
        _close(o2, o1, 1e-12, "shift invariance O")
        _close(lse2 - 0.5 * (q @ c), lse1, 1e-12, "shift invariance LSE")


def pin_value_shift(impl):
    """V -> V + 1 b^T gives O + 1 b^T (rows of P sum to one)."""
    q, k, v = _rand_head(4)
    b = _rng(5).standard_normal(v.shape[1])
    o1, _ = impl.head(q, k, v, 0.7, True)
    o2, _ = impl.head(q, k, v + b[None, :], 0.7, True)
    _close(o2, o1 + b[None, :], 1e-12, "value shift")


def pin_permutation(impl):
    """Non-causal attention is invariant to a joint permutation of the (K, V) rows."""
    q, k, v = _rand_head(6)
    perm = _rng(7).permutation(k.shape[0])
    o1, lse1 = impl.head(q, k, v, 0.6)
    o2, lse2 = impl.head(q, k[perm], v[perm], 0.6)
    _close(o2, o1, 1e-12, "permutation O")
    _close(lse2, lse1, 1e-12, "permutation LSE")


def pin_zero_query(impl):
    """Q = 0 gives uniform weights: O is the column mean of V over visible keys."""
    q, k, v = _rand_head(8)
    q[:] = 0.0
    o, lse = impl.head(q, k, v, 1.0, False, 7)
    _close(o[:7], np.broadcast_to(v[:7].mean(axis=0), (7, v.shape[1])), 1e-14, "zero query")
    _close(lse[:7], np.full(7, math.log(7)), 1e-14, "zero query LSE")
    o, _ = impl.head(q, k, v, 1.0, True)
    want = np.cumsum(v, axis=0) / np.arange(1, v.shape[0] + 1)[:, None]
    _close(o, want, 1e-13, "zero query causal (running mean)")


def pin_causal_first_row(impl):
    """Causal row 0 sees key 0 only: O_0 = V_0 and LSE_0 = scale q_0 . k_0."""
    q, k, v = _rand_head(9)
    o, lse = impl.head(q, k, v, 0.3, True)
    _close(o[0], v[0], 0.0, "causal row 0")
    assert abs(lse[0] - 0.3 * float(q[0] @ k[0])) <= 1e-14


def pin_single_key(impl):
    """N = 1: the only key has weight 1, so O = V."""
    q, k, v = _rand_head(10, n=1)
    o, lse = impl.head(q, k, v, 0.9)
    _close(o, v, 0.0, "N=1")


def pin_padding(impl):
    """Padded batch ([OpOpt] §二): rows at or beyond the length are not computed
    (O = 0, LSE = -inf) and valid rows equal attention over the unpadded sequence."""
    q, k, v = _rand_head(11, n=16)
    for causal in (False, True):
        for L in (0, 1, 5, 16):
            o, lse = impl.head(q, k, v, 0.45, causal, L)
            assert np.all(o[L:] == 0.0) and np.all(np.isneginf(lse[L:]))
            if L:
                o_t, lse_t = impl.head(q[:L], k[:L], v[:L], 0.45, causal)
                _close(o[:L], o_t, 1e-14, "padding vs truncated")
                _close(lse[:L], lse_t, 1e-14, "padding LSE vs truncated")


def pin_identical_queries(impl):
    """[AIInfra] §3.1 stress case: identical query vectors give identical output rows,
    and a query equal (up to a large factor) to every key gives uniform weights."""
    q, k, v = _rand_head(12)
    q[:] = q[0]
    o, _ = impl.head(q, k, v, 0.5)
    _close(o, np.broadcast_to(o[0], o.shape), 0.0, "identical queries")
    k2 = np.broadcast_to(q[0] * 40.0, k.shape).copy()
    o2, _ = impl.head(q, k2, v, 0.5)
    _close(o2, np.broadcast_to(v.mean(axis=0), o2.shape), 1e-13, "query equal to every key")


def pin_large_scores(impl):
    """[AIInfra] §3.1 stress case: a very large Q K^T range stays finite and exact.

    Scores of order 1e4 overflow exp() unless the row maximum is subtracted
    ([SafeSoftmax] §2). The row with one dominant key must return that key's value.
    """
    q, k, v = _rand_head(13, scale_mag=30.0)
    o, lse = impl.head(q, k, v, 1.0)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    _, _, p = impl.head(q, k, v, 1.0, return_p=True)
    _close(p.sum(axis=1), np.ones(q.shape[0]), 1e-13, "large-score row sums")
    # dominant key: q . k_j = 1e4 for j = 3, tiny elsewhere
    q1 = np.zeros((1, 2)); q1[0, 0] = 100.0
    k1 = np.zeros((5, 2)); k1[3, 0] = 100.0
    v1 = np.arange(10.0).reshape(5, 2)
    o1, lse1 = impl.head(q1, k1, v1, 1.0)
    _close(o1[0], v1[3], 0.0, "dominant key")
    assert abs(lse1[0] - 1e4) <= 1e-9


def pin_torch_sdpa(impl):
    """Library special case: torch's CPU scaled_dot_product_attention in fp64
    (a boolean mask marks visible keys) must agree with the oracle."""
    for seed, causal, L in [(20, False, None), (21, True, None), (22, False, 11), (23, True, 9)]:
        q, k, v = _rand_head(seed, n=17, d=6)
        o, lse = impl.head(q, k, v, 0.37, causal, L)
        n = q.shape[0]
        LL = n if L is None else L
        visible = np.arange(n)[None, :] < LL
        if causal:
            visible = visible & (np.arange(n)[None, :] <= np.arange(n)[:, None])
        tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
        ref = torch.nn.functional.scaled_dot_product_attention(
            tq, tk, tv, attn_mask=torch.from_numpy(visible), scale=0.37).numpy()
        s = (tq @ tk.T) * 0.37
        s = s.masked_fill(~torch.from_numpy(visible), float("-inf"))
        ref_lse = torch.logsumexp(s, dim=-1).numpy()
        _close(o[:LL], ref[:LL], 1e-13, "torch sdpa O")
        _close(lse[:LL], ref_lse[:LL], 1e-13, "torch logsumexp")


def online_merge_reference(q, k, v, scale, causal=False, valid_len=None, block=4):
    """The tiled FA2-form forward ([SafeSoftmax] §3.2 merge rule, [AIInfra] §2.1 loop),
    written here independently of the oracle to pin the merge rule against the
    three-pass definition: state (m, l, acc) per row, rescaled by exp(m_old - m_new)."""
    n = k.shape[0]
    L = n if valid_len is None else valid_len
    rows = q.shape[0]
    m = np.full(rows, -np.inf)
    l = np.zeros(rows)
    acc = np.zeros((rows, v.shape[1]))
    for j0 in range(0, n, block):
        j = np.arange(j0, min(j0 + block, n))
        s = scale * (q @ k[j].T)
        vis = np.broadcast_to(j[None, :] < L, (rows, len(j)))
        if causal:
            vis = vis & (j[None, :] <= np.arange(rows)[:, None])
        s = np.where(vis, s, -np.inf)
        m_new = np.maximum(m, s.max(axis=1))
        live = np.isfinite(m_new)
        alpha = np.where(live, np.exp(np.where(live, m - m_new, 0.0)), 1.0)
        pt = np.where(vis & live[:, None], np.exp(s - np.where(live, m_new, 0.0)[:, None]), 0.0)
        l = alpha * l + pt.sum(axis=1)
        acc = alpha[:, None] * acc + pt @ v[j]
        m = m_new
    o = np.where(l[:, None] > 0, acc / np.where(l > 0, l, 1.0)[:, None], 0.0)
    return o


def pin_online_merge(impl):
    """The online merge (tiled, rescaled) equals the three-pass oracle to rounding."""
    for seed, causal, L, blk in [(30, False, None, 4), (31, True, None, 3), (32, False, 10, 5),
                                 (33, True, 7, 2)]:
        q, k, v = _rand_head(seed, n=19, d=7)
        o, _ = impl.head(q, k, v, 0.41, causal, L)
        o2 = online_merge_reference(q, k, v, 0.41, causal, L, blk)
        LL = q.shape[0] if L is None else L
        _close(o[:LL], o2[:LL], 1e-13, "online merge vs three-pass")


# -------------------------------------------------------------------- backward

def _loss_grad_fd(impl, q, k, v, do, scale, causal, L, eps=1e-6):
    """Central finite differences of L = sum(O o dO) with respect to Q, K, V."""
    def loss(qq, kk, vv):
        o, _ = impl.head(qq, kk, vv, scale, causal, L)
        return float(np.sum(o * do))
    grads = []
    for which in range(3):
        base = [q.copy(), k.copy(), v.copy()]
        g = np.zeros_like(base[which])
        for idx in np.ndindex(g.shape):
            plus = [x.copy() for x in base]
            minus = [x.copy() for x in base]
            plus[which][idx] += eps
            minus[which][idx] -= eps
            g[idx] = (loss(*plus) - loss(*minus)) / (2 * eps)
        grads.append(g)
    return grads


def pin_bwd_finite_difference(impl):
    """[AIInfra] §4.3 numerical-gradient check: the analytic backward must match
    central finite differences of L = sum(O o dO) in fp64."""
    for seed, causal, L in [(40, False, None), (41, True, None), (42, False, 4), (43, True, 5)]:
        r = _rng(seed)
        n, d = 6, 3
        q, k, v, do = (r.standard_normal((n, d)) for _ in range(4))
        dq, dk, dv = impl.bwd_head(q, k, v, do, 0.8, causal, L)
        fq, fk, fv = _loss_grad_fd(impl, q, k, v, do, 0.8, causal, L)
        for a, b, nm in [(dq, fq, "dQ"), (dk, fk, "dK"), (dv, fv, "dV")]:
            err = np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-30)
            assert err <= 1e-7, f"{nm}: finite-difference rel err {err:.2e} (seed {seed})"


def pin_bwd_torch_autograd(impl):
    """Library special case: autograd through torch's fp64 CPU SDPA."""
    for seed, causal in [(50, False), (51, True)]:
        r = _rng(seed)
        n, d = 21, 8
        q, k, v, do = (r.standard_normal((n, d)) for _ in range(4))
        dq, dk, dv = impl.bwd_head(q, k, v, do, 0.33, causal)
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal,
                                                               scale=0.33)
        out.backward(torch.from_numpy(do))
        for a, t, nm in [(dq, tq, "dQ"), (dk, tk, "dK"), (dv, tv, "dV")]:
            _close(a, t.grad.numpy(), 1e-12, f"autograd {nm}")


def pin_bwd_invariants(impl):
    """Rows of dS sum to zero, so sum_j dK_j = 0; and sum_j dV_j = sum_i dO_i
    (every row of P sums to one). Padded keys and padded queries get zero gradient."""
    r = _rng(60)
    n, d = 15, 4
    q, k, v, do = (r.standard_normal((n, d)) for _ in range(4))
    for causal in (False, True):
        dq, dk, dv = impl.bwd_head(q, k, v, do, 0.5, causal)
        _close(dk.sum(axis=0), np.zeros(d), 1e-12, "sum dK")
        _close(dv.sum(axis=0), do.sum(axis=0), 1e-12, "sum dV")
        dq, dk, dv = impl.bwd_head(q, k, v, do, 0.5, causal, 9)
        assert np.all(dq[9:] == 0) and np.all(dk[9:] == 0) and np.all(dv[9:] == 0)
        _close(dv.sum(axis=0), do[:9].sum(axis=0), 1e-12, "sum dV (padded)")


# ------------------------------------------------------ grouped K/V heads
# These pins take the batch-level entry points: impl.fwd(q, k, v, scale, causal,
# seqlens) -> (O, LSE) and impl.bwd(q, k, v, do, scale, causal, seqlens) ->
# (dQ, dK, dV), with q [B,H,N,d] and k, v [B,H_kv,N,d].

def pin_gqa_torch_sdpa(impl):
    """Library special case: torch's fp64 CPU SDPA with enable_gqa, whose K/V
    head for query head h is h // (H // H_kv) ([OpOpt] §五's grouping with
    consecutive query heads per group), forward and autograd backward."""
    for seed, (B, H, H_kv), causal in [(70, (2, 6, 2), False), (71, (1, 4, 1), True),
                                       (72, (2, 8, 4), True)]:
        r = _rng(seed)
        n, d = 11, 5
        q = r.standard_normal((B, H, n, d))
        k, v = r.standard_normal((B, H_kv, n, d)), r.standard_normal((B, H_kv, n, d))
        do = r.standard_normal((B, H, n, d))
        o, _ = impl.fwd(q, k, v, 0.6, causal)
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal,
                                                               scale=0.6, enable_gqa=True)
        _close(o, out.detach().numpy(), 1e-12, f"GQA O (H={H}, H_kv={H_kv})")
        out.backward(torch.from_numpy(do))
        dq, dk, dv = impl.bwd(q, k, v, do, 0.6, causal)
        for a, t, nm in [(dq, tq, "dQ"), (dk, tk, "dK"), (dv, tv, "dV")]:
            _close(a, t.grad.numpy(), 1e-12, f"GQA {nm} (H={H}, H_kv={H_kv})")


def pin_gqa_finite_difference(impl):
    """A shared K/V head's gradient is the derivative of L = sum(O o dO) through
    every query head that reads it: central finite differences in fp64."""
    r = _rng(73)
    B, H, H_kv, n, d = 1, 3, 1, 5, 3
    q = r.standard_normal((B, H, n, d))
    k, v = r.standard_normal((B, H_kv, n, d)), r.standard_normal((B, H_kv, n, d))
    do = r.standard_normal((B, H, n, d))
    for causal in (False, True):
        _, dk, dv = impl.bwd(q, k, v, do, 0.7, causal)
        for which, g in ((1, dk), (2, dv)):
            fd = np.zeros_like(g)
            for idx in np.ndindex(g.shape):
                args = [q, k.copy(), v.copy()]
                args[which][idx] += 1e-6
                lp = float(np.sum(impl.fwd(*args, 0.7, causal)[0] * do))
                args[which][idx] -= 2e-6
                lm = float(np.sum(impl.fwd(*args, 0.7, causal)[0] * do))
                fd[idx] = (lp - lm) / 2e-6
            err = np.max(np.abs(g - fd)) / max(np.max(np.abs(fd)), 1e-30)
            assert err <= 1e-7, f"GQA {'dK' if which == 1 else 'dV'} finite-difference err {err:.2e}"


def pin_gqa_padding(impl):
    """Grouped heads with a padded batch: every query head of sequence b sees
    only its first L_b keys; padded rows are 0 / -inf and get zero gradient."""
    r = _rng(74)
    B, H, H_kv, n, d = 2, 4, 2, 9, 3
    q = r.standard_normal((B, H, n, d))
    k, v = r.standard_normal((B, H_kv, n, d)), r.standard_normal((B, H_kv, n, d))
    do = r.standard_normal((B, H, n, d))
    sl = np.array([6, 9])
    o, lse = impl.fwd(q, k, v, 0.5, False, sl)
    for h in range(H):
        g = h // (H // H_kv)
        ref_o, ref_l = impl.head(q[0, h, :6], k[0, g, :6], v[0, g, :6], 0.5)
        _close(o[0, h, :6], ref_o, 1e-13, "GQA padded O")
        _close(lse[0, h, :6], ref_l, 1e-13, "GQA padded LSE")
    assert np.all(o[0, :, 6:] == 0) and np.all(np.isneginf(lse[0, :, 6:]))
    dq, dk, dv = impl.bwd(q, k, v, do, 0.5, False, sl)
    assert np.all(dq[0, :, 6:] == 0) and np.all(dk[0, :, 6:] == 0) and np.all(dv[0, :, 6:] == 0)


GQA_PINS = [pin_gqa_torch_sdpa, pin_gqa_finite_difference, pin_gqa_padding]


# ------------------------------------------------------------------ decode
# impl.decode(q, k, v, scale, causal, kv_lens) -> (O, LSE), q [B,H,Nq,d].

def pin_decode_is_last_forward_rows(impl):
    """Decoding the last Nq positions gives exactly the last Nq rows of the
    full forward over the same sequence (causal or not, padded or not)."""
    r = _rng(80)
    B, H, H_kv, n, d, nq = 2, 4, 2, 12, 3, 3
    q = r.standard_normal((B, H, n, d))
    k, v = r.standard_normal((B, H_kv, n, d)), r.standard_normal((B, H_kv, n, d))
    for causal in (False, True):
        for sl in (None, np.array([7, 12])):
            fo, fl = impl.fwd(q, k, v, 0.9, causal, sl)
            lens = [n, n] if sl is None else sl.tolist()
            qd = np.stack([q[b, :, L - nq:L] for b, L in enumerate(lens)])
            do_, dl = impl.decode(qd, k, v, 0.9, causal, sl)
            for b, L in enumerate(lens):
                _close(do_[b], fo[b, :, L - nq:L], 1e-13, f"decode O (causal={causal}, L={L})")
                _close(dl[b], fl[b, :, L - nq:L], 1e-13, f"decode LSE (causal={causal}, L={L})")


def pin_decode_torch_lower_right(impl):
    """Library special case: torch's fp64 SDPA with the lower-right causal bias
    (the last Nq query positions against Nk keys) and with no mask."""
    from torch.nn.attention.bias import causal_lower_right
    r = _rng(81)
    B, H, nq, nk, d = 2, 3, 4, 10, 5
    q = r.standard_normal((B, H, nq, d))
    k, v = r.standard_normal((B, H, nk, d)), r.standard_normal((B, H, nk, d))
    for causal in (False, True):
        o, _ = impl.decode(q, k, v, 0.7, causal)
        tq, tk, tv = (torch.tensor(x) for x in (q, k, v))
        mask = causal_lower_right(nq, nk) if causal else None
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=0.7)
        _close(o, ref.numpy(), 1e-12, f"decode vs torch (causal={causal})")


def pin_decode_no_visible_key(impl):
    """More queries than valid keys under the causal mask: positions below 0
    see nothing (O = 0, LSE = -inf); an empty sequence likewise."""
    r = _rng(82)
    q = r.standard_normal((2, 1, 4, 3))
    k, v = r.standard_normal((2, 1, 6, 3)), r.standard_normal((2, 1, 6, 3))
    o, l = impl.decode(q, k, v, 1.0, True, np.array([2, 0]))
    assert np.all(o[0, 0, :2] == 0) and np.all(np.isneginf(l[0, 0, :2]))
    assert np.all(np.isfinite(l[0, 0, 2:]))
    ref_o, _ = impl.head(q[0, 0, 3:4], k[0, 0, :2], v[0, 0, :2], 1.0)
    _close(o[0, 0, 3:4], ref_o, 1e-13, "last query sees both keys")
    assert np.all(o[1] == 0) and np.all(np.isneginf(l[1]))


def pin_e4m3_values(impl):
    """The E4M3 decoder: hand values of the format (1.0, the largest finite 448,
    the smallest subnormal 2^-9, -0, NaN) and, for all 256 bytes, torch's own
    float8_e4m3fn conversion (a library special case)."""
    f = impl.e4m3
    assert f([0x38])[0] == 1.0 and f([0x7E])[0] == 448.0 and f([0x01])[0] == 2.0 ** -9
    assert f([0x08])[0] == 2.0 ** -6 and f([0xC0])[0] == -2.0
    assert f([0x80])[0] == 0.0 and np.signbit(f([0x80])[0])
    assert np.isnan(f([0x7F])[0]) and np.isnan(f([0xFF])[0])
    allb = np.arange(256)
    ref = torch.tensor(allb, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = f(allb)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert np.all(same), f"E4M3 bytes {allb[~same][:8]} decode differently"


def pin_dequant_fp8_values(impl):
    """FP8 cache dequantisation ([OpOpt] §六: each cached token's K or V row is
    stored as E4M3 bytes with one fp32 scale per token, value = byte value x
    scale). Hand-worked values: three tokens (Nk = 3) of two columns (d = 2),
    so a scale broadcast along the wrong axis cannot even line up, with a
    different scale per token (0.5, 3, 10), none of them 1, so dividing
    instead of multiplying or reusing one token's scale changes the result.
    Bytes: 0x38 = 1, 0xC0 = -2, 0x40 = 2, 0x30 = 0.5, 0x7E = 448 (largest
    finite), 0x01 = 2^-9 (smallest subnormal)."""
    f = impl.dequant
    x8 = np.array([[0x38, 0xC0], [0x40, 0x30], [0x7E, 0x01]], dtype=np.uint8)
    sc = np.array([0.5, 3.0, 10.0])
    want = np.array([[0.5, -1.0], [6.0, 1.5], [4480.0, 10.0 * 2.0 ** -9]])
    got = f(x8, sc)
    assert got.shape == want.shape, f"dequant shape {got.shape} vs {want.shape}"
    assert np.array_equal(got, want), f"dequant values {got} vs {want}"
    # A [B=1, H_kv=2, Nk=3, d=4] cache: the scale of (head g, token j) multiplies
    # only that row. Row (g, j) holds the byte 0x38 + 8*j (1, 2, 4 for j = 0..2)
    # in every column; scales 1 + g + 10 j (head 0: 1, 11, 21; head 1: 2, 12, 22).
    x8 = np.zeros((1, 2, 3, 4), dtype=np.uint8)
    sc = np.zeros((1, 2, 3))
    for g in range(2):
        for j in range(3):
            x8[0, g, j, :] = 0x38 + 8 * j
            sc[0, g, j] = 1 + g + 10 * j
    want = np.array([[[[1.0] * 4, [22.0] * 4, [84.0] * 4],
                      [[2.0] * 4, [24.0] * 4, [88.0] * 4]]])
    got = f(x8, sc)
    assert got.shape == want.shape and np.array_equal(got, want), f"dequant 4-d values {got}"
    # torch tensors (the form the tests hand over) give the same values
    got_t = f(torch.from_numpy(x8), torch.from_numpy(sc).to(torch.float32))
    assert np.array_equal(got_t, want)


DECODE_PINS = [pin_decode_is_last_forward_rows, pin_decode_torch_lower_right,
               pin_decode_no_visible_key, pin_e4m3_values, pin_dequant_fp8_values]

FWD_PINS = [pin_two_block_example, pin_merge_example, pin_safe_softmax_example,
            pin_hand_case_noncausal, pin_hand_case_causal, pin_hand_case_scaled,
            pin_rows_sum_to_one, pin_shift_invariance, pin_value_shift, pin_permutation,
            pin_zero_query, pin_causal_first_row, pin_single_key, pin_padding,
            pin_identical_queries, pin_large_scores, pin_torch_sdpa, pin_online_merge]
BWD_PINS = [pin_bwd_finite_difference, pin_bwd_torch_autograd, pin_bwd_invariants]
ALL_PINS = FWD_PINS + BWD_PINS + GQA_PINS + DECODE_PINS
