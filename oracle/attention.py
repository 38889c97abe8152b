"""Plain fp64 CPU oracle for exact scaled dot-product attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or run
this module: only the test suite, the package smoke check and the benchmark's
CPU-baseline leg do. It shares no code with the HIP library (no kernels,
headers, helpers, tables or constants); the two meet only in the seeded input
generator module, which holds none of the method's arithmetic.

Pages cited in this file (by title):
  [SafeSoftmax]  "FlashAttention：从 Safe Softmax 到分块计算" (liumengxuan04.github.io)
  [Viper]        "FlashAttention算子优化" (ViperEkura's Blog)
  [OpOpt]        "Attention 算子优化:从物化 N×N 矩阵到 FlashAttention 与 PagedAttention"
                 (geek-doc.cn)
  [AIInfra]      the AIInfra FlashAttention data-flow note on dpshk.com (its HTML
                 title, "企业官网建设流程全解析", is unrelated to its body)
  [Tiling]       "FlashAttention分块计算优化大模型训练效率" (intelliparadigm.com)

What is computed. FlashAttention reaches exactly (up to rounding order) the
result of standard attention O = softmax(scale * Q K^T) V ([SafeSoftmax] §1 and
§10: same mathematical result, no approximation). So this oracle is that plain
definition written out, per (batch, head), in float64, materialising the N x N
score matrix S and probability matrix P:

  1. S = scale * Q K^T                                   [SafeSoftmax] §1, [Viper] §1
  2. masked scores set to -inf: future keys j > i when causal
     ([SafeSoftmax] §5.2), and keys at or beyond the sequence's valid length in
     a padded batch ([OpOpt] §二, padding masked to -inf before the softmax)
  3. three-pass safe softmax, row by row ([SafeSoftmax] §2 and the three
     scans listed at the start of §3; [Viper] §1, the conventional softmax):
       pass 1  m_i = max_j S_ij
       pass 2  l_i = sum_j exp(S_ij - m_i)
       pass 3  P_ij = exp(S_ij - m_i) / l_i
  4. O = P V                                             [SafeSoftmax] §1
  5. LSE_i = m_i + ln l_i, the per-row log-sum-exp statistic saved for the
     backward ([SafeSoftmax] §8)

Readings taken where the pages are silent (each is listed in the design notes):
  * A row with no visible key (a padded query row, or a sequence of length 0)
    has no softmax; its output row is 0 and its LSE is -inf.
  * Queries and keys of one sequence share one valid length; causal alignment
    is top-left (query i sees keys 0..i).
  * Grouped K/V heads ([OpOpt] §五: query heads fall into groups and each group
    shares one K/V head; H_kv = 1 is multi-query attention): with k, v of shape
    [B, H_kv, N, d], query head h uses K/V head h // (H // H_kv), i.e. groups
    are runs of consecutive query heads (the pages do not fix the order; this
    is the plain reading). In the backward a K/V head's gradient is the sum of
    the per-query-head gradients of its group (the chain rule through the
    shared tensor).
  * Decode ([OpOpt] §五: each new token's query attends to the cached K, V of
    all earlier tokens): the Nq queries of sequence b are its last Nq positions
    L_b - Nq .. L_b - 1, so under the causal mask query i sees keys
    j <= L_b - Nq + i (bottom-right alignment; for Nq = L_b it is the
    forward's mask). Without the mask it sees every valid key.
  * FP8 K/V cache ([OpOpt] §六: K, V stored as FP8 E4M3 with per-token
    scales, dequantised before use): the oracle decodes each byte by the OCP
    E4M3 definition (sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
    exponent 0 is subnormal; 0x7F and 0xFF are NaN; no infinities) and
    multiplies by the token's scale in fp64; attention then runs on those
    values exactly as above.
  * Backward ([AIInfra] §2.3 gives dV = P^T dO and dS = P o (dP - rowsum(dP o P))
    with dP = dO V^T; the scale factor on dQ and dK is not on the pages and
    follows from S = scale * Q K^T by the chain rule):
       dV = P^T dO,  dP = dO V^T,  D_i = sum_j dP_ij P_ij,
       dS = P o (dP - D),  dQ = scale * dS K,  dK = scale * dS^T Q.
"""
from __future__ import annotations

import numpy as np

__all__ = ["scores", "mask", "softmax_three_pass", "attn_ref_head", "kv_head", "attn_ref_fwd",
           "attn_ref_rows", "attn_ref_decode", "e4m3_decode", "dequant_fp8",
           "attn_ref_bwd_head", "attn_ref_bwd"]


def _f64(x) -> np.ndarray:
    """Exact upcast to float64 (bf16, fp16 and fp32 values are representable)."""
    if hasattr(x, "detach"):  # a torch tensor: go through fp32, which holds bf16/fp16 exactly
        import torch
        x = x.detach().to("cpu")
        if x.dtype in (torch.bfloat16, torch.float16):
            x = x.to(torch.float32)
        x = x.numpy()
    return np.asarray(x, dtype=np.float64)


def scores(q: np.ndarray, k: np.ndarray, scale: float) -> np.ndarray:
    """Step 1: S = scale * Q K^T for one head (q: [M, d], k: [N, d])."""
    return scale * (q @ k.T)


def mask(s: np.ndarray, row_index: np.ndarray, causal: bool, valid_len: int) -> np.ndarray:
    """Step 2: set masked scores to -inf.

    ``row_index[r]`` is the sequence position of row r of ``s`` (so a subset of
    rows can be evaluated on its own). Key j is visible to query i iff
    j < valid_len and (not causal or j <= i).
    """
    s = s.copy()
    n_keys = s.shape[1]
    key_index = np.arange(n_keys)[None, :]
    hidden = key_index >= valid_len
    if causal:
        hidden = hidden | (key_index > row_index[:, None])
    s[np.broadcast_to(hidden, s.shape)] = -np.inf
    return s


def softmax_three_pass(s: np.ndarray):
    """Step 3: row-wise safe softmax in three passes over S.

    Returns (P, m, l). Rows with no finite score (fully masked) get P = 0,
    m = -inf and l = 0.
    """
    rows, cols = s.shape
    # pass 1: row maximum
    m = np.full(rows, -np.inf)
    for i in range(rows):
        m[i] = np.max(s[i]) if cols else -np.inf
    # pass 2: sum of exponentials relative to the row maximum
    l = np.zeros(rows)
    for i in range(rows):
        if np.isfinite(m[i]):
            l[i] = np.sum(np.exp(s[i] - m[i]))
    # pass 3: normalise
    p = np.zeros_like(s)
    for i in range(rows):
        if l[i] > 0.0:
            p[i] = np.exp(s[i] - m[i]) / l[i]
    return p, m, l


def _valid_len(seqlens, b: int, n: int) -> int:
    if seqlens is None:
        return n
    return int(min(max(int(np.asarray(seqlens)[b]), 0), n))


def attn_ref_head(q, k, v, scale: float, causal: bool = False, valid_len=None,
                  rows=None, return_p: bool = False):
    """Attention for one head, following steps 1-5 above.

    q: [N, d]; k, v: [N, d]. ``rows`` optionally restricts the query rows that
    are evaluated (the definition is row by row, so a subset of rows is
    computed exactly as in the full matrix). Query rows at or beyond
    ``valid_len`` are padding: O = 0, LSE = -inf.
    Returns (O [R, d], LSE [R]) and P [R, N] when ``return_p``.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    n = k.shape[0]
    valid = n if valid_len is None else int(valid_len)
    row_index = np.arange(q.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    qr = q[row_index]
    s = mask(scores(qr, k, scale), row_index, causal, valid)
    p, m, l = softmax_three_pass(s)
    o = p @ v
    with np.errstate(divide="ignore"):
        lse = np.where(l > 0.0, m + np.log(np.where(l > 0.0, l, 1.0)), -np.inf)
    padded = row_index >= valid
    o[padded] = 0.0
    lse[padded] = -np.inf
    if return_p:
        p[padded] = 0.0
        return o, lse, p
    return o, lse


def kv_head(h: int, H: int, H_kv: int) -> int:
    """K/V head read by query head h when H_kv K/V heads serve H query heads
    ([OpOpt] §五): consecutive runs of H // H_kv query heads share one."""
    if H_kv < 1 or H % H_kv:
        raise ValueError(f"{H_kv} K/V heads cannot serve {H} query heads")
    return h // (H // H_kv)


def attn_ref_fwd(q, k, v, scale: float, causal: bool = False, seqlens=None):
    """Forward over [B, H, N, d] queries and [B, H_kv, N, d] keys/values (any
    float type, upcast exactly to fp64; H_kv = H is plain multi-head attention).

    Returns (O [B,H,N,d] fp64, LSE [B,H,N] fp64 natural log).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, d = q.shape
    H_kv = k.shape[1]
    o = np.zeros((B, H, N, v.shape[-1]))
    lse = np.zeros((B, H, N))
    for b in range(B):
        L = _valid_len(seqlens, b, N)
        for h in range(H):
            g = kv_head(h, H, H_kv)
            o[b, h], lse[b, h] = attn_ref_head(q[b, h], k[b, g], v[b, g], scale, causal, L)
    return o, lse


def attn_ref_decode(q, k, v, scale: float, causal: bool = False, kv_lens=None, heads=None):
    """Decode: q [B, H, Nq, d] holds the last Nq positions of each sequence and
    k, v [B, H_kv, Nk, d] its keys and values, sequence b having L_b valid keys
    (kv_lens, default Nk). Steps 1-5 with row positions L_b - Nq + i.
    Returns (O [B,H,Nq,d], LSE [B,H,Nq]) fp64; ``heads`` optionally restricts
    the (b, h) pairs evaluated (the others are left 0)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, Nq, _ = q.shape
    H_kv, Nk = k.shape[1], k.shape[2]
    o = np.zeros((B, H, Nq, v.shape[-1]))
    lse = np.zeros((B, H, Nq))
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    for b, h in pairs:
        L = _valid_len(kv_lens, b, Nk)
        g = kv_head(h, H, H_kv)
        pos = L - Nq + np.arange(Nq)
        s = mask(scores(q[b, h], k[b, g], scale), pos, causal, L)
        p, m, l = softmax_three_pass(s)
        o[b, h] = p @ v[b, g]
        with np.errstate(divide="ignore"):
            lse[b, h] = np.where(l > 0.0, m + np.log(np.where(l > 0.0, l, 1.0)), -np.inf)
    return o, lse


def e4m3_decode(byte_values) -> np.ndarray:
    """The value of each FP8 E4M3 byte, by the format's definition."""
    u = np.asarray(byte_values, dtype=np.int64)
    sign = np.where(u >> 7, -1.0, 1.0)
    e = (u >> 3) & 15
    m = (u & 7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e - 7.0)
    sub = (m / 8.0) * np.exp2(-6.0)
    v = sign * np.where(e == 0, sub, normal)
    return np.where((e == 15) & ((u & 7) == 7), np.nan, v)


def dequant_fp8(x8, scale) -> np.ndarray:
    """FP8 cache [..., N, d] (uint8 bytes) and per-token scales [..., N] ->
    fp64 values x8 * scale."""
    b = x8.detach().cpu().numpy() if hasattr(x8, "detach") else np.asarray(x8)
    return e4m3_decode(b) * _f64(scale)[..., None]


def attn_ref_rows(q, k, v, b: int, h: int, rows, scale: float, causal: bool = False,
                  seqlens=None):
    """Oracle values for selected query rows of one (b, h) head of a [B,H,N,d] batch.

    Used to check full-size GPU runs on sampled outputs.
    """
    N = q.shape[2]
    L = _valid_len(seqlens, b, N)
    g = kv_head(h, q.shape[1], k.shape[1])
    return attn_ref_head(q[b, h], k[b, g], v[b, g], scale, causal, L, rows=rows)


def attn_ref_bwd_head(q, k, v, do, scale: float, causal: bool = False, valid_len=None):
    """Backward for one head by the chain rule, with P recomputed by the forward steps.

    Returns (dQ, dK, dV), each [N, d] fp64. Padded query rows and padded keys
    carry P = 0, so they receive zero gradient.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    _, _, p = attn_ref_head(q, k, v, scale, causal, valid_len, return_p=True)
    dv = p.T @ do                                     # dV = P^T dO
    dp = do @ v.T                                     # dP = dO V^T
    D = np.sum(dp * p, axis=1)                        # rowsum(dP o P)
    ds = p * (dp - D[:, None])                        # dS = P o (dP - D)
    dq = scale * (ds @ k)                             # S = scale Q K^T  =>  dQ = scale dS K
    dk = scale * (ds.T @ q)                           #                      dK = scale dS^T Q
    return dq, dk, dv


def attn_ref_bwd(q, k, v, do, scale: float, causal: bool = False, seqlens=None):
    """Backward over [B, H, N, d] queries and [B, H_kv, N, d] keys/values.
    Returns (dQ, dK, dV) fp64; dK and dV have the K/V shape, each K/V head
    summing the gradients of the query heads that read it."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, H, N, d = q.shape
    H_kv = k.shape[1]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        L = _valid_len(seqlens, b, N)
        for h in range(H):
            g = kv_head(h, H, H_kv)
            dq[b, h], dk_h, dv_h = attn_ref_bwd_head(
                q[b, h], k[b, g], v[b, g], do[b, h], scale, causal, L)
            dk[b, g] += dk_h
            dv[b, g] += dv_h
    return dq, dk, dv
