/*
 * attn.h - C ABI of an exact-attention library for AMD MI355X (gfx950).
 *
 * The library computes exact scaled dot-product attention
 *
 *     O = softmax(scale * Q K^T) V
 *
 * the FlashAttention way: Q is cut into row tiles, each tile streams over K/V
 * tiles held on chip, and an online-softmax state (running row max m, running
 * exponential sum l, unnormalised output accumulator) is rescaled by
 * exp(m_old - m_new) whenever the max grows, so the N x N score and probability
 * matrices never reach device memory. The result equals standard attention up
 * to floating-point rounding order.
 *
 * Pages this interface follows (cited by title):
 *  - "FlashAttention：从 Safe Softmax 到分块计算": §1 (the definition),
 *    §3.1-§3.2 (the (m, l, u) state and its merge rule), §5 (tiling), §5.2
 *    (causal mask: query i sees keys j <= i), §7 (forward loop, rows with no
 *    visible key in a tile are left untouched), §8 (a per-row log-sum-exp saved
 *    for a recompute-based backward).
 *  - "Attention 算子优化:从物化 N×N 矩阵到 FlashAttention 与 PagedAttention":
 *    §二 (a padded variable-length batch with a key-padding mask), §四 (causal
 *    block skipping; the backward recomputes P from Q, K, V).
 *  - the AIInfra FlashAttention note on dpshk.com: §2.1 (finite initial row
 *    max), §2.3 (dV = P^T dO, dS = P o (dP - rowsum(dP o P)), dP = dO V^T).
 *  - "Attention 算子优化..." §五 (grouped- and multi-query attention: several
 *    query heads share one K/V head; decode reads the whole K/V cache per new
 *    token and is bandwidth-bound).
 *  - "FlashAttention：从 Safe Softmax 到分块计算" §10 (splitting the K/V range
 *    across workgroups for decode, partial states combined by the §3.2 merge).
 *  - "Attention 算子优化..." §六 (FP8 E4M3 K/V cache with per-token scales,
 *    dequantised on chip; softmax and accumulation in fp32, products in 16-bit).
 *
 * Conventions shared by every entry point
 *  - Tensors are [B, H, N, d], contiguous, d fastest (element (b,h,i,c) sits at
 *    ((b*H + h)*N + i)*d + c). Q, K, V, O, dO, dQ, dK, dV share one shape.
 *  - All tensor pointers are DEVICE pointers. The caller allocates and owns
 *    every buffer; the library allocates nothing and keeps no state between
 *    calls (the one exception is attn_bwd_noalloc's static device scratch).
 *    Buffers must be 16-byte aligned.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *    null stream). No entry point synchronises the host.
 *  - Argument errors are detected on the host before anything is launched and
 *    are returned as a status; nothing is thrown across the ABI. A failed HIP
 *    launch returns ATTN_ERR_HIP.
 *  - seqlens: optional DEVICE int32 array [B]. Sequence b has L_b valid
 *    positions (queries and keys alike); positions >= L_b are padding. Query
 *    rows >= L_b are not computed: their O (and dQ) rows are written as 0 and
 *    their LSE as -inf; keys >= L_b get zero weight (and zero dK, dV). NULL
 *    means L_b = N for every b. Values must lie in [0, N]; values outside are
 *    clamped into [0, N] by the kernels (the host cannot check device memory
 *    without a synchronisation).
 *  - causal != 0 masks keys j > i for query i (top-left alignment, within
 *    each sequence's valid length). Both masks may be combined.
 *  - scale must be finite and > 0 (usually 1/sqrt(d)).
 */
#ifndef EXACT_ATTENTION_ATTN_H
#define EXACT_ATTENTION_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

struct ihipStream_t;
/* Same type as hipStream_t. */
typedef struct ihipStream_t* attn_stream_t;

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARG = 1, /* null pointer, non-positive size, bad scale, misalignment */
  ATTN_ERR_UNSUPPORTED = 2, /* valid request this library does not implement (e.g. d not in {64,128}) */
  ATTN_ERR_HIP = 3          /* a HIP runtime call or kernel launch failed */
} attn_status;

typedef enum {
  ATTN_DTYPE_F32 = 0,  /* fp32 storage, fp32 arithmetic throughout */
  ATTN_DTYPE_BF16 = 1, /* bf16 storage; products on bf16 MFMA with fp32 accumulation;
                          softmax in fp32; outputs rounded to bf16 (nearest-even) */
  ATTN_DTYPE_F16 = 2   /* fp16 storage, the same kernels on fp16 MFMA; P (<= 256 by the
                          lazy rescale) and dS are rounded to fp16 before their
                          products, so |dP - D| must stay below 65504 */
} attn_dtype;

/*
 * attn_fwd - attention forward.
 *
 * Defined by "FlashAttention：从 Safe Softmax 到分块计算" §1 (O = softmax(scale *
 * Q K^T) V, row-wise softmax), computed by its §5/§7 tiled loop with the §3.1
 * state and §3.2 merge; the mask of §5.2 (causal) and of "Attention 算子优化..."
 * §二 (key padding); the row log-sum-exp of §8.
 *
 * Computes, per (b, h) and valid query row i, O_i = sum_j P_ij V_j with
 * P_ij = exp(scale*q_i.k_j - LSE_i) over the visible keys j, and
 * LSE_i = ln(sum_j exp(scale*q_i.k_j)) (natural log).
 *
 *  q, k, v   [B,H,N,d] of `dtype`, read only.
 *  o         [B,H,N,d] of `dtype`, written (padded rows written as 0).
 *  lse       [B,H,N] fp32, written; may be NULL when no backward will follow.
 *  B, H, N   >= 1.   d: 64 or 128 (ATTN_ERR_UNSUPPORTED otherwise).
 *
 * The 16-bit forwards are deterministic: the same inputs give bit-identical outputs.
 */
attn_status attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int H, int N, int d, attn_dtype dtype, float scale, int causal,
                     const int32_t* seqlens, attn_stream_t stream);

/*
 * attn_fwd_gqa - attn_fwd with grouped K/V heads ("Attention 算子优化..." §五).
 *
 * q, o are [B,H,N,d]; k, v are [B,H_kv,N,d]. Query head h attends with K/V
 * head h / (H / H_kv): H_kv = H is attn_fwd, H_kv = 1 is multi-query
 * attention. H_kv must divide H (ATTN_ERR_INVALID_ARG otherwise). All other
 * arguments and outputs as for attn_fwd.
 */
attn_status attn_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
                         int B, int H, int H_kv, int N, int d, attn_dtype dtype, float scale,
                         int causal, const int32_t* seqlens, attn_stream_t stream);

/*
 * attn_fwd_fp8 - attention forward over FP8 inputs, both products on the FP8
 * matrix cores ("FlashAttention：从 Safe Softmax 到分块计算" §9.2: an FP8 path
 * handles scaling, accumulation and error control; "Attention 算子优化..."
 * §六: softmax and accumulation stay in fp32).
 *
 *  q8        [B,H,N,d] bytes, OCP FP8 E4M3 (as for attn_decode_fp8kv), read only.
 *  k8, v8    [B,H_kv,N,d] bytes, E4M3, read only; H_kv divides H as for
 *            attn_fwd_gqa.
 *  q_scale   [B,H,N] fp32 per-token scales, k_scale and v_scale [B,H_kv] fp32
 *            per-head scales: the inputs are Q_i = q8_i * q_scale_i,
 *            K = k8 * k_scale, V = v8 * v_scale, and the result is attn_fwd_gqa
 *            of those values. Scales must be finite and > 0 (the kernel
 *            takes the row max of the unscaled scores).
 *  o         [B,H,N,d] in out_dtype (ATTN_DTYPE_BF16 or ATTN_DTYPE_F16;
 *            ATTN_DTYPE_F32 gives ATTN_ERR_UNSUPPORTED).
 *  lse, B, H, N, scale, causal, seqlens, stream: as for attn_fwd.
 *  d         128 (ATTN_ERR_UNSUPPORTED otherwise).
 * Precision: the scores are exact products of E4M3 values summed in fp32 on
 * the matrix cores; the LSE uses the fp32 weights (as attn_fwd). For the V
 * product each unnormalised weight w (<= 2^8) is rounded to E4M3 (nearest
 * even): error <= 2^-4 w for w >= 2^-6, <= 2^-10 below. So
 * |O_i - O_exact_i| <= v_scale * sum_j err_ij |v8_j| / l_i, plus the rounding
 * of O to out_dtype, where l_i is the row's sum of weights measured against a
 * reference no larger than the row max (so l_i >= 1).
 */
attn_status attn_fwd_fp8(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8,
                         const float* q_scale, const float* k_scale, const float* v_scale,
                         void* o, float* lse, int B, int H, int H_kv, int N, int d,
                         attn_dtype out_dtype, float scale, int causal, const int32_t* seqlens,
                         attn_stream_t stream);

/*
 * attn_bwd_workspace_bytes - device workspace that attn_bwd needs for these sizes
 * (it holds -D_i = -rowsum(dO_i o O_i) and LSE_i * log2(e), fp32 [B,H,N] each).
 * Returns 0 for invalid sizes.
 */
size_t attn_bwd_workspace_bytes(int B, int H, int N, int d, attn_dtype dtype);

/*
 * attn_bwd - recompute-based attention backward.
 *
 * Defined by the AIInfra FlashAttention note on dpshk.com §2.3 (dV = P^T dO,
 * dP = dO V^T, dS = P o (dP - rowsum(dP o P))) and "Attention 算子优化..." §四
 * (P recomputed tile by tile from Q, K and the saved LSE instead of being
 * stored); the scale factor of dQ and dK follows from S = scale * Q K^T.
 *
 * Given the forward's inputs q, k, v, its output o and lse, and the upstream
 * gradient dO, recomputes P tile by tile from q, k and lse and writes
 *   dV = P^T dO,   dP = dO V^T,   D_i = rowsum(dO_i o O_i) (= rowsum(dP o P)),
 *   dS = P o (dP - D),   dQ = scale * dS K,   dK = scale * dS^T Q.
 *
 *  q, k, v, o, dO   [B,H,N,d] of `dtype`, read only.
 *  lse              [B,H,N] fp32 from attn_fwd with the same arguments.
 *  dq, dk, dv       [B,H,N,d] of `dtype`, written (fully overwritten).
 *  workspace        device buffer of at least attn_bwd_workspace_bytes(...)
 *                   bytes, 256-byte aligned; contents on entry are ignored.
 *  workspace_bytes  its size; smaller than required gives ATTN_ERR_INVALID_ARG.
 * ATTN_DTYPE_BF16 and ATTN_DTYPE_F16 are implemented (ATTN_ERR_UNSUPPORTED for fp32).
 * Deterministic: no atomics are used.
 */
attn_status attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO,
                     const float* lse, void* dq, void* dk, void* dv, void* workspace,
                     size_t workspace_bytes, int B, int H, int N, int d, attn_dtype dtype,
                     float scale, int causal, const int32_t* seqlens, attn_stream_t stream);

/*
 * attn_bwd_gqa - attn_bwd with grouped K/V heads (see attn_fwd_gqa).
 *
 * q, o, dO, dq are [B,H,N,d]; k, v, dk, dv are [B,H_kv,N,d]. dK and dV of a
 * K/V head are the sums of the contributions of the H / H_kv query heads that
 * read it, accumulated in a fixed order (deterministic). The workspace is
 * attn_bwd_workspace_bytes(B, H, N, d, dtype) with the query head count H.
 */
attn_status attn_bwd_gqa(const void* q, const void* k, const void* v, const void* o,
                         const void* dO, const float* lse, void* dq, void* dk, void* dv,
                         void* workspace, size_t workspace_bytes, int B, int H, int H_kv, int N,
                         int d, attn_dtype dtype, float scale, int causal,
                         const int32_t* seqlens, attn_stream_t stream);

/*
 * attn_bwd_noalloc - attn_bwd_gqa without a workspace argument, for callers
 * that cannot allocate device memory at all (code under HIP graph capture,
 * tight serving or training loops, harnesses that forbid allocation).
 *
 * The workspace of attn_bwd_gqa (-D and LSE * log2(e), fp32 [B,H,N] each)
 * lives instead in a static device array of ATTN_NOALLOC_SCRATCH_BYTES bytes
 * that the library holds on each GPU it runs on until the process ends; its
 * device address is looked up once per device (on the first call with that
 * device current) and kept. The call allocates nothing, neither directly nor
 * through any library routine. Every other argument, output and error is as
 * for attn_bwd_gqa (H_kv = H is plain attn_bwd), and the results are
 * bit-identical to it: the same kernels run.
 *
 * Limit: B * H * N <= ATTN_NOALLOC_MAX_ROWS (2^21 query rows, e.g. B=2, H=32,
 * N=32768); larger sizes return ATTN_ERR_UNSUPPORTED before anything is
 * launched (attn_last_error() names the limit).
 * Concurrency: every call on one GPU uses that GPU's one scratch array. Calls
 * on the same stream are ordered and safe; calls that may overlap on one GPU
 * (different streams, or different host threads without ordering) race on the
 * scratch and give undefined results. The scratch needs no clearing: each
 * call writes every entry it reads before reading it.
 */
#define ATTN_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
#define ATTN_NOALLOC_MAX_ROWS ((long long)1 << 21)
attn_status attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                             const void* dO, const float* lse, void* dq, void* dk, void* dv,
                             int B, int H, int H_kv, int N, int d, attn_dtype dtype, float scale,
                             int causal, const int32_t* seqlens, attn_stream_t stream);

/*
 * attn_decode_workspace_bytes - device workspace attn_decode needs for these
 * sizes and this num_splits (0 = automatic; the same value must be passed to
 * attn_decode). It holds each split's partial state: fp32 O [B*H*Nq][splits][d]
 * and (m, l) [B*H*Nq][splits][2]. Returns 0 for invalid or unsupported sizes.
 */
size_t attn_decode_workspace_bytes(int B, int H, int H_kv, int Nq, int Nk, int d,
                                   attn_dtype dtype, int num_splits);

/*
 * attn_decode - split-KV attention for a few new queries against a long K/V
 * cache (decode).
 *
 *  q         [B,H,Nq,d] of `dtype` (bf16 or fp16), read only.
 *  k, v      [B,H_kv,Nk,d] of `dtype`, read only; query head h reads K/V head
 *            h / (H / H_kv) as in attn_fwd_gqa.
 *  o         [B,H,Nq,d] of `dtype`, written.
 *  lse       [B,H,Nq] fp32 natural-log log-sum-exp, written; may be NULL.
 *  kv_lens   optional DEVICE int32 [B]: sequence b has L_b valid keys (clamped
 *            into [0, Nk]); NULL means Nk for every b.
 *  causal    the Nq queries of sequence b are its last Nq positions,
 *            L_b - Nq .. L_b - 1; with causal != 0 query i sees keys
 *            j <= L_b - Nq + i (with Nq = L_b: the mask of attn_fwd), otherwise
 *            every valid key. A query that sees no key gets O = 0, LSE = -inf.
 *  num_splits  splits of the keys per (batch, K/V head), split s of S
 *            taking the 32-key chunks s, s + S, s + 2S, ...; 0 picks a count
 *            that gives about 512 workgroups for one-wave workgroups over a
 *            16-bit cache, about 768 for query columns in pairs of 32-column
 *            blocks (two-wave workgroups) and about 1024 over an FP8 cache.
 *            Results do not depend on it beyond rounding.
 *  workspace device buffer of attn_decode_workspace_bytes(...) bytes, 256-byte
 *            aligned; contents on entry are ignored.
 *
 * Two launches on `stream`: the split kernel (partial softmax states) and the
 * merge. fp32 and d outside {64, 128} return ATTN_ERR_UNSUPPORTED.
 */
attn_status attn_decode(const void* q, const void* k, const void* v, void* o, float* lse,
                        int B, int H, int H_kv, int Nq, int Nk, int d, attn_dtype dtype,
                        float scale, int causal, const int32_t* kv_lens, int num_splits,
                        void* workspace, size_t workspace_bytes, attn_stream_t stream);

/*
 * attn_decode_fp8kv - attn_decode over an FP8 K/V cache.
 *
 *  k8, v8    [B,H_kv,Nk,d] bytes, OCP FP8 E4M3 (sign, 4 exponent bits with bias
 *            7, 3 mantissa bits; 0x7F/0xFF are NaN, no infinities), read only.
 *  k_scale, v_scale  [B,H_kv,Nk] fp32 per-token scales: the keys and values
 *            are K_j = k8_j * k_scale_j and V_j = v8_j * v_scale_j.
 * q, o, lse, dtype (of q and o), kv_lens, causal, num_splits and the workspace
 * (attn_decode_workspace_bytes with the same arguments) are as for attn_decode.
 * d is 64 or 128 as for attn_decode. HBM and LDS carry the 8-bit K/V; each
 * MFMA operand is widened to the 16-bit format on chip (exact), the scales are
 * applied in fp32 to the scores and to the weights before the V product.
 * With fp16 queries the weights (each <= 1: the running max is exact there)
 * times v_scale are rounded to fp16, so v_scale must stay below 65504; with
 * bf16 queries the fp32 exponent range applies.
 */
attn_status attn_decode_fp8kv(const void* q, const uint8_t* k8, const uint8_t* v8,
                              const float* k_scale, const float* v_scale, void* o, float* lse,
                              int B, int H, int H_kv, int Nq, int Nk, int d, attn_dtype dtype,
                              float scale, int causal, const int32_t* kv_lens, int num_splits,
                              void* workspace, size_t workspace_bytes, attn_stream_t stream);

/* Human-readable name of a status code (static storage, never NULL). */
const char* attn_status_string(attn_status s);

/* Message of the last HIP error seen by this library on the calling thread
 * ("" if none). */
const char* attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_ATTENTION_ATTN_H */
