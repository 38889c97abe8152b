// Attention backward kernels for gfx950: recompute P from Q, K and the saved
// row log-sum-exp instead of storing it.
//
// Pages cited (by title):
//   [SafeSoftmax] "FlashAttention：从 Safe Softmax 到分块计算"
//   [OpOpt]       "Attention 算子优化:从物化 N×N 矩阵到 FlashAttention 与 PagedAttention"
//   [AIInfra]     the AIInfra FlashAttention note on dpshk.com
//
// The forward saves LSE_i per query row ([SafeSoftmax] §8); the backward
// re-reads Q, K, V and recomputes each tile of P = exp(scale*Q K^T - LSE)
// ([OpOpt] §四: recompute instead of storing the N x N matrix). The gradient
// formulas are those of [AIInfra] §2.3: dV = P^T dO, dP = dO V^T,
// dS = P o (dP - rowsum(dP o P)); rowsum(dP o P) equals rowsum(dO o O)
// (sum_j P_ij dO_i.V_j = dO_i.O_i), which is what the first kernel computes.
// With S = scale*Q K^T, dQ = scale*dS K and dK = scale*dS^T Q.
//
// Three launches on one stream:
//   bwd_pre:  -delta_i = -rowsum(dO_i o O_i) and LSE_i*log2(e)  (HBM-bound)
//   bwd_dkdv: one workgroup per 128 keys; loops over the query tiles that can
//             see those keys, accumulating dK and dV in registers
//   bwd_dq:   one workgroup per 128 queries; loops over the key tiles they
//             see, accumulating dQ in registers (no atomics: deterministic)
// Tiles reach LDS through direct buffer->LDS loads into XOR-swizzled layouts,
// one LDS array per stage and tensor, as in the forward kernel. Every load is
// bounded by the sequence's valid length L, so padded positions are never
// read: they enter the products as zeros.
#include "attn_common.h"
#include "attn_kernels.h"
#include "attn_sched.h"
#include "attn_tile.h"

#include <math.h>

namespace attn {

namespace {

__device__ __forceinline__ int seq_len(const BwdArgs& a, int b) {
  return a.seqlens ? min(max(a.seqlens[b], 0), a.N) : a.N;
}

// ---------------------------------------------------------------------------
// delta_i = sum_d dO_i[d] * O_i[d] in fp32, stored negated (the dK/dV kernel
// starts its dP accumulators at -delta, so dP - delta comes out of the MFMA),
// and lse2_i = LSE_i * log2(e); both 0 for padded rows.
// ---------------------------------------------------------------------------
template <int D, bool F16>
__global__ void __launch_bounds__(256) bwd_pre_kernel(BwdArgs a) {
  constexpr int TPR = D / 8, RPB = 256 / TPR;
  const int tid = threadIdx.x;
  const long long total = (long long)a.B * a.H * a.N;
  const long long row = (long long)blockIdx.x * RPB + tid / TPR;
  const int c = tid % TPR;
  float part = 0.f;
  bool valid = false;
  if (row < total) {
    const int bh = (int)(row / a.N), q = (int)(row % a.N);
    valid = q < seq_len(a, bh / a.H);
    if (valid) {
      const u32x4 o = gload16((const e16_t*)a.o + row * D + c * 8);
      const u32x4 g = gload16((const e16_t*)a.dO + row * D + c * 8);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        part += unpack_lo<F16>(o[i]) * unpack_lo<F16>(g[i]) + unpack_hi<F16>(o[i]) * unpack_hi<F16>(g[i]);
    }
  }
#pragma unroll
  for (int m = TPR / 2; m >= 1; m >>= 1) part += __shfl_xor(part, m, TPR);
  if (row < total && c == 0) {
    a.delta[row] = valid ? -part : 0.f;
    a.lse2[row] = valid ? a.lse[row] * kLog2e : 0.f;
  }
}

// Output-row staging for the epilogues: 32 rows of D 16-bit values per wave,
// 16-byte chunk c of row r at chunk c ^ (r mod chunks-per-row), so that the
// 8-byte accumulator writes and the 16-byte row reads spread over the banks.
template <int D>
struct RowStage {
  static constexpr int RB = D * 2, CPRO = RB / 16, RPI = 64 / CPRO;
  __device__ static __forceinline__ uint32_t off(int r, int byte) {
    return (uint32_t)(r * RB + ((((byte >> 4) ^ (r & (CPRO - 1))) << 4) | (byte & 15)));
  }
};

// ---------------------------------------------------------------------------
// dK, dV: workgroup = 4 waves x 32 keys. Each wave keeps its K and V rows in
// VGPRs (B operands of S = Q K^T and dP = dO V^T) and accumulates dK^T, dV^T.
// Query tiles of 64 rows (Q, dO, and the rows' lse2 and delta) are
// double-buffered in LDS and processed as two 32-row sub-blocks:
//   S  (q x key)   = Q  K^T        A = Q rows (LDS),   B = K (VGPR)
//   P              = exp2(S*scale*log2e - LSE*log2e), masked
//   dV^T (d x key) += dO^T P       A = dO^T (transposing LDS read), B = P
//   dP (q x key)   = dO V^T        A = dO rows (LDS),  B = V (VGPR)
//   dS             = P o (dP - delta)  (dP's accumulator starts at -delta)
//   dK^T (d x key) += Q^T dS       A = Q^T (transposing LDS read),  B = dS
// The products are built from v_mfma_f32_16x16x32 blocks (as in the forward,
// for the clock the power limit allows; measured 6% faster for this kernel
// than 32x32x16 blocks). Lane l: c = l % 16, g = l / 16, keys kw + c and
// kw + 16 + c. The score accumulators hold queries 16*qb + 4*g + i of a
// sub-block, so one 16-byte read of the statistics tile gives a lane its four
// rows' LSE or delta (the latter is the dP accumulator's start). For the dV
// and dK products the MFMA k index 8g + e stands for query 4g + e (e < 4) or
// 16 + 4g + e - 4 of the sub-block, so P and dS are packed in place and dO^T,
// Q^T are read in that order. Q and dO tiles, read both ways, use the
// TILE_T16 layout.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL, bool F16>
__device__ __forceinline__ void bwd_dkdv_body(const BwdArgs& a) {
  constexpr int BN = 128, BM = 64;
  constexpr int TILE = BM * D * 2;
  constexpr int CH = D / 8;
  constexpr int DC = D / 32, DBK = D / 16;

  __shared__ __attribute__((aligned(1024))) char q0_[TILE], q1_[TILE], o0_[TILE], o1_[TILE];
  __shared__ __attribute__((aligned(256))) char st0_[2 * BM * 4], st1_[2 * BM * 4];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c16 = lane & 15, g = lane >> 4;
  const int N = a.N;
  const int nkt = (N + BN - 1) / BN;
  int bkv, kt;
  tile_order(blockIdx.x, nkt, a.B * a.H_kv, 1, false, bkv, kt);
  const int b = bkv / a.H_kv, G = a.H / a.H_kv;
  const int hq0 = b * a.H + (bkv % a.H_kv) * G;  // first query head of the group
  const int L = seq_len(a, b);
  const int n0 = kt * BN;
  const size_t kvoff = (size_t)bkv * N * D;
  const e16_t* __restrict__ Kh = (const e16_t*)a.k + kvoff;
  const e16_t* __restrict__ Vh = (const e16_t*)a.v + kvoff;
  e16_t* __restrict__ dKh = (e16_t*)a.dk + kvoff;
  e16_t* __restrict__ dVh = (e16_t*)a.dv + kvoff;
  const u32x4 zero4 = {0u, 0u, 0u, 0u};

  if (n0 >= L) {  // every key of this tile is padding: zero gradients
    const int rows = min(BN, N - n0);
    for (int c = tid; c < rows * CH; c += 256) {
      const size_t off = (size_t)(n0 + c / CH) * D + (c % CH) * 8;
      gstore16(dKh + off, zero4);
      gstore16(dVh + off, zero4);
    }
    return;
  }

  const int kw = n0 + wave * 32;                    // first key of this wave
  constexpr int RB = RowStage<D>::RB, CPRO = RowStage<D>::CPRO, RPI = RowStage<D>::RPI;
  auto stage_off = [](int r, int byte) { return RowStage<D>::off(r, byte); };
  const int keys[2] = {kw + c16, kw + 16 + c16};    // this lane's keys (kb = 0, 1)
  const int q_begin = CAUSAL ? (n0 / BM) * BM : 0;
  const int nqt = ((L - q_begin + BM - 1) / BM + 1) & ~1;
  const float c2 = a.scale_log2;

  TileDma<D, BM, 4, TILE_T16> qdma((const e16_t*)a.q, L, wave, lane);
  TileDma<D, BM, 4, TILE_T16> odma((const e16_t*)a.dO, L, wave, lane);
  const float* lse2_h = a.lse2;
  const float* delta_h = a.delta;
  auto load_tile = [&](int q0, int st) {
    qdma.load(lds_base(st ? q1_ : q0_), q0);
    odma.load(lds_base(st ? o1_ : o0_), q0);
    const int odd = wave & 1;
    vec64_dma(lds_base(st ? st1_ : st0_) + odd * (BM * 4), odd ? delta_h : lse2_h, L, q0, lane);
  };

  // K^T, V^T as B operands: key keys[kb], d = 32*dc + 8*g .. +7.
  e16x8 kreg[2][DC], vreg[2][DC];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) {
      const size_t off = (size_t)keys[kb] * D + dc * 32 + g * 8;
      kreg[kb][dc] = as_e16x8(keys[kb] < L ? gload16(Kh + off) : zero4);
      vreg[kb][dc] = as_e16x8(keys[kb] < L ? gload16(Vh + off) : zero4);
    }
  // LDS offsets: row operands (query 16*qb + c, columns 32*dc + 8*g ..) and
  // transposed operands (rows 4*g + c/4 (+16), columns 16*db + 4*(c%4) ..);
  // whole 16-row blocks leave the layout unchanged.
  uint32_t roff[DC], toff[DBK];
#pragma unroll
  for (int dc = 0; dc < DC; ++dc) roff[dc] = (uint32_t)tile_off_lay<D, TILE_T16>(c16, dc * 32 + g * 8);
#pragma unroll
  for (int db = 0; db < DBK; ++db)
    toff[db] = (uint32_t)tile_off_lay<D, TILE_T16>(4 * g + (c16 >> 2), db * 16 + 4 * (c16 & 3));

  f32x4 dk[DBK][2], dv[DBK][2];  // dK^T, dV^T blocks (d 16*db + 4*g + i, key keys[kb])
#pragma unroll
  for (int db = 0; db < DBK; ++db)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) { dk[db][kb][i] = 0.f; dv[db][kb][i] = 0.f; }

  // Statistics and Q/dO row operands of sub-block sb of the tile in stage st:
  // queries 32*sb + 16*qb + 4*g + i in the accumulators.
  auto read_stats = [&](int st, int sb, f32x4* l4, f32x4* d4) {
    const lds_t* lse_t = lds_base(st ? st1_ : st0_);
    const lds_t* del_t = lse_t + BM * 4;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int rl = sb * 32 + qb * 16 + g * 4;
      l4[qb] = *(const ATTN_LDS f32x4*)(lse_t + rl * 4);
      d4[qb] = *(const ATTN_LDS f32x4*)(del_t + rl * 4);
    }
  };
  auto read_rows = [&](int st, int sb, e16x8 (*qo)[DC][2]) {  // qo[qb][dc] = {Q, dO}
    const lds_t* Qt = lds_base(st ? q1_ : q0_);
    const lds_t* dOt = lds_base(st ? o1_ : o0_);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) {
        const int r0 = (sb * 32 + qb * 16) * (D * 2);
        qo[qb][dc][0] = as_e16x8(lds_load16(Qt + r0 + roff[dc]));
        qo[qb][dc][1] = as_e16x8(lds_load16(dOt + r0 + roff[dc]));
      }
  };
  // Sub-block A's operands are read one phase early: the step before issues
  // them under its last MFMAs (the loop prologues issue the first ones).
  e16x8 ra[2][DC][2];
  f32x4 lA[2], dA[2];

  auto step = [&](int t, const int st, const bool MASKED) {
    const int qt0 = q_begin + t * BM;
    load_tile(qt0 + BM, st ^ 1);
    const lds_t* Qt = lds_base(st ? q1_ : q0_);
    const lds_t* dOt = lds_base(st ? o1_ : o0_);

    // S = Q K^T and dP - delta = dO V^T - delta (the accumulator starts at -delta).
    auto scores = [&](e16x8 (*qo)[DC][2], const f32x4* d4, f32x4 (*s)[2], f32x4 (*dp)[2]) {
#pragma unroll
      for (int dc = 0; dc < DC; ++dc)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
            s[qb][kb] = mfma16x16x32<F16>(qo[qb][dc][0], kreg[kb][dc], dc == 0 ? z : s[qb][kb]);
            dp[qb][kb] = mfma16x16x32<F16>(qo[qb][dc][1], vreg[kb][dc], dc == 0 ? d4[qb] : dp[qb][kb]);
          }
    };
    // P and dS of sub-block sb, packed as B operands: k index 8g + e stands for
    // query 32*sb + 4g + e (e < 4, block qb = 0) or 32*sb + 16 + 4g + e - 4.
    auto softmax_grad = [&](int sb, f32x4 (*s)[2], f32x4 (*dp)[2], const f32x4* l4, e16x8* pb,
                            e16x8* gb) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          // query qt0 + 32sb + 16qb + 4g + i sees key keys[kb] iff i >= lo
          const int lo = keys[kb] - (qt0 + sb * 32 + qb * 16 + 4 * g);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float p = fast_exp2(fmaf(s[qb][kb][i], c2, -l4[qb][i]));
            if (MASKED) p = i >= lo ? p : 0.f;
            s[qb][kb][i] = p;
            dp[qb][kb][i] = p * dp[qb][kb][i];
          }
        }
        const u32x4 wp = {pack2<F16>(s[0][kb][0], s[0][kb][1]), pack2<F16>(s[0][kb][2], s[0][kb][3]),
                          pack2<F16>(s[1][kb][0], s[1][kb][1]), pack2<F16>(s[1][kb][2], s[1][kb][3])};
        const u32x4 wg = {pack2<F16>(dp[0][kb][0], dp[0][kb][1]), pack2<F16>(dp[0][kb][2], dp[0][kb][3]),
                          pack2<F16>(dp[1][kb][0], dp[1][kb][1]), pack2<F16>(dp[1][kb][2], dp[1][kb][3])};
        pb[kb] = as_e16x8(wp);
        gb[kb] = as_e16x8(wg);
      }
    };
    auto read_tr = [&](int sb, e16x8 (*qo)[2]) {  // qo[db] = {dO^T, Q^T}
#pragma unroll
      for (int db = 0; db < DBK; ++db) {
        const int r0 = sb * 32 * (D * 2) + toff[db];
        qo[db][0] = join_e16x8(lds_load_tr16(dOt + r0), lds_load_tr16(dOt + r0 + 16 * (D * 2)));
        qo[db][1] = join_e16x8(lds_load_tr16(Qt + r0), lds_load_tr16(Qt + r0 + 16 * (D * 2)));
      }
    };
    auto grad_mfma = [&](e16x8 (*qo)[2], const e16x8* pb, const e16x8* gb) {
#pragma unroll
      for (int db = 0; db < DBK; ++db)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          dv[db][kb] = mfma16x16x32<F16>(qo[db][0], pb[kb], dv[db][kb]);
          dk[db][kb] = mfma16x16x32<F16>(qo[db][1], gb[kb], dk[db][kb]);
        }
    };

    // The tile is two 32-query sub-blocks A (rows 0-31) and B (rows 32-63),
    // laid out in phases separated by scheduling fences so that the exp/VALU
    // work of one sub-block runs under the MFMAs of the other and every LDS
    // read is issued a phase ahead of the MFMA that consumes it.
    constexpr int PM = 8 * DC;  // MFMAs per phase
    // Phase 1: S_A, dP_A - delta_A; reads: statistics and row operands of B.
    f32x4 sA[2][2], dpA[2][2];
    scores(ra, dA, sA, dpA);
    f32x4 lB[2], dB[2];
    read_stats(st, 1, lB, dB);
    e16x8 rb[2][DC][2];
    read_rows(st, 1, rb);
#pragma unroll
    for (int i = 0; i < PM / 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    // Phase 2: S_B, dP_B - delta_B; VALU of A; reads: transposed operands of A.
    f32x4 sB[2][2], dpB[2][2];
    scores(rb, dB, sB, dpB);
    e16x8 pA[2], gA[2];
    softmax_grad(0, sA, dpA, lA, pA, gA);
    e16x8 trA[DBK][2];
    read_tr(0, trA);
#pragma unroll
    for (int i = 0; i < PM / 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x002 | 0x400, 5, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    // Phase 3: dV, dK += sub-block A; VALU of B; reads: transposed operands of B.
    grad_mfma(trA, pA, gA);
    e16x8 pB[2], gB[2];
    softmax_grad(1, sB, dpB, lB, pB, gB);
    e16x8 trB[DBK][2];
    read_tr(1, trB);
#pragma unroll
    for (int i = 0; i < PM / 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x002 | 0x400, 5, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    // The next tile has landed (this wave's loads, then every wave's) and no
    // wave reads this stage any more; phase 4 reads nothing from LDS.
    dma_wait();
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    // Phase 4: dV, dK += sub-block B; reads: sub-block A of the next tile.
    grad_mfma(trB, pB, gB);
    read_stats(st ^ 1, 0, lA, dA);
    read_rows(st ^ 1, 0, ra);
#pragma unroll
    for (int i = 0; i < PM / 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      if (i < 10) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // Heads of the group one after another; the causal diagonal pairs of all
  // heads run first and the unmasked tiles after, so each loop body holds one
  // variant of the tile code (with both in one loop the register allocator
  // went past its budget and spilled).
  auto set_head = [&](int hg) {
    const size_t qoff = (size_t)(hq0 + hg) * N;
    qdma.head = (const e16_t*)a.q + qoff * D;
    odma.head = (const e16_t*)a.dO + qoff * D;
    lse2_h = a.lse2 + qoff;
    delta_h = a.delta + qoff;
  };
  // Every loop iteration starts by filling stage 0 once every wave is past
  // its last read of it (the early reads of the step before, whose values
  // are not used), then reads sub-block A of that tile.
  if (CAUSAL) {  // query tiles [n0, n0 + 128): the diagonal
    for (int hg = 0; hg < G; ++hg) {
      set_head(hg);
      __syncthreads();
      load_tile(q_begin, 0);
      dma_wait();
      __syncthreads();
      read_stats(0, 0, lA, dA);
      read_rows(0, 0, ra);
      step(0, 0, true);
      step(1, 1, true);
    }
  }
  const int t0 = CAUSAL ? 2 : 0;
  for (int hg = 0; hg < G; ++hg) {
    set_head(hg);
    __syncthreads();
    load_tile(q_begin + t0 * BM, 0);
    dma_wait();
    __syncthreads();
    read_stats(0, 0, lA, dA);
    read_rows(0, 0, ra);
    for (int t = t0; t < nqt; t += 2) {
      step(t, 0, false);
      step(t + 1, 1, false);
    }
  }

  // Each wave stages its 32 dK and dV rows in the idle Q/dO stage buffers
  // (the last step's barrier has passed, no load is in flight) and stores
  // whole rows.
  lds_t* const kst_o = lds_base(wave < 2 ? q0_ : o0_) + (wave & 1) * (32 * RB);
  lds_t* const vst_o = lds_base(wave < 2 ? q1_ : o1_) + (wave & 1) * (32 * RB);
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const bool kv = keys[kb] < L;
    const int r = kb * 16 + c16;
#pragma unroll
    for (int db = 0; db < DBK; ++db) {
      const u32x2 wk = {kv ? pack2<F16>(dk[db][kb][0] * a.scale, dk[db][kb][1] * a.scale) : 0u,
                        kv ? pack2<F16>(dk[db][kb][2] * a.scale, dk[db][kb][3] * a.scale) : 0u};
      const u32x2 wv = {kv ? pack2<F16>(dv[db][kb][0], dv[db][kb][1]) : 0u,
                        kv ? pack2<F16>(dv[db][kb][2], dv[db][kb][3]) : 0u};
      lds_store8(kst_o + stage_off(r, db * 32 + g * 8), wk);
      lds_store8(vst_o + stage_off(r, db * 32 + g * 8), wv);
    }
  }
#pragma unroll
  for (int it = 0; it < 32 / RPI; ++it) {
    const int r = it * RPI + lane / CPRO, c = lane % CPRO;
    const u32x4 wk = lds_load16(kst_o + stage_off(r, c * 16));
    const u32x4 wv = lds_load16(vst_o + stage_off(r, c * 16));
    if (kw + r < N) {
      gstore16(dKh + (size_t)(kw + r) * D + c * 8, wk);
      gstore16(dVh + (size_t)(kw + r) * D + c * 8, wv);
    }
  }
}

// ---------------------------------------------------------------------------
// dQ: workgroup = 4 waves x 32 queries; Q and dO rows stay in VGPRs (B
// operands), K/V tiles of 64 keys are double-buffered in LDS. The products are
// built from v_mfma_f32_16x16x32 blocks (as in the forward, for the clock the
// power limit allows; measured 7% faster for this kernel than 32x32x16
// blocks). Lane l: c = l % 16, g = l / 16, queries qw + c and qw + 16 + c:
//   S^T  (key x q) = K Q^T     A = K rows (LDS),  B = Q (VGPR)
//   dP^T (key x q) = V dO^T    A = V rows (LDS),  B = dO (VGPR)
//   dS^T = P^T o (dP^T - delta)   (LSE and delta are per-query scalars)
//   dQ^T (d x q)  += K^T dS^T  A = K^T (transposing LDS read), B = dS^T
// Each K or V operand read feeds both 16-query blocks. The score accumulators
// hold keys 16*kb + 4*g + i; for the dQ product the MFMA k index 8g + e stands
// for key 32h + 4g + e (e < 4) or 32h + 16 + 4g + e - 4 of half h, so dS^T is
// packed in place and K^T is read in that key order. V tiles use the
// TILE_K16 layout; K tiles, read both ways, use TILE_T16 (conflict-free for
// the transposing read).
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL, bool F16>
__device__ __forceinline__ void bwd_dq_body(const BwdArgs& a) {
  constexpr int BM = 128, BN = 64;
  constexpr int TILE = BN * D * 2;
  constexpr int CH = D / 8;
  constexpr int DC = D / 32, DBK = D / 16;

  __shared__ __attribute__((aligned(1024))) char k0_[TILE], v0_[TILE], k1_[TILE], v1_[TILE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c16 = lane & 15, g = lane >> 4;
  const int N = a.N;
  const int nm = (N + BM - 1) / BM;
  int bh, mt;
  tile_order(blockIdx.x, nm, a.B * a.H, a.H / a.H_kv, CAUSAL, bh, mt);
  const int L = seq_len(a, bh / a.H);
  const int m0 = mt * BM;
  const size_t hoff = (size_t)bh * N * D;
  const size_t kvoff = (size_t)((bh / a.H) * a.H_kv + (bh % a.H) / (a.H / a.H_kv)) * N * D;
  const e16_t* __restrict__ Qh = (const e16_t*)a.q + hoff;
  const e16_t* __restrict__ dOh = (const e16_t*)a.dO + hoff;
  e16_t* __restrict__ dQh = (e16_t*)a.dq + hoff;
  const u32x4 zero4 = {0u, 0u, 0u, 0u};

  if (m0 >= L) {
    const int rows = min(BM, N - m0);
    for (int c = tid; c < rows * CH; c += 256)
      gstore16(dQh + (size_t)(m0 + c / CH) * D + (c % CH) * 8, zero4);
    return;
  }

  const int qw = m0 + wave * 32;
  const int qq[2] = {qw + c16, qw + 16 + c16};
  const bool qv[2] = {qq[0] < L, qq[1] < L};
  const int kv_end = CAUSAL ? min(L, m0 + BM) : L;
  const int nt = ((kv_end + BN - 1) / BN + 1) & ~1;
  const float c2 = a.scale_log2;

  const TileDma<D, BN, 4, TILE_T16> kdma((const e16_t*)a.k + kvoff, L, wave, lane);
  const TileDma<D, BN, 4, TILE_K16> vdma((const e16_t*)a.v + kvoff, L, wave, lane);
  kdma.load(lds_base(k0_), 0);
  vdma.load(lds_base(v0_), 0);

  float lse2[2], negd[2];
  e16x8 qreg[2][DC], doreg[2][DC];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    lse2[qb] = qv[qb] ? a.lse2[(size_t)bh * N + qq[qb]] : 0.f;
    negd[qb] = qv[qb] ? a.delta[(size_t)bh * N + qq[qb]] : 0.f;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) {
      const size_t off = (size_t)qq[qb] * D + dc * 32 + g * 8;
      qreg[qb][dc] = as_e16x8(qv[qb] ? gload16(Qh + off) : zero4);
      doreg[qb][dc] = as_e16x8(qv[qb] ? gload16(dOh + off) : zero4);
    }
  }
  uint32_t koff[DC], vroff[DC], ktoff[DBK];
#pragma unroll
  for (int dc = 0; dc < DC; ++dc) {
    koff[dc] = (uint32_t)tile_off_lay<D, TILE_T16>(c16, dc * 32 + g * 8);
    vroff[dc] = (uint32_t)tile_off_lay<D, TILE_K16>(c16, dc * 32 + g * 8);
  }
#pragma unroll
  for (int db = 0; db < DBK; ++db)
    ktoff[db] = (uint32_t)tile_off_lay<D, TILE_T16>(4 * g + (c16 >> 2), db * 16 + 4 * (c16 & 3));

  f32x4 acc[DBK][2];
#pragma unroll
  for (int db = 0; db < DBK; ++db)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[db][qb][i] = 0.f;

  auto step = [&](int j, const int st, const bool MASKED) {
    const int n0 = j * BN;
    kdma.load(lds_base(st ? k0_ : k1_), n0 + BN);
    vdma.load(lds_base(st ? v0_ : v1_), n0 + BN);
    const lds_t* Kt = lds_base(st ? k1_ : k0_);
    const lds_t* Vt = lds_base(st ? v1_ : v0_);

    // Half h holds keys 32h .. 32h+31 (key blocks 2h, 2h+1).
    auto scores = [&](int h, f32x4 (&s)[2][2], f32x4 (&dp)[2][2]) {
#pragma unroll
      for (int dc = 0; dc < DC; ++dc)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const int r0 = (2 * h + kk) * 16 * (D * 2);
          const e16x8 kop = as_e16x8(lds_load16(Kt + r0 + koff[dc]));
          const e16x8 vop = as_e16x8(lds_load16(Vt + r0 + vroff[dc]));
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) {
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
            s[kk][qb] = mfma16x16x32<F16>(kop, qreg[qb][dc], dc == 0 ? z : s[kk][qb]);
            dp[kk][qb] = mfma16x16x32<F16>(vop, doreg[qb][dc], dc == 0 ? z : dp[kk][qb]);
          }
        }
    };
    auto softmax_grad = [&](int h, f32x4 (&s)[2][2], f32x4 (&dp)[2][2], e16x8 (&gb)[2]) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const int lim = (CAUSAL ? min(qq[qb], L - 1) : L - 1) - n0 - 32 * h - 4 * g;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float p = fast_exp2(fmaf(s[kk][qb][i], c2, -lse2[qb]));
            if (MASKED) p = (16 * kk + i <= lim) ? p : 0.f;
            dp[kk][qb][i] = p * (dp[kk][qb][i] + negd[qb]);
          }
        const u32x4 w = {pack2<F16>(dp[0][qb][0], dp[0][qb][1]), pack2<F16>(dp[0][qb][2], dp[0][qb][3]),
                         pack2<F16>(dp[1][qb][0], dp[1][qb][1]), pack2<F16>(dp[1][qb][2], dp[1][qb][3])};
        gb[qb] = as_e16x8(w);
      }
    };
    auto dq_mfma = [&](int h, const e16x8 (&gb)[2]) {
#pragma unroll
      for (int db = 0; db < DBK; ++db) {
        const lds_t* p = Kt + 32 * h * (D * 2) + ktoff[db];
        const e16x8 kt = join_e16x8(lds_load_tr16(p), lds_load_tr16(p + 16 * (D * 2)));
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) acc[db][qb] = mfma16x16x32<F16>(kt, gb[qb], acc[db][qb]);
      }
    };
    constexpr int NR = 4 * DC;  // b128 reads per half (K and V)
    f32x4 s0[2][2], dp0[2][2];
    scores(0, s0, dp0);
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      if (i < NR - 4) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    f32x4 s1[2][2], dp1[2][2];
    scores(1, s1, dp1);
    e16x8 g0[2];
    softmax_grad(0, s0, dp0, g0);
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x002 | 0x400, 5, 0);
      if (i < NR - 4) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    dq_mfma(0, g0);
    e16x8 g1[2];
    softmax_grad(1, s1, dp1, g1);
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < 2 * DBK; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002 | 0x400, 5, 0);
      if (i < 2 * DBK - 4) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    dq_mfma(1, g1);
    dma_wait();
    __syncthreads();
  };

  dma_wait();
  __syncthreads();
  int j = 0;
  for (; j < nt - 2; j += 2) {
    step(j, 0, false);
    step(j + 1, 1, false);
  }
  step(j, 0, true);
  step(j + 1, 1, true);

#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    if (qq[qb] < N) {
      e16_t* rowp = dQh + (size_t)qq[qb] * D;
#pragma unroll
      for (int db = 0; db < DBK; ++db) {
        const uint32_t w0 = pack2<F16>(acc[db][qb][0] * a.scale, acc[db][qb][1] * a.scale);
        const uint32_t w1 = pack2<F16>(acc[db][qb][2] * a.scale, acc[db][qb][3] * a.scale);
        const u32x2 w = {qv[qb] ? w0 : 0u, qv[qb] ? w1 : 0u};
        gstore8(rowp + db * 16 + 4 * g, w);
      }
    }
  }
}

// Thin __global__ wrappers: with the buffer builtins inside a __global__
// template body, the host pass dropped some of the launch stubs.
template <int D, bool CAUSAL, bool F16>
__global__ void __launch_bounds__(256, 1) bwd_dkdv_kernel(BwdArgs a) {
  bwd_dkdv_body<D, CAUSAL, F16>(a);
}
template <int D, bool CAUSAL, bool F16>
__global__ void __launch_bounds__(256, 2) bwd_dq_kernel(BwdArgs a) {
  bwd_dq_body<D, CAUSAL, F16>(a);
}

template <int D, bool CAUSAL, bool F16>
hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t stream) {
  const long long rows = (long long)a.B * a.H * a.N;
  constexpr int RPB = 256 / (D / 8);
  hipLaunchKernelGGL((bwd_pre_kernel<D, F16>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0,
                     stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int heads = a.B * a.H;
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, F16>),
                     dim3((unsigned)(a.B * a.H_kv * ((a.N + 127) / 128))),
                     dim3(256), 0, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, F16>), dim3((unsigned)(heads * ((a.N + 127) / 128))),
                     dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <bool F16>
hipError_t launch_bwd_fmt(const BwdArgs& a, int d, bool causal, hipStream_t stream) {
  if (d == 64)
    return causal ? launch_bwd_t<64, true, F16>(a, stream) : launch_bwd_t<64, false, F16>(a, stream);
  return causal ? launch_bwd_t<128, true, F16>(a, stream) : launch_bwd_t<128, false, F16>(a, stream);
}

}  // namespace

hipError_t launch_bwd_16(const BwdArgs& a, int d, bool causal, bool f16, hipStream_t stream) {
  return f16 ? launch_bwd_fmt<true>(a, d, causal, stream) : launch_bwd_fmt<false>(a, d, causal, stream);
}

}  // namespace attn
