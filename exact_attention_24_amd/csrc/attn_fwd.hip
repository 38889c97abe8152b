// Attention forward kernels for gfx950.
//
// Pages cited (by title):
//   [SafeSoftmax] "FlashAttention：从 Safe Softmax 到分块计算"
//   [OpOpt]       "Attention 算子优化:从物化 N×N 矩阵到 FlashAttention 与 PagedAttention"
//   [AIInfra]     the AIInfra FlashAttention note on dpshk.com
//
// Each workgroup owns one row tile of Q for one (batch, head) and streams the
// K/V tiles of that head through LDS ([SafeSoftmax] §5). Per query row it keeps
// the online-softmax state of [SafeSoftmax] §3.1: running max m, running
// exponential sum l and the unnormalised output accumulator; each new tile is
// merged by rescaling the old state with exp(m_old - m_new) ([SafeSoftmax]
// §3.2, in the single-exponential form of the [AIInfra] §2.1 loop: the tile's
// weights are taken relative to m_new directly). Causal tiles above the
// diagonal are never visited ([OpOpt] §四); keys past a sequence's valid
// length are masked ([OpOpt] §二); the output is divided by l once at the end
// and the row log-sum-exp is written for the backward ([SafeSoftmax] §8).
#include "attn_common.h"
#include "attn_kernels.h"
#include "attn_sched.h"
#include "attn_tile.h"

#include <math.h>

namespace attn {

namespace {

// ----------------------------------------------------------------------------
// 16-bit inputs (bf16, or fp16 with F16), MFMA products, fp32 softmax and
// accumulation.
//
// Workgroup: 4 waves, 128 query rows (32 per wave), K/V tiles of 64 keys,
// double-buffered in LDS and filled by direct global->LDS loads
// (global_load_lds_dwordx4, no VGPR staging). Scores are computed transposed,
// S^T = K Q^T, from v_mfma_f32_16x16x32_bf16 (_f16) blocks: K (from LDS) is
// the A operand and Q (held in VGPRs for the whole loop) the B operand. Lane
// l (c = l % 16, g = l / 16) holds the queries qw + c and qw + 16 + c, each
// with the keys 16*kb + 4*g + i of the tile (kb, i = 0..3), so one query's 64
// keys lie in the lanes c, c+16, c+32, c+48. Each K operand read feeds both
// 16-query blocks, which keeps the LDS bytes per FLOP of 32x32x16 blocks,
// while the 16x16 shape holds a higher clock under the GPU's power limit
// (measured ~1.93 against ~1.76 GHz for the same kernel on 32x32x16 blocks at
// d = 128, +5% net). The output is accumulated transposed as well,
// O^T += V^T P^T: the MFMA k index 8g + e stands for key 32jj + 4g + e (e < 4)
// or 32jj + 16 + 4g + e - 4, the order in which the score accumulators already
// hold P^T, so the weights are packed in place as B operands, and V^T is read
// from the row-major V tile with the transposing LDS load in that key order.
// K and V tiles use the TILE_K16 and TILE_T16 layouts, in which these reads
// are free of bank conflicts.
//
// Softmax arithmetic per score: one FMA (s*scale*log2e - m*scale*log2e), one
// v_exp_f32 (exp2), one fp32 add into the lane's partial row sum and a share
// of a 16-bit pack; statistics stay in fp32 and only the P V product sees
// 16-bit weights. The rescale of [SafeSoftmax] §3.2 is applied lazily against
// a reference max m: the first tile sets m to its exact row max (the only
// per-tile use of the two lane exchanges), and later tiles are weighted
// against m without taking their own max. A weight can exceed 2^8 only if its
// lane's partial row sum does, so that sum (needed anyway) is the check; when
// it fails (rare: a score more than 8/(scale*log2e) above the reference) the
// tile's scores are recomputed, m moves to the exact max, and O and l are
// rescaled. Weights stay <= 256, far from fp32 or bf16 range limits, and O / l
// and LSE use the same reference, so the result is the same softmax. The P V
// phase runs at raised wave priority (s_setprio): with two waves per SIMD (one
// from each resident workgroup), the wave holding P V MFMAs is issued first
// when both are ready (measured 2-4% faster).
// ----------------------------------------------------------------------------
constexpr float kLazyRescaleW = 256.0f;  // largest unnormalised weight kept without rescaling

template <int D, bool CAUSAL, bool F16>
__device__ __forceinline__ void fwd_16_body(const FwdArgs& a) {
  constexpr int BM = 128, BN = 64;
  constexpr int TILE = BN * D * 2;
  constexpr int CH = D / 8;
  constexpr int DC = D / 32, DBK = D / 16;  // 32-wide d chunks (Q, K), 16-wide d blocks (O, V)

  __shared__ __attribute__((aligned(1024))) char k0_[TILE], v0_[TILE], k1_[TILE], v1_[TILE];
  lds_t* const kst[2] = {lds_base(k0_), lds_base(k1_)};
  lds_t* const vst[2] = {lds_base(v0_), lds_base(v1_)};

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c16 = lane & 15, g = lane >> 4;
  const int N = a.N;
  const int nm = (N + BM - 1) / BM;
  int bh, mt;
  const int group = a.H / a.H_kv;
  if (a.seqlens && a.B <= 64 && ((a.H / group) & 7) == 0) {
    int rank, h;
    varlen_order(blockIdx.x, nm, a.H, group, CAUSAL, rank, h, mt);
    bh = batch_of_rank(a.seqlens, a.B, N, rank) * a.H + h;
  } else {
    tile_order(blockIdx.x, nm, a.B * a.H, group, CAUSAL, bh, mt);
  }
  const int b = bh / a.H;
  int L = N;
  if (a.seqlens) L = min(max(a.seqlens[b], 0), N);
  const int m0 = mt * BM;
  const size_t hoff = (size_t)bh * N * D;
  const size_t kvoff = (size_t)(b * a.H_kv + (bh % a.H) / (a.H / a.H_kv)) * N * D;
  const e16_t* __restrict__ Qh = (const e16_t*)a.q + hoff;
  e16_t* __restrict__ Oh = (e16_t*)a.o + hoff;
  float* __restrict__ lse_h = a.lse ? a.lse + (size_t)bh * N : nullptr;
  const u32x4 zero4 = {0u, 0u, 0u, 0u};

  if (m0 >= L) {  // the whole row tile is padding: O = 0, LSE = -inf
    const int rows = min(BM, N - m0);
    for (int c = tid; c < rows * CH; c += 256)
      gstore16(Oh + (size_t)(m0 + c / CH) * D + (c % CH) * 8, zero4);
    if (lse_h)
      for (int r = tid; r < rows; r += 256) lse_h[m0 + r] = -INFINITY;
    return;
  }

  const int kv_end = CAUSAL ? min(L, m0 + BM) : L;
  const int nt = (kv_end + BN - 1) / BN;                 // tiles the workgroup loads
  const int qw = m0 + wave * 32;                         // first query row of this wave
  const int qq[2] = {qw + c16, qw + 16 + c16};           // this lane's queries (qb = 0, 1)
  const int w_end = (qw >= L) ? 0 : (CAUSAL ? min(L, qw + 32) : L);
  const int wnt = (w_end + BN - 1) / BN;                 // tiles this wave computes

  // K/V rows at or past L are never fetched (the DMA reads zeros there).
  const TileDma<D, BN, 4, TILE_K16> kdma((const e16_t*)a.k + kvoff, L, wave, lane);
  const TileDma<D, BN, 4, TILE_T16> vdma((const e16_t*)a.v + kvoff, L, wave, lane);
  kdma.load(kst[0], 0);
  vdma.load(vst[0], 0);

  // Q as B operands: query qq[qb], d = 32*dc + 8*g .. +7.
  e16x8 qr[2][DC];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int dc = 0; dc < DC; ++dc)
      qr[qb][dc] = as_e16x8(qq[qb] < L ? gload16(Qh + (size_t)qq[qb] * D + dc * 32 + g * 8) : zero4);

  // Per-lane LDS offsets. K operand: key 16*kb + c, columns 32*dc + 8*g .. +7.
  // V^T operand: row 4*g + c/4 (+16 for the upper half), columns
  // 16*db + 4*(c%4) .. +3. Offsets of whole 16-row blocks leave both swizzles
  // unchanged and become immediates.
  uint32_t koff[DC], voff[DBK];
#pragma unroll
  for (int dc = 0; dc < DC; ++dc) koff[dc] = (uint32_t)tile_off_lay<D, TILE_K16>(c16, dc * 32 + g * 8);
#pragma unroll
  for (int db = 0; db < DBK; ++db)
    voff[db] = (uint32_t)tile_off_lay<D, TILE_T16>(4 * g + (c16 >> 2), db * 16 + 4 * (c16 & 3));

  f32x4 o[DBK][2];  // O^T block (d 16*db + 4*g + i, query qq[qb])
#pragma unroll
  for (int db = 0; db < DBK; ++db)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int i = 0; i < 4; ++i) o[db][qb][i] = 0.f;
  float m_ref[2] = {kMaxInit, kMaxInit}, l_part[2] = {0.f, 0.f};
  const float c2 = a.scale_log2;

  auto tile_step = [&](int j, const int ST) {
    const int n0 = j * BN;
    if (j + 1 < nt) {
      kdma.load(kst[ST ^ 1], n0 + BN);
      vdma.load(vst[ST ^ 1], n0 + BN);
    }
    if (j < wnt) {
      const lds_t* kt = kst[ST];
      const lds_t* vt = vst[ST];
      f32x4 s[4][2];
      // S^T blocks, masked; each K operand read feeds both query blocks.
      auto scores = [&]() {
#pragma unroll
        for (int dc = 0; dc < DC; ++dc)
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) {
            const e16x8 kop = as_e16x8(lds_load16(kt + kb * 16 * (D * 2) + koff[dc]));
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
              const f32x4 z = {0.f, 0.f, 0.f, 0.f};
              s[kb][qb] = mfma16x16x32<F16>(kop, qr[qb][dc], dc == 0 ? z : s[kb][qb]);
            }
          }
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int i = 0; i < 4 * DC; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
          if (i < 4 * DC - 4) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        // Key n0 + 16*kb + 4*g + i is visible iff 16*kb + i <= lim.
        if (n0 + BN > L || (CAUSAL && n0 + BN - 1 > qw)) {
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) {
            const int lim = (CAUSAL ? min(qq[qb], L - 1) : L - 1) - n0 - 4 * g;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
              for (int i = 0; i < 4; ++i) s[kb][qb][i] = kb * 16 + i <= lim ? s[kb][qb][i] : -INFINITY;
          }
        }
      };
      auto row_max = [&](int qb) {
        float mx = fmaxf(s[0][qb][0], s[0][qb][1]);
#pragma unroll
        for (int e = 2; e < 16; e += 2) mx = max3f(mx, s[e >> 2][qb][e & 3], s[e >> 2][qb][(e & 3) + 1]);
        return max_quarters(mx);
      };
      float sum[2];
      auto weights = [&]() {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const float mc = m_ref[qb] * c2;
          sum[qb] = 0.f;
#pragma unroll
          for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              s[kb][qb][i] = fast_exp2(fmaf(s[kb][qb][i], c2, -mc));
              sum[qb] += s[kb][qb][i];
            }
        }
      };
      scores();
      // The first tile sets each query's reference max (every query sees key 0).
      if (j == 0) {
        m_ref[0] = row_max(0);
        m_ref[1] = row_max(1);
      }
      weights();
      // Stale reference (rare): recompute the scores, move to the exact max,
      // rescale O and l.
      if (__builtin_amdgcn_ballot_w64(!(sum[0] <= kLazyRescaleW) || !(sum[1] <= kLazyRescaleW))) {
        scores();
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const float m_new = fmaxf(m_ref[qb], row_max(qb));
          const float alpha = fast_exp2((m_ref[qb] - m_new) * c2);
          l_part[qb] *= alpha;
#pragma unroll
          for (int db = 0; db < DBK; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i) o[db][qb][i] *= alpha;
          m_ref[qb] = m_new;
        }
        weights();
      }
      l_part[0] += sum[0];
      l_part[1] += sum[1];
      // P^T B operands for k-step jj (keys 32jj ..), query block qb.
      e16x8 pb[2][2];
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const f32x4& x0 = s[2 * jj][qb];
          const f32x4& x1 = s[2 * jj + 1][qb];
          const u32x4 w = {pack2<F16>(x0[0], x0[1]), pack2<F16>(x0[2], x0[3]),
                           pack2<F16>(x1[0], x1[1]), pack2<F16>(x1[2], x1[3])};
          pb[jj][qb] = as_e16x8(w);
        }
      __builtin_amdgcn_s_setprio(1);
      // O^T (D x 32) += V^T (D x 64) P^T (64 x 32); each V^T operand feeds both
      // query blocks.
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int db = 0; db < DBK; ++db) {
          const lds_t* p = vt + jj * 32 * (D * 2) + voff[db];
          const e16x8 vop = join_e16x8(lds_load_tr16(p), lds_load_tr16(p + 16 * (D * 2)));
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) o[db][qb] = mfma16x16x32<F16>(vop, pb[jj][qb], o[db][qb]);
        }
      __builtin_amdgcn_sched_group_barrier(0x100, 6, 1);
#pragma unroll
      for (int i = 0; i < 4 * DBK; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
        if (i < 4 * DBK - 6) __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    dma_wait();
    __syncthreads();
  };

  dma_wait();
  __syncthreads();
  for (int j = 0; j < nt; j += 2) {
    tile_step(j, 0);
    if (j + 1 < nt) tile_step(j + 1, 1);
  }

  // Epilogue: O = O_acc / l, rounded to 16 bits; LSE = m*scale + ln l. Each
  // wave stages its 32 rows in LDS (the K/V stages are idle now; the last
  // step's barrier has passed and no load is in flight) and stores them as
  // whole rows: 16-byte pieces, a row per 16 lanes.
  constexpr int RB = D * 2;                     // bytes per O row
  constexpr int CPRO = RB / 16;                 // 16-byte chunks per row
  lds_t* const ost = (wave < 2 ? kst[0] : vst[0]) + (wave & 1) * (32 * RB);
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float l_tot = sum_quarters(l_part[qb]);
    const int q = qq[qb];
    const bool valid = q < L && l_tot > 0.f;
    const float inv = valid ? 1.f / l_tot : 0.f;
    const int r = qb * 16 + c16;                // row within the wave's 32
#pragma unroll
    for (int db = 0; db < DBK; ++db) {
      const u32x2 w = {pack2<F16>(o[db][qb][0] * inv, o[db][qb][1] * inv),
                       pack2<F16>(o[db][qb][2] * inv, o[db][qb][3] * inv)};
      const int byte = db * 32 + g * 8;         // columns 16 db + 4 g .. +3
      lds_store8(ost + r * RB + ((((byte >> 4) ^ (r & (CPRO - 1))) << 4) | (byte & 15)), w);
    }
    if (q < N && lse_h && g == 0) lse_h[q] = valid ? m_ref[qb] * a.scale + logf(l_tot) : -INFINITY;
  }
  constexpr int RPI = 64 / CPRO;                // rows per store instruction
#pragma unroll
  for (int it = 0; it < 32 / RPI; ++it) {
    const int r = it * RPI + lane / CPRO, c = lane % CPRO;
    const u32x4 w = lds_load16(ost + r * RB + ((c ^ (r & (CPRO - 1))) << 4));
    if (qw + r < N) gstore16(Oh + (size_t)(qw + r) * D + c * 8, w);
  }
}

// The kernel is a thin wrapper: with the body in a __device__ template, the
// host compilation pass emits every instantiation's launch stub (with the
// buffer-load builtins directly in a __global__ template body it silently
// dropped some of them).
template <int D, bool CAUSAL, bool F16>
__global__ void __launch_bounds__(256, 2) fwd_16_kernel(FwdArgs a) {
  fwd_16_body<D, CAUSAL, F16>(a);
}

template <int D, bool CAUSAL, bool F16>
hipError_t launch_16_t(const FwdArgs& a, hipStream_t stream) {
  constexpr int BM = 128;
  const int nm = (a.N + BM - 1) / BM;
  dim3 grid((unsigned)(nm * a.B * a.H)), block(256);
  hipLaunchKernelGGL((fwd_16_kernel<D, CAUSAL, F16>), grid, block, 0, stream, a);
  return hipGetLastError();
}

template <bool F16>
hipError_t launch_16_fmt(const FwdArgs& a, int d, bool causal, hipStream_t stream) {
  if (d == 64)
    return causal ? launch_16_t<64, true, F16>(a, stream) : launch_16_t<64, false, F16>(a, stream);
  return causal ? launch_16_t<128, true, F16>(a, stream) : launch_16_t<128, false, F16>(a, stream);
}

}  // namespace

hipError_t launch_fwd_16(const FwdArgs& a, int d, bool causal, bool f16, hipStream_t stream) {
  return f16 ? launch_16_fmt<true>(a, d, causal, stream) : launch_16_fmt<false>(a, d, causal, stream);
}

}  // namespace attn
