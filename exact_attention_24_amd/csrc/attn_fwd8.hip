// FP8 attention forward for gfx950: Q, K and V in FP8 E4M3, both products on
// the FP8 matrix cores, softmax and accumulation in fp32.
//
// Pages cited (by title):
//   [SafeSoftmax] "FlashAttention：从 Safe Softmax 到分块计算"
//   [OpOpt]       "Attention 算子优化:从物化 N×N 矩阵到 FlashAttention 与 PagedAttention"
//
// Same method as the 16-bit forward ([SafeSoftmax] §3.1-§3.2, §5, §7, §8): one
// workgroup per 128-row tile of Q, K/V tiles streamed through LDS, online
// softmax with the lazy rescale of the 16-bit kernel, causal block skipping
// ([OpOpt] §四), keys past a sequence's length masked ([OpOpt] §二). What
// changes is the number format ([SafeSoftmax] §9.2 names scaling, accumulation
// and error control as the points an FP8 path has to handle; [OpOpt] §六 keeps
// softmax and accumulation in fp32):
//  - Q, K, V are FP8 E4M3 with scales: Q per token (q_scale[b,h,i]), K and V
//    per (batch, K/V head). The Q and K scales and the softmax scale fold into
//    one fp32 constant per query, so the scores need no extra operation; the V
//    scale folds into the final division by l.
//  - S^T = K Q^T from v_mfma_scale_f32_16x16x128_f8f6f4 (E4M3 x E4M3, block
//    scales 1): one MFMA per 16 keys x 16 queries covers d = 128.
//  - The weights (each <= 2^8 by the lazy-rescale check, inside E4M3's range
//    of 448) are rounded to E4M3 (nearest even) for O^T += V^T P^T on the same
//    MFMA with 128 keys per instruction. The row sum l is taken over the fp32
//    weights, so the LSE is that of the exact softmax; O carries the rounding
//    of the weights to 3 mantissa bits.
// K and V tiles hold 128 keys (16 KiB each, two stages: 64 KiB per workgroup).
#include "attn_common.h"
#include "attn_kernels.h"
#include "attn_sched.h"
#include "attn_tile.h"

#include <math.h>

namespace attn {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

// D(16x16) += A(16x128) B(128x16) on E4M3 operands with unit block scales.
// Lane l (r = l % 16, g = l / 16) holds A row r and B column r at 32 k values
// of group g; the product pairs byte j of A's group-g lanes with byte j of B's
// group-g lanes (checked on the device against a host product), so any fixed
// assignment of k indices to (g, j) serves both operands. D: lane l holds
// column l % 16, rows 4 * (l / 16) + i, as for the 16-bit 16x16x32 MFMA.
__device__ __forceinline__ f32x4 mfma_f8(i32x8 a, i32x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ i32x8 join8(u32x4 lo, u32x4 hi) {
  i32x8 v = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
             (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  return v;
}

// Four fp32 values rounded to E4M3 (nearest even), bytes in order.
__device__ __forceinline__ int pack4_e4m3(f32x4 x) {
  int w = 0;
  w = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], w, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], w, true);
}

constexpr float kLazyRescaleW8 = 256.0f;  // largest unnormalised weight kept without rescaling

template <bool CAUSAL, bool F16>
__device__ __forceinline__ void fwd8_body(const Fwd8Args& a) {
  constexpr int D = 128;                 // head dimension = bytes per row
  constexpr int BM = 128, BN = 128;
  constexpr int TILE = BN * D;           // 16 KiB
  constexpr int KB = BN / 16;            // 16-key blocks per tile
  constexpr int DB = D / 16;             // 16-wide d blocks of O
  constexpr int CH = D / 8;              // 16-byte chunks of a 16-bit O row

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
  const int hkv = b * a.H_kv + (bh % a.H) / group;
  int L = N;
  if (a.seqlens) L = min(max(a.seqlens[b], 0), N);
  const int m0 = mt * BM;
  const size_t hoff = (size_t)bh * N * D;   // bytes of q8, elements of O
  const size_t kvoff = (size_t)hkv * N * D;
  const uint8_t* __restrict__ Qh = a.q + hoff;
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

  // Tiles in 16-bit units (a 128-byte row is 64 of them); rows at or past L
  // are never fetched.
  const TileDma<64, BN, 4, TILE_K16> kdma((const e16_t*)(a.k + kvoff), L, wave, lane);
  const TileDma<64, BN, 4, TILE_V8> vdma((const e16_t*)(a.v + kvoff), L, wave, lane);
  kdma.load(kst[0], 0);
  vdma.load(vst[0], 0);

  // Q as B operands: query qq[qb], bytes 16g .. 16g + 15 and 64 + 16g .. +15
  // of its row (the k assignment the K operands below use).
  i32x8 qr[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const bool in = qq[qb] < L;
    const uint8_t* row = Qh + (size_t)qq[qb] * D + 16 * g;
    qr[qb] = join8(in ? gload16(row) : zero4, in ? gload16(row + 64) : zero4);
  }
  // Scores to exp2 arguments: scale * log2(e) * q_scale[query] * k_scale[head].
  // Rows past L (zero Q, output discarded) take q_scale = 1: any positive
  // finite factor keeps a masked score's -inf from turning into NaN.
  const float kv_s = a.k_scale[hkv], v_s = a.v_scale[hkv];
  float c2[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
    c2[qb] = a.scale * kLog2e * kv_s * (qq[qb] < L ? a.q_scale[(size_t)bh * N + qq[qb]] : 1.f);

  // K operand: key 16*kb + c16, 16-byte chunks g and g + 4 of the row (bytes
  // 16g .. and 64 + 16g ..), so each read touches four consecutive chunks of
  // 16 rows: conflict-free under TILE_K16 (chunks 2g, 2g + 1 measured four
  // extra cycles per read); the row's swizzle does not depend on kb. V^T operand, read t: source lane (c16, g)
  // addresses key row 32t + 16*(x/4) + 4g + x%4 (x = c16 / 2) at bytes
  // 16*db + 8*(c16 % 2) .. +7, so the transposing read hands lane (c16, g) the
  // column d = 16*db + c16 of the keys 16*kb + 4g + i (kb = 2t, 2t+1; i < 4):
  // the keys, in the order, that the lane's score accumulators hold.
  uint32_t koff[2], voff[DB];
#pragma unroll
  for (int h = 0; h < 2; ++h) koff[h] = (uint32_t)tile_off_lay<64, TILE_K16>(c16, 8 * (g + 4 * h));
  const int x = c16 >> 1;
  const int vrow = 16 * (x >> 2) + 4 * g + (x & 3);
#pragma unroll
  for (int db = 0; db < DB; ++db)
    voff[db] = (uint32_t)tile_off_lay<64, TILE_V8>(vrow, 8 * db + 4 * (c16 & 1));

  f32x4 o[DB][2];  // O^T block (d 16*db + 4*g + i, query qq[qb])
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int i = 0; i < 4; ++i) o[db][qb][i] = 0.f;
  float m_ref[2] = {kMaxInit, kMaxInit}, l_part[2] = {0.f, 0.f};

  auto tile_step = [&](int j, const int ST) {
    const int n0 = j * BN;
    if (j + 1 < nt) {
      kdma.load(kst[ST ^ 1], n0 + BN);
      vdma.load(vst[ST ^ 1], n0 + BN);
    }
    if (j < wnt) {
      const lds_t* kt = kst[ST];
      const lds_t* vt = vst[ST];
      f32x4 s[KB][2];
      // S^T blocks, masked; each K operand feeds both query blocks.
      auto scores = [&]() {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const lds_t* p = kt + kb * 16 * D;
          const i32x8 kop = join8(lds_load16(p + koff[0]), lds_load16(p + koff[1]));
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) {
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
            s[kb][qb] = mfma_f8(kop, qr[qb], z);
          }
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
        for (int i = 0; i < KB; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
          if (i < KB - 3) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        // Key n0 + 16*kb + 4*g + i is visible iff 16*kb + i <= lim.
        if (n0 + BN > L || (CAUSAL && n0 + BN - 1 > qw)) {
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) {
            const int lim = (CAUSAL ? min(qq[qb], L - 1) : L - 1) - n0 - 4 * g;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
              for (int i = 0; i < 4; ++i) s[kb][qb][i] = kb * 16 + i <= lim ? s[kb][qb][i] : -INFINITY;
          }
        }
      };
      auto row_max = [&](int qb) {
        float mx = fmaxf(s[0][qb][0], s[0][qb][1]);
#pragma unroll
        for (int e = 2; e < 4 * KB; e += 2) mx = max3f(mx, s[e >> 2][qb][e & 3], s[e >> 2][qb][(e & 3) + 1]);
        return max_quarters(mx);
      };
      float sum[2];
      auto weights = [&]() {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const float mc = m_ref[qb] * c2[qb];
          sum[qb] = 0.f;
#pragma unroll
          for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              s[kb][qb][i] = fast_exp2(fmaf(s[kb][qb][i], c2[qb], -mc));
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
      if (__builtin_amdgcn_ballot_w64(!(sum[0] <= kLazyRescaleW8) || !(sum[1] <= kLazyRescaleW8))) {
        scores();
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const float m_new = fmaxf(m_ref[qb], row_max(qb));
          const float alpha = fast_exp2((m_ref[qb] - m_new) * c2[qb]);
          l_part[qb] *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i) o[db][qb][i] *= alpha;
          m_ref[qb] = m_new;
        }
        weights();
      }
      l_part[0] += sum[0];
      l_part[1] += sum[1];
      // P^T B operands: byte j of group g is the weight of key 16*(j/4) + 4g + j%4.
      i32x8 pb[2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) pb[qb][kb] = pack4_e4m3(s[kb][qb]);
      __builtin_amdgcn_s_setprio(1);
      // O^T (D x 32) += V^T (D x 128) P^T (128 x 32); each V^T operand feeds
      // both query blocks.
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const lds_t* p = vt + voff[db];
        u32x2 t[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) t[r] = lds_load_tr8(p + r * 32 * D);
        const i32x8 vop = {(int)t[0][0], (int)t[0][1], (int)t[1][0], (int)t[1][1],
                           (int)t[2][0], (int)t[2][1], (int)t[3][0], (int)t[3][1]};
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) o[db][qb] = mfma_f8(vop, pb[qb], o[db][qb]);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 1);
#pragma unroll
      for (int i = 0; i < DB; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 1);
        if (i < DB - 2) __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);
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

  // Epilogue: O = v_scale * O_acc / l, rounded to 16 bits; LSE in natural log
  // units, m * scale * q_scale * k_scale + ln l. As in the 16-bit forward, each
  // wave stages its 32 rows in LDS (idle K/V stages, no load in flight) and
  // stores whole rows, 16-byte pieces, a row per 16 lanes.
  constexpr int RB = D * 2;                     // bytes per O row (16-bit)
  constexpr int CPRO = RB / 16;                 // 16-byte chunks per row
  lds_t* const ost = (wave < 2 ? kst[0] : vst[0]) + (wave & 1) * (32 * RB);
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float l_tot = sum_quarters(l_part[qb]);
    const int q = qq[qb];
    const bool valid = q < L && l_tot > 0.f;
    const float inv = valid ? v_s / l_tot : 0.f;
    const int r = qb * 16 + c16;                // row within the wave's 32
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const u32x2 w = {pack2<F16>(o[db][qb][0] * inv, o[db][qb][1] * inv),
                       pack2<F16>(o[db][qb][2] * inv, o[db][qb][3] * inv)};
      const int byte = db * 32 + g * 8;         // columns 16 db + 4 g .. +3
      lds_store8(ost + r * RB + ((((byte >> 4) ^ (r & (CPRO - 1))) << 4) | (byte & 15)), w);
    }
    if (q < N && lse_h && g == 0) lse_h[q] = valid ? m_ref[qb] * c2[qb] * kLn2 + logf(l_tot) : -INFINITY;
  }
  constexpr int RPI = 64 / CPRO;                // rows per store instruction
#pragma unroll
  for (int it = 0; it < 32 / RPI; ++it) {
    const int r = it * RPI + lane / CPRO, c = lane % CPRO;
    const u32x4 w = lds_load16(ost + r * RB + ((c ^ (r & (CPRO - 1))) << 4));
    if (qw + r < N) gstore16(Oh + (size_t)(qw + r) * D + c * 8, w);
  }
}

template <bool CAUSAL, bool F16>
__global__ void __launch_bounds__(256, 2) fwd8_kernel(Fwd8Args a) {
  fwd8_body<CAUSAL, F16>(a);
}

template <bool CAUSAL, bool F16>
hipError_t launch8_t(const Fwd8Args& a, hipStream_t stream) {
  const int nm = (a.N + 127) / 128;
  dim3 grid((unsigned)(nm * a.B * a.H)), block(256);
  hipLaunchKernelGGL((fwd8_kernel<CAUSAL, F16>), grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_fp8(const Fwd8Args& a, bool causal, bool f16_out, hipStream_t stream) {
  if (f16_out) return causal ? launch8_t<true, true>(a, stream) : launch8_t<false, true>(a, stream);
  return causal ? launch8_t<true, false>(a, stream) : launch8_t<false, false>(a, stream);
}

}  // namespace attn
