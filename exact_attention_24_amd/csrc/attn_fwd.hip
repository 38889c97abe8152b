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

#include <math.h>

namespace attn {

namespace {

// ----------------------------------------------------------------------------
// bf16 inputs, MFMA products, fp32 softmax and accumulation.
//
// Workgroup: 4 waves, 128 query rows (32 per wave), K/V tiles of 64 keys,
// double-buffered in LDS. Scores are computed transposed, S^T = K Q^T, with
// v_mfma_f32_32x32x16_bf16: K (from LDS) is the A operand and Q (held in
// VGPRs for the whole loop) is the B operand, so each lane's accumulator holds
// 16 keys of ONE query. Row max and row sum are then 32 in-lane operations plus
// one exchange between the two 32-lane halves. The output is accumulated
// transposed as well, O^T += V^T P^T: P^T stays in the accumulator lanes it
// was computed in (B operand), and V^T is read from the row-major V tile with
// the transposing LDS load ds_read_b64_tr_b16, in the same key order as P^T's
// lanes hold. All exponentials are exp2 with log2(e) folded into the scale.
// ----------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ void __launch_bounds__(256, 2) fwd_bf16_kernel(FwdArgs a) {
  constexpr int BM = 128, BN = 64;
  constexpr int KS = D * 2 + 16;      // K row stride in LDS (bytes): 16 consecutive rows hit distinct banks
  constexpr int VS = D * 2 + 64;      // V row stride in LDS (bytes), for the transposing reads
  constexpr int KB = BN * KS, VB = BN * VS, STAGE = KB + VB;
  constexpr int CH = D / 8;           // 16-byte chunks per row
  constexpr int LOADS = BN * CH / 256;
  constexpr int DS = D / 16, DB = D / 32;

  extern __shared__ __attribute__((aligned(16))) char smem_generic[];
  lds_t* smem = lds_base(smem_generic);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int N = a.N;
  const int nm = (N + BM - 1) / BM;
  int bh, mt;
  tile_order(blockIdx.x, nm, a.B * a.H, CAUSAL, bh, mt);
  const int b = bh / a.H;
  int L = N;
  if (a.seqlens) L = min(max(a.seqlens[b], 0), N);
  const int m0 = mt * BM;
  const size_t hoff = (size_t)bh * N * D;
  const bf16_t* __restrict__ Qh = (const bf16_t*)a.q + hoff;
  const bf16_t* __restrict__ Kh = (const bf16_t*)a.k + hoff;
  const bf16_t* __restrict__ Vh = (const bf16_t*)a.v + hoff;
  bf16_t* __restrict__ Oh = (bf16_t*)a.o + hoff;
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
  const int q = qw + l32;                                // this lane's query row
  const int w_end = (qw >= L) ? 0 : (CAUSAL ? min(L, qw + 32) : L);
  const int wnt = (w_end + BN - 1) / BN;                 // tiles this wave computes

  // Q rows -> VGPRs, B-operand layout: lane holds query q, d = 16*ds + 8*hi .. +7.
  bf16x8 qr[DS];
#pragma unroll
  for (int ds = 0; ds < DS; ++ds)
    qr[ds] = as_bf16x8(q < N ? gload16(Qh + (size_t)q * D + ds * 16 + hi * 8) : zero4);

  u32x4 kr[LOADS], vr[LOADS];
  auto gload_tile = [&](int n0) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int c = tid + 256 * i, row = c / CH, col = c % CH, g = n0 + row;
      kr[i] = g < N ? gload16(Kh + (size_t)g * D + col * 8) : zero4;
      vr[i] = g < N ? gload16(Vh + (size_t)g * D + col * 8) : zero4;
    }
  };
  auto lds_store_tile = [&](int st) {
    lds_t* kb = smem + st * STAGE;
    lds_t* vb = kb + KB;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int c = tid + 256 * i, row = c / CH, col = c % CH;
      lds_store16(kb + row * KS + col * 16, kr[i]);
      lds_store16(vb + row * VS + col * 16, vr[i]);
    }
  };

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
  float m_run = kMaxInit, l_run = 0.f;
  const float c2 = a.scale_log2;

  // Lane-constant parts of the LDS addresses.
  const int k_lane = l32 * KS + hi * 16;
  const int v_lane = (hi * 4 + ((lane & 15) >> 2)) * VS + (((lane >> 4) & 1) * 16 + 4 * (lane & 3)) * 2;

  gload_tile(0);
  lds_store_tile(0);
  __syncthreads();

  for (int j = 0; j < nt; ++j) {
    const int st = j & 1, n0 = j * BN;
    if (j + 1 < nt) gload_tile(n0 + BN);
    if (j < wnt) {
      const lds_t* kb = smem + st * STAGE;
      const lds_t* vb = kb + KB;
      // S^T (64 keys x 32 queries) as two 32x32 blocks.
      f32x16 s0, s1;
#pragma unroll
      for (int i = 0; i < 16; ++i) { s0[i] = 0.f; s1[i] = 0.f; }
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) {
        const bf16x8 k0 = as_bf16x8(lds_load16(kb + k_lane + ds * 32));
        const bf16x8 k1 = as_bf16x8(lds_load16(kb + k_lane + 32 * KS + ds * 32));
        s0 = mfma32x32x16(k0, qr[ds], s0);
        s1 = mfma32x32x16(k1, qr[ds], s1);
      }
      // Mask keys past the valid length and, for causal, keys after the query.
      if (n0 + BN > L || (CAUSAL && n0 + BN - 1 > qw)) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = n0 + (i >> 2) * 8 + hi * 4 + (i & 3);
          if (key >= L || (CAUSAL && key > q)) s0[i] = -INFINITY;
          if (key + 32 >= L || (CAUSAL && key + 32 > q)) s1[i] = -INFINITY;
        }
      }
      float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, fmaxf(s0[i], s1[i]));
      mx = max_halves(mx);
      const float m_new = fmaxf(m_run, mx);
      const float mc = m_new * c2;
      const float alpha = fast_exp2((m_run - m_new) * c2);
      float ls = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s0[i] = fast_exp2(fmaf(s0[i], c2, -mc));
        s1[i] = fast_exp2(fmaf(s1[i], c2, -mc));
        ls += s0[i] + s1[i];
      }
      l_run = alpha * l_run + ls;
      m_run = m_new;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
      // P^T -> bf16 B operands, one per 16-key step.
      bf16x8 pb[4];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        u32x4 w0 = {pack_bf16x2(s0[8 * h + 0], s0[8 * h + 1]), pack_bf16x2(s0[8 * h + 2], s0[8 * h + 3]),
                    pack_bf16x2(s0[8 * h + 4], s0[8 * h + 5]), pack_bf16x2(s0[8 * h + 6], s0[8 * h + 7])};
        u32x4 w1 = {pack_bf16x2(s1[8 * h + 0], s1[8 * h + 1]), pack_bf16x2(s1[8 * h + 2], s1[8 * h + 3]),
                    pack_bf16x2(s1[8 * h + 4], s1[8 * h + 5]), pack_bf16x2(s1[8 * h + 6], s1[8 * h + 7])};
        pb[h] = as_bf16x8(w0);
        pb[2 + h] = as_bf16x8(w1);
      }
      // O^T (D x 32) += V^T (D x 64) P^T (64 x 32). For key step ks the lane
      // half hi holds keys ks*16 + hi*4 + {0..3} and ks*16 + 8 + hi*4 + {0..3};
      // the two transposing reads fetch exactly those keys of V for d = lane%32.
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const lds_t* p = vb + v_lane + ks * 16 * VS + db * 64;
          const u32x2 lo = lds_load_tr16(p);
          const u32x2 up = lds_load_tr16(p + 8 * VS);
          o[db] = mfma32x32x16(join_bf16x8(lo, up), pb[ks], o[db]);
        }
      }
    }
    if (j + 1 < nt) lds_store_tile(st ^ 1);
    __syncthreads();
  }

  // Epilogue: O = O_acc / l, rounded to bf16; LSE = m*scale + ln l.
  const float l_tot = sum_halves(l_run);
  const bool valid = q < L && l_tot > 0.f;
  const float inv = valid ? 1.f / l_tot : 0.f;
  if (q < N) {
    bf16_t* orow = Oh + (size_t)q * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const u32x2 w = {pack_bf16x2(o[db][4 * g + 0] * inv, o[db][4 * g + 1] * inv),
                         pack_bf16x2(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv)};
        gstore8(orow + db * 32 + g * 8 + hi * 4, w);
      }
    if (lse_h && hi == 0) lse_h[q] = valid ? m_run * a.scale + logf(l_tot) : -INFINITY;
  }
}

// ----------------------------------------------------------------------------
// fp32 inputs: plain VALU kernel, one query row per lane, 64 rows per
// workgroup, K/V tiles of 32 keys in LDS (read as broadcasts). Same online
// softmax; the exponent is formed as (s - m) * scale*log2(e) so its rounding
// error scales with s - m, which keeps fp32 results within a few ulps.
// ----------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ void __launch_bounds__(64) fwd_f32_kernel(FwdArgs a) {
  constexpr int BM = 64, BN = 32, C4 = D / 4;
  __shared__ float4 ks[BN][C4];
  __shared__ float4 vs[BN][C4];
  const int lane = threadIdx.x;
  const int N = a.N;
  const int nm = (N + BM - 1) / BM;
  const int bh = blockIdx.x / nm, mt = blockIdx.x % nm;
  const int b = bh / a.H;
  int L = N;
  if (a.seqlens) L = min(max(a.seqlens[b], 0), N);
  const int m0 = mt * BM, q = m0 + lane;
  const size_t hoff = (size_t)bh * N * D;
  const float4* Qh = (const float4*)((const float*)a.q + hoff);
  const float4* Kh = (const float4*)((const float*)a.k + hoff);
  const float4* Vh = (const float4*)((const float*)a.v + hoff);
  float4* Oh = (float4*)((float*)a.o + hoff);
  const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);

  float4 qv[C4], acc[C4];
#pragma unroll
  for (int c = 0; c < C4; ++c) {
    qv[c] = q < N ? Qh[(size_t)q * C4 + c] : z;
    acc[c] = z;
  }
  float m_run = kMaxInit, l_run = 0.f;
  const float c2 = a.scale_log2;
  const int kv_end = m0 >= L ? 0 : (CAUSAL ? min(L, m0 + BM) : L);
  for (int n0 = 0; n0 < kv_end; n0 += BN) {
    __syncthreads();
    for (int e = lane; e < BN * C4; e += 64) {
      const int r = e / C4, c = e % C4, g = n0 + r;
      ks[r][c] = g < N ? Kh[(size_t)g * C4 + c] : z;
      vs[r][c] = g < N ? Vh[(size_t)g * C4 + c] : z;
    }
    __syncthreads();
    float s[BN];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < BN; ++j) {
      float d0 = 0.f, d1 = 0.f, d2 = 0.f, d3 = 0.f;
#pragma unroll
      for (int c = 0; c < C4; ++c) {
        const float4 kk = ks[j][c];
        d0 = fmaf(qv[c].x, kk.x, d0);
        d1 = fmaf(qv[c].y, kk.y, d1);
        d2 = fmaf(qv[c].z, kk.z, d2);
        d3 = fmaf(qv[c].w, kk.w, d3);
      }
      const int key = n0 + j;
      s[j] = (key >= L || (CAUSAL && key > q)) ? -INFINITY : (d0 + d1) + (d2 + d3);
      mx = fmaxf(mx, s[j]);
    }
    const float m_new = fmaxf(m_run, mx);
    const float alpha = fast_exp2((m_run - m_new) * c2);
    float ls = 0.f;
#pragma unroll
    for (int j = 0; j < BN; ++j) {
      s[j] = fast_exp2((s[j] - m_new) * c2);
      ls += s[j];
    }
    l_run = alpha * l_run + ls;
    m_run = m_new;
#pragma unroll
    for (int c = 0; c < C4; ++c) {
      float4 t = acc[c];
      t.x *= alpha; t.y *= alpha; t.z *= alpha; t.w *= alpha;
#pragma unroll
      for (int j = 0; j < BN; ++j) {
        const float4 vv = vs[j][c];
        t.x = fmaf(s[j], vv.x, t.x);
        t.y = fmaf(s[j], vv.y, t.y);
        t.z = fmaf(s[j], vv.z, t.z);
        t.w = fmaf(s[j], vv.w, t.w);
      }
      acc[c] = t;
    }
  }
  if (q < N) {
    const bool valid = q < L && l_run > 0.f;
    const float inv = valid ? 1.f / l_run : 0.f;
#pragma unroll
    for (int c = 0; c < C4; ++c) {
      float4 t = acc[c];
      t.x *= inv; t.y *= inv; t.z *= inv; t.w *= inv;
      Oh[(size_t)q * C4 + c] = t;
    }
    if (a.lse) a.lse[(size_t)bh * N + q] = valid ? m_run * a.scale + logf(l_run) : -INFINITY;
  }
}

template <int D, bool CAUSAL>
hipError_t launch_bf16_t(const FwdArgs& a, hipStream_t stream) {
  constexpr int BM = 128, BN = 64;
  constexpr int lds = 2 * (BN * (D * 2 + 16) + BN * (D * 2 + 64));
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)fwd_bf16_kernel<D, CAUSAL>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int nm = (a.N + BM - 1) / BM;
  dim3 grid((unsigned)(nm * a.B * a.H)), block(256);
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL>), grid, block, lds, stream, a);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_f32_t(const FwdArgs& a, hipStream_t stream) {
  const int nm = (a.N + 63) / 64;
  dim3 grid((unsigned)(nm * a.B * a.H)), block(64);
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, int d, bool causal, hipStream_t stream) {
  if (d == 64) return causal ? launch_bf16_t<64, true>(a, stream) : launch_bf16_t<64, false>(a, stream);
  return causal ? launch_bf16_t<128, true>(a, stream) : launch_bf16_t<128, false>(a, stream);
}

hipError_t launch_fwd_f32(const FwdArgs& a, int d, bool causal, hipStream_t stream) {
  if (d == 64) return causal ? launch_f32_t<64, true>(a, stream) : launch_f32_t<64, false>(a, stream);
  return causal ? launch_f32_t<128, true>(a, stream) : launch_f32_t<128, false>(a, stream);
}

void tile_order_host(int block, int num_tiles, int num_heads, bool heavy_first, int* head, int* tile) {
  int h, t;
  tile_order(block, num_tiles, num_heads, heavy_first, h, t);
  *head = h;
  *tile = t;
}

}  // namespace attn
