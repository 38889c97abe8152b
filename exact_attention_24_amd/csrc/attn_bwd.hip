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
//   bwd_pre:  delta_i = rowsum(dO_i o O_i)                    (HBM-bound)
//   bwd_dkdv: one workgroup per 128 keys; loops over the query tiles that can
//             see those keys, accumulating dK and dV in registers
//   bwd_dq:   one workgroup per 128 queries; loops over the key tiles they
//             see, accumulating dQ in registers (no atomics: deterministic)
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

// Store a transposed 32-row accumulator block: lane holds column `row` of the
// result and values for d = db*32 + g*8 + hi*4 + {0..3}.
template <int DB>
__device__ __forceinline__ void store_rowT(bf16_t* rowp, const f32x16* acc, float mul, int hi) {
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const u32x2 w = {pack_bf16x2(acc[db][4 * g + 0] * mul, acc[db][4 * g + 1] * mul),
                       pack_bf16x2(acc[db][4 * g + 2] * mul, acc[db][4 * g + 3] * mul)};
      gstore8(rowp + db * 32 + g * 8 + hi * 4, w);
    }
}

// ---------------------------------------------------------------------------
// delta_i = sum_d dO_i[d] * O_i[d] in fp32; 0 for padded rows.
// ---------------------------------------------------------------------------
template <int D>
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
      const u32x4 o = gload16((const bf16_t*)a.o + row * D + c * 8);
      const u32x4 g = gload16((const bf16_t*)a.dO + row * D + c * 8);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        part += bf16_lo(o[i]) * bf16_lo(g[i]) + bf16_hi(o[i]) * bf16_hi(g[i]);
    }
  }
#pragma unroll
  for (int m = TPR / 2; m >= 1; m >>= 1) part += __shfl_xor(part, m, TPR);
  if (row < total && c == 0) a.delta[row] = valid ? part : 0.f;
}

// ---------------------------------------------------------------------------
// dK, dV: workgroup = 4 waves x 32 keys. Each wave keeps its K and V rows in
// VGPRs (B operands of S = Q K^T and dP = dO V^T) and accumulates dK^T, dV^T.
// Query tiles of 64 rows (Q, dO, log2-scaled LSE, delta) are double-buffered in
// LDS and processed as two 32-row sub-blocks:
//   S  (q x key)   = Q  K^T        A = Q rows (LDS),   B = K (VGPR)
//   P              = exp2(S*scale*log2e - LSE*log2e), masked
//   dV^T (d x key) += dO^T P       A = dO^T (transposing LDS read), B = P
//   dP (q x key)   = dO V^T        A = dO rows (LDS),  B = V (VGPR)
//   dS             = P o (dP - delta)
//   dK^T (d x key) += Q^T dS       A = Q^T (transposing LDS read),  B = dS
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ void __launch_bounds__(256, 1) bwd_dkdv_kernel(BwdArgs a) {
  constexpr int BN = 128, BM = 64;
  constexpr int TILE = BM * D * 2;
  constexpr int STAGE = 2 * TILE + 2 * BM * 4;
  constexpr int CH = D / 8, LOADS = BM * CH / 256;
  constexpr int DS = D / 16, DB = D / 32;

  extern __shared__ __attribute__((aligned(16))) char smem_generic[];
  lds_t* smem = lds_base(smem_generic);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int N = a.N;
  const int nkt = (N + BN - 1) / BN;
  int bh, kt;
  tile_order(blockIdx.x, nkt, a.B * a.H, false, bh, kt);
  const int L = seq_len(a, bh / a.H);
  const int n0 = kt * BN;
  const size_t hoff = (size_t)bh * N * D;
  const bf16_t* __restrict__ Qh = (const bf16_t*)a.q + hoff;
  const bf16_t* __restrict__ Kh = (const bf16_t*)a.k + hoff;
  const bf16_t* __restrict__ Vh = (const bf16_t*)a.v + hoff;
  const bf16_t* __restrict__ dOh = (const bf16_t*)a.dO + hoff;
  const float* __restrict__ lse_h = a.lse + (size_t)bh * N;
  const float* __restrict__ del_h = a.delta + (size_t)bh * N;
  bf16_t* __restrict__ dKh = (bf16_t*)a.dk + hoff;
  bf16_t* __restrict__ dVh = (bf16_t*)a.dv + hoff;
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

  const int kw = n0 + wave * 32;  // first key of this wave
  const int key = kw + l32;       // this lane's key (B-operand column)
  bf16x8 kreg[DS], vreg[DS];
#pragma unroll
  for (int ds = 0; ds < DS; ++ds) {
    const size_t off = (size_t)key * D + ds * 16 + hi * 8;
    kreg[ds] = as_bf16x8(key < N ? gload16(Kh + off) : zero4);
    vreg[ds] = as_bf16x8(key < N ? gload16(Vh + off) : zero4);
  }

  const int q_begin = CAUSAL ? (n0 / BM) * BM : 0;
  const int nqt = (L - q_begin + BM - 1) / BM;
  const float c2 = a.scale_log2;

  u32x4 qr[LOADS], dor[LOADS];
  float lr = 0.f, dr = 0.f;
  auto gload_tile = [&](int q0) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int c = tid + 256 * i, row = c / CH, col = c % CH, g = q0 + row;
      qr[i] = g < N ? gload16(Qh + (size_t)g * D + col * 8) : zero4;
      dor[i] = g < N ? gload16(dOh + (size_t)g * D + col * 8) : zero4;
    }
    if (tid < BM) {
      const int g = q0 + tid;
      lr = g < L ? lse_h[g] * kLog2e : 0.f;
      dr = g < L ? del_h[g] : 0.f;
    }
  };
  auto lds_store_tile = [&](int st) {
    lds_t* qt = smem + st * STAGE;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int c = tid + 256 * i, row = c / CH, col = c % CH;
      lds_store16(qt + tile_off<D>(row, col), qr[i]);
      lds_store16(qt + TILE + tile_off<D>(row, col), dor[i]);
    }
    if (tid < BM) {
      lds_storef(qt + 2 * TILE + tid * 4, lr);
      lds_storef(qt + 2 * TILE + BM * 4 + tid * 4, dr);
    }
  };

  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) { dk[db][i] = 0.f; dv[db][i] = 0.f; }

  gload_tile(q_begin);
  lds_store_tile(0);
  __syncthreads();

  for (int t = 0; t < nqt; ++t) {
    const int st = t & 1, qt0 = q_begin + t * BM;
    if (t + 1 < nqt) gload_tile(qt0 + BM);
    const lds_t* Qt = smem + st * STAGE;
    const lds_t* dOt = Qt + TILE;
    const lds_t* lse_t = Qt + 2 * TILE;
    const lds_t* del_t = lse_t + BM * 4;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const int qs = qt0 + sb * 32;
      if (kw >= L || qs >= L || (CAUSAL && qs + 31 < kw)) continue;
      f32x16 s, dp;
#pragma unroll
      for (int i = 0; i < 16; ++i) { s[i] = 0.f; dp[i] = 0.f; }
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) {
        const bf16x8 qa = as_bf16x8(lds_load16(Qt + tile_off<D>(sb * 32 + l32, ds * 2 + hi)));
        const bf16x8 da = as_bf16x8(lds_load16(dOt + tile_off<D>(sb * 32 + l32, ds * 2 + hi)));
        s = mfma32x32x16(qa, kreg[ds], s);
        dp = mfma32x32x16(da, vreg[ds], dp);
      }
      const bool need_mask = qs + 32 > L || kw + 32 > L || (CAUSAL && qs < kw + 31);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int rl = sb * 32 + g * 8 + hi * 4;  // first of 4 consecutive query rows
        const f32x4 l4 = *(const ATTN_LDS f32x4*)(lse_t + rl * 4);
        const f32x4 d4 = *(const ATTN_LDS f32x4*)(del_t + rl * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * g + e;
          float p = fast_exp2(fmaf(s[i], c2, -l4[e]));
          if (need_mask) {
            const int q = qt0 + rl + e;
            if (key >= L || q >= L || (CAUSAL && key > q)) p = 0.f;
          }
          s[i] = p;
          dp[i] = p * (dp[i] - d4[e]);
        }
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const bf16x8 pb = pack8(s, h);
        const bf16x8 sb16 = pack8(dp, h);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          dv[db] = mfma32x32x16(tr_operand<D>(dOt, sb * 32 + h * 16, db * 32, lane), pb, dv[db]);
          dk[db] = mfma32x32x16(tr_operand<D>(Qt, sb * 32 + h * 16, db * 32, lane), sb16, dk[db]);
        }
      }
    }
    if (t + 1 < nqt) lds_store_tile(st ^ 1);
    __syncthreads();
  }

  if (key < N) {
    store_rowT<DB>(dKh + (size_t)key * D, dk, a.scale, hi);
    store_rowT<DB>(dVh + (size_t)key * D, dv, 1.f, hi);
  }
}

// ---------------------------------------------------------------------------
// dQ: workgroup = 4 waves x 32 queries; Q and dO rows stay in VGPRs (B
// operands), K/V tiles of 64 keys are double-buffered in LDS:
//   S^T  (key x q) = K Q^T     A = K rows (LDS),  B = Q (VGPR)
//   dP^T (key x q) = V dO^T    A = V rows (LDS),  B = dO (VGPR)
//   dS^T = P^T o (dP^T - delta)   (LSE and delta are per-lane scalars)
//   dQ^T (d x q)  += K^T dS^T  A = K^T (transposing LDS read), B = dS^T
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ void __launch_bounds__(256, 2) bwd_dq_kernel(BwdArgs a) {
  constexpr int BM = 128, BN = 64;
  constexpr int TILE = BN * D * 2;
  constexpr int STAGE = 2 * TILE;
  constexpr int CH = D / 8, LOADS = BN * CH / 256;
  constexpr int DS = D / 16, DB = D / 32;

  extern __shared__ __attribute__((aligned(16))) char smem_generic[];
  lds_t* smem = lds_base(smem_generic);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int N = a.N;
  const int nm = (N + BM - 1) / BM;
  int bh, mt;
  tile_order(blockIdx.x, nm, a.B * a.H, CAUSAL, bh, mt);
  const int L = seq_len(a, bh / a.H);
  const int m0 = mt * BM;
  const size_t hoff = (size_t)bh * N * D;
  const bf16_t* __restrict__ Qh = (const bf16_t*)a.q + hoff;
  const bf16_t* __restrict__ Kh = (const bf16_t*)a.k + hoff;
  const bf16_t* __restrict__ Vh = (const bf16_t*)a.v + hoff;
  const bf16_t* __restrict__ dOh = (const bf16_t*)a.dO + hoff;
  bf16_t* __restrict__ dQh = (bf16_t*)a.dq + hoff;
  const u32x4 zero4 = {0u, 0u, 0u, 0u};

  if (m0 >= L) {
    const int rows = min(BM, N - m0);
    for (int c = tid; c < rows * CH; c += 256)
      gstore16(dQh + (size_t)(m0 + c / CH) * D + (c % CH) * 8, zero4);
    return;
  }

  const int qw = m0 + wave * 32, q = qw + l32;
  const bool qvalid = q < L;
  const float lse2 = qvalid ? a.lse[(size_t)bh * N + q] * kLog2e : 0.f;
  const float dq_delta = qvalid ? a.delta[(size_t)bh * N + q] : 0.f;
  bf16x8 qreg[DS], doreg[DS];
#pragma unroll
  for (int ds = 0; ds < DS; ++ds) {
    const size_t off = (size_t)q * D + ds * 16 + hi * 8;
    qreg[ds] = as_bf16x8(q < N ? gload16(Qh + off) : zero4);
    doreg[ds] = as_bf16x8(q < N ? gload16(dOh + off) : zero4);
  }

  const int kv_end = CAUSAL ? min(L, m0 + BM) : L;
  const int nt = (kv_end + BN - 1) / BN;
  const int w_end = (qw >= L) ? 0 : (CAUSAL ? min(L, qw + 32) : L);
  const int wnt = (w_end + BN - 1) / BN;
  const float c2 = a.scale_log2;

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
    lds_t* kt = smem + st * STAGE;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int c = tid + 256 * i, row = c / CH, col = c % CH;
      lds_store16(kt + tile_off<D>(row, col), kr[i]);
      lds_store16(kt + TILE + tile_off<D>(row, col), vr[i]);
    }
  };

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;

  gload_tile(0);
  lds_store_tile(0);
  __syncthreads();

  for (int j = 0; j < nt; ++j) {
    const int st = j & 1, n0 = j * BN;
    if (j + 1 < nt) gload_tile(n0 + BN);
    if (j < wnt) {
      const lds_t* Kt = smem + st * STAGE;
      const lds_t* Vt = Kt + TILE;
      const bool need_mask = n0 + BN > L || qw + 32 > L || (CAUSAL && n0 + BN - 1 > qw);
      // One 32-key block at a time keeps only one S^T and one dP^T block live.
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        f32x16 s, dp;
#pragma unroll
        for (int i = 0; i < 16; ++i) { s[i] = 0.f; dp[i] = 0.f; }
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
          const bf16x8 ka = as_bf16x8(lds_load16(Kt + tile_off<D>(kb * 32 + l32, ds * 2 + hi)));
          const bf16x8 va = as_bf16x8(lds_load16(Vt + tile_off<D>(kb * 32 + l32, ds * 2 + hi)));
          s = mfma32x32x16(ka, qreg[ds], s);
          dp = mfma32x32x16(va, doreg[ds], dp);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float p = fast_exp2(fmaf(s[i], c2, -lse2));
          if (need_mask) {
            const int key = n0 + kb * 32 + (i >> 2) * 8 + hi * 4 + (i & 3);
            if (key >= L || !qvalid || (CAUSAL && key > q)) p = 0.f;
          }
          dp[i] = p * (dp[i] - dq_delta);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const bf16x8 dsb = pack8(dp, h);
#pragma unroll
          for (int db = 0; db < DB; ++db)
            acc[db] = mfma32x32x16(tr_operand<D>(Kt, kb * 32 + h * 16, db * 32, lane), dsb, acc[db]);
        }
      }
    }
    if (j + 1 < nt) lds_store_tile(st ^ 1);
    __syncthreads();
  }

  if (q < N) store_rowT<DB>(dQh + (size_t)q * D, acc, qvalid ? a.scale : 0.f, hi);
}

template <int D, bool CAUSAL>
hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t stream) {
  constexpr int lds_dkdv = 2 * (2 * 64 * D * 2 + 2 * 64 * 4);
  constexpr int lds_dq = 2 * (2 * 64 * D * 2);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)bwd_dkdv_kernel<D, CAUSAL>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds_dkdv);
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute((const void*)bwd_dq_kernel<D, CAUSAL>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, lds_dq);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const long long rows = (long long)a.B * a.H * a.N;
  constexpr int RPB = 256 / (D / 8);
  hipLaunchKernelGGL((bwd_pre_kernel<D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0,
                     stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int heads = a.B * a.H;
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3((unsigned)(heads * ((a.N + 127) / 128))),
                     dim3(256), lds_dkdv, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), dim3((unsigned)(heads * ((a.N + 127) / 128))),
                     dim3(256), lds_dq, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdArgs& a, int d, bool causal, hipStream_t stream) {
  if (d == 64) return causal ? launch_bwd_t<64, true>(a, stream) : launch_bwd_t<64, false>(a, stream);
  return causal ? launch_bwd_t<128, true>(a, stream) : launch_bwd_t<128, false>(a, stream);
}

}  // namespace attn
