// fp32 attention forward for gfx950 (VALU arithmetic, no matrix cores).
//
// Pages cited (by title):
//   [SafeSoftmax] "FlashAttention：从 Safe Softmax 到分块计算"
//   [OpOpt]       "Attention 算子优化:从物化 N×N 矩阵到 FlashAttention 与 PagedAttention"
//   [AIInfra]     the AIInfra FlashAttention note on dpshk.com
//
// The same method as the 16-bit forward: one workgroup per row tile of Q and
// (batch, head), K/V tiles streamed through LDS ([SafeSoftmax] §5), the
// online-softmax state (m, l, unnormalised O) of [SafeSoftmax] §3.1 merged
// tile by tile with the rescale of §3.2 (single-exponential form of the
// [AIInfra] §2.1 loop, finite initial max), causal tiles above the diagonal
// never visited and padded keys masked ([OpOpt] §四, §二), O divided by l at
// the end and the row log-sum-exp written ([SafeSoftmax] §8).
#include "attn_common.h"
#include "attn_kernels.h"

#include <math.h>

namespace attn {

namespace {

// ----------------------------------------------------------------------------
// fp32 inputs: VALU kernel. Four lanes (a DPP quad) share a query row; lane
// slice s of the quad holds the 16-byte column chunks 4c + s of q and of the
// output accumulator, so a score is the sum of four partial dot products (two
// quad exchanges, after which all four lanes hold the same score and run the
// same softmax arithmetic on it). 16 rows per wave, 64 per 256-thread
// workgroup. K/V tiles of 32 keys: the workgroup loads tile t+1 into
// registers (all its loads in flight at once) while it computes tile t from
// LDS; the quad's four lanes read four consecutive chunks of one key row, the
// other quads the same bytes (a broadcast). The running max moves to the
// exact max of every tile (no lazy reference as in the 16-bit kernels), and
// the exponent is formed as (s - m) * scale*log2(e) so its rounding error
// scales with s - m, which keeps fp32 results within a few ulps.
// ----------------------------------------------------------------------------

// Sum over the four lanes of a quad; every lane gets the same bits (both
// steps add the same two operands in either order).
__device__ __forceinline__ float sum_quad(float x) {
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));  // lanes 1,0,3,2
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));  // lanes 2,3,0,1
  return x;
}

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(256) fwd_f32_kernel(FwdArgs a) {
  constexpr int BM = 64, BN = 32, D4 = D / 4, C4 = D4 / 4;
  constexpr int LPT = BN * D4 / 256;  // float4 loads per thread, tensor and tile
  __shared__ f32x4 ks[BN][D4];
  __shared__ f32x4 vs[BN][D4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, slice = lane & 3;
  const int N = a.N;
  const int nm = (N + BM - 1) / BM;
  const int bh = blockIdx.x / nm, mt = blockIdx.x % nm;
  const int b = bh / a.H;
  int L = N;
  if (a.seqlens) L = min(max(a.seqlens[b], 0), N);
  const int m0 = mt * BM, q = m0 + wave * 16 + (lane >> 2);
  const size_t hoff = (size_t)bh * N * D;
  const size_t kvoff = (size_t)(b * a.H_kv + (bh % a.H) / (a.H / a.H_kv)) * N * D;
  const f32x4* Qh = (const f32x4*)((const float*)a.q + hoff);
  const f32x4* Kh = (const f32x4*)((const float*)a.k + kvoff);
  const f32x4* Vh = (const f32x4*)((const float*)a.v + kvoff);
  f32x4* Oh = (f32x4*)((float*)a.o + hoff);
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};

  f32x4 qv[C4], acc[C4];
#pragma unroll
  for (int c = 0; c < C4; ++c) {
    qv[c] = q < L ? Qh[(size_t)q * D4 + 4 * c + slice] : z;
    acc[c] = z;
  }
  const int kv_end = m0 >= L ? 0 : (CAUSAL ? min(L, m0 + BM) : L);
  const int nt = (kv_end + BN - 1) / BN;
  f32x4 kreg[LPT], vreg[LPT];
  auto fetch = [&](int n0) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int e = tid + 256 * i, g = n0 + e / D4;
      kreg[i] = g < L ? Kh[(size_t)g * D4 + e % D4] : z;
      vreg[i] = g < L ? Vh[(size_t)g * D4 + e % D4] : z;
    }
  };
  if (nt > 0) fetch(0);
  float m_run = kMaxInit, l_run = 0.f;
  const float c2 = a.scale_log2;
  for (int t = 0; t < nt; ++t) {
    const int n0 = t * BN;
    __syncthreads();  // every wave is done with tile t-1
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int e = tid + 256 * i;
      ks[e / D4][e % D4] = kreg[i];
      vs[e / D4][e % D4] = vreg[i];
    }
    __syncthreads();
    if (t + 1 < nt) fetch(n0 + BN);
    float s[BN];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < BN; ++j) {
      float d0 = 0.f, d1 = 0.f, d2 = 0.f, d3 = 0.f;
#pragma unroll
      for (int c = 0; c < C4; ++c) {
        const f32x4 kk = ks[j][4 * c + slice];
        d0 = fmaf(qv[c][0], kk[0], d0);
        d1 = fmaf(qv[c][1], kk[1], d1);
        d2 = fmaf(qv[c][2], kk[2], d2);
        d3 = fmaf(qv[c][3], kk[3], d3);
      }
      const float dot = sum_quad((d0 + d1) + (d2 + d3));
      const int key = n0 + j;
      s[j] = (key >= L || (CAUSAL && key > q)) ? -INFINITY : dot;
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
      f32x4 u = acc[c] * alpha;
#pragma unroll
      for (int j = 0; j < BN; ++j) {
        const f32x4 vv = vs[j][4 * c + slice];
#pragma unroll
        for (int i = 0; i < 4; ++i) u[i] = fmaf(s[j], vv[i], u[i]);
      }
      acc[c] = u;
    }
  }
  if (q < N) {
    const bool valid = q < L && l_run > 0.f;
    const float inv = valid ? 1.f / l_run : 0.f;
#pragma unroll
    for (int c = 0; c < C4; ++c) {
      Oh[(size_t)q * D4 + 4 * c + slice] = acc[c] * inv;
    }
    if (a.lse && slice == 0) a.lse[(size_t)bh * N + q] = valid ? m_run * a.scale + logf(l_run) : -INFINITY;
  }
}

template <int D, bool CAUSAL>
hipError_t launch_f32_t(const FwdArgs& a, hipStream_t stream) {
  const int nm = (a.N + 63) / 64;
  dim3 grid((unsigned)(nm * a.B * a.H)), block(256);
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a, int d, bool causal, hipStream_t stream) {
  if (d == 64) return causal ? launch_f32_t<64, true>(a, stream) : launch_f32_t<64, false>(a, stream);
  return causal ? launch_f32_t<128, true>(a, stream) : launch_f32_t<128, false>(a, stream);
}

}  // namespace attn
