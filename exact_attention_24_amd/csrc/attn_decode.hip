// Split-KV decode for gfx950: a few new queries per sequence against a long
// K/V cache.
//
// Pages cited (by title):
//   [SafeSoftmax] "FlashAttention：从 Safe Softmax 到分块计算"
//   [OpOpt]       "Attention 算子优化:从物化 N×N 矩阵到 FlashAttention 与 PagedAttention"
//
// Decode reads the whole K/V cache for very little arithmetic, so it is bound
// by HBM bandwidth, not by the matrix cores ([OpOpt] §五). With one query row
// per (batch, head) a forward-style launch would have B*H workgroups each
// walking the full key range; here the keys of every K/V head are dealt to
// splits that run in parallel ([SafeSoftmax] §10: split the K/V dimension
// across workgroups), each keeping the online-softmax state (m, l,
// unnormalised O) of [SafeSoftmax] §3.1 for its keys, and a second kernel
// combines the splits with the merge rule of [SafeSoftmax] §3.2 (which does
// not depend on which keys a split holds). Split s of S takes the 32-key
// chunks s, s + S, s + 2S, ...: the splits of one head then read neighbouring
// chunks at the same time, which streams from HBM faster than S separate
// contiguous ranges (measured 3-4% on the eight-token and FP8 workloads).
//
// Split kernel: one wave per 32-column block. The G = H / H_kv query heads
// that share a K/V head ([OpOpt] §五) and their N_q queries are packed into
// the columns of MFMA blocks (column c = g*N_q + i, 32 per block), so each K/V
// byte is read from HBM once for all of them; two blocks of the same (batch,
// K/V head, split) run as the two waves of one workgroup and share every
// chunk load. K/V chunks of 32 keys stream through a ring in LDS by direct
// buffer->LDS loads (three stages, two chunks in flight; FP8: four stages,
// three in flight, fewer bytes); S^T = K Q^T and O^T += V^T P^T run on
// v_mfma_f32_32x32x16 exactly as in the forward kernel.
//
// FP8 K/V cache ([OpOpt] §六): K and V stored as OCP E4M3 bytes with one fp32
// scale per token (K_j = k8_j * ks_j, V_j = v8_j * vs_j). HBM and LDS carry the
// 8-bit form; each MFMA operand is read from the FP8 tile (V through the 8-bit
// transposing read) and widened exactly to the 16-bit format of Q in
// registers (every E4M3 value is exact in bf16 and in fp16), and the products
// run on the matching MFMA. The scales are applied in fp32:
// ks_j to the scores after the K product (S_ij = ks_j * (q_i . k8_j)), vs_j
// to the weights before they are rounded for the V product (the row sums use
// the unscaled weights), so the softmax and accumulation stay fp32.
//
// Query positions: the N_q queries of sequence b are its last N_q positions,
// L_b - N_q .. L_b - 1, so with causal masking query i sees keys
// j <= L_b - N_q + i (when N_q = L_b this is the forward's top-left mask).
#include "attn_common.h"
#include "attn_kernels.h"
#include "attn_tile.h"

#include <math.h>

namespace attn {

namespace {

constexpr float kLazyRescaleDecW = 256.0f;  // largest unnormalised weight kept without rescaling

// Two E4M3 bytes (the low or high half of w) widened exactly to the 16-bit
// format (every E4M3 value is representable in bf16 and in fp16). The scale
// operand is 1.0: these conversions use only the exponent of their scale.
template <bool F16>
__device__ __forceinline__ uint32_t widen2(uint32_t w, bool high) {
  if constexpr (F16)
    return __builtin_bit_cast(uint32_t, high ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.f, true)
                                             : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.f, false));
  else
    return __builtin_bit_cast(uint32_t, high ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.f, true)
                                             : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.f, false));
}

// A operand of the score MFMA for k step ds, straight from an FP8 tile in the
// layout above: lane l takes key row l%32, bytes 16*ds + 8*(l/32) .. +7 (eight
// consecutive d), widened exactly in registers (no 16-bit copy of K in LDS).
template <int D, bool F16>
__device__ __forceinline__ e16x8 fp8_row_operand(const lds_t* tile, int ds, int lane) {
  const int r = lane & 31;
  const u32x2 w = lds_load8(tile + r * D + ((ds ^ swz<D / 2>(r)) << 4) + (lane >> 5) * 8);
  const u32x4 e = {widen2<F16>(w[0], false), widen2<F16>(w[0], true), widen2<F16>(w[1], false),
                   widen2<F16>(w[1], true)};
  return as_e16x8(e);
}

// A operand of the P V MFMA (V^T rows d = col0 + l%32, the 8 keys of 16-key
// step row0 that the score accumulator lanes hold: row0 + hi*4 + {0..3} and
// row0 + 8 + hi*4 + {0..3}) straight from an FP8 V tile, with one transposing
// 8-bit read: source lane src of each 16-lane group addresses key slot src/2
// at columns 8*(src%2) .. +7 of its 16-column half, and lane j receives the
// byte (j%16)%8 of sources (j%16)/8 + 2s, i.e. column col0 + l%32 of key slot
// s. Widened exactly in registers.
template <int D, bool F16>
__device__ __forceinline__ e16x8 fp8_tr_operand(const lds_t* tile, int row0, int col0, int lane) {
  const int g = lane >> 4, src = lane & 15, s = src >> 1;
  const int key = row0 + (s < 4 ? (g >> 1) * 4 + s : 8 + (g >> 1) * 4 + (s - 4));
  const int c = col0 + 16 * (g & 1) + 8 * (src & 1);
  const u32x2 w = lds_load_tr8(tile + key * D + (((c >> 4) ^ swz<D / 2>(key)) << 4) + (c & 15));
  const u32x4 e = {widen2<F16>(w[0], false), widen2<F16>(w[0], true), widen2<F16>(w[1], false),
                   widen2<F16>(w[1], true)};
  return as_e16x8(e);
}

template <int D, bool F16, bool KV8, int NW>
__device__ __forceinline__ void decode_split_body(const DecArgs& a) {
  constexpr int BN = 32;  // keys per chunk
  constexpr int DD = KV8 ? D / 2 : D;  // row width in 16-bit units as stored in HBM
  constexpr int TILE = BN * DD * 2;    // bytes of one stored chunk
  constexpr int DS = D / 16, DB = D / 32;
  constexpr int LPC = 2 * TileDma<DD, BN, NW>::ITER + (KV8 ? 2 : 0);  // loads per chunk and wave
  // Ring of NST chunk stages, NST - 1 chunks in flight. An FP8 chunk is half
  // the bytes of a 16-bit one, so its ring is one stage deeper. Measured on
  // the B=8, 64:8-head, 8192-position workloads with the caches in HBM only:
  // 3 stages (16-bit) and 4 (FP8) with the split counts chosen in the host
  // code were the best of ring depths 2-7 and 256-1536 workgroups.
  constexpr int NST = KV8 ? 4 : 3;
  __shared__ __attribute__((aligned(1024))) char kr_[NST][TILE], vr_[NST][TILE];
  // FP8 only: per-stage token scales (64 floats fetched, the first 32 used).
  // K and V operands are widened in registers from the FP8 tiles.
  __shared__ __attribute__((aligned(256))) float ks_[KV8 ? NST : 1][64], vs_[KV8 ? NST : 1][64];

  // NW waves share each chunk: wave w takes column block cg0 + w of the same
  // (batch, K/V head, split), so the chunk is fetched once for all of them.
  const int lane = threadIdx.x & 63, l32 = lane & 31, hi = lane >> 5;
  const int wave = NW > 1 ? __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) : 0;
  const int G = a.H / a.H_kv;
  int bid = blockIdx.x;
  const int s = bid % a.splits;
  bid /= a.splits;
  const int cg = (bid % (a.col_groups / NW)) * NW + wave;
  bid /= a.col_groups / NW;
  const int bkv = bid;  // b * H_kv + kv head
  const int b = bkv / a.H_kv, kvh = bkv % a.H_kv;
  const int L = a.kv_lens ? min(max(a.kv_lens[b], 0), a.Nk) : a.Nk;

  // This lane's query column.
  const int col = cg * 32 + l32;
  const bool cvalid = col < G * a.Nq;
  const int g = cvalid ? col / a.Nq : 0, qi = cvalid ? col % a.Nq : 0;
  const int h = kvh * G + g;
  const size_t qrow = ((size_t)(b * a.H + h) * a.Nq + qi);  // row of q, o, lse, partials
  const int pos = L - a.Nq + qi;                           // this query's position

  const int j_begin = s * BN;                  // first key of this split's first chunk
  const int CS = a.splits * BN;                 // keys between this split's chunks
  const int nchunks = (L + BN - 1) / BN;
  const int nch = nchunks > s ? (nchunks - s + a.splits - 1) / a.splits : 0;
  const int j_end = L;

  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  e16x8 qr[DS];
#pragma unroll
  for (int ds = 0; ds < DS; ++ds)
    qr[ds] = as_e16x8(cvalid ? gload16((const e16_t*)a.q + qrow * D + ds * 16 + hi * 8) : zero4);

  const size_t kvoff = (size_t)bkv * a.Nk * DD;  // in 16-bit units
  const TileDma<DD, BN, NW> kdma((const e16_t*)a.k + kvoff, j_end, wave, lane);
  const TileDma<DD, BN, NW> vdma((const e16_t*)a.v + kvoff, j_end, wave, lane);
  auto kst = [&](int st) { return lds_base(kr_[st]); };
  auto vst = [&](int st) { return lds_base(vr_[st]); };
  const float* ksh = KV8 ? a.k_scale + (size_t)bkv * a.Nk : nullptr;
  const float* vsh = KV8 ? a.v_scale + (size_t)bkv * a.Nk : nullptr;
  auto load_chunk = [&](int st, int j0) {
    kdma.load(kst(st), j0);
    vdma.load(vst(st), j0);
    if constexpr (KV8) {  // every wave fetches the same scales to the same place
      vec64_dma(lds_base((char*)ks_[st]), ksh, j_end, j0, lane);
      vec64_dma(lds_base((char*)vs_[st]), vsh, j_end, j0, lane);
    }
  };
#pragma unroll
  for (int c = 0; c < NST - 1; ++c)
    if (c < nch) load_chunk(c, j_begin + c * CS);

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
  float m_ref = kMaxInit, l_part = 0.f;
  const float c2 = a.scale_log2;
  // Last visible key of this column (keys past it are masked).
  const int last = a.causal ? min(pos, L - 1) : L - 1;

  auto chunk = [&](int t, const int st) {
    const int j0 = j_begin + t * CS;
    // Chunk t + NST - 1 goes into the stage chunk t - 1 used; chunk t is
    // waited for (the loads of a wave complete in issue order, so "all but the
    // newest n"). One wave: issue first, then wait. Several: wait for this
    // wave's share of chunk t, meet at the barrier (every share has landed and
    // every wave is done with chunk t - 1), then issue.
    const bool more = t + NST - 1 < nch;
    if (NW == 1 && more) load_chunk((st + NST - 1) % NST, j0 + (NST - 1) * CS);
    const int after = min(NW == 1 ? NST - 1 : NST - 2, nch - 1 - t);  // chunks issued after t
    if (after >= 4) dma_wait_allbut<(NST > 4 ? 4 : 1) * LPC>();
    else if (after == 3) dma_wait_allbut<(NST > 3 ? 3 : 1) * LPC>();
    else if (after == 2) dma_wait_allbut<2 * LPC>();
    else if (after == 1) dma_wait_allbut<LPC>();
    else dma_wait();
    if constexpr (NW > 1) {
      __syncthreads();
      if (more) load_chunk((st + NST - 1) % NST, j0 + (NST - 1) * CS);
    }
    const lds_t* Kt = kst(st);
    const lds_t* Vt = vst(st);
    f32x4 ksc[4], vsc[4];  // FP8: token scales of this lane's 16 keys
    if constexpr (KV8) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        ksc[gq] = *(const f32x4*)&ks_[st][gq * 8 + hi * 4];
        vsc[gq] = *(const f32x4*)&vs_[st][gq * 8 + hi * 4];
      }
    }
    auto kop = [&](int ds) {
      if constexpr (KV8) return fp8_row_operand<D, F16>(Kt, ds, lane);
      else return row_operand<D>(Kt, 0, ds * 2, lane);
    };
    f32x16 sc = mfma32x32x16_z<F16>(kop(0), qr[0]);
#pragma unroll
    for (int ds = 1; ds < DS; ++ds) sc = mfma32x32x16<F16>(kop(ds), qr[ds], sc);
    if constexpr (KV8) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[i] *= ksc[i >> 2][i & 3];
    }
    // Element i is key j0 + hi*4 + c (c = (i/4)*8 + i%4); visible iff c <= lim.
    const int lim = last - j0 - hi * 4;
    if (__builtin_amdgcn_ballot_w64(lim < BN - 1)) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[i] = ((i >> 2) * 8 + (i & 3)) <= lim ? sc[i] : -INFINITY;
    }
    auto chunk_max = [&](const f32x16& x) {
      float mx = max3f(x[0], x[1], x[2]);
#pragma unroll
      for (int i = 3; i < 15; i += 2) mx = max3f(mx, x[i], x[i + 1]);
      return max_halves(fmaxf(mx, x[15]));
    };
    auto weights = [&](f32x16& x) {
      const float mc = m_ref * c2;
      float sa = 0.f, sb = 0.f;
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        x[i] = fast_exp2(fmaf(x[i], c2, -mc));
        x[i + 1] = fast_exp2(fmaf(x[i + 1], c2, -mc));
        sa += x[i];
        sb += x[i + 1];
      }
      return sa + sb;
    };
    // The split's first chunk sets the reference max (a column that sees none
    // of its keys keeps the initial value and gets zero weights). Later chunks
    // are weighted against the reference without taking their max; a weight
    // above 2^8 forces the lane's partial sum above 2^8, and only then (rare)
    // does the reference move to the exact max, rescaling O and l.
    //
    // fp16 queries over an FP8 cache multiply each weight by its token's value
    // scale before rounding it to fp16, whose range ends at 65504: there the
    // reference is the exact running max of every chunk, so weights stay <= 1
    // and weight * scale stays finite for any scale up to 65504.
    float sum;
    if constexpr (F16 && KV8) {
      const float m_new = fmaxf(m_ref, chunk_max(sc));
      if (__builtin_amdgcn_ballot_w64(m_new > m_ref)) {
        const float alpha = fast_exp2((m_ref - m_new) * c2);
        l_part *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
      }
      m_ref = m_new;
      sum = weights(sc);
    } else {
      if (t == 0) m_ref = fmaxf(m_ref, chunk_max(sc));
      const f32x16 raw = sc;
      sum = weights(sc);
      if (__builtin_amdgcn_ballot_w64(!(sum <= kLazyRescaleDecW))) {
        const float m_new = fmaxf(m_ref, chunk_max(raw));
        const float alpha = fast_exp2((m_ref - m_new) * c2);
        l_part *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
        m_ref = m_new;
        sc = raw;
        sum = weights(sc);
      }
    }
    l_part += sum;
    if constexpr (KV8) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[i] *= vsc[i >> 2][i & 3];
    }
    const e16x8 p0 = pack8<F16>(sc, 0), p1 = pack8<F16>(sc, 1);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      if constexpr (KV8) {
        o[db] = mfma32x32x16<F16>(fp8_tr_operand<D, F16>(Vt, 0, db * 32, lane), p0, o[db]);
        o[db] = mfma32x32x16<F16>(fp8_tr_operand<D, F16>(Vt, 16, db * 32, lane), p1, o[db]);
      } else {
        o[db] = mfma32x32x16<F16>(tr_operand<D>(Vt, 0, db * 32, lane), p0, o[db]);
        o[db] = mfma32x32x16<F16>(tr_operand<D>(Vt, 16, db * 32, lane), p1, o[db]);
      }
    }
  };
  for (int t = 0; t < nch; t += NST) {
#pragma unroll
    for (int st = 0; st < NST; ++st)
      if (t + st < nch) chunk(t + st, st);
  }

  // Partial state of this split: m in log2 units (m_ref * scale * log2 e), the
  // weight sum l and the unnormalised O, all relative to m. An empty split (or
  // a column that saw no key) leaves l = 0, which the merge ignores.
  const float l_tot = sum_halves(l_part);
  if (cvalid) {
    const size_t prow = qrow * a.splits + s;
    float* po = a.part_o + prow * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const f32x4 w = {o[db][4 * gq + 0], o[db][4 * gq + 1], o[db][4 * gq + 2], o[db][4 * gq + 3]};
        *(f32x4*)(po + db * 32 + gq * 8 + hi * 4) = w;
      }
    if (hi == 0) {
      a.part_ml[2 * prow + 0] = l_tot > 0.f ? m_ref * c2 : -INFINITY;
      a.part_ml[2 * prow + 1] = l_tot;
    }
  }
}

// Thin __global__ wrapper (the host pass drops launch stubs of __global__
// templates whose body holds the buffer-load builtins directly).
template <int D, bool F16, bool KV8, int NW>
__global__ void __launch_bounds__(64 * NW) decode_split_kernel(DecArgs a) {
  decode_split_body<D, F16, KV8, NW>(a);
}

// Merge the splits of one query row ([SafeSoftmax] §3.2): with M = max_s m_s,
// l = sum_s 2^(m_s - M) l_s and O = sum_s 2^(m_s - M) O_s / l; LSE = (M +
// log2 l) ln 2. A row with l = 0 saw no key: O = 0, LSE = -inf.
template <int D, bool F16>
__global__ void __launch_bounds__(D) decode_merge_kernel(DecArgs a) {
  const size_t row = blockIdx.x;
  const int t = threadIdx.x;
  const float* ml = a.part_ml + row * a.splits * 2;
  const float* po = a.part_o + row * a.splits * D + t;
  // One pass with a running max (the merge rule applied split by split), in
  // blocks of 16 splits whose loads are all issued before any is used (one
  // memory round trip per block). No branches: an empty split (l = 0, O = 0,
  // m = -inf) or a slot past the last split (m taken as -inf) adds nothing,
  // and a factor whose max did not move is 1 (so -inf - -inf never occurs).
  float M = -INFINITY, l = 0.f, acc = 0.f;
  for (int s0 = 0; s0 < a.splits; s0 += 16) {
    float ms[16], ls[16], os[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int s = min(s0 + i, a.splits - 1);
      ms[i] = s0 + i < a.splits ? ml[2 * s] : -INFINITY;
      ls[i] = ml[2 * s + 1];
      os[i] = po[(size_t)s * D];
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float Mn = fmaxf(M, ms[i]);
      const float a0 = M == Mn ? 1.f : fast_exp2(M - Mn);
      const float a1 = ms[i] == Mn ? 1.f : fast_exp2(ms[i] - Mn);
      l = l * a0 + ls[i] * a1;
      acc = acc * a0 + os[i] * a1;
      M = Mn;
    }
  }
  const bool valid = l > 0.f;
  const float out = valid ? acc / l : 0.f;
  const uint32_t packed = pack2<F16>(out, 0.f);
  ((uint16_t*)a.o)[row * D + t] = (uint16_t)(packed & 0xffffu);
  if (t == 0 && a.lse) a.lse[row] = valid ? (M + log2f(l)) * kLn2 : -INFINITY;
}

template <int D, bool F16, bool KV8>
hipError_t launch_decode_t(const DecArgs& a, hipStream_t stream) {
  // Two waves per workgroup share the K/V chunks when the column blocks pair up.
  const int nw = decode_waves(a.col_groups);
  const unsigned wgs = (unsigned)(a.B * a.H_kv * (a.col_groups / nw) * a.splits);
  if (nw == 2)
    hipLaunchKernelGGL((decode_split_kernel<D, F16, KV8, 2>), dim3(wgs), dim3(128), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_split_kernel<D, F16, KV8, 1>), dim3(wgs), dim3(64), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_merge_kernel<D, F16>), dim3((unsigned)(a.B * a.H * a.Nq)), dim3(D), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_16(const DecArgs& a, int d, bool f16, hipStream_t stream) {
  if (a.k_scale) {  // FP8 K/V
    if (d == 64)
      return f16 ? launch_decode_t<64, true, true>(a, stream) : launch_decode_t<64, false, true>(a, stream);
    return f16 ? launch_decode_t<128, true, true>(a, stream) : launch_decode_t<128, false, true>(a, stream);
  }
  if (d == 64)
    return f16 ? launch_decode_t<64, true, false>(a, stream) : launch_decode_t<64, false, false>(a, stream);
  return f16 ? launch_decode_t<128, true, false>(a, stream) : launch_decode_t<128, false, false>(a, stream);
}

}  // namespace attn
