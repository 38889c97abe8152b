// Device helpers shared by the gfx950 attention kernels: vector types, MFMA
// wrappers, LDS access through address-space-3 pointers, lane exchanges and
// 16-bit packing. Everything here is written for CDNA4 (wave64, gfx950) only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

#define ATTN_LDS __attribute__((address_space(3)))

// 16-bit elements: bf16 or fp16 (the kernels take the format as a template
// flag F16; storage, LDS layout and loads are the same for both).
typedef uint16_t e16_t;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 e16x8;  // MFMA operand
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

typedef ATTN_LDS char lds_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Finite initial row maximum: below any real score, so exp2 of the rescale
// factor underflows to 0 instead of forming (-inf) - (-inf).
constexpr float kMaxInit = -1.0e30f;

// D += A(32x16) * B(16x32), 16-bit inputs (bf16, or fp16 when F16), fp32
// accumulate. A: lane l holds row l%32, k = 8*(l/32) .. +7.  B: lane l holds
// column l%32, k = 8*(l/32) .. +7.  D: lane l holds column l%32, rows
// (i/4)*8 + 4*(l/32) + i%4. Both formats use the same lane layout.
template <bool F16>
__device__ __forceinline__ f32x16 mfma32x32x16(e16x8 a, e16x8 b, f32x16 c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// Same product with a zero accumulator (no VGPRs need clearing first).
template <bool F16>
__device__ __forceinline__ f32x16 mfma32x32x16_z(e16x8 a, e16x8 b) {
  const f32x16 z = {};
  return mfma32x32x16<F16>(a, b, z);
}

// D += A(16x32) * B(32x16), 16-bit inputs, fp32 accumulate. A: lane l holds
// row l%16, k = 8*(l/16) .. +7.  B: lane l holds column l%16, k = 8*(l/16) ..
// +7.  D: lane l holds column l%16, rows 4*(l/16) + i, i = 0..3 (layout
// checked on the device with an in-bounds probe against a host product).
template <bool F16>
__device__ __forceinline__ f32x4 mfma16x16x32(e16x8 a, e16x8 b, f32x4 c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float max3f(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

__device__ __forceinline__ e16x8 as_e16x8(u32x4 v) { return __builtin_bit_cast(e16x8, v); }

// ---- LDS access (address space 3, so the compiler emits ds_* instructions)
__device__ __forceinline__ lds_t* lds_base(char* generic) { return (lds_t*)generic; }

__device__ __forceinline__ u32x4 lds_load16(const lds_t* p) { return *(const ATTN_LDS u32x4*)p; }
__device__ __forceinline__ void lds_store16(lds_t* p, u32x4 v) { *(ATTN_LDS u32x4*)p = v; }
__device__ __forceinline__ u32x2 lds_load8(const lds_t* p) { return *(const ATTN_LDS u32x2*)p; }
__device__ __forceinline__ void lds_store8(lds_t* p, u32x2 v) { *(ATTN_LDS u32x2*)p = v; }
__device__ __forceinline__ float lds_loadf(const lds_t* p) { return *(const ATTN_LDS float*)p; }
__device__ __forceinline__ void lds_storef(lds_t* p, float v) { *(ATTN_LDS float*)p = v; }

// Transposing LDS read of four 16-bit values. Within each group of 16 lanes,
// let M[src][s] be the four values at lane src's address; lane j receives
// M[(j >> 2) + 4*s][j & 3] for s = 0..3.
__device__ __forceinline__ u32x2 lds_load_tr16(const lds_t* p) {
  s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ATTN_LDS s16x4*)p);
  return __builtin_bit_cast(u32x2, v);
}

// Transposing LDS read of eight 8-bit values. Within each group of 16 lanes,
// let M[src][b] be the eight bytes at lane src's address; lane j receives
// M[(j >> 3) + 2*s][j & 7] as its byte s, s = 0..7 (layout measured on the
// device with an in-bounds probe).
__device__ __forceinline__ u32x2 lds_load_tr8(const lds_t* p) {
  typedef __attribute__((__vector_size__(2 * sizeof(int)))) int i32x2;
  i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((ATTN_LDS i32x2*)p);
  return __builtin_bit_cast(u32x2, v);
}

__device__ __forceinline__ e16x8 join_e16x8(u32x2 lo, u32x2 hi) {
  u32x4 v = {lo[0], lo[1], hi[0], hi[1]};
  return as_e16x8(v);
}

// ---- global access
__device__ __forceinline__ u32x4 gload16(const void* p) { return *(const u32x4*)p; }
__device__ __forceinline__ void gstore16(void* p, u32x4 v) { *(u32x4*)p = v; }
__device__ __forceinline__ void gstore8(void* p, u32x2 v) { *(u32x2*)p = v; }

// ---- lane exchange between the two 32-lane halves of a wave
// v_permlane32_swap on two copies of x leaves the low half's values in the
// first result and the high half's in the second, in every lane: lane l sees
// x[l % 32] and x[l % 32 + 32].
__device__ __forceinline__ void split_halves(float x, float& lo, float& hi) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  lo = __builtin_bit_cast(float, (uint32_t)r[0]);
  hi = __builtin_bit_cast(float, (uint32_t)r[1]);
}

// Combine the values of lanes l and l ^ 32; both lanes get the same bits.
__device__ __forceinline__ float max_halves(float x) {
  float lo, hi;
  split_halves(x, lo, hi);
  return fmaxf(lo, hi);
}
__device__ __forceinline__ float sum_halves(float x) {
  float lo, hi;
  split_halves(x, lo, hi);
  return lo + hi;
}

// Max / sum over the four lanes l % 16 + {0, 16, 32, 48} (every one of them
// gets the result).
__device__ __forceinline__ float max_quarters(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float sum_quarters(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}

// ---- 16-bit packing: one v_cvt_pk_bf16_f32 / v_cvt_pk_f16_f32 (round to
// nearest even) per pair
typedef float f32x2_t __attribute__((ext_vector_type(2)));
template <bool F16>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  if constexpr (F16)
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
  else
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// The two 16-bit values of a 32-bit word, widened exactly to fp32.
template <bool F16>
__device__ __forceinline__ float unpack_lo(uint32_t u) {
  if constexpr (F16) return (float)__builtin_bit_cast(_Float16, (uint16_t)(u & 0xffffu));
  else return __builtin_bit_cast(float, u << 16);
}
template <bool F16>
__device__ __forceinline__ float unpack_hi(uint32_t u) {
  if constexpr (F16) return (float)__builtin_bit_cast(_Float16, (uint16_t)(u >> 16));
  else return __builtin_bit_cast(float, u & 0xffff0000u);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// The batch index of the sequence at position `rank` in the order of
// decreasing length (ties: lower index first), for B <= 64: lane j holds
// sequence j's length and counts the sequences ahead of it. Same result in
// every lane and wave.
__device__ __forceinline__ int batch_of_rank(const int32_t* seqlens, int B, int N, int rank) {
  const int lane = threadIdx.x & 63;
  const int len = lane < B ? min(max(seqlens[lane], 0), N) : -1;
  int ahead = 0;
  for (int j = 0; j < B; ++j) {
    const int lj = __builtin_amdgcn_readlane(len, j);
    ahead += (lj > len) | ((lj == len) & (j < lane));
  }
  const unsigned long long hit = __builtin_amdgcn_ballot_w64(lane < B && ahead == rank);
  return __builtin_ffsll((long long)hit) - 1;
}

}  // namespace attn
