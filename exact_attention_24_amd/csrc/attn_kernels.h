// Internal interface between the C-ABI layer (attn_api.cpp) and the kernel
// translation units. Not installed; the public interface is include/attn.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace attn {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;               // may be null
  const int32_t* seqlens;   // may be null
  int B, H, N;
  int H_kv;                 // K/V heads; query head h reads K/V head h / (H / H_kv)
  float scale;              // softmax scale applied to q.k
  float scale_log2;         // scale * log2(e)
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dO;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* delta;             // workspace: -rowsum(dO o O), fp32 [B,H,N]
  float* lse2;              // workspace: LSE * log2(e), fp32 [B,H,N] (0 on padded rows)
  const int32_t* seqlens;
  int B, H, N;
  int H_kv;                 // K/V heads; query head h reads K/V head h / (H / H_kv)
  float scale;
  float scale_log2;
};

// FP8 forward: q, k, v are E4M3 bytes [B,H,N,128] / [B,H_kv,N,128]; scores
// scale by scale * q_scale[b,h,i] * k_scale[b,hkv], O by v_scale[b,hkv].
struct Fwd8Args {
  const uint8_t* q;
  const uint8_t* k;
  const uint8_t* v;
  const float* q_scale;     // [B,H,N]
  const float* k_scale;     // [B,H_kv]
  const float* v_scale;     // [B,H_kv]
  void* o;                  // [B,H,N,128] bf16 or fp16
  float* lse;               // may be null
  const int32_t* seqlens;   // may be null
  int B, H, N;
  int H_kv;
  float scale;
};

// Split-KV decode: q, o [B,H,Nq,D], k, v [B,H_kv,Nk,D], split kernel partials
// in the workspace, merged into o and lse.
struct DecArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;               // may be null
  const int32_t* kv_lens;   // may be null (every sequence has Nk keys)
  const float* k_scale;     // FP8 K/V only: per-token scales [B,H_kv,Nk]; null for 16-bit K/V
  const float* v_scale;
  float* part_o;            // workspace: [B*H*Nq][splits][D] unnormalised partial O
  float* part_ml;           // workspace: [B*H*Nq][splits][2] = (m * scale * log2 e, l)
  int B, H, H_kv, Nq, Nk;
  int splits;               // splits per (batch, K/V head); split s takes the 32-key chunks s, s + splits, ...
  int col_groups;           // ceil((H / H_kv) * Nq / 32) query-column blocks
  int causal;
  float scale, scale_log2;
};

// Waves per decode workgroup: two column blocks of the same (batch, K/V head,
// split) share one workgroup (and each fetched chunk) when they pair up.
inline int decode_waves(int col_groups) { return col_groups % 2 == 0 ? 2 : 1; }

// Each launcher enqueues its kernels on `stream` and returns the launch status.
// 16-bit formats: bf16, or fp16 when f16 is set.
hipError_t launch_fwd_16(const FwdArgs& a, int d, bool causal, bool f16, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdArgs& a, int d, bool causal, hipStream_t stream);
hipError_t launch_fwd_fp8(const Fwd8Args& a, bool causal, bool f16_out, hipStream_t stream);
hipError_t launch_bwd_16(const BwdArgs& a, int d, bool causal, bool f16, hipStream_t stream);
hipError_t launch_decode_16(const DecArgs& a, int d, bool f16, hipStream_t stream);

}  // namespace attn
