// C-ABI entry points (declared in include/attn.h): argument validation on the
// host, then dispatch to the gfx950 kernels on the caller's stream. Nothing
// here allocates device memory or synchronises.
#include "../../include/attn.h"

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "attn_kernels.h"

// Static device scratch of attn_bwd_noalloc: the backward workspace for
// callers that cannot allocate. Each GPU holds its own copy of the array; in
// host code `scratch` is only a host-side stand-in for it, so kernels and
// copies get the device address that hipGetSymbolAddress returns, looked up
// once per device with that device current (scratch_ptr below).
static_assert(2 * ((ATTN_NOALLOC_MAX_ROWS * 4 + 255) / 256 * 256) <= (long long)ATTN_NOALLOC_SCRATCH_BYTES,
              "the scratch holds both fp32 sections for the largest row count");
static __device__ __attribute__((aligned(256))) char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local char g_last_error[256] = "";

void record_hip_error(hipError_t e, const char* where) {
  snprintf(g_last_error, sizeof(g_last_error), "%s: %s (%d)", where, hipGetErrorString(e), (int)e);
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

attn_status check_sizes(int B, int H, int N, int d, attn_dtype dtype) {
  if (B < 1 || H < 1 || N < 1 || d < 1) return ATTN_ERR_INVALID_ARG;
  if (dtype != ATTN_DTYPE_F32 && dtype != ATTN_DTYPE_BF16 && dtype != ATTN_DTYPE_F16)
    return ATTN_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  // Workgroup counts and per-head row offsets must fit the kernels' 32-bit
  // index arithmetic: (B*H) * ceil(N/64) workgroups and N*d elements per head.
  const long long heads = (long long)B * H;
  const long long tiles = heads * ((N + 63) / 64);
  if (tiles > 0x7fffffffLL || (long long)N * d > 0x7fffffffLL) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

bool scale_ok(float scale) { return isfinite(scale) && scale > 0.f; }

// Grouped K/V heads: H_kv must divide H (H_kv = H is plain multi-head
// attention, H_kv = 1 multi-query attention).
attn_status check_heads(int H, int H_kv) {
  if (H_kv < 1 || H_kv > H || H % H_kv != 0) return ATTN_ERR_INVALID_ARG;
  return ATTN_OK;
}

// Split plan of the decode: `splits` splits per (batch, K/V head), split s
// taking the 32-key chunks s, s + splits, ... (so each holds about
// `chunk_keys` keys, a multiple of 32). 0 requested splits picks enough for
// one resident round of workgroups on 256 CUs (three per CU for the 16-bit
// split kernel's 48 KiB of LDS, four for the FP8 kernel's 34 KiB). More,
// shorter workgroups were measured slower (each pays its start-up latency
// again; B=8, 8 K/V heads, 8192 keys: 32 splits 52.7 us, 12 splits 49.6 us
// for bf16, 53.7 -> 46.9 us for FP8 K/V).
struct DecodePlan {
  int splits, chunk_keys, col_groups;
};
// Automatic split count: about `target` workgroups. Measured on the B=8,
// H=64, H_kv=8, Nk=8192 workloads with the caches in HBM only (each call timed
// after a 512 MiB read): one-wave workgroups over a 16-bit cache do best at
// ~512 (fewer splits also shrink the merge), two-wave workgroups at ~768, FP8
// caches (smaller workgroups: a 32 KiB ring) at ~1024. The FP8 plan never has
// fewer splits, so it sizes the workspace for all.
DecodePlan decode_plan(int B, int H, int H_kv, int Nq, int Nk, int num_splits, bool kv8) {
  DecodePlan p;
  p.col_groups = ((H / H_kv) * Nq + 31) / 32;
  long long want = num_splits;
  if (want <= 0) {
    const int nw = attn::decode_waves(p.col_groups);
    const long long target = kv8 ? 1024 : (nw == 1 ? 512 : 768);
    const long long units = (long long)B * H_kv * (p.col_groups / nw);
    want = (target + units - 1) / units;
  }
  const long long max_splits = (Nk + 31) / 32;
  if (want > max_splits) want = max_splits;
  if (want < 1) want = 1;
  const long long per = (Nk + want - 1) / want;
  p.chunk_keys = (int)((per + 31) / 32 * 32);
  p.splits = (Nk + p.chunk_keys - 1) / p.chunk_keys;
  return p;
}

size_t decode_part_o_bytes(int B, int H, int Nq, int d, int splits) {
  return (((size_t)B * H * Nq * splits * d * sizeof(float)) + 255) / 256 * 256;
}

attn_status check_decode(int B, int H, int H_kv, int Nq, int Nk, int d, attn_dtype dtype,
                         int num_splits) {
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || d < 1 || num_splits < 0) return ATTN_ERR_INVALID_ARG;
  if (dtype != ATTN_DTYPE_F32 && dtype != ATTN_DTYPE_BF16 && dtype != ATTN_DTYPE_F16)
    return ATTN_ERR_INVALID_ARG;
  if (H_kv < 1 || H_kv > H || H % H_kv != 0) return ATTN_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  if (dtype == ATTN_DTYPE_F32) return ATTN_ERR_UNSUPPORTED;
  if ((long long)Nk * d > 0x7fffffffLL || (long long)Nq * d > 0x7fffffffLL) return ATTN_ERR_UNSUPPORTED;
  const DecodePlan p = decode_plan(B, H, H_kv, Nq, Nk, num_splits, true);
  if ((long long)B * H_kv * p.col_groups * p.splits > 0x7fffffffLL ||
      (long long)B * H * Nq > 0x7fffffffLL)
    return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

size_t attn_bwd_section_bytes(int B, int H, int N) {
  const size_t rows = (size_t)B * H * N;
  return ((rows * sizeof(float) + 255) / 256) * 256;
}

// Device addresses of the static scratch array (below), one per device.
constexpr int kMaxDevices = 256;
void* scratch_dev[kMaxDevices];
std::mutex scratch_mu;

// Device address of the current device's scratch array (looked up on first use).
hipError_t scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    scratch_dev[dev] = p;
  }
  *out = scratch_dev[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

const char* attn_status_string(attn_status s) {
  switch (s) {
    case ATTN_OK: return "ATTN_OK";
    case ATTN_ERR_INVALID_ARG: return "ATTN_ERR_INVALID_ARG";
    case ATTN_ERR_UNSUPPORTED: return "ATTN_ERR_UNSUPPORTED";
    case ATTN_ERR_HIP: return "ATTN_ERR_HIP";
  }
  return "ATTN_STATUS_UNKNOWN";
}

const char* attn_last_error(void) { return g_last_error; }

attn_status attn_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                         int H, int H_kv, int N, int d, attn_dtype dtype, float scale, int causal,
                         const int32_t* seqlens, attn_stream_t stream) {
  attn_status st = check_sizes(B, H, N, d, dtype);
  if (st != ATTN_OK) return st;
  if ((st = check_heads(H, H_kv)) != ATTN_OK) return st;
  if (!q || !k || !v || !o) return ATTN_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16))
    return ATTN_ERR_INVALID_ARG;
  if ((lse && !aligned(lse, 4)) || (seqlens && !aligned(seqlens, 4))) return ATTN_ERR_INVALID_ARG;
  if (!scale_ok(scale)) return ATTN_ERR_INVALID_ARG;

  attn::FwdArgs a;
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse; a.seqlens = seqlens;
  a.B = B; a.H = H; a.N = N; a.H_kv = H_kv;
  a.scale = scale;
  a.scale_log2 = scale * 1.4426950408889634f;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = dtype == ATTN_DTYPE_F32
                     ? attn::launch_fwd_f32(a, d, causal != 0, s)
                     : attn::launch_fwd_16(a, d, causal != 0, dtype == ATTN_DTYPE_F16, s);
  if (e != hipSuccess) {
    record_hip_error(e, "attn_fwd launch");
    return ATTN_ERR_HIP;
  }
  return ATTN_OK;
}

attn_status attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                     int N, int d, attn_dtype dtype, float scale, int causal,
                     const int32_t* seqlens, attn_stream_t stream) {
  return attn_fwd_gqa(q, k, v, o, lse, B, H, H, N, d, dtype, scale, causal, seqlens, stream);
}

attn_status attn_fwd_fp8(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8,
                         const float* q_scale, const float* k_scale, const float* v_scale,
                         void* o, float* lse, int B, int H, int H_kv, int N, int d,
                         attn_dtype out_dtype, float scale, int causal, const int32_t* seqlens,
                         attn_stream_t stream) {
  if (out_dtype != ATTN_DTYPE_BF16 && out_dtype != ATTN_DTYPE_F16) {
    if (out_dtype == ATTN_DTYPE_F32) return ATTN_ERR_UNSUPPORTED;
    return ATTN_ERR_INVALID_ARG;
  }
  attn_status st = check_sizes(B, H, N, d, out_dtype);
  if (st != ATTN_OK) return st;
  if (d != 128) return ATTN_ERR_UNSUPPORTED;
  if ((st = check_heads(H, H_kv)) != ATTN_OK) return st;
  if (!q8 || !k8 || !v8 || !q_scale || !k_scale || !v_scale || !o) return ATTN_ERR_INVALID_ARG;
  if (!aligned(q8, 16) || !aligned(k8, 16) || !aligned(v8, 16) || !aligned(o, 16))
    return ATTN_ERR_INVALID_ARG;
  if (!aligned(q_scale, 4) || !aligned(k_scale, 4) || !aligned(v_scale, 4))
    return ATTN_ERR_INVALID_ARG;
  if ((lse && !aligned(lse, 4)) || (seqlens && !aligned(seqlens, 4))) return ATTN_ERR_INVALID_ARG;
  if (!scale_ok(scale)) return ATTN_ERR_INVALID_ARG;

  attn::Fwd8Args a;
  a.q = q8; a.k = k8; a.v = v8;
  a.q_scale = q_scale; a.k_scale = k_scale; a.v_scale = v_scale;
  a.o = o; a.lse = lse; a.seqlens = seqlens;
  a.B = B; a.H = H; a.N = N; a.H_kv = H_kv;
  a.scale = scale;
  hipError_t e = attn::launch_fwd_fp8(a, causal != 0, out_dtype == ATTN_DTYPE_F16, (hipStream_t)stream);
  if (e != hipSuccess) {
    record_hip_error(e, "attn_fwd_fp8 launch");
    return ATTN_ERR_HIP;
  }
  return ATTN_OK;
}

size_t attn_bwd_workspace_bytes(int B, int H, int N, int d, attn_dtype dtype) {
  if (check_sizes(B, H, N, d, dtype) != ATTN_OK) return 0;
  // delta and log2-scaled LSE, one fp32 per row each, each section 256-byte aligned
  return 2 * attn_bwd_section_bytes(B, H, N);
}

attn_status attn_bwd_gqa(const void* q, const void* k, const void* v, const void* o,
                         const void* dO, const float* lse, void* dq, void* dk, void* dv,
                         void* workspace, size_t workspace_bytes, int B, int H, int H_kv, int N,
                         int d, attn_dtype dtype, float scale, int causal, const int32_t* seqlens,
                         attn_stream_t stream) {
  attn_status st = check_sizes(B, H, N, d, dtype);
  if (st != ATTN_OK) return st;
  if ((st = check_heads(H, H_kv)) != ATTN_OK) return st;
  if (!q || !k || !v || !o || !dO || !lse || !dq || !dk || !dv || !workspace)
    return ATTN_ERR_INVALID_ARG;
  const void* t16[] = {q, k, v, o, dO, dq, dk, dv};
  for (const void* p : t16)
    if (!aligned(p, 16)) return ATTN_ERR_INVALID_ARG;
  if (!aligned(lse, 4) || !aligned(workspace, 256) || (seqlens && !aligned(seqlens, 4)))
    return ATTN_ERR_INVALID_ARG;
  if (workspace_bytes < attn_bwd_workspace_bytes(B, H, N, d, dtype)) return ATTN_ERR_INVALID_ARG;
  if (!scale_ok(scale)) return ATTN_ERR_INVALID_ARG;
  if (dtype == ATTN_DTYPE_F32) return ATTN_ERR_UNSUPPORTED;

  attn::BwdArgs a;
  a.q = q; a.k = k; a.v = v; a.o = o; a.dO = dO; a.lse = lse;
  a.dq = dq; a.dk = dk; a.dv = dv;
  a.delta = (float*)workspace;
  a.lse2 = (float*)((char*)workspace + attn_bwd_section_bytes(B, H, N));
  a.seqlens = seqlens;
  a.B = B; a.H = H; a.N = N; a.H_kv = H_kv;
  a.scale = scale;
  a.scale_log2 = scale * 1.4426950408889634f;
  hipError_t e = attn::launch_bwd_16(a, d, causal != 0, dtype == ATTN_DTYPE_F16, (hipStream_t)stream);
  if (e != hipSuccess) {
    record_hip_error(e, "attn_bwd launch");
    return ATTN_ERR_HIP;
  }
  return ATTN_OK;
}

attn_status attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO,
                     const float* lse, void* dq, void* dk, void* dv, void* workspace,
                     size_t workspace_bytes, int B, int H, int N, int d, attn_dtype dtype,
                     float scale, int causal, const int32_t* seqlens, attn_stream_t stream) {
  return attn_bwd_gqa(q, k, v, o, dO, lse, dq, dk, dv, workspace, workspace_bytes, B, H, H, N, d,
                      dtype, scale, causal, seqlens, stream);
}

attn_status attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                             const void* dO, const float* lse, void* dq, void* dk, void* dv, int B,
                             int H, int H_kv, int N, int d, attn_dtype dtype, float scale,
                             int causal, const int32_t* seqlens, attn_stream_t stream) {
  // Every size check comes before the scratch lookup, so a rejected call makes
  // no HIP call at all.
  attn_status st = check_sizes(B, H, N, d, dtype);
  if (st != ATTN_OK) return st;
  if ((long long)B * H * N > ATTN_NOALLOC_MAX_ROWS) {
    snprintf(g_last_error, sizeof(g_last_error),
             "attn_bwd_noalloc: B*H*N = %lld query rows exceed the static scratch's limit of %lld",
             (long long)B * H * N, (long long)ATTN_NOALLOC_MAX_ROWS);
    return ATTN_ERR_UNSUPPORTED;
  }
  if ((st = check_heads(H, H_kv)) != ATTN_OK) return st;
  if (!q || !k || !v || !o || !dO || !lse || !dq || !dk || !dv) return ATTN_ERR_INVALID_ARG;
  if (!scale_ok(scale)) return ATTN_ERR_INVALID_ARG;
  if (dtype == ATTN_DTYPE_F32) return ATTN_ERR_UNSUPPORTED;
  void* ws = nullptr;
  hipError_t e = scratch_ptr(&ws);
  if (e != hipSuccess) {
    record_hip_error(e, "attn_bwd_noalloc scratch lookup");
    return ATTN_ERR_HIP;
  }
  return attn_bwd_gqa(q, k, v, o, dO, lse, dq, dk, dv, ws, ATTN_NOALLOC_SCRATCH_BYTES, B, H, H_kv,
                      N, d, dtype, scale, causal, seqlens, stream);
}

size_t attn_decode_workspace_bytes(int B, int H, int H_kv, int Nq, int Nk, int d,
                                   attn_dtype dtype, int num_splits) {
  if (check_decode(B, H, H_kv, Nq, Nk, d, dtype, num_splits) != ATTN_OK) return 0;
  const DecodePlan p = decode_plan(B, H, H_kv, Nq, Nk, num_splits, true);
  const size_t ml = (((size_t)B * H * Nq * p.splits * 2 * sizeof(float)) + 255) / 256 * 256;
  return decode_part_o_bytes(B, H, Nq, d, p.splits) + ml;
}

namespace {

attn_status decode_common(const void* q, const void* k, const void* v, const float* k_scale,
                          const float* v_scale, void* o, float* lse, int B, int H, int H_kv,
                          int Nq, int Nk, int d, attn_dtype dtype, float scale, int causal,
                          const int32_t* kv_lens, int num_splits, void* workspace,
                          size_t workspace_bytes, attn_stream_t stream) {
  attn_status st = check_decode(B, H, H_kv, Nq, Nk, d, dtype, num_splits);
  if (st != ATTN_OK) return st;
  if (!q || !k || !v || !o || !workspace) return ATTN_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(workspace, 256))
    return ATTN_ERR_INVALID_ARG;
  if ((lse && !aligned(lse, 4)) || (kv_lens && !aligned(kv_lens, 4))) return ATTN_ERR_INVALID_ARG;
  if (!scale_ok(scale)) return ATTN_ERR_INVALID_ARG;
  if (workspace_bytes < attn_decode_workspace_bytes(B, H, H_kv, Nq, Nk, d, dtype, num_splits))
    return ATTN_ERR_INVALID_ARG;
  const DecodePlan p = decode_plan(B, H, H_kv, Nq, Nk, num_splits, k_scale != nullptr);
  attn::DecArgs a;
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse; a.kv_lens = kv_lens;
  a.k_scale = k_scale; a.v_scale = v_scale;
  a.part_o = (float*)workspace;
  a.part_ml = (float*)((char*)workspace + decode_part_o_bytes(B, H, Nq, d, p.splits));
  a.B = B; a.H = H; a.H_kv = H_kv; a.Nq = Nq; a.Nk = Nk;
  a.splits = p.splits; a.col_groups = p.col_groups;
  a.causal = causal != 0;
  a.scale = scale;
  a.scale_log2 = scale * 1.4426950408889634f;
  hipError_t e = attn::launch_decode_16(a, d, dtype == ATTN_DTYPE_F16, (hipStream_t)stream);
  if (e != hipSuccess) {
    record_hip_error(e, "attn_decode launch");
    return ATTN_ERR_HIP;
  }
  return ATTN_OK;
}

}  // namespace

attn_status attn_decode(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                        int H, int H_kv, int Nq, int Nk, int d, attn_dtype dtype, float scale,
                        int causal, const int32_t* kv_lens, int num_splits, void* workspace,
                        size_t workspace_bytes, attn_stream_t stream) {
  return decode_common(q, k, v, nullptr, nullptr, o, lse, B, H, H_kv, Nq, Nk, d, dtype, scale,
                       causal, kv_lens, num_splits, workspace, workspace_bytes, stream);
}

attn_status attn_decode_fp8kv(const void* q, const uint8_t* k8, const uint8_t* v8,
                              const float* k_scale, const float* v_scale, void* o, float* lse,
                              int B, int H, int H_kv, int Nq, int Nk, int d, attn_dtype dtype,
                              float scale, int causal, const int32_t* kv_lens, int num_splits,
                              void* workspace, size_t workspace_bytes, attn_stream_t stream) {
  attn_status st = check_decode(B, H, H_kv, Nq, Nk, d, dtype, num_splits);
  if (st != ATTN_OK) return st;
  if (!k_scale || !v_scale || !aligned(k_scale, 4) || !aligned(v_scale, 4))
    return ATTN_ERR_INVALID_ARG;
  return decode_common(q, k8, v8, k_scale, v_scale, o, lse, B, H, H_kv, Nq, Nk, d, dtype, scale,
                       causal, kv_lens, num_splits, workspace, workspace_bytes, stream);
}

}  // extern "C"
