// LDS tile layouts, direct global->LDS tile loads and MFMA operand helpers
// shared by the attention kernels (gfx950, wave64). The forward and backward
// read 16x16x32 MFMA operands from the TILE_K16 / TILE_T16 layouts below; the
// decode reads 32x32x16 operands from the swz layout.
#pragma once

#include "attn_common.h"

namespace attn {

// A row-major [rows][D] 16-bit tile in LDS, no padding; the 16-byte chunk c of
// row r sits at chunk c ^ swz(r). The XOR keeps the 32x32x16 operand reads
// free of bank conflicts on gfx950's 64 LDS banks: 32 consecutive rows read at
// two chunks (ds_read_b128 operands), and 4 consecutive rows read as 4
// consecutive chunks (ds_read_b64_tr_b16 transposed operands). It is a bijection on the
// chunks of each row, so a wave can fill whole rows with one 1 KB
// global_load_lds_dwordx4 by fetching, for physical chunk p, logical chunk
// p ^ swz(r).
template <int D>
__device__ __forceinline__ int swz(int r) {
  static_assert(D == 128 || D == 64 || D == 32, "16 / 8 / 4 chunks per row");
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else if constexpr (D == 64) return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  else return (r >> 2) & 3;  // 64-byte rows (FP8 rows of 64 elements)
}
template <int D>
__device__ __forceinline__ int tile_off(int r, int chunk) {
  return r * (D * 2) + ((chunk ^ swz<D>(r)) << 4);
}

// Two more layouts for tiles read by 16x16x32 MFMA operands (both bijections
// on each row's chunks; measured with SQ_LDS_BANK_CONFLICT, against which swz
// above conflicts for the first pattern):
//  - TILE_K16, for ds_read_b128 operands that take 16 consecutive rows at 4
//    consecutive chunks: chunk c of row r at c ^ (r % 16) for 128 columns,
//    c ^ ((r / 2) % 8) for 64 (two rows per bank line); conflict-free;
//  - TILE_T16, for transposing reads that take eight consecutive rows at two
//    consecutive chunks per half-wave: chunk c of row r at c ^ (2 * (r % 8)),
//    or c ^ (2 * ((r / 2) % 4)) for 64 columns; conflict-free for those reads
//    and, as measured in the backward kernels, for the b128 pattern above too.
//  - TILE_V8, for 128-byte rows of 8-bit values read by ds_read_b64_tr_b8
//    with each half-wave addressing the 16 rows r0 + {0..7, 16..23} (r0 a
//    multiple of 8) at one 16-byte chunk: chunk c of row r at
//    c ^ (((r / 2) % 4) | 4 * ((r / 16) % 2)), which puts the eight even and
//    the eight odd rows of that set on eight distinct chunks each.
enum TileLayout { TILE_SWZ = 0, TILE_K16 = 1, TILE_T16 = 2, TILE_V8 = 3 };
template <int D, int LAYOUT>
__device__ __forceinline__ int layout_swz(int r) {
  if constexpr (LAYOUT == TILE_K16) return D == 128 ? (r & 15) : ((r >> 1) & 7);
  else if constexpr (LAYOUT == TILE_T16) return D == 128 ? 2 * (r & 7) : 2 * ((r >> 1) & 3);
  else if constexpr (LAYOUT == TILE_V8) return ((r >> 1) & 3) | ((r >> 2) & 4);
  else return swz<D>(r);
}
// Byte offset of element column `col` (a multiple of 4) of row r.
template <int D, int LAYOUT>
__device__ __forceinline__ int tile_off_lay(int r, int col) {
  return r * (D * 2) + (((col >> 3) ^ layout_swz<D, LAYOUT>(r)) << 4) + ((col >> 2) & 1) * 8;
}
// Byte offset of element column `col` (a multiple of 4) of row r.
template <int D>
__device__ __forceinline__ int tile_off_col(int r, int col) {
  return tile_off<D>(r, col >> 3) + ((col >> 2) & 1) * 8;
}

// A operand (32 rows x 16 k) read straight from a tile: lane holds row
// row0 + lane%32 and k = chunk*8 + 8*(lane/32) .. +7.
template <int D>
__device__ __forceinline__ e16x8 row_operand(const lds_t* tile, int row0, int chunk, int lane) {
  return as_e16x8(lds_load16(tile + tile_off<D>(row0 + (lane & 31), chunk + (lane >> 5))));
}

// Transposed operand from a row-major tile T (rows = the contraction index):
// lane receives T[row0 + hi*4 + {0..3}][col] and T[row0 + 8 + hi*4 + {0..3}][col]
// with col = col0 + lane%32 and hi = lane/32. That is exactly the k order in
// which a 32x32 accumulator's lane holds its 16 rows (i/4)*8 + hi*4 + i%4, so a
// score block produced by one MFMA feeds the next MFMA as the other operand
// without any data exchange between lanes. ds_read_b64_tr_b16 gives lane j of
// each 16-lane group the values M[(j>>2) + 4s][j&3] (s = 0..3) of the 8-byte
// pieces M[src] its group addressed, so lane src addresses row
// row0 + hi*4 + (src>>2) at column col0 + 16*((lane>>4)&1) + 4*(src&3).
template <int D>
__device__ __forceinline__ e16x8 tr_operand(const lds_t* tile, int row0, int col0, int lane) {
  const int r = row0 + (lane >> 5) * 4 + ((lane & 15) >> 2);
  const int col = col0 + ((lane >> 4) & 1) * 16 + 4 * (lane & 3);
  const u32x2 lo = lds_load_tr16(tile + tile_off_col<D>(r, col));
  const u32x2 up = lds_load_tr16(tile + tile_off_col<D>(r + 8, col));
  return join_e16x8(lo, up);
}

// Accumulator values 8h .. 8h+7 packed to 16 bits (round to nearest even):
// the B operand for the 16-row k step h of the next product.
template <bool F16>
__device__ __forceinline__ e16x8 pack8(const f32x16& s, int h) {
  u32x4 w = {pack2<F16>(s[8 * h + 0], s[8 * h + 1]), pack2<F16>(s[8 * h + 2], s[8 * h + 3]),
             pack2<F16>(s[8 * h + 4], s[8 * h + 5]), pack2<F16>(s[8 * h + 6], s[8 * h + 7])};
  return as_e16x8(w);
}

// Direct global -> LDS tile loads (buffer_load_dwordx4 ... lds) for one
// (batch, head). Each load builds a buffer resource whose base is the tile's
// first row and whose range ends at row n_rows, so rows at or past n_rows read
// as zeros (hardware range check on the per-lane offset; the scalar offset is
// left at 0): the tile never holds stale LDS bytes that could be NaN bit
// patterns, rows past the end are never fetched, and no clamping is needed.
// LAYOUT selects the chunk layout (swz unless stated). NWAVES waves share a tile of
// ROWS rows; the calling wave fills the 1 KB row
// groups g = wave, wave + NWAVES, ... (64/(D/8) rows each), lane l writing
// physical chunk l % (D/8) of row l / (D/8), i.e. logical chunk
// (l % (D/8)) ^ swz(row). The per-lane byte offsets do not depend on which
// tile is loaded, so they are computed once.
template <int D, int ROWS, int NWAVES, int LAYOUT = TILE_SWZ>
struct TileDma {
  static_assert(LAYOUT == TILE_SWZ || D == 128 || D == 64, "16x16 layouts: 64 or 128 columns");
  static_assert(LAYOUT != TILE_V8 || D == 64, "TILE_V8: 128-byte rows");
  static constexpr int CPR = D / 8;      // 16-byte chunks per row
  static constexpr int RPG = 64 / CPR;   // rows per 1 KB wave load
  static constexpr int ITER = ROWS / RPG / NWAVES;
  static_assert(ITER * RPG * NWAVES == ROWS, "tile rows must split evenly over the waves");

  const e16_t* head;
  int n_rows;
  uint32_t voff[ITER];
  int wave;

  __device__ __forceinline__ TileDma(const e16_t* head_, int n_rows_, int wave_, int lane) {
    head = head_;
    n_rows = n_rows_;
    wave = wave_;
    const int rsub = lane / CPR, pc = lane % CPR;
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      const int r = (wave + it * NWAVES) * RPG + rsub;
      voff[it] = (uint32_t)(r * D * 2 + ((pc ^ layout_swz<D, LAYOUT>(r)) << 4));
    }
  }
  // Enqueue the loads of rows [row0, row0 + ROWS) into `tile`.
  __device__ __forceinline__ void load(lds_t* tile, int row0) const {
    const uint32_t bytes = (uint32_t)max(n_rows - row0, 0) * (uint32_t)(D * 2);
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(head + (size_t)row0 * D), (short)0, (int)bytes, 0x00020000);
#pragma unroll
    for (int it = 0; it < ITER; ++it)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsrc, (ATTN_LDS void*)(tile + (wave + it * NWAVES) * 1024), 16, voff[it], 0, 0, 0);
  }
};

// One 4-byte value per lane, 64 lanes, straight into LDS: values
// [row0, row0 + 64) of an fp32 array of n_rows entries (zeros at or past
// n_rows), written to lds[0 .. 256).
__device__ __forceinline__ void vec64_dma(lds_t* lds, const float* base, int n_rows, int row0,
                                          int lane) {
  const uint32_t bytes = (uint32_t)max(n_rows - row0, 0) * 4u;
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)(base + row0), (short)0, (int)bytes, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (ATTN_LDS void*)lds, 4, lane * 4, 0, 0, 0);
}

// Wait until this wave's direct-to-LDS loads have landed (vmcnt = 0).
__device__ __forceinline__ void dma_wait() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Wait until at most N of this wave's most recent vector-memory loads are
// still in flight (they complete in issue order).
template <int N>
__device__ __forceinline__ void dma_wait_allbut() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

}  // namespace attn
