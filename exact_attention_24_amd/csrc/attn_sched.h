// Workgroup -> (batch*head, row tile) mapping shared by the attention kernels.
#pragma once

namespace attn {

// MI355X dispatches consecutive workgroups round-robin over its 8 XCDs, each
// with a private L2. Workgroups are ordered by row tile first: with
// heavy_first (causal masks, where the last row tiles visit the most KV
// tiles) every head's heaviest tile is launched before any lighter one, so
// the longest workgroups start earliest and the launch ends on short ones.
// Within one row tile the heads are split over the XCDs: when the head count
// is a multiple of 8, workgroup b runs on XCD b % 8 and only ever touches
// heads xcd*H/8 .. xcd*H/8 + H/8 - 1, so each head's K/V is cached in one L2.
__host__ __device__ inline void tile_order(int block, int num_tiles, int num_heads,
                                           bool heavy_first, int& head, int& tile) {
  int r;
  if ((num_heads & 7) == 0) {
    const int xcd = block & 7, slot = block >> 3;
    const int heads_per_xcd = num_heads >> 3;
    head = xcd * heads_per_xcd + slot % heads_per_xcd;
    r = slot / heads_per_xcd;
  } else {
    head = block % num_heads;
    r = block / num_heads;
  }
  tile = heavy_first ? num_tiles - 1 - r : r;
}

}  // namespace attn
