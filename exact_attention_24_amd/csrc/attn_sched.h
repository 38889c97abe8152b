// Workgroup -> (batch*head, row tile) mapping shared by the attention kernels.
#pragma once

namespace attn {

// MI355X dispatches consecutive workgroups round-robin over its 8 XCDs, each
// with a private L2. When the head count is a multiple of 8 the mapping keeps
// every tile of one (batch, head) on one XCD, so that head's K/V tiles are
// fetched from HBM into that XCD's L2 and reused there by all its row tiles.
// Within an XCD the heads are visited one after another; with heavy_first
// (causal masks) each head's tiles go from the last row tile (most KV tiles
// to visit) to the first, so the longest workgroups start earliest and the
// launch ends on short ones.
__host__ __device__ inline void tile_order(int block, int num_tiles, int num_heads,
                                           bool heavy_first, int& head, int& tile) {
  int r;
  if ((num_heads & 7) == 0) {
    const int xcd = block & 7, slot = block >> 3;
    const int heads_per_xcd = num_heads >> 3;
    head = xcd * heads_per_xcd + slot / num_tiles;
    r = slot % num_tiles;
  } else {
    head = block % num_heads;
    r = block / num_heads;
  }
  tile = heavy_first ? num_tiles - 1 - r : r;
}

}  // namespace attn
