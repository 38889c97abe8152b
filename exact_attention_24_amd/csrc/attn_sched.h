// Workgroup -> (batch*head, row tile) mapping shared by the attention kernels.
#pragma once

namespace attn {

// MI355X dispatches consecutive workgroups round-robin over its 8 XCDs, each
// with a private L2. Workgroups are ordered by row tile first: with
// heavy_first (causal masks, where the last row tiles visit the most KV
// tiles) every head's heaviest tile is launched before any lighter one, so
// the longest workgroups start earliest and the launch ends on short ones.
// Within one row tile the heads are dealt to the XCDs: when the head count is
// a multiple of 8 groups, workgroup b runs on XCD b % 8 and only ever touches
// the heads of that XCD, so each head's K/V is cached in one L2. Heads are
// dealt in units of `group` consecutive heads (the query heads that share one
// K/V head, which then share that L2 too), and the units are interleaved over
// the XCDs (unit u on XCD u % 8): every XCD gets heads of every sequence, so a
// padded batch whose sequences differ in length still loads the XCDs evenly.
__host__ __device__ inline void tile_order(int block, int num_tiles, int num_heads, int group,
                                           bool heavy_first, int& head, int& tile) {
  int r;
  if (group >= 1 && num_heads % group == 0 && ((num_heads / group) & 7) == 0) {
    const int xcd = block & 7, slot = block >> 3;
    const int heads_per_xcd = num_heads >> 3;
    const int s = slot % heads_per_xcd;        // which of this XCD's heads
    const int unit = (s / group) * 8 + xcd;    // units u with u % 8 == xcd
    head = unit * group + s % group;
    r = slot / heads_per_xcd;
  } else {
    head = block % num_heads;
    r = block / num_heads;
  }
  tile = heavy_first ? num_tiles - 1 - r : r;
}

// Padded batches (per-sequence lengths on the device): a workgroup's run time
// grows with its sequence's length, so the longest sequences go first. Block
// b maps to (rank, head, tile): rank is the position of the sequence in the
// order of decreasing length (the caller turns it into a batch index), and
// within one rank the heads and tiles are laid out as in tile_order above
// (XCD b % 8 holds the same heads of every sequence; heavy_first puts each
// head's last tile first). Needs num_heads / group to be a multiple of 8.
__host__ __device__ inline void varlen_order(int block, int num_tiles, int num_heads, int group,
                                             bool heavy_first, int& rank, int& head, int& tile) {
  const int xcd = block & 7, slot = block >> 3;
  const int heads_per_xcd = num_heads >> 3;
  const int per_rank = heads_per_xcd * num_tiles;
  rank = slot / per_rank;
  const int rem = slot % per_rank;
  const int r = rem / heads_per_xcd, s = rem % heads_per_xcd;
  head = ((s / group) * 8 + xcd) * group + s % group;
  tile = heavy_first ? num_tiles - 1 - r : r;
}

}  // namespace attn
