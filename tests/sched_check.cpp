// Host check of the workgroup -> (head, row tile) order used by the kernels
// (attn_sched.h): the map is a bijection, each head's workgroups stay on one
// XCD (block % 8), the heads sharing a K/V head stay together, every XCD gets
// heads of every sequence, and heavy-first puts each head's last tile first.
// Prints "ok" or the first failure.
#define __host__
#define __device__
#include <cstdio>
#include <vector>
#include "attn_sched.h"

static int check(int tiles, int heads, int group, int seq_heads, bool heavy) {
  const int n = tiles * heads;
  std::vector<int> seen(n, 0), xcd_of_head(heads, -1);
  for (int b = 0; b < n; ++b) {
    int h, t;
    attn::tile_order(b, tiles, heads, group, heavy, h, t);
    if (h < 0 || h >= heads || t < 0 || t >= tiles) { printf("out of range %d\n", b); return 1; }
    if (seen[h * tiles + t]++) { printf("duplicate (%d,%d)\n", h, t); return 1; }
    if (heavy && b < heads && t != tiles - 1) { printf("heavy-first violated at %d\n", b); return 1; }
    const bool xcd_mode = heads % group == 0 && ((heads / group) % 8) == 0;
    if (xcd_mode) {
      if (xcd_of_head[h] == -1) xcd_of_head[h] = b % 8;
      if (xcd_of_head[h] != b % 8) { printf("head %d on two XCDs\n", h); return 1; }
    }
  }
  const bool xcd_mode = heads % group == 0 && ((heads / group) % 8) == 0;
  if (xcd_mode) {
    for (int h = 0; h < heads; ++h)
      if (xcd_of_head[h] != xcd_of_head[(h / group) * group]) { printf("group split %d\n", h); return 1; }
    if (seq_heads % (8 * group) == 0)
      for (int s0 = 0; s0 < heads; s0 += seq_heads)
        for (int x = 0; x < 8; ++x) {
          int cnt = 0;
          for (int h = s0; h < s0 + seq_heads; ++h) cnt += xcd_of_head[h] == x;
          if (cnt != seq_heads / 8) { printf("sequence at head %d: XCD %d has %d heads\n", s0, x, cnt); return 1; }
        }
  }
  return 0;
}

// varlen_order: a bijection onto (rank, head, tile); ranks in launch order;
// each (rank, head) on one XCD, grouped heads together; heavy-first within a
// rank.
static int check_varlen(int tiles, int B, int heads, int group, bool heavy) {
  const int n = B * heads * tiles;
  std::vector<int> seen(n, 0), xcd(B * heads, -1);
  int last_rank = 0;
  for (int b = 0; b < n; ++b) {
    int r, h, t;
    attn::varlen_order(b, tiles, heads, group, heavy, r, h, t);
    if (r < 0 || r >= B || h < 0 || h >= heads || t < 0 || t >= tiles) { printf("varlen out of range %d\n", b); return 1; }
    if (seen[(r * heads + h) * tiles + t]++) { printf("varlen duplicate (%d,%d,%d)\n", r, h, t); return 1; }
    if (r < last_rank) { printf("varlen rank order at %d\n", b); return 1; }
    last_rank = r > last_rank ? r : last_rank;
    if (xcd[r * heads + h] == -1) xcd[r * heads + h] = b % 8;
    if (xcd[r * heads + h] != b % 8) { printf("varlen head on two XCDs\n"); return 1; }
    if (xcd[r * heads + (h / group) * group] != -1 && xcd[r * heads + (h / group) * group] != b % 8) {
      printf("varlen group split\n"); return 1;
    }
    const int first_of_rank = r * heads * tiles;
    if (heavy && b - first_of_rank < heads && t != tiles - 1) { printf("varlen heavy-first at %d\n", b); return 1; }
  }
  return 0;
}

int main() {
  const int vcases[][4] = {{16, 8, 16, 1}, {32, 3, 32, 4}, {5, 7, 8, 1}, {1, 2, 64, 8}};
  for (const auto& c : vcases)
    for (int heavy = 0; heavy < 2; ++heavy)
      if (check_varlen(c[0], c[1], c[2], c[3], heavy)) {
        printf("varlen case tiles=%d B=%d heads=%d group=%d heavy=%d\n", c[0], c[1], c[2], c[3], heavy);
        return 1;
      }
  const int cases[][4] = {{16, 128, 1, 16}, {32, 64, 1, 32}, {16, 64, 4, 32}, {7, 24, 3, 24},
                          {5, 12, 1, 6}, {1, 8, 8, 8}, {64, 32, 1, 16}, {3, 48, 2, 48}};
  for (const auto& c : cases)
    for (int heavy = 0; heavy < 2; ++heavy)
      if (check(c[0], c[1], c[2], c[3], heavy)) {
        printf("case tiles=%d heads=%d group=%d heavy=%d\n", c[0], c[1], c[2], heavy);
        return 1;
      }
  printf("ok\n");
  return 0;
}
