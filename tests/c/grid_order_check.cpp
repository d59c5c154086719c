// Host-side check of the grid-order functions the tiled kernels share (fa_common.h): xcd_remap and
// head_tile, compiled for the host from the same header the kernels include.  For every checked
// grid:
//   * xcd_remap is a bijection of [0, total) and puts logical item L on XCD L / (total / 8) when the
//     launcher chooses the XCD order (use_xcd_order in fa_launch.h);
//   * head_tile is a bijection of [0, heads · tiles) onto (head, tile) pairs;
//   * within a head, tiles start in order (the item of tile t precedes the item of tile t + 1), so
//     that under the causal mask each head's heaviest tiles start first;
//   * in the XCD order with grouped heads, every head's items lie in one XCD's eighth;
//   * a group of heads never spans more than kHeadGroup + 3 heads, and its items alternate between
//     the heads tile by tile (items g·t + i → tile t of the group's head i).
// Prints "all checks passed" and exits 0, or names the first failing grid and exits 1.
#include "fa_common.h"
#include "fa_launch.h"

#include <cstdio>
#include <vector>

namespace {

int fail(const char* what, int heads, int tiles, int remap, int per_cu, long item) {
  std::printf("FAIL %s: heads=%d tiles=%d remap=%d per_cu=%d item=%ld\n", what, heads, tiles, remap,
              per_cu, item);
  return 1;
}

int check_remap(uint32_t total) {
  std::vector<char> seen(total, 0);
  for (uint32_t b = 0; b < total; ++b) {
    const uint32_t l = fa::xcd_remap(b, total);
    if (l >= total || seen[l]) return fail("xcd_remap not a bijection", 0, 0, 1, 0, (long)b);
    seen[l] = 1;
    // Workgroup b is dispatched to XCD b % 8; its logical item must lie in that XCD's eighth.
    if (l / (total / 8u) != b % 8u) return fail("xcd_remap eighth", 0, 0, 1, 0, (long)b);
  }
  return 0;
}

int check_grid(int heads, int tiles, int remap, int per_cu) {
  const long total = (long)heads * tiles;
  std::vector<long> item_of((size_t)total, -1);
  std::vector<int> head_of((size_t)total), tile_of((size_t)total);
  for (long it = 0; it < total; ++it) {
    int h = -1, t = -1;
    fa::head_tile((uint32_t)it, tiles, heads, remap, per_cu, h, t);
    if (h < 0 || h >= heads || t < 0 || t >= tiles)
      return fail("out of range", heads, tiles, remap, per_cu, it);
    long& slot = item_of[(size_t)h * tiles + t];
    if (slot >= 0) return fail("pair mapped twice", heads, tiles, remap, per_cu, it);
    slot = it;
    head_of[(size_t)it] = h;
    tile_of[(size_t)it] = t;
  }
  const bool grouped = !(tiles >= 32 * per_cu || (remap && heads % 8 != 0));
  for (int h = 0; h < heads; ++h) {
    for (int t = 0; t + 1 < tiles; ++t)
      if (item_of[(size_t)h * tiles + t] >= item_of[(size_t)h * tiles + t + 1])
        return fail("tiles of a head out of order", heads, tiles, remap, per_cu, h);
    if (remap && grouped) {
      const long eighth = total / 8;
      const long x0 = item_of[(size_t)h * tiles] / eighth;
      for (int t = 1; t < tiles; ++t)
        if (item_of[(size_t)h * tiles + t] / eighth != x0)
          return fail("head spans two XCD eighths", heads, tiles, remap, per_cu, h);
    }
  }
  if (grouped && tiles > 1) {
    // Walk the groups: a group of g heads opens with g items of tile 0 (its heads' first tiles),
    // and its items g·t + i must be tile t of its heads h0 + i, consecutive heads.  (With one tile
    // per head every order is head by head, and there is nothing more to check.)
    long it = 0;
    while (it < total) {
      int g = 0;
      while (it + g < total && tile_of[(size_t)(it + g)] == 0) ++g;
      const int h0 = head_of[(size_t)it];
      if (g < 1 || g > fa::kHeadGroup + 3 || h0 + g > heads)
        return fail("group size", heads, tiles, remap, per_cu, it);
      for (int t = 0; t < tiles; ++t)
        for (int i = 0; i < g; ++i)
          if (item_of[(size_t)(h0 + i) * tiles + t] != it + (long)g * t + i)
            return fail("group not interleaved tile by tile", heads, tiles, remap, per_cu, it);
      it += (long)g * tiles;
    }
  }
  return 0;
}

}  // namespace

int main() {
  int bad = 0;
  for (uint32_t total = 8; total <= 4096 && !bad; total += 8) bad |= check_remap(total);
  bad |= check_remap(8u * 4u * 32u * 32u);  // causal 4 × 32 heads × 32 tiles
  long grids = 0;
  for (int per_cu = 1; per_cu <= 3 && !bad; ++per_cu)
    for (int heads = 1; heads <= 72 && !bad; ++heads)
      for (int tiles = 1; tiles <= 100 && !bad; tiles += (tiles < 40 ? 1 : 7))
        for (int remap = 0; remap <= 1 && !bad; ++remap) {
          // The launcher chooses the XCD order only for totals that are multiples of 8.
          if (remap && fa::use_xcd_order((uint32_t)(heads * tiles), heads, 1) == 0 &&
              fa::use_xcd_order((uint32_t)(heads * tiles), heads, 0) == 0)
            continue;
          bad |= check_grid(heads, tiles, remap, per_cu);
          ++grids;
        }
  // The two headline grids: causal 4 × 32 heads of 4096 keys (32 query tiles of 128) at one to three
  // resident workgroups per compute unit, and 32 heads of 16384 keys (128 tiles: one head at a time).
  for (int per_cu = 1; per_cu <= 3 && !bad; ++per_cu) {
    bad |= check_grid(128, 32, 1, per_cu);
    bad |= check_grid(32, 128, 1, per_cu);
    grids += 2;
  }
  if (bad) return 1;
  std::printf("%ld grids: all checks passed\n", grids);
  return 0;
}
