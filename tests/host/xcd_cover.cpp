// Host check of the unit -> XCD slot deals: the chunked deal shared by the
// single-row attend and the merge kernel, and the kv-head block deal of the
// sparse row tiles.  Over each launch's workgroups every unit below the count
// is visited exactly once, for many unit counts and kv head counts.
#include <cstdio>
#include <vector>

#include "msa_internal.h"

int main() {
  const int hkvs[] = {1, 2, 3, 4, 8, 16};
  for (int hkv : hkvs) {
    for (int units = hkv; units <= 70000; units += (units < 600 ? hkv : 97 * hkv)) {
      const int64_t groups = msa::xcd_groups(units, hkv);
      std::vector<int> seen(units, 0);
      for (int64_t b = 0; b < groups * msa::kXcdSlots; ++b) {
        const int u = msa::xcd_unit(units, hkv, (int)(b % msa::kXcdSlots),
                                    (int)(b / msa::kXcdSlots));
        if (u < 0) { std::printf("negative unit\n"); return 1; }
        if (u < units) ++seen[u];
      }
      for (int u = 0; u < units; ++u) {
        if (seen[u] != 1) {
          std::printf("units %d hkv %d: unit %d seen %d times\n", units, hkv, u, seen[u]);
          return 1;
        }
      }
    }
  }
  // Sparse row tiles: chunks of kTileBlock tiles of one kv head per slot.
  for (int hkv : hkvs) {
    for (int tiles = 1; tiles <= 9000; tiles += (tiles < 300 ? 1 : 89)) {
      const int units = tiles * hkv;
      const int64_t groups = msa::tile_block_groups(tiles, hkv);
      std::vector<int> seen(units, 0);
      for (int64_t b = 0; b < groups * msa::kXcdSlots; ++b) {
        const int slot = (int)(b % msa::kXcdSlots);
        const int u = msa::tile_block_unit(tiles, hkv, slot, (int)(b / msa::kXcdSlots));
        if (u >= units) { std::printf("unit past the launch\n"); return 1; }
        if (u >= 0) {
          ++seen[u];
          // every unit of one chunk (kv head, block of tiles) sits on one slot
          const int tile = u / hkv, h = u % hkv;
          const int chunk = (tile / msa::kTileBlock) * hkv + h;
          if (chunk % msa::kXcdSlots != slot) { std::printf("chunk off its slot\n"); return 1; }
        }
      }
      for (int u = 0; u < units; ++u) {
        if (seen[u] != 1) {
          std::printf("tiles %d hkv %d: unit %d seen %d times\n", tiles, hkv, u, seen[u]);
          return 1;
        }
      }
    }
  }
  std::printf("ok\n");
  return 0;
}
