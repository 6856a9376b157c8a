// Host check of the unit -> XCD slot deal shared by the single-row attend and
// the merge kernel: over the launch's workgroups every unit below the count is
// visited exactly once, for many unit counts and kv head counts.
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
  std::printf("ok\n");
  return 0;
}
