// Host check of how work units are dealt to workgroup slots (no GPU; built by
// tests/test_launch_order.py with hipcc, host code only).
//
// For both orders of launch_order.h and many unit counts and run lengths
// (whole and partial last runs), the slots that slots_for() asks for, mapped
// by unit_of_slot(), give every unit in [0, units) exactly one slot and give
// the other slots units at or past `units` (which do nothing). In the
// interleaved order the units of one run also share an XCD (slot mod 8).
// Prints "ok" and exits 0 when every check holds.

#include "../../group_scale_factor_amd/csrc/launch_order.h"

#include <cstdio>
#include <random>
#include <vector>

namespace {

int failures = 0;

template <bool IL>
void check(int64_t units, int64_t per_block) {
  const int64_t slots = slots_for(IL, units, per_block);
  if (slots % 8 != 0 || slots < units) {
    if (failures++ < 20) std::fprintf(stderr, "slots %lld for %lld units\n", (long long)slots, (long long)units);
    return;
  }
  std::vector<int> hits(size_t(units), 0);
  std::vector<int> xcd_of_block(size_t((units + per_block - 1) / per_block), -1);
  for (int64_t s = 0; s < slots; ++s) {
    const int64_t u = unit_of_slot<IL>(s, slots, per_block);
    if (u < 0) {
      if (failures++ < 20) std::fprintf(stderr, "negative unit at slot %lld\n", (long long)s);
      continue;
    }
    if (u >= units) continue;
    ++hits[size_t(u)];
    if (IL) {
      int &x = xcd_of_block[size_t(u / per_block)];
      if (x < 0) x = int(s & 7);
      else if (x != int(s & 7) && failures++ < 20)
        std::fprintf(stderr, "run %lld on two XCDs\n", (long long)(u / per_block));
    }
  }
  for (int64_t u = 0; u < units; ++u)
    if (hits[size_t(u)] != 1) {
      if (failures++ < 20)
        std::fprintf(stderr, "%s: unit %lld of %lld (per block %lld) has %d slots\n", IL ? "interleaved" : "contiguous",
                     (long long)u, (long long)units, (long long)per_block, hits[size_t(u)]);
      break;
    }
}

}  // namespace

int main() {
  std::mt19937_64 rng(7);
  for (int64_t units = 0; units <= 300; ++units)
    for (int64_t per_block : {1, 2, 3, 4, 7, 8, 11, 13, 32, 33, 44}) {
      check<false>(units, per_block);
      check<true>(units, per_block);
    }
  for (int it = 0; it < 2000; ++it) {
    const int64_t per_block = 1 + int64_t(rng() % 200);
    const int64_t units = int64_t(rng() % 200000);
    check<false>(units, per_block);
    check<true>(units, per_block);
  }
  if (failures) return 1;
  std::printf("ok\n");
  return 0;
}
