// run_bits_check.cpp -- host-side exhaustive check of the partial-tile run
// bitmask (attn_common.h) against the per-element definition of a run.
//
// A lane's 32 elements of a 64-wide tile sit at indices
// base + elem_offset(e / 16, e % 16), base = tile start + 4 h.  For every
// run [s, e) with 0 <= s <= e <= N, every tile start and both lane halves,
// bit t of run_bits(s, e - s, base) must be set exactly when
// s <= index(t) < e, and every index must be numbered in increasing order.
// Prints "ok <checks>" and exits 0, or the first mismatch and exits 1.
#include <cstdio>
#include <cstdlib>

#include "../runtime_metadata_attention_amd/csrc/attn_common.h"

using namespace cm::attn;

int main(int argc, char** argv) {
  const int N = argc > 1 ? std::atoi(argv[1]) : 200;
  long checks = 0;
  for (int t0 = 0; t0 < N + 64; t0 += 64) {
    for (int h = 0; h < 2; ++h) {
      const uint32_t base = uint32_t(t0 + 4 * h);
      uint32_t prev = 0;
      for (int e = 0; e < 32; ++e) {
        const uint32_t j = base + elem_offset(e >> 4, e & 15);
        if (e > 0 && j <= prev) {
          std::printf("element order: base %u element %d index %u after %u\n", base, e, j, prev);
          return 1;
        }
        prev = j;
      }
      for (int s = 0; s <= N; ++s) {
        for (int en = s; en <= N; ++en) {
          const uint32_t bits = run_bits(uint32_t(s), uint32_t(en - s), base);
          for (int e = 0; e < 32; ++e) {
            const uint32_t j = base + elem_offset(e >> 4, e & 15);
            const bool want = uint32_t(s) <= j && j < uint32_t(en);
            const bool got = (bits >> e) & 1u;
            ++checks;
            if (want != got) {
              std::printf("mismatch: run [%d, %d) base %u element %d (index %u): bit %d, want %d\n", s, en, base,
                          e, j, int(got), int(want));
              return 1;
            }
          }
        }
      }
    }
  }
  std::printf("ok %ld\n", checks);
  return 0;
}
