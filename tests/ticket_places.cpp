// Host check of the late-workgroup ticket rule (csrc/tickets.h): for every
// claimer count and counter start value, the claimers' places form a
// permutation of [0, claimers). The increments are applied one after another,
// as the device's atomics serialise them (their order does not change the set
// of values returned). Prints "ok <cases>" or the first failure; exit status 1
// on failure.
#include <cstdio>
#include <vector>

#include "tickets.h"

int main() {
  long cases = 0;
  const uint32_t big[] = {0x7fffffffu, 0x80000000u, 0xfffffffeu, 0xffffffffu};
  for (uint32_t n = 1; n <= 300; ++n) {
    std::vector<uint32_t> starts;
    for (uint32_t c = 0; c <= n + 8; ++c) starts.push_back(c);
    for (uint32_t b : big) starts.push_back(b);
    for (uint32_t c0 : starts) {
      uint32_t counter = c0;
      std::vector<int> seen(n, 0);
      for (uint32_t k = 0; k < n; ++k) {
        const uint32_t old = counter;
        counter = pkv::ticket_counter_next(old, n - 1);
        const uint32_t place = pkv::ticket_place(old, n);
        if (place >= n) {
          std::printf("claimers %u start %u: place %u out of range\n", n, c0, place);
          return 1;
        }
        seen[place] += 1;
      }
      for (uint32_t p = 0; p < n; ++p) {
        if (seen[p] != 1) {
          std::printf("claimers %u start %u: place %u taken %d times\n", n, c0, p, seen[p]);
          return 1;
        }
      }
      // a clean counter stays clean; any start within the range is kept
      if (c0 <= n - 1 && counter != c0) {
        std::printf("claimers %u start %u: counter ends at %u\n", n, c0, counter);
        return 1;
      }
      ++cases;
    }
  }
  // Without the clamp, a start value past the limit leaves one place
  // untaken: the rule above is what makes those cases pass.
  long raw_fail = 0;
  for (uint32_t n = 1; n <= 300; ++n) {
    uint32_t counter = n + 3;
    std::vector<int> seen(n, 0);
    for (uint32_t k = 0; k < n; ++k) {
      const uint32_t old = counter;
      counter = pkv::ticket_counter_next(old, n - 1);
      if (old < n) seen[old] += 1;
    }
    for (uint32_t p = 0; p < n; ++p) raw_fail += seen[p] != 1;
  }
  std::printf("ok %ld %ld\n", cases, raw_fail);
  return 0;
}
