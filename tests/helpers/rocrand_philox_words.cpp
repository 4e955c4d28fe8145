// Prints the Philox4x32-10 word that rocRAND's engine yields for each query
// line "seed b h j" on stdin: the engine is seeded with `seed`, moved to
// subsequence b and skipped by h * 2^34 + j numbers, then asked for one word.
// Used only to pin the CPU oracle's Philox against an independent
// implementation (rocRAND's host-callable engine).
#include <rocrand/rocrand_philox4x32_10.h>

#include <cstdio>

int main() {
  unsigned long long seed, b, h, j;
  while (std::scanf("%llu %llu %llu %llu", &seed, &b, &h, &j) == 4) {
    rocrand_device::philox4x32_10_engine e(seed, b, (h << 34) + j);
    std::printf("%u\n", e.next());
  }
  return 0;
}
