// Host check of the multiply-shift division the kernels use for row maps and
// block coordinates (fast_div / fdiv in common.h): fdiv(n, fast_div(d)) must
// equal n / d for every 0 <= n < 2^31 and 1 <= d < 2^31.  Edge cases
// (powers of two and their neighbours, the largest numerators, d = 1 and the
// largest d) plus a seeded sample; prints the failures and exits 1 on any.
#include <cstdint>
#include <cstdio>
#include <random>
#include <vector>
#include "common.h"

using vggt::fast_div;
using vggt::fdiv;

static int check(int n, int64_t d, long* fails) {
  const int q = fdiv(n, fast_div(d));
  const int want = (int)((int64_t)n / d);
  if (q != want) {
    if (*fails < 10) std::printf("n=%d d=%lld: %d, want %d\n", n, (long long)d, q, want);
    ++*fails;
  }
  return 0;
}

int main() {
  long fails = 0, count = 0;
  const int64_t top = ((int64_t)1 << 31) - 1;
  std::vector<int64_t> ds = {1, 2, 3, 5, 7, 17, 64, 1031, 1088, 4096, 65535, 65536, 65537,
                             top - 1, top};
  for (int k = 1; k < 31; ++k)
    for (int e = -1; e <= 1; ++e) ds.push_back(((int64_t)1 << k) + e);
  std::vector<int> ns = {0, 1, 2, 3, 1030, 1031, 1032, 65535, 65536, (int)top - 1, (int)top};
  for (int k = 1; k < 31; ++k)
    for (int e = -1; e <= 1; ++e) ns.push_back((int)(((int64_t)1 << k) + e));
  for (int64_t d : ds)
    for (int n : ns) {
      check(n, d, &fails);
      ++count;
      // the multiples of d and their neighbours (where a wrong quotient shows)
      for (int64_t m : {(int64_t)n / d, (int64_t)n / d + 1})
        for (int e = -1; e <= 0; ++e) {
          const int64_t x = m * d + e;
          if (x >= 0 && x <= top) {
            check((int)x, d, &fails);
            ++count;
          }
        }
    }
  std::mt19937_64 rng(20261204);
  for (int i = 0; i < 4000000; ++i) {
    const int bits = 1 + (int)(rng() % 31);
    const int64_t d = 1 + (int64_t)(rng() % (uint64_t)(((int64_t)1 << bits) - 1));
    const int n = (int)(rng() & (uint64_t)top);
    check(n, d, &fails);
    ++count;
  }
  std::printf("%ld checks, %ld failures\n", count, fails);
  return fails ? 1 : 0;
}
