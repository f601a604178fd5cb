// Host check of FastDiv (pa_common.h), the kernels' multiply-and-shift
// division by launch constants: every quotient and remainder it gives is
// compared with plain integer division. Prints "ok" and exits 0 when all agree.
#include <cstdio>
#include <cstdint>
#include <random>

#include "pa_common.h"

static int bad = 0;

static void check(uint32_t d, int n) {
  const pa::FastDiv f = pa::FastDiv::make(d);
  const int q = f.div(n), r = f.mod(n);
  if (q != (int)((uint32_t)n / d) || r != (int)((uint32_t)n % d)) {
    if (bad < 10) std::printf("d %u n %d: got %d r %d, want %u r %u\n", d, n, q, r,
                              (uint32_t)n / d, (uint32_t)n % d);
    ++bad;
  }
}

int main() {
  const int kTop = 0x7fffffff;
  // Every divisor up to 4096 (split sizes, head counts, bins, items per
  // entry): all numerators below 2^16, then numerators near multiples of d
  // and near 2^31.
  for (uint32_t d = 1; d <= 4096; ++d) {
    for (int n = 0; n < (1 << 16); ++n) check(d, n);
    for (int64_t k = 1; k * d < (int64_t)kTop; k = k * 3 + 1)
      for (int e = -1; e <= 1; ++e) {
        const int64_t n = k * d + e;
        if (n >= 0 && n <= kTop) check(d, (int)n);
      }
    for (int n = kTop; n > kTop - 64; --n) check(d, n);
  }
  // Powers of two and their neighbours up to 2^31 - 1, and random pairs.
  for (int l = 0; l <= 31; ++l)
    for (int64_t dd = (1ll << l) - 1; dd <= (1ll << l) + 1; ++dd)
      if (dd >= 1 && dd <= kTop)
        for (int n : {0, 1, 2, (int)dd - 1 < 0 ? 0 : (int)dd - 1, kTop, kTop - 1, kTop / 2})
          if (n >= 0) check((uint32_t)dd, n);
  std::mt19937_64 rng(12345);
  for (int i = 0; i < 20000000; ++i) {
    const uint32_t d = 1 + (uint32_t)(rng() % (uint64_t)kTop);
    const uint32_t dsmall = 1 + (uint32_t)(rng() % 70000);
    const int n = (int)(rng() % ((uint64_t)kTop + 1));
    check(i & 1 ? d : dsmall, n);
  }
  if (bad) {
    std::printf("%d mismatches\n", bad);
    return 1;
  }
  std::printf("ok\n");
  return 0;
}
