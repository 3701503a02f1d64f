// Host check of the partition arithmetic shared by the decode kernels:
// floor_div against exact integer division over the whole range the host
// admits (numerators below 2^51), and PartGrid against its integer
// definition (partition g owns units [floor(gT/G), floor((g+1)T/G))).
#include <cstdio>
#include <random>

#include "mla_common.h"

int main() {
  std::mt19937_64 rng(1);
  long bad = 0, n = 0;
  auto check = [&](int64_t num, int64_t den) {
    ++n;
    const int64_t q = mla::floor_div(num, den);
    if (q != num / den && bad++ < 5)
      std::printf("floor_div(%lld, %lld) = %lld, want %lld\n", (long long)num, (long long)den,
                  (long long)q, (long long)(num / den));
  };
  const int64_t kNumMax = int64_t(1) << 51;
  for (int i = 0; i < 1000000; ++i) {
    const int64_t den = 1 + int64_t(rng() % ((uint64_t(1) << 31) - 1));
    const int64_t k = int64_t(rng() % uint64_t(kNumMax / den + 1));
    for (int d = -1; d <= 1; ++d) {
      const int64_t num = k * den + d;
      if (num >= 0 && num < kNumMax) check(num, den);
    }
  }
  for (int64_t den : {1, 2, 3, 7, 1 << 20, (1 << 20) + 1, 2147483647})
    for (int64_t num : {int64_t(0), int64_t(1), kNumMax - 1, kNumMax - 2, den * (kNumMax / den) - 1})
      if (num >= 0) check(num, den);
  // partition grid: boundaries and owners agree with the integer definition
  for (int i = 0; i < 2000; ++i) {
    const int64_t T = 1 + int64_t(rng() % (i < 1000 ? 5000 : 2147483647));
    const int G = int(std::min<int64_t>(T, 1 + int64_t(rng() % (1 << 20))));
    const mla::PartGrid pg(T, G);
    for (int s = 0; s < 50; ++s) {
      const int g = int(rng() % uint64_t(G + 1));
      ++n;
      if (pg.lo(g) != int64_t(g) * T / G && bad++ < 5)
        std::printf("lo(%d) T=%lld G=%d wrong\n", g, (long long)T, G);
      const int64_t u = int64_t(rng() % uint64_t(T));
      const int p = pg.part_of(u);
      ++n;
      if ((p < 0 || p >= G || pg.lo(p) > u || pg.lo(p + 1) <= u) && bad++ < 5)
        std::printf("part_of(%lld) = %d, T=%lld G=%d\n", (long long)u, p, (long long)T, G);
    }
  }
  std::printf("%ld checks, %ld wrong\n", n, bad);
  return bad != 0;
}
