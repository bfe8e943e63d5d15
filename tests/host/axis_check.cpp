// Host check of the GEMM output-address division (multiply-shift reciprocal):
// floor(x / d) for 0 <= x < 2^31 across many divisors.  Exit status 0 = pass.
#include <cstdio>
#include <cstdint>
#include <random>
#include "txl_internal.h"

int main() {
  using namespace txl;
  std::mt19937_64 rng(12345);
  std::vector<int32_t> divs = {1, 2, 3, 5, 7, 31, 32, 33, 41, 48, 64, 100, 150, 160, 300, 1728,
                               3928, 3968, 65535, 65536, 65537, (1 << 20) + 7, 1 << 30,
                               (1 << 30) + 1, 0x7ffffffe};
  for (int i = 0; i < 2000; ++i) divs.push_back(1 + (int32_t)(rng() % 0x7ffffffeu));
  for (int i = 0; i < 2000; ++i) divs.push_back(1 + (int32_t)(rng() % 5000));
  long checked = 0;
  for (int32_t d : divs) {
    AxisMap a = make_axis(d, 7, 3);
    auto check = [&](int64_t x) {
      if (x < 0 || x > 0x7fffffff) return true;
      const int32_t q = axis_quot(a, (int32_t)x);
      ++checked;
      if (q != (int32_t)(x / d)) {
        std::printf("FAIL d=%d x=%lld q=%d want=%lld\n", d, (long long)x, q, (long long)(x / d));
        return false;
      }
      const int64_t off = axis_offset(a, (int32_t)x);
      if (off != (x / d) * 7 + (x % d) * 3) {
        std::printf("FAIL offset d=%d x=%lld\n", d, (long long)x);
        return false;
      }
      return true;
    };
    for (int64_t x = 0; x < 4096; ++x) if (!check(x)) return 1;
    for (int64_t k = 1; k < 64; ++k)
      for (int64_t e = -1; e <= 1; ++e) if (!check(k * (int64_t)d + e)) return 1;
    for (int64_t m = 0x7fffffffLL / d - 2; m <= 0x7fffffffLL / d + 1; ++m)
      for (int64_t e = -1; e <= 1; ++e) if (!check(m * (int64_t)d + e)) return 1;
    for (int i = 0; i < 2000; ++i) if (!check((int64_t)(rng() % 0x80000000ull))) return 1;
    if (!check(0x7fffffff)) return 1;
  }
  AxisMap lin = make_axis(kLinearDiv, 0, 5);
  for (int64_t x : {0LL, 1LL, 12345LL, 0x7ffffffeLL})
    if (axis_offset(lin, (int32_t)x) != x * 5) { std::printf("FAIL linear\n"); return 1; }
  std::printf("ok %ld checks\n", checked);
  return 0;
}
