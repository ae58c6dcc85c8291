// Host check of DivBy (the launch-invariant division of the kernels' block
// decoding) against plain integer division: every divisor up to 4096 and the
// powers of two and their neighbours up to 2^31 - 1, each with dividends
// 0 .. 4095, the last 4096 below 2^31, multiples of the divisor and their
// neighbours, and a pseudo-random spread.  Prints "ok <checks>" or the first
// mismatch.
#include <cstdint>
#include <cstdio>
#include <vector>

#include "npa_internal.hpp"

using npa::DivBy;

static bool check_one(int32_t d, int32_t n, const DivBy& b, long long& count) {
  ++count;
  if (n < 0) return true;
  const int32_t q = b.div(n), r = b.mod(n);
  if (q != n / d || r != n % d) {
    std::printf("mismatch: %d / %d -> %d rem %d (expected %d rem %d)\n", n, d, q, r, n / d, n % d);
    return false;
  }
  return true;
}

int main() {
  std::vector<int32_t> divisors;
  for (int32_t d = 1; d <= 4096; ++d) divisors.push_back(d);
  for (int k = 12; k <= 30; ++k)
    for (int32_t e = -3; e <= 3; ++e) divisors.push_back((int32_t)((1u << k) + e));
  divisors.push_back(2147483646);
  divisors.push_back(2147483647);
  const int32_t top = 2147483647;
  long long count = 0;
  uint64_t x = 0x9E3779B97F4A7C15ull;
  for (int32_t d : divisors) {
    const DivBy b = DivBy::of(d);
    for (int32_t n = 0; n < 4096; ++n)
      if (!check_one(d, n, b, count)) return 1;
    for (int32_t n = top - 4095; n >= 0 && n <= top - 0; ++n) {
      if (!check_one(d, n, b, count)) return 1;
      if (n == top) break;
    }
    for (int64_t k = 1; k <= 64; ++k) {
      const int64_t m = (int64_t)d * k * 33331;
      for (int64_t e = -1; e <= 1; ++e)
        if (m + e >= 0 && m + e <= top && !check_one(d, (int32_t)(m + e), b, count)) return 1;
    }
    for (int i = 0; i < 256; ++i) {
      x ^= x << 13;
      x ^= x >> 7;
      x ^= x << 17;
      if (!check_one(d, (int32_t)(x & 0x7FFFFFFF), b, count)) return 1;
    }
  }
  std::printf("ok %lld\n", count);
  return 0;
}
