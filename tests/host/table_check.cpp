// Host checks of the code tables the library builds (compiled with address
// and undefined-behaviour sanitizers by tests/test_host_tables.py; CPU only).
//
// For every table: ascending levels spanning [-1, 1]; each threshold is the
// smallest fp32 number above its midpoint (equal levels share one threshold);
// on a sweep of fp32 quotients the one-comparison bucket search, when the
// table allows it, gives the same code as counting the 15 thresholds, and that
// count is the nearest level with the lowest index on a tie; the decode
// levels are bf16(kappa * L) with kappa * L exact in bf16 for kappa > 1.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "nf4_table.h"

using namespace qlora;

static int failures = 0;
#define CHECK(cond, ...)                      \
  do {                                        \
    if (!(cond)) {                            \
      std::printf("FAIL %s: ", #cond);        \
      std::printf(__VA_ARGS__);               \
      std::printf("\n");                      \
      if (++failures > 20) return;            \
    }                                         \
  } while (0)

static float from_bits(uint32_t b) {
  float f;
  std::memcpy(&f, &b, 4);
  return f;
}

static uint32_t count_code(float x, const Nf4Table& t) {
  uint32_t c = 0;
  for (int j = 0; j < 15; ++j) c += x >= t.thr[j];
  return c;
}

// nearest level, lowest index on a tie, decided exactly: for fp32 x and
// levels a < b, x is nearer to b iff 2x > a + b, and 2x, a + b are exact in
// long double (64-bit significand) for the magnitudes here, or x is tiny and
// the comparison is decided by sign
static uint32_t nearest(float x, const Nf4Table& t) {
  uint32_t best = 0;
  for (uint32_t i = 1; i < 16; ++i) {
    const long double a = t.level[best], b = t.level[i];
    if (b == a) continue;
    const long double d2 = 2.0L * (long double)x, s = a + b;
    if (d2 > s) best = i;   // strictly nearer to the higher level i (levels ascend)
  }
  return best;
}

static void check_table(int ty) {
  const Nf4Table& t = code_table(ty);
  const Nf4Buckets& bk = code_buckets(ty);
  const DecodeLevels& dl = decode_levels(ty);
  CHECK(t.level[0] == -1.0f && t.level[15] == 1.0f, "table %d span", ty);
  for (int i = 0; i < 15; ++i) CHECK(t.level[i] <= t.level[i + 1], "table %d level %d", ty, i);
  for (int j = 0; j < 15; ++j) {
    if (t.level[j] == t.level[j + 1]) {
      CHECK(j < 14 && t.thr[j] == t.thr[j + 1], "table %d duplicate level %d", ty, j);
      continue;
    }
    const long double mid = ((long double)t.level[j] + (long double)t.level[j + 1]) / 2.0L;
    CHECK((long double)t.thr[j] > mid, "table %d thr %d above", ty, j);
    CHECK((long double)std::nextafter(t.thr[j], -INFINITY) <= mid, "table %d thr %d smallest", ty, j);
  }
  // the sweep: every 101st fp32 pattern in [-1, 1] (both signs), plus the
  // neighbours of every threshold and of every bucket edge
  uint64_t n = 0;
  auto one = [&](float x) {
    const uint32_t c = count_code(x, t);
    CHECK(c == nearest(x, t), "table %d x %a: count %u nearest %u", ty, (double)x, c, nearest(x, t));
    if (bk.ok) {
      int q = (int)std::fma(x, 16.0f, 16.0f);
      q = q < 0 ? 0 : q > 32 ? 32 : q;
      const uint32_t cb = bk.base[q] + (x >= bk.thr[q] ? 1u : 0u);
      CHECK(cb == c, "table %d x %a: bucket %u count %u", ty, (double)x, cb, c);
    }
    ++n;
  };
  for (uint32_t b = 0; b <= 0x3F800000u; b += 101) {
    one(from_bits(b));
    one(from_bits(b | 0x80000000u));
  }
  for (int j = 0; j < 15; ++j) {
    float x = t.thr[j];
    for (int k = 0; k < 4; ++k) x = std::nextafter(x, -INFINITY);
    for (int k = 0; k < 9; ++k, x = std::nextafter(x, INFINITY)) one(x);
  }
  for (int q = 0; q <= 32; ++q) {
    float x = (float)(q / 16.0 - 1.0);
    for (int k = 0; k < 4; ++k) x = std::nextafter(x, -INFINITY);
    for (int k = 0; k < 9; ++k, x = std::nextafter(x, INFINITY))
      if (std::fabs(x) <= 1.0f) one(x);
  }
  // decode levels
  CHECK(dl.kappa >= 1.0f && dl.kappa == std::floor(dl.kappa), "table %d kappa %g", ty, (double)dl.kappa);
  for (int i = 0; i < 16; ++i) {
    const double v = (double)dl.kappa * t.level[i];
    const uint32_t bits = (uint32_t)dl.bf16[i] << 16;
    const double b = from_bits(bits);
    if (dl.kappa > 1.0f)
      CHECK(std::fabs(b - v) <= std::ldexp(std::fabs(v), -20), "table %d decode level %d", ty, i);
    else
      CHECK(std::fabs(b - v) <= std::ldexp(std::fabs(v), -8), "table %d decode level %d", ty, i);
  }
  std::printf("table %d: %llu quotients, buckets %s, kappa %g\n", ty, (unsigned long long)n,
              bk.ok ? "on" : "off", (double)dl.kappa);
}

int main() {
  for (int ty = 0; ty < kCodeTables; ++ty) check_table(ty);
  std::printf("%s\n", failures ? "FAILED" : "OK");
  return failures ? 1 : 0;
}
