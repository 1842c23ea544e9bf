// Host construction of the NF4 code table and its decision thresholds.
//
// itwiki "QLoRA", NF4 section: the 16 levels are standard-normal quantiles.
// The positive half uses 8 probabilities spaced evenly from 0.5 (excluded) up
// to the offset 0.9677083, the negative half the negated quantiles of 7 such
// probabilities, plus an exact zero; the set is divided by its largest
// magnitude so that it spans [-1, 1].
//
// The inverse normal CDF is solved here by Newton's method on
// Phi(x) = erfc(-x / sqrt(2)) / 2 in long double, which is far more accurate
// than the fp32 rounding of the levels needs (every level sits more than 1e-3
// fp32 ulp away from an fp32 rounding tie).
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "nf4_table.h"

namespace qlora {
namespace {

constexpr long double kOffset = 0.9677083L;

long double normal_quantile(long double p) {
  const long double sqrt2 = 1.41421356237309504880168872420969808L;
  const long double inv_sqrt_2pi = 0.398942280401432677939946059934381868L;
  long double x = 0.0L;
  for (int it = 0; it < 100; ++it) {
    const long double cdf = 0.5L * std::erfc(-x / sqrt2);
    const long double pdf = inv_sqrt_2pi * std::exp(-0.5L * x * x);
    const long double step = (cdf - p) / pdf;
    x -= step;
    if (std::fabs(step) < 1e-19L) break;
  }
  return x;
}

// Smallest fp32 number strictly greater than the exact midpoint m.
float next_f32_above(long double m) {
  float f = (float)m;
  if ((long double)f <= m) f = std::nextafter(f, INFINITY);
  while ((long double)std::nextafter(f, -INFINITY) > m) f = std::nextafter(f, -INFINITY);
  return f;
}

Nf4Table build_table() {
  long double v[16];
  int k = 0;
  for (int i = 7; i >= 1; --i) v[k++] = -normal_quantile(0.5L + (kOffset - 0.5L) * i / 7.0L);
  v[k++] = 0.0L;
  for (int i = 1; i <= 8; ++i) v[k++] = normal_quantile(0.5L + (kOffset - 0.5L) * i / 8.0L);
  long double mx = 0.0L;
  for (int i = 0; i < 16; ++i) mx = std::fmax(mx, std::fabs(v[i]));
  Nf4Table t;
  for (int i = 0; i < 16; ++i) t.level[i] = (float)(v[i] / mx);
  for (int j = 0; j < 15; ++j) {
    const long double mid = ((long double)t.level[j] + (long double)t.level[j + 1]) / 2.0L;
    t.thr[j] = next_f32_above(mid);
  }
  return t;
}

uint16_t bf16_rne(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

float bf16_value(uint16_t b) {
  const uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

}  // namespace

const Nf4HiLo& nf4_hilo() {
  static Nf4HiLo hl;
  static std::once_flag once;
  std::call_once(once, [] {
    const Nf4Table& t = nf4_table();
    for (int i = 0; i < 16; ++i) {
      const uint16_t hi = bf16_rne(t.level[i]);
      const uint16_t lo = bf16_rne(t.level[i] - bf16_value(hi));
      hl.word[i] = (uint32_t)hi | ((uint32_t)lo << 16);
    }
  });
  return hl;
}

const Nf4Buckets& nf4_buckets() {
  static Nf4Buckets b;
  static std::once_flag once;
  std::call_once(once, [] {
    const Nf4Table& t = nf4_table();
    b.ok = 1;
    for (int q = 0; q <= 32; ++q) {
      const double lo = q / 16.0 - 1.0, hi = (q + 1) / 16.0 - 1.0;
      b.thr[q] = INFINITY;
      b.base[q] = 0;
      int inside = 0;
      for (int j = 0; j < 15; ++j) {
        const double v = t.thr[j];
        if (v < lo) ++b.base[q];
        if (v >= lo && v < hi) {
          b.thr[q] = t.thr[j];
          ++inside;
        }
        if (std::fabs(v - lo) <= std::ldexp(1.0, -20)) b.ok = 0;
      }
      if (inside > 1) b.ok = 0;
    }
  });
  return b;
}

const Nf4Table& nf4_table() {
  static Nf4Table table;
  static std::once_flag once;
  std::call_once(once, [] { table = build_table(); });
  return table;
}

}  // namespace qlora
