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

// Decision thresholds of an ascending level table: code(x) = #{j : x >= thr[j]}
// picks the nearest level, the lowest code on a tie.  Where two codes share
// a level (FP4's two zeros) the upper one is never the lowest nearest code, so
// its boundary coincides with the next one and both are crossed together.
void set_thresholds(Nf4Table& t) {
  for (int j = 14; j >= 0; --j) {
    if (t.level[j] == t.level[j + 1] && j < 14) {
      t.thr[j] = t.thr[j + 1];
      continue;
    }
    const long double mid = ((long double)t.level[j] + (long double)t.level[j + 1]) / 2.0L;
    t.thr[j] = next_f32_above(mid);
  }
}

Nf4Table build_nf4() {
  long double v[16];
  int k = 0;
  for (int i = 7; i >= 1; --i) v[k++] = -normal_quantile(0.5L + (kOffset - 0.5L) * i / 7.0L);
  v[k++] = 0.0L;
  for (int i = 1; i <= 8; ++i) v[k++] = normal_quantile(0.5L + (kOffset - 0.5L) * i / 8.0L);
  long double mx = 0.0L;
  for (int i = 0; i < 16; ++i) mx = std::fmax(mx, std::fabs(v[i]));
  Nf4Table t;
  for (int i = 0; i < 16; ++i) t.level[i] = (float)(v[i] / mx);
  set_thresholds(t);
  return t;
}

// Uniform 4-bit: 16 evenly spaced levels on [-1, 1] (itwiki "QLoRA", NF4
// section: the comparison grid of the worked example), each the fp32 rounding
// of -1 + 2 i / 15 as an fp64 number -1 + i * (2 / 15).
Nf4Table build_uniform4() {
  Nf4Table t;
  const double step = 2.0 / 15.0;
  for (int i = 0; i < 16; ++i) t.level[i] = i == 15 ? 1.0f : (float)(-1.0 + i * step);
  set_thresholds(t);
  return t;
}

// FP4: the 4-bit float E2M1 -- sign, 2 exponent bits with bias 1, 1
// mantissa bit, subnormals at exponent field 0, no infinity or NaN -- with
// every magnitude pattern 0..7 decoded as its significand (in halves) times a
// power of two, scaled by the largest magnitude (6) to span [-1, 1] like the
// other tables.  Ascending order puts -0 and +0 at codes 7 and 8; both are
// stored as +0, so code 7 stays the zero level.  The pages name FP4
// (irregular6612 "QLoRA - Efficient Finetuning of Quantized LLMs"; itwiki
// "QLoRA": bitsandbytes' default 4-bit type) but give no grid: this one is a
// reading.
Nf4Table build_fp4() {
  double mag[8];
  for (int c = 0; c < 8; ++c) {
    const int e = c >> 1, m = c & 1;
    // subnormal: m/2 * 2^(1-1); normal: (2 + m)/2 * 2^(e-1)
    mag[c] = e == 0 ? std::ldexp((double)m, -1) : std::ldexp((double)(2 + m), e - 2);
  }
  Nf4Table t;
  for (int i = 0; i < 8; ++i) {
    t.level[7 - i] = i == 0 ? 0.0f : (float)(-mag[i] / mag[7]);
    t.level[8 + i] = (float)(mag[i] / mag[7]);
  }
  set_thresholds(t);
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

const Nf4Table& code_table(int type) {
  static Nf4Table tables[kCodeTables];
  static std::once_flag once;
  std::call_once(once, [] {
    tables[kTableNf4] = build_nf4();
    tables[kTableUniform4] = build_uniform4();
    tables[kTableFp4] = build_fp4();
  });
  return tables[type];
}

const DecodeLevels& decode_levels(int type) {
  static DecodeLevels dl[kCodeTables];
  static std::once_flag once;
  std::call_once(once, [] {
    for (int ty = 0; ty < kCodeTables; ++ty) {
      const Nf4Table& t = code_table(ty);
      int kappa = 1;
      for (int k = 1; k <= 64; ++k) {
        bool exact = true;
        for (int i = 0; i < 16; ++i) {
          const double v = (double)k * t.level[i];
          const double b = bf16_value(bf16_rne((float)v));
          exact = exact && std::fabs(b - v) <= std::ldexp(std::fabs(v), -20);
        }
        if (exact) {
          kappa = k;
          break;
        }
      }
      dl[ty].kappa = (float)kappa;
      for (int i = 0; i < 16; ++i) dl[ty].bf16[i] = bf16_rne((float)((double)kappa * t.level[i]));
    }
  });
  return dl[type];
}

const Nf4Buckets& code_buckets(int type) {
  static Nf4Buckets bk[kCodeTables];
  static std::once_flag once;
  std::call_once(once, [] {
    for (int ty = 0; ty < kCodeTables; ++ty) {
      const Nf4Table& t = code_table(ty);
      Nf4Buckets& b = bk[ty];
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
    }
  });
  return bk[type];
}

}  // namespace qlora
