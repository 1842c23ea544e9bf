// Exact mean of non-negative fp32 values, rounded once to fp32.
//
// Every finite fp32 value is M * 2^(b-150) with an integer mantissa M < 2^24 and
// b = max(biased exponent, 1).  Summing the mantissas per b in 64-bit integers
// ("buckets") loses nothing, and the exact total is
//     S * 2^-149,   S = sum_b bucket[b] * 2^(b-1).
// mean_from_buckets() forms S as a multi-word integer, divides by n and rounds
// the quotient to the nearest fp32 (ties to even), subnormals included.  It is
// plain integer code, so it runs the same on the host and on the GPU.
#pragma once

#include <stdint.h>

#ifdef __HIPCC__
#define QLORA_HD __host__ __device__
#else
#define QLORA_HD
#endif

namespace qlora {

constexpr int kMeanBuckets = 256;  // indices 1..254 used

namespace detail {

constexpr int kLimbs = 16;  // 512-bit integers in 32-bit limbs

QLORA_HD inline int bitlen_big(const uint32_t* x) {
  for (int i = kLimbs - 1; i >= 0; --i)
    if (x[i]) return 32 * i + (32 - __builtin_clz(x[i]));
  return 0;
}

QLORA_HD inline int bitlen64(uint64_t v) { return v ? 64 - __builtin_clzll(v) : 0; }

// x += v << shift  (v < 2^64, shift >= 0, result < 2^512)
QLORA_HD inline void add_shifted(uint32_t* x, uint64_t v, int shift) {
  int li = shift >> 5;
  const int bo = shift & 31;
  // v << bo spans up to 96 bits
  uint32_t parts[3];
  parts[0] = (uint32_t)(v << bo);
  parts[1] = (uint32_t)((bo ? (v >> (32 - bo)) : (v >> 32)));
  parts[2] = bo ? (uint32_t)(v >> (64 - bo)) : 0u;
  uint64_t carry = 0;
  for (int k = 0; k < 3 || carry; ++k, ++li) {
    if (li >= kLimbs) break;
    uint64_t s = (uint64_t)x[li] + (k < 3 ? parts[k] : 0u) + carry;
    x[li] = (uint32_t)s;
    carry = s >> 32;
  }
}

// Bits [0, nbits) of x are all zero?
QLORA_HD inline bool low_bits_zero(const uint32_t* x, int nbits) {
  for (int i = 0; i < kLimbs && nbits > 0; ++i, nbits -= 32) {
    const uint32_t mask = nbits >= 32 ? 0xFFFFFFFFu : ((1u << nbits) - 1u);
    if (x[i] & mask) return false;
  }
  return true;
}

// y = x << s (s >= 0) or x >> -s
QLORA_HD inline void shift_big(const uint32_t* x, int s, uint32_t* y) {
  for (int i = 0; i < kLimbs; ++i) y[i] = 0;
  if (s >= 0) {
    const int ls = s >> 5, bs = s & 31;
    for (int i = kLimbs - 1; i >= 0; --i) {
      const int src = i - ls;
      if (src < 0) break;
      uint32_t v = x[src] << bs;
      if (bs && src - 1 >= 0) v |= x[src - 1] >> (32 - bs);
      y[i] = v;
    }
  } else {
    const int r = -s, ls = r >> 5, bs = r & 31;
    for (int i = 0; i < kLimbs; ++i) {
      const int src = i + ls;
      if (src >= kLimbs) break;
      uint32_t v = x[src] >> bs;
      if (bs && src + 1 < kLimbs) v |= x[src + 1] << (32 - bs);
      y[i] = v;
    }
  }
}

}  // namespace detail

// bucket[b] = sum of integer mantissas of the values whose max(exponent,1) is b.
// Returns the fp32 bit pattern of the correctly rounded mean of n values.
// The rounded mean of S * 2^-149 over n values (S: kLimbs-limb integer).
QLORA_HD inline uint32_t mean_from_sum(const uint32_t* S, uint64_t n) {
  using namespace detail;
  const int ls = bitlen_big(S);
  if (ls == 0 || n == 0) return 0u;
  const int ln = bitlen64(n);
  const int sh = 26 - (ls - ln);  // scales S/n into [2^25, 2^27)
  uint32_t T[kLimbs];
  shift_big(S, sh, T);
  bool sticky = sh < 0 ? !low_bits_zero(S, -sh) : false;
  // long division of T by n in 16-bit digits (remainder < n < 2^48), from
  // T's highest nonzero limb (the leading zero digits add nothing)
  uint64_t rem = 0, Q = 0;
  for (int i = (bitlen_big(T) + 31) / 32 - 1; i >= 0; --i) {
    for (int h = 1; h >= 0; --h) {
      const uint64_t cur = (rem << 16) | ((T[i] >> (16 * h)) & 0xFFFFu);
      const uint64_t q = cur / n;
      rem = cur - q * n;
      Q = (Q << 16) | q;
    }
  }
  sticky = sticky || rem != 0;
  const int bq = bitlen64(Q);                 // 26 or 27
  int E = bq - 1 - sh - 149;                  // floor(log2(mean))
  int drop = E >= -126 ? bq - 24 : sh;        // bits below the fp32 ulp
  if (drop >= 40) return 0u;                  // far below half the smallest subnormal
  uint64_t keep = Q >> drop;
  const uint64_t low = Q & ((1ull << drop) - 1ull);
  const uint64_t half = 1ull << (drop - 1);
  const bool up = low > half || (low == half && (sticky || (keep & 1ull)));
  keep += up ? 1ull : 0ull;
  if (E < -126) return (uint32_t)keep;        // subnormal (2^23 is the smallest normal)
  if (keep == (1ull << 24)) {
    keep >>= 1;
    E += 1;
  }
  return ((uint32_t)(E + 127) << 23) | ((uint32_t)keep & 0x7FFFFFu);
}

// The rounded mean of n values from their exponent buckets (see above).
QLORA_HD inline uint32_t mean_from_buckets(const unsigned long long* bucket, uint64_t n) {
  using namespace detail;
  uint32_t S[kLimbs];
  for (int i = 0; i < kLimbs; ++i) S[i] = 0;
  for (int b = 1; b < 255; ++b)
    if (bucket[b]) add_shifted(S, bucket[b], b - 1);
  return mean_from_sum(S, n);
}

}  // namespace qlora
