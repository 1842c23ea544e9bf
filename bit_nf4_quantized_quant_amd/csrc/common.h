// Device-side building blocks shared by the QLoRA NF4 kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nf4_table.h"

namespace qlora {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBlock = 64;     // weights per first-level constant
constexpr int kDqBlock = 256;  // constants per second-level constant

// --------------------------------------------------------------- bf16

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v[0] = (__bf16)lo;  // v_cvt_pk_bf16_f32: round to nearest even
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// --------------------------------------------------------------- E4M3 (OCP e4m3fn)

// Exact decode of an E4M3 byte (never NaN here: the encoder saturates at 448).
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  const uint32_t sign = (c & 0x80u) << 24;
  const uint32_t e = (c >> 3) & 0xFu;
  const uint32_t m = c & 0x7u;
  float mag;
  if (e == 0) {
    mag = (float)m * 0.001953125f;  // m * 2^-9 (subnormal)
  } else {
    mag = __uint_as_float(((e + 120u) << 23) | (m << 20));  // (1 + m/8) * 2^(e-7)
  }
  return __uint_as_float(__float_as_uint(mag) | sign);
}

// fp32 -> E4M3 byte: round to nearest, ties to even, saturate to +-448, keep
// the sign of zero.  Written on the fp32 bit pattern.
__device__ __forceinline__ uint32_t f32_to_e4m3(float t) {
  const uint32_t bits = __float_as_uint(t);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const float a = __uint_as_float(bits & 0x7FFFFFFFu);
  uint32_t code;
  if (a >= 448.0f) {
    code = 0x7Eu;
  } else if (a < 0.015625f) {  // below 2^-6: E4M3 subnormal grid of step 2^-9
    code = (uint32_t)__builtin_rintf(a * 512.0f);  // exact scaling, rint = ties to even; 8 -> 0x08
  } else {
    const uint32_t ab = bits & 0x7FFFFFFFu;
    const uint32_t e = (ab >> 23) - 120u;  // E4M3 exponent field, 1..15
    const uint32_t frac = ab & 0x7FFFFFu;
    const uint32_t m = frac >> 20;
    const uint32_t rest = frac & 0xFFFFFu;
    const uint32_t up = (rest > 0x80000u) || (rest == 0x80000u && (m & 1u));
    code = ((e << 3) | m) + up;  // a mantissa carry moves into the exponent
  }
  return code | sign;
}

// c_hat = fp32( fp32(e4m3(c2) * c1) + mean ), two separate roundings.
__device__ __forceinline__ float dequant_constant(uint32_t c2, float c1, float mean) {
  const float p = __fmul_rn(e4m3_to_f32(c2), c1);
  return __fadd_rn(p, mean);
}

__device__ __forceinline__ uint32_t nf4_code(float x, const Nf4Table& t) {
  uint32_t c = 0;
#pragma unroll
  for (int j = 0; j < 15; ++j) c += (x >= t.thr[j]) ? 1u : 0u;
  return c;
}

}  // namespace qlora
