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

// --------------------------------------------------------------- buffer resources

// A raw buffer over `bytes` bytes at `base`: loads take a 32-bit byte offset
// (vector part + scalar part + immediate) and return zero past the end.
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

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

// Exact decode of an E4M3 byte: gfx950's v_cvt_f32_fp8 takes the OCP e4m3fn
// format (bias 7, subnormals, max 448); every E4M3 value is exact in fp32.
// `sel` picks the byte of `w` (a constant, encoded in the instruction).
template <int sel>
__device__ __forceinline__ float e4m3_byte_to_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_f32_fp8((int)w, sel);
}

__device__ __forceinline__ float e4m3_to_f32(uint32_t c) { return e4m3_byte_to_f32<0>(c); }

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

// The same for byte `sel` of a word holding four c2 codes.
template <int sel>
__device__ __forceinline__ float dequant_constant_byte(uint32_t c2w, float c1, float mean) {
  return __fadd_rn(__fmul_rn(e4m3_byte_to_f32<sel>(c2w), c1), mean);
}

__device__ __forceinline__ uint32_t nf4_code(float x, const Nf4Table& t) {
  uint32_t c = 0;
#pragma unroll
  for (int j = 0; j < 15; ++j) c += (x >= t.thr[j]) ? 1u : 0u;
  return c;
}

}  // namespace qlora
