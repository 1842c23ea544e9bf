// Internal launchers behind the C ABI (host side).  Every launcher queues its
// kernels on the given stream and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qlora {

// Compute units of the current device (cached per device).
int cu_count();
// Raises a kernel's dynamic-LDS limit to at least `bytes` on the current
// device, once per device and kernel.
hipError_t ensure_lds_limit(const void* kernel, size_t bytes);

// table: the code table (0 NF4, 1 uniform 4-bit, 2 FP4; checked by the caller)
hipError_t launch_nf4_quantize(const float* W, int64_t N, int64_t K, int table, uint8_t* codes, float* absmax,
                               hipStream_t s);
hipError_t launch_nf4_quantize_bf16(const uint16_t* W, int64_t N, int64_t K, int table, uint8_t* codes,
                                    float* absmax, hipStream_t s);
size_t double_quant_workspace_bytes();
hipError_t launch_double_quant(const float* absmax, int64_t n, uint8_t* c2, float* c1, float* mean,
                               void* workspace, hipStream_t s);
hipError_t launch_nf4_dequant(const uint8_t* codes, const uint8_t* c2, const float* c1, const float* mean,
                              int table, int64_t N, int64_t K, uint16_t* out, hipStream_t s);
hipError_t launch_nf4_merge(const uint8_t* codes, const uint8_t* c2, const float* c1, const float* mean, int table,
                            int64_t N,
                            int64_t K, const uint16_t* A, const uint16_t* B, int64_t r, float s, uint16_t* out,
                            hipStream_t st);

// The quantized weight as the matrix kernels see it.
struct Nf4Weight {
  const uint8_t* codes;  // [N, K/2]
  const uint8_t* c2;     // [N*K/64]
  const float* c1;       // [ceil(N*K/16384)]
  const float* mean;     // [1]
  int table;             // code table (0 NF4, 1 uniform 4-bit, 2 FP4)
};

struct FwdArgs {
  const uint16_t* X;
  int64_t M, N, K, r;
  Nf4Weight w;
  const uint16_t* A;
  const uint16_t* B;
  float scale;      // alpha / r
  uint16_t* Y;
  float* H;         // [M, r] fp32 (caller's H_out or the workspace)
  void* workspace;  // remaining workspace past H
};

struct BwdArgs {
  const uint16_t* dY;
  const uint16_t* X;
  int64_t M, N, K, r;
  Nf4Weight w;
  const uint16_t* A;
  const uint16_t* B;
  float scale;
  const float* H;  // may be null: recomputed into the workspace
  uint16_t* dX;    // may be null
  uint16_t* dA;
  uint16_t* dB;
  void* workspace;
};

hipError_t launch_linear_bwd(const BwdArgs& a, hipStream_t s);

}  // namespace qlora
