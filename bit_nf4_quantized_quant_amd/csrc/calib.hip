// Reference kernels for the benchmark's attainable-floor figures (gfx950):
// an empty kernel (launch-to-launch cost of one dispatch) and a plain
// streaming read of a buffer (the bandwidth a kernel that only reads the
// bytes reaches).  They compute nothing of the layer; the benchmark times them
// in the same mode as the layer's kernels to show what the platform itself
// allows at a given size.  Built as libqlora_calib.so, separate from the
// layer's library.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ void calib_empty_kernel() {}

// Each workgroup reads one contiguous chunk of 16-byte words, eight loads in
// flight per thread, and folds them with XOR; the fold is stored only when it
// equals a value the caller never passes, so the loads cannot be removed and
// nothing is written.
constexpr int kThreads = 256;
constexpr int kUnroll = 8;

__global__ void __launch_bounds__(kThreads) calib_read_kernel(const u32x4* src, uint64_t n16, uint64_t per_wg,
                                                             uint32_t never, uint32_t* sink) {
  const uint64_t beg = (uint64_t)blockIdx.x * per_wg;
  const uint64_t end = beg + per_wg < n16 ? beg + per_wg : n16;
  uint32_t acc = 0;
  for (uint64_t i = beg + threadIdx.x; i < end; i += (uint64_t)kThreads * kUnroll) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint64_t k = i + (uint64_t)u * kThreads;
      v[u] = k < end ? __builtin_nontemporal_load(src + k) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  if (acc == never) sink[0] = acc;
}

}  // namespace

extern "C" {

// One empty kernel on `stream`.  Returns a hipError_t value.
int calib_empty(void* stream) {
  hipLaunchKernelGGL(calib_empty_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream);
  return (int)hipGetLastError();
}

// Reads `bytes` (a multiple of 16; `src` 16-byte aligned) with `workgroups`
// workgroups of 256 threads on `stream`.  `sink` is one device uint32 that is
// never written in practice.  Returns a hipError_t value.
int calib_read(const void* src, uint64_t bytes, int workgroups, uint32_t* sink, void* stream) {
  if (bytes % 16 != 0 || workgroups <= 0 || (reinterpret_cast<uintptr_t>(src) % 16) != 0) return (int)hipErrorInvalidValue;
  const uint64_t n16 = bytes / 16;
  const uint64_t per_wg = (n16 + workgroups - 1) / workgroups;
  hipLaunchKernelGGL(calib_read_kernel, dim3((unsigned)workgroups), dim3(kThreads), 0, (hipStream_t)stream,
                     static_cast<const u32x4*>(src), n16, per_wg, 0x9E3779B9u, sink);
  return (int)hipGetLastError();
}

}  // extern "C"
