// Blockwise NF4 quantization, double quantization of the constants and
// standalone dequantization to bf16 (gfx950).
//
// itwiki "QLoRA", NF4 section: each run of 64 weights is divided by its
// absmax and every quotient is replaced by the index of the nearest of the 16
// NF4 levels.  Double quantization section: the absmax constants are centred
// on their mean and stored as 8-bit floats in runs of 256, with one fp32
// constant per run.  Section on the computation: doubleDequant gives the bf16
// weight used by the matrix products.
//
// All three passes stream HBM once with 16-byte vector accesses; none of them
// needs a matrix core.
#include "common.h"
#include "exact_mean.h"
#include "launch.h"

namespace qlora {
namespace {

// ------------------------------------------------------------------ quantize
//
// One thread per 4 weights: 16 consecutive lanes hold one 64-element block.
// The weights are fp32, or bf16 (minnong511 "quantization", the QLoRA
// pipeline: a base model in FP16/BF16 is quantized to 4 bits), widened
// exactly to fp32 first, so bf16 input gives the codes of its fp32 values.  The
// block absmax is a 4-step xor-shuffle reduction inside the 16-lane group; the
// quotient uses IEEE fp32 division.  Its level index is the count of
// thresholds at or below it: with kBuckets, one comparison against the single
// threshold of the quotient's 1/16-wide bucket (a 33-entry table in LDS; the
// count of the 15 thresholds is what limits the pass otherwise), else all 15
// comparisons.  Codes leave as one 16-bit store per thread (4 nibbles), i.e.
// 128 contiguous bytes per wave.
__device__ __forceinline__ uint32_t nf4_code_bucket(float x, const float2* lut) {
  int q = (int)__builtin_fmaf(x, 16.0f, 16.0f);   // |x| <= 1: 16 (x + 1), rounded, truncated
  q = min(max(q, 0), 32);
  const float2 e = lut[q];
  return __float_as_uint(e.y) + (x >= e.x ? 1u : 0u);
}

// kBf16: the weights come as bf16 (4 per 8-byte load), widened exactly to fp32.
template <bool kBuckets, bool kBf16>
__global__ void __launch_bounds__(256) nf4_quantize_kernel(const void* __restrict__ Wv, uint64_t n_vec4,
                                                           uint16_t* __restrict__ codes,
                                                           float* __restrict__ absmax, Nf4Table tab,
                                                           Nf4Buckets bk) {
  __shared__ float2 lut[33];
  if (kBuckets) {
    if (threadIdx.x < 33) lut[threadIdx.x] = make_float2(bk.thr[threadIdx.x], __uint_as_float(bk.base[threadIdx.x]));
    __syncthreads();
  }
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_vec4; i += stride) {
    float4 w;
    if constexpr (kBf16) {
      const uint2 b = reinterpret_cast<const uint2*>(Wv)[i];
      w = make_float4(__uint_as_float(b.x << 16), __uint_as_float(b.x & 0xFFFF0000u), __uint_as_float(b.y << 16),
                      __uint_as_float(b.y & 0xFFFF0000u));
    } else {
      w = reinterpret_cast<const float4*>(Wv)[i];
    }
    float a = fmaxf(fmaxf(fabsf(w.x), fabsf(w.y)), fmaxf(fabsf(w.z), fabsf(w.w)));
    a = fmaxf(a, __shfl_xor(a, 1));
    a = fmaxf(a, __shfl_xor(a, 2));
    a = fmaxf(a, __shfl_xor(a, 4));
    a = fmaxf(a, __shfl_xor(a, 8));
    uint32_t packed;
    if (a > 0.0f) {
      uint32_t c[4];
      const float x[4] = {w.x / a, w.y / a, w.z / a, w.w / a};
#pragma unroll
      for (int e = 0; e < 4; ++e) c[e] = kBuckets ? nf4_code_bucket(x[e], lut) : nf4_code(x[e], tab);
      packed = c[0] | (c[1] << 4) | (c[2] << 8) | (c[3] << 12);
    } else {
      packed = 0x7777u;  // the zero level
    }
    codes[i] = (uint16_t)packed;
    if ((threadIdx.x & 15) == 0) absmax[i >> 4] = a;
  }
}

// ------------------------------------------------------------------ double quant

// Zero the global mean buckets (a fill kernel, so the pass stays capturable).
__global__ void dq_zero_kernel(unsigned long long* buckets) {
  buckets[threadIdx.x] = 0ull;
}

__device__ __forceinline__ unsigned long long wave_sum_u64(unsigned long long v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// Exact per-exponent mantissa sums.  A wave handles 64 constants at a time:
// it repeatedly takes the exponent of the first pending lane, sums the
// mantissas of all lanes with that exponent and adds the sum to an LDS bucket,
// so there is one LDS atomic per distinct exponent per wave (a handful).
__global__ void __launch_bounds__(256) dq_bucket_kernel(const float* __restrict__ absmax, uint64_t n,
                                                        unsigned long long* __restrict__ buckets) {
  __shared__ unsigned long long lb[kMeanBuckets];
  lb[threadIdx.x] = 0ull;
  __syncthreads();
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t wave = threadIdx.x >> 6;
  const uint64_t stride = (uint64_t)gridDim.x * 256;
  for (uint64_t base = (uint64_t)blockIdx.x * 256 + wave * 64; base < n; base += stride) {
    const uint64_t i = base + lane;
    const bool valid = i < n;
    const uint32_t bits = valid ? __float_as_uint(absmax[i]) : 0u;
    const uint32_t e = (bits >> 23) & 0xFFu;
    const uint32_t b = e ? e : 1u;
    const unsigned long long m = (bits & 0x7FFFFFu) | (e ? 0x800000u : 0u);
    bool pending = valid && m != 0ull;
    while (true) {
      const unsigned long long mask = __ballot(pending);
      if (mask == 0ull) break;
      const int leader = __builtin_ctzll(mask);
      const uint32_t eb = __shfl(b, leader);
      const bool mine = pending && b == eb;
      const unsigned long long s = wave_sum_u64(mine ? m : 0ull);
      if (lane == 0) atomicAdd(&lb[eb], s);
      pending = pending && !mine;
    }
  }
  __syncthreads();
  const unsigned long long v = lb[threadIdx.x];
  if (v) atomicAdd(&buckets[threadIdx.x], v);
}

// The buckets come into LDS with one load per thread and a mask of the
// nonzero ones (the constants of a tensor span a few exponents), so the one
// thread that forms the exact sum touches only those: walking all 254 from
// global memory, each load waited on before the next, took 25-30 us.
__global__ void __launch_bounds__(kMeanBuckets) dq_mean_kernel(const unsigned long long* __restrict__ buckets,
                                                               uint64_t n, float* __restrict__ mean) {
  __shared__ unsigned long long lb[kMeanBuckets];
  __shared__ unsigned long long nz[kMeanBuckets / 64];
  const unsigned long long v = buckets[threadIdx.x];
  lb[threadIdx.x] = v;
  const unsigned long long m = __ballot(v != 0ull);
  if ((threadIdx.x & 63) == 0) nz[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t S[detail::kLimbs];
    for (int i = 0; i < detail::kLimbs; ++i) S[i] = 0;
    for (int w = 0; w < kMeanBuckets / 64; ++w) {
      for (unsigned long long bits = nz[w]; bits; bits &= bits - 1ull) {
        const int b = 64 * w + __builtin_ctzll(bits);
        if (b >= 1 && b < 255) detail::add_shifted(S, lb[b], b - 1);
      }
    }
    mean[0] = __uint_as_float(mean_from_sum(S, n));
  }
}

// One workgroup per run of 256 constants: centre on the mean, find the run's
// largest magnitude, scale to +-448 and round to E4M3.
__global__ void __launch_bounds__(256) dq_encode_kernel(const float* __restrict__ absmax, uint64_t n,
                                                        const float* __restrict__ mean,
                                                        uint8_t* __restrict__ c2,
                                                        float* __restrict__ c1) {
  __shared__ float wmax[4];
  const uint64_t i = (uint64_t)blockIdx.x * kDqBlock + threadIdx.x;
  const bool valid = i < n;
  const float mu = mean[0];
  const float x = valid ? __fsub_rn(absmax[i], mu) : 0.0f;
  float m = fabsf(x);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  const float amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const float scale = amax / 448.0f;
  uint32_t code = 0u;
  if (scale > 0.0f) code = f32_to_e4m3(x / scale);
  if (valid) c2[i] = (uint8_t)code;
  if (threadIdx.x == 0) c1[blockIdx.x] = scale;
}

// ------------------------------------------------------------------ dequant
//
// One thread per 16 bytes of codes (32 weights, half a block); the level table
// sits in LDS (16 banks, no conflicts) and the output leaves as four 16-byte
// stores.
__global__ void __launch_bounds__(256) nf4_dequant_kernel(const uint4* __restrict__ codes, uint64_t n_units,
                                                          const uint8_t* __restrict__ c2,
                                                          const float* __restrict__ c1,
                                                          const float* __restrict__ mean,
                                                          uint4* __restrict__ out, Nf4Table tab) {
  __shared__ float lut[16];
  if (threadIdx.x < 16) lut[threadIdx.x] = tab.level[threadIdx.x];
  __syncthreads();
  const float mu = mean[0];
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t u = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; u < n_units; u += stride) {
    const uint64_t blk = u >> 1;
    const float chat = dequant_constant(c2[blk], c1[blk >> 8], mu);
    const uint4 q = codes[u];
    const uint32_t words[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int wi = 0; wi < 4; ++wi) {
      const uint32_t w = words[wi];
      uint4 o;
      uint32_t* op = reinterpret_cast<uint32_t*>(&o);
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const float lo = __fmul_rn(lut[(w >> (8 * p)) & 15u], chat);
        const float hi = __fmul_rn(lut[(w >> (8 * p + 4)) & 15u], chat);
        op[p] = pack_bf16x2(lo, hi);
      }
      out[u * 4 + wi] = o;
    }
  }
}

// ------------------------------------------------------------------ merge
//
// W' = bf16( W_deq + s B A ) for the whole weight, in fp64: per output, the
// products B[n][j] A[j][k] (exact: two bf16 numbers) summed over j in
// ascending order by fused multiply-adds (one rounding per addition), times
// s (one rounding), plus W_deq (one rounding), then rounded to bf16 once.
// Bound by the fp64 multiply-adds (r per weight).  A workgroup takes 64
// columns and 256 rows (two chunks of 128); thread (row group, column group)
// holds 4 rows x 8 columns of sums.  A's 64 columns and the chunk's B rows sit
// in LDS as fp32 (exact for bf16), sized by r (dynamic LDS: 49 KB at r = 64,
// three workgroups per CU); B rows are padded to r + 1 so that the row groups
// of one j spread over the banks.
constexpr int kMgCols = 64, kMgRows = 128, kMgChunks = 2, kMgMaxR = 128;

// fp64 -> bf16, rounded to nearest even in effect: the fp64 value is first
// rounded to fp32 by round-to-odd (truncate, then set the last bit if
// anything was dropped), which keeps enough information for the second
// rounding (24 >= 8 + 2 bits) to give the same result as one rounding.
__device__ __forceinline__ uint32_t f64_to_bf16(double u) {
  const float f = __double2float_rn(u);
  uint32_t b = __float_as_uint(f);
  const double back = (double)f;
  if (back != u) {
    if (fabs(back) > fabs(u)) b -= 1u;   // one fp32 step toward zero (|f| > 0 here)
    b |= 1u;
  }
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

__global__ void __launch_bounds__(256) nf4_merge_kernel(const uint8_t* __restrict__ codes,
                                                        const uint8_t* __restrict__ c2,
                                                        const float* __restrict__ c1,
                                                        const float* __restrict__ mean, int64_t N, int64_t K,
                                                        const uint16_t* __restrict__ A,
                                                        const uint16_t* __restrict__ B, int r, float s,
                                                        uint16_t* __restrict__ out, Nf4Table tab) {
  __shared__ float lut[16];
  // sized by r (dynamic), so that at the common ranks several workgroups
  // share a CU: A[j][k0 ..] (r x 64), then B[n][j] of the chunk (128 x (r + 1))
  extern __shared__ __attribute__((aligned(16))) float mg_smem[];
  const int pitch = r + 1;
  float* at = mg_smem;
  float* bt = mg_smem + r * kMgCols;
  const int64_t k0 = (int64_t)blockIdx.x * kMgCols;
  const int64_t nbase = (int64_t)blockIdx.y * (kMgRows * kMgChunks);
  if (threadIdx.x < 16) lut[threadIdx.x] = tab.level[threadIdx.x];
  for (int i = threadIdx.x; i < r * kMgCols; i += 256)
    at[i] = __uint_as_float((uint32_t)A[(int64_t)(i / kMgCols) * K + k0 + (i % kMgCols)] << 16);
  const float mu = mean[0];
  const double s64 = (double)s;
  const int cg = threadIdx.x & 7, rg = threadIdx.x >> 3;
  const int64_t k = k0 + 8 * cg;
  for (int chunk = 0; chunk < kMgChunks; ++chunk) {
    const int64_t n0 = nbase + (int64_t)chunk * kMgRows;
    if (n0 >= N) break;
    __syncthreads();   // (A and the level table; the previous chunk's B rows are no longer read)
    for (int i = threadIdx.x; i < kMgRows * r; i += 256) {
      const int row = i / r, j = i - row * r;
      bt[row * pitch + j] = n0 + row < N ? __uint_as_float((uint32_t)B[(n0 + row) * r + j] << 16) : 0.f;
    }
    __syncthreads();
    double acc[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[i][e] = 0.0;
    for (int j = 0; j < r; ++j) {
      const float4 a0 = *reinterpret_cast<const float4*>(&at[j * kMgCols + 8 * cg]);
      const float4 a1 = *reinterpret_cast<const float4*>(&at[j * kMgCols + 8 * cg + 4]);
      const double a[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const double b = (double)bt[(4 * rg + i) * pitch + j];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[i][e] = __fma_rn(b, a[e], acc[i][e]);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t n = n0 + 4 * rg + i;
      if (n >= N) continue;
      const uint32_t word = *reinterpret_cast<const uint32_t*>(codes + n * (K / 2) + k / 2);
      const int64_t bi = n * (K / 64) + k / 64;
      const float chat = dequant_constant(c2[bi], c1[bi >> 8], mu);
      uint32_t o[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        uint32_t h[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const uint32_t code = (word >> (4 * (e + q))) & 15u;
          const uint32_t wb = pack_bf16x2(__fmul_rn(lut[code], chat), 0.f) & 0xFFFFu;   // W_deq
          const double w = (double)__uint_as_float(wb << 16);
          h[q] = f64_to_bf16(__dadd_rn(w, __dmul_rn(s64, acc[i][e + q])));
        }
        o[e / 2] = h[0] | (h[1] << 16);
      }
      *reinterpret_cast<uint4*>(out + n * K + k) = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
}

unsigned grid_for(uint64_t work_items, unsigned per_block, unsigned cap) {
  uint64_t g = (work_items + per_block - 1) / per_block;
  if (g > cap) g = cap;
  return g ? (unsigned)g : 1u;
}

}  // namespace

hipError_t launch_nf4_quantize(const float* W, int64_t N, int64_t K, int table, uint8_t* codes, float* absmax,
                               hipStream_t s) {
  const uint64_t n_vec4 = (uint64_t)N * (uint64_t)K / 4;
  const Nf4Buckets& bk = code_buckets(table);
  hipLaunchKernelGGL((bk.ok ? nf4_quantize_kernel<true, false> : nf4_quantize_kernel<false, false>),
                     dim3(grid_for(n_vec4, 256, 65536)), dim3(256), 0, s, static_cast<const void*>(W), n_vec4,
                     reinterpret_cast<uint16_t*>(codes), absmax, code_table(table), bk);
  return hipGetLastError();
}

hipError_t launch_nf4_quantize_bf16(const uint16_t* W, int64_t N, int64_t K, int table, uint8_t* codes,
                                    float* absmax, hipStream_t s) {
  const uint64_t n_vec4 = (uint64_t)N * (uint64_t)K / 4;
  const Nf4Buckets& bk = code_buckets(table);
  hipLaunchKernelGGL((bk.ok ? nf4_quantize_kernel<true, true> : nf4_quantize_kernel<false, true>),
                     dim3(grid_for(n_vec4, 256, 65536)), dim3(256), 0, s, static_cast<const void*>(W), n_vec4,
                     reinterpret_cast<uint16_t*>(codes), absmax, code_table(table), bk);
  return hipGetLastError();
}

size_t double_quant_workspace_bytes() { return kMeanBuckets * sizeof(unsigned long long); }

hipError_t launch_double_quant(const float* absmax, int64_t n, uint8_t* c2, float* c1, float* mean,
                               void* workspace, hipStream_t s) {
  auto* buckets = reinterpret_cast<unsigned long long*>(workspace);
  hipLaunchKernelGGL(dq_zero_kernel, dim3(1), dim3(kMeanBuckets), 0, s, buckets);
  hipLaunchKernelGGL(dq_bucket_kernel, dim3(grid_for((uint64_t)n, 256 * 8, 2048)), dim3(256), 0, s,
                     absmax, (uint64_t)n, buckets);
  hipLaunchKernelGGL(dq_mean_kernel, dim3(1), dim3(kMeanBuckets), 0, s, buckets, (uint64_t)n, mean);
  const uint64_t nb = ((uint64_t)n + kDqBlock - 1) / kDqBlock;
  hipLaunchKernelGGL(dq_encode_kernel, dim3((unsigned)nb), dim3(256), 0, s, absmax, (uint64_t)n, mean,
                     c2, c1);
  return hipGetLastError();
}

hipError_t launch_nf4_dequant(const uint8_t* codes, const uint8_t* c2, const float* c1, const float* mean,
                              int table, int64_t N, int64_t K, uint16_t* out, hipStream_t s) {
  const uint64_t n_units = (uint64_t)N * (uint64_t)K / 32;
  hipLaunchKernelGGL(nf4_dequant_kernel, dim3(grid_for(n_units, 256, 65536)), dim3(256), 0, s,
                     reinterpret_cast<const uint4*>(codes), n_units, c2, c1, mean,
                     reinterpret_cast<uint4*>(out), code_table(table));
  return hipGetLastError();
}

hipError_t launch_nf4_merge(const uint8_t* codes, const uint8_t* c2, const float* c1, const float* mean, int table,
                            int64_t N, int64_t K, const uint16_t* A, const uint16_t* B, int64_t r, float s, uint16_t* out,
                            hipStream_t st) {
  const dim3 grid((unsigned)(K / kMgCols), (unsigned)((N + kMgRows * kMgChunks - 1) / (kMgRows * kMgChunks)));
  const size_t lds = (size_t)(r * kMgCols + kMgRows * (r + 1)) * sizeof(float);
  // the limit is raised once per device, for r = kMgMaxR
  const size_t max_lds = (size_t)(kMgMaxR * kMgCols + kMgRows * (kMgMaxR + 1)) * sizeof(float);
  const hipError_t e = ensure_lds_limit(reinterpret_cast<const void*>(nf4_merge_kernel), max_lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(nf4_merge_kernel, grid, dim3(256), lds, st, codes, c2, c1, mean, N, K, A, B, (int)r, s, out,
                     code_table(table));
  return hipGetLastError();
}

}  // namespace qlora
