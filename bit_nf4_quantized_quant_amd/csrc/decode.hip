// Fused QLoRA forward for decode-sized batches (M <= 16), gfx950.
//
// Y = bf16( X W_deq^T + s (X A^T) B^T )   (itwiki "QLoRA", section on the
// computation; minnong511 "quantization", y = W x + (alpha/r) B A x).
//
// At M <= 16 the layer is bound by HBM bandwidth on the 4-bit weight.  The
// pages describe the slow path as a separate dequantization kernel whose bf16
// output makes a round trip through memory before the matrix product
// (irregular6612 "QLoRA - Efficient Finetuning of Quantized LLMs", the
// inference-speed discussion); here the packed codes are streamed once and
// expanded in registers straight into bf16 matrix-core operands.
//
// One launch does everything:
//   * Workgroups take tile tickets from an atomic counter in the workspace.
//     The first tickets are "LoRA-down" tiles: 16 rows of A times a K slice,
//     giving partial sums of H = X A^T.  The last of them to finish adds the
//     partials up into H.
//   * The remaining tickets are weight tiles: 16 output rows, all of K, split
//     over the 8 waves of the workgroup.  Each 64-element NF4 block is one
//     scaling unit: the levels go into bf16 16x16x32 MFMAs as a hi + lo pair
//     (exact to ~2^-17), and the block's fp32 constant c_hat scales the block
//     partial product in fp32 afterwards.
//   * A weight tile then waits (bounded) until H is complete, adds s H B^T in
//     fp32 and stores bf16 Y.
//   Tickets make the wait safe: a workgroup holding a weight ticket knows that
//   every LoRA-down ticket was taken by a workgroup that is already running,
//   and those never wait on anything.  The last workgroup to finish resets the
//   counters, so the workspace is ready for the next call.
#include "common.h"
#include "launch.h"

namespace qlora {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kRows = 16;         // output rows per weight tile
constexpr int kLutCopies = 16;    // pair table replicated per lane%16 (no LDS bank conflicts)
constexpr int kHSplit = 8;        // K slices per LoRA-down row group
constexpr unsigned kSpinLimit = 1u << 24;

// Workspace layout (all offsets in bytes)
constexpr size_t kCtrBytes = 256;
//   ctr[0] ticket, ctr[1] LoRA-down tiles done, ctr[2] H published,
//   ctr[3] workgroups finished, ctr[4] wait timed out (diagnostic)

struct DecodeParams {
  const uint16_t* X;
  int M;
  int N;
  int K;
  int r;
  const uint8_t* codes;
  const uint8_t* c2;
  const float* c1;
  const float* mean;
  const uint16_t* A;
  const uint16_t* B;
  float scale;
  uint16_t* Y;
  float* H;        // final H [M, r]
  float* Hpart;    // [kHSplit][M][r16] partial sums (r16 = r rounded up to 16)
  unsigned* ctr;
  int n_htiles;
  int n_wtiles;
  Nf4HiLo hilo;
};

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ u32x4 load16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// X operand: lane (m = lane & 15) supplies 8 consecutive k; rows past M are 0.
__device__ __forceinline__ u32x4 load_x8(const DecodeParams& p, int m, int k) {
  if (m < p.M) return load16(p.X + (size_t)m * p.K + k);
  return u32x4{0u, 0u, 0u, 0u};
}

// ---------------------------------------------------------------- LoRA-down tile
// rows j0..j0+15 of A, K slice ks; wave w covers every 8th 32-wide k step.
__device__ void lora_down_tile(const DecodeParams& p, int tile, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rg = tile / kHSplit, ks = tile % kHSplit;
  const int j0 = rg * kRows;
  const int jl = lane & 15, g = lane >> 4;
  const int steps = p.K / 32;
  const int per = (steps + kHSplit - 1) / kHSplit;
  const int s_beg = ks * per, s_end = min(steps, s_beg + per);
  const int jrow = min(j0 + jl, p.r - 1);
  const uint16_t* arow = p.A + (size_t)jrow * p.K;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = s_beg + wave; s < s_end; s += kWaves) {
    const int k = s * 32 + 8 * g;
    const u32x4 av = load16(arow + k);
    const u32x4 xv = load_x8(p, jl, k);
    acc = mfma16(as_bf16x8(xv), as_bf16x8(av), acc);
  }
  // acc[v] = partial H[m = 4g + v][j0 + jl]; reduce over the 8 waves
#pragma unroll
  for (int v = 0; v < 4; ++v) red[wave * 256 + (4 * g + v) * 16 + jl] = acc[v];
  __syncthreads();
  if (threadIdx.x < 256) {
    const int m = threadIdx.x >> 4, jj = threadIdx.x & 15;
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) sum += red[w * 256 + threadIdx.x];
    const int r16 = (p.r + 15) & ~15;
    if (m < p.M) p.Hpart[((size_t)ks * p.M + m) * r16 + j0 + jj] = sum;
  }
}

// ---------------------------------------------------------------- weight tile
__device__ void weight_tile(const DecodeParams& p, int tile, const uint2* lut, float* red,
                            float* hs) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n0 = tile * kRows;
  const int nl = lane & 15, g = lane >> 4;
  const int row = min(n0 + nl, p.N - 1);
  const bool row_ok = n0 + nl < p.N;
  const int nblk = p.K / 64;
  const uint8_t* crow = p.codes + (size_t)row * (p.K / 2);
  const size_t blk_row = (size_t)row * nblk;
  const float mu = *p.mean;
  const uint32_t cb = (uint32_t)(lane & 15) * 8u;  // this lane's table copy (bytes)
  const char* lutb = reinterpret_cast<const char*>(lut);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};

  for (int b = wave; b < nblk; b += kWaves) {
    // this lane: row n0+nl, elements 64b + 16g .. +16 (8 code bytes)
    const u32x2 cw = *reinterpret_cast<const u32x2*>(crow + 32 * b + 8 * g);
    const size_t bi = blk_row + b;
    const float chat = row_ok ? dequant_constant(p.c2[bi], p.c1[bi >> 8], mu) : 0.0f;
    const int kx = 64 * b + 16 * g;
    const u32x4 x0 = load_x8(p, nl, kx);
    const u32x4 x1 = load_x8(p, nl, kx + 8);
    f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t w = cw[h];
      u32x4 whi, wlo;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t byte = (w >> (8 * q)) & 0xFFu;
        const uint2 e = *reinterpret_cast<const uint2*>(lutb + ((byte << 7) | cb));
        whi[q] = e.x;
        wlo[q] = e.y;
      }
      const bf16x8 xa = as_bf16x8(h ? x1 : x0);
      t = mfma16(xa, as_bf16x8(whi), t);
      t = mfma16(xa, as_bf16x8(wlo), t);
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[v] = __builtin_fmaf(chat, t[v], acc[v]);
  }
  // acc[v] = partial Y0[m = 4g + v][n0 + nl]
#pragma unroll
  for (int v = 0; v < 4; ++v) red[wave * 256 + (4 * g + v) * 16 + nl] = acc[v];

  // wait for H (published by the last LoRA-down tile), then stage it in LDS
  if (threadIdx.x == 0) {
    unsigned spins = 0;
    while (__hip_atomic_load(&p.ctr[2], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u) {
      __builtin_amdgcn_s_sleep(2);
      if (++spins > kSpinLimit) {
        atomicExch(&p.ctr[4], 1u);
        break;
      }
    }
    __threadfence();
  }
  __syncthreads();
  for (int i = threadIdx.x; i < p.M * p.r; i += kThreads)
    hs[i] = __hip_atomic_load(&p.H[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();

  if (threadIdx.x < 256) {
    const int m = threadIdx.x >> 4, nn = threadIdx.x & 15;
    float y = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) y += red[w * 256 + threadIdx.x];
    const int n = n0 + nn;
    if (m < p.M && n < p.N) {
      const uint16_t* brow = p.B + (size_t)n * p.r;
      const float* hrow = hs + m * p.r;
      float lora = 0.f;
      for (int j = 0; j < p.r; ++j) lora = __builtin_fmaf(hrow[j], __uint_as_float((uint32_t)brow[j] << 16), lora);
      y = __builtin_fmaf(p.scale, lora, y);
      p.Y[(size_t)m * p.N + n] = (uint16_t)(pack_bf16x2(y, 0.f) & 0xFFFFu);
    }
  }
}

__global__ void __launch_bounds__(kThreads) qlora_decode_kernel(DecodeParams p) {
  __shared__ uint2 lut[256 * kLutCopies];       // 32 KiB
  __shared__ float red[kWaves * 256];           // 8 KiB
  __shared__ float hs[16 * 128];                // 8 KiB: H rows for the epilogue
  __shared__ int ticket;
  if (threadIdx.x == 0) ticket = (int)atomicAdd(&p.ctr[0], 1u);
  __syncthreads();
  const int tile = ticket;

  if (tile < p.n_htiles) {
    lora_down_tile(p, tile, red);
    __syncthreads();
    if (threadIdx.x == 0) {
      __threadfence();
      const unsigned done = atomicAdd(&p.ctr[1], 1u);
      ticket = (done == (unsigned)p.n_htiles - 1u) ? 1 : 0;  // last LoRA-down tile?
    }
    __syncthreads();
    if (ticket) {
      __threadfence();
      const int r16 = (p.r + 15) & ~15;
      for (int i = threadIdx.x; i < p.M * p.r; i += kThreads) {
        const int m = i / p.r, j = i % p.r;
        float s = 0.f;
        for (int ks = 0; ks < kHSplit; ++ks)
          s += __hip_atomic_load(&p.Hpart[((size_t)ks * p.M + m) * r16 + j], __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
        p.H[i] = s;
      }
      __syncthreads();
      if (threadIdx.x == 0) {
        __threadfence();
        atomicExch(&p.ctr[2], 1u);
      }
    }
  } else {
    // pair table: entry for code byte e holds the hi and lo bf16 pairs of
    // (level[e & 15], level[e >> 4]), one copy per lane%16
    for (int i = threadIdx.x; i < 256 * kLutCopies; i += kThreads) {
      const int e = i >> 4;
      const uint32_t w0 = p.hilo.word[e & 15], w1 = p.hilo.word[e >> 4];
      lut[i] = make_uint2((w0 & 0xFFFFu) | (w1 << 16), (w0 >> 16) | (w1 & 0xFFFF0000u));
    }
    __syncthreads();
    weight_tile(p, tile - p.n_htiles, lut, red, hs);
  }

  // the last workgroup out resets the counters for the next call
  __syncthreads();
  if (threadIdx.x == 0) {
    __threadfence();
    const unsigned fin = atomicAdd(&p.ctr[3], 1u);
    if (fin == gridDim.x - 1u) {
      p.ctr[0] = 0u;
      p.ctr[1] = 0u;
      p.ctr[2] = 0u;
      p.ctr[3] = 0u;
      __threadfence();
    }
  }
}

}  // namespace

size_t decode_workspace_bytes(int64_t M, int64_t r) {
  const int64_t r16 = (r + 15) & ~15;
  return kCtrBytes + (size_t)(kHSplit * M * r16 + M * r) * sizeof(float);
}

hipError_t launch_decode_fwd(const FwdArgs& a, hipStream_t s) {
  DecodeParams p;
  p.X = a.X;
  p.M = (int)a.M;
  p.N = (int)a.N;
  p.K = (int)a.K;
  p.r = (int)a.r;
  p.codes = a.w.codes;
  p.c2 = a.w.c2;
  p.c1 = a.w.c1;
  p.mean = a.w.mean;
  p.A = a.A;
  p.B = a.B;
  p.scale = a.scale;
  p.Y = a.Y;
  char* ws = reinterpret_cast<char*>(a.workspace);
  p.ctr = reinterpret_cast<unsigned*>(ws);
  const int64_t r16 = (a.r + 15) & ~15;
  p.Hpart = reinterpret_cast<float*>(ws + kCtrBytes);
  p.H = a.H ? a.H : p.Hpart + kHSplit * a.M * r16;
  p.n_htiles = (int)(r16 / kRows) * kHSplit;
  p.n_wtiles = (int)((a.N + kRows - 1) / kRows);
  p.hilo = nf4_hilo();
  hipLaunchKernelGGL(qlora_decode_kernel, dim3(p.n_htiles + p.n_wtiles), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace qlora
