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
//   * Workgroups 0 .. n_htiles-1 are "LoRA-down" tiles: 16 rows of A times a
//     quarter of K, giving partial sums of H = X A^T.  They never wait.
//   * The remaining workgroups are weight tiles: 16 output rows, all of K,
//     split over the 8 waves of the workgroup.  Each 64-element NF4 block is
//     one scaling unit: the levels enter bf16 16x16x32 MFMAs as a hi + lo pair
//     (together exact to ~2^-17) and the block's fp32 constant c_hat scales
//     the block's partial product in fp32 afterwards.  Loads use buffer
//     instructions with immediate offsets; rows past N read as zero.
//   * A weight tile then waits (bounded spin) until the LoRA-down partials of
//     this launch are published, sums them into H, adds s H B^T in fp32 and
//     stores bf16 Y.  Workgroups are dispatched in index order, so the
//     LoRA-down tiles are running or done before any weight tile waits.
//
// Launch epochs instead of counter resets: every launch adds exactly 2^20 to
// each counter it uses, however many workgroups share the counter.  A weight
// tile's own counter update returns (epoch << 20) + something < 2^20, which
// names the epoch; the partials of this launch are complete once the
// LoRA-down counter reaches (epoch + 1) << 20.  Weight tiles spread their
// updates over 8 counters so no address sees more than ~1/8 of them.  The
// counter updates are issued at the start and their results are only needed
// at the wait, so their latency hides behind the weight stream.
#include "common.h"
#include "launch.h"

namespace qlora {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kRows = 16;          // output rows per weight tile
constexpr int kLutCopies = 16;     // pair table replicated per lane%16
constexpr int kHSplit = 4;         // K slices per LoRA-down row group
constexpr int kSlots = 8;          // weight-tile epoch counters
constexpr uint64_t kEpoch = uint64_t(1) << 20;
constexpr unsigned kSpinLimit = 1u << 24;
constexpr int kXLdsBytes = 16384;  // X staged in LDS when M*K*2 fits

// Workspace layout (bytes): [0] LoRA-down counter (u64), [128*(1+s)] weight
// counter s (u64), [128*9] timeout flag (u32), [kHpartOff..] partial sums.
constexpr size_t kHpartOff = 2048;

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
  float* H;        // H [M, r] for the caller, or null
  float* Hpart;    // [kHSplit][M][r16] partial sums (r16 = r rounded up to 16)
  char* ws;
  int n_htiles;
  int n_wtiles;
  Nf4HiLo hilo;
};

typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }

// Cross-workgroup data (H partials, counters) moves only through relaxed
// agent-scope atomics, which are coherent across the XCDs' separate L2 caches
// on their own.  Ordering comes from waiting for this thread's stores to
// complete (s_waitcnt 0) before a barrier and the counter update, so no L2
// write-back/invalidate fence is ever issued.
__device__ __forceinline__ void st_shared_f32(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_shared_f32(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_ctr(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t add_ctr(uint64_t* p, uint64_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_stores() { __builtin_amdgcn_s_waitcnt(0); }

// i-th of n equal integer shares of 2^20 (the shares add up to exactly 2^20)
__device__ __forceinline__ uint64_t epoch_share(uint32_t i, uint32_t n) {
  return kEpoch / n + ((i < kEpoch % n) ? 1u : 0u);
}

// ---------------------------------------------------------------- LoRA-down tile
// Rows j0..j0+15 of A over a quarter of K; each wave takes a contiguous run of
// 32-wide steps and issues the loads of 8 steps at a time.  MFMA rows past M
// carry copies of row M-1; their outputs are discarded.
constexpr int kHBatch = 8;

__device__ void lora_down_tile(const DecodeParams& p, int tile, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rg = tile / kHSplit, ks = tile % kHSplit;
  const int j0 = rg * kRows;
  const int jl = lane & 15, g = lane >> 4;
  const int steps = p.K / 32;
  const int per_split = (steps + kHSplit - 1) / kHSplit;
  const int s_lo = ks * per_split, s_hi = min(steps, s_lo + per_split);
  const int per_wave = (s_hi - s_lo + kWaves - 1) / kWaves;
  const int s_beg = s_lo + wave * per_wave, s_end = min(s_hi, s_beg + per_wave);
  const rsrc_t ra = make_rsrc(p.A, (uint32_t)p.r * p.K * 2);
  const rsrc_t rx = make_rsrc(p.X, (uint32_t)p.M * p.K * 2);
  const uint32_t a_off = ((uint32_t)(j0 + jl) * p.K + 8 * g) * 2;   // rows >= r read as 0
  const uint32_t x_off = ((uint32_t)min(jl, p.M - 1) * p.K + 8 * g) * 2;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = s_beg; s0 < s_end; s0 += kHBatch) {
    u32x4 av[kHBatch], xv[kHBatch];
#pragma unroll
    for (int i = 0; i < kHBatch; ++i) {
      const uint32_t k2 = (uint32_t)min(s0 + i, s_end - 1) * 64;   // 32 elements * 2 bytes
      av[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, a_off + k2, 0, 0));
      xv[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, x_off + k2, 0, 0));
    }
#pragma unroll
    for (int i = 0; i < kHBatch; ++i)
      if (s0 + i < s_end) acc = mfma16(as_bf16x8(xv[i]), as_bf16x8(av[i]), acc);
  }
  // acc[v] = partial H[m = 4g + v][j0 + jl]; reduce over the waves
#pragma unroll
  for (int v = 0; v < 4; ++v) red[wave * 256 + (4 * g + v) * 16 + jl] = acc[v];
  __syncthreads();
  if (threadIdx.x < 256) {
    const int m = threadIdx.x >> 4, jj = threadIdx.x & 15;
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) sum += red[w * 256 + threadIdx.x];
    const int r16 = (p.r + 15) & ~15;
    if (m < p.M) st_shared_f32(&p.Hpart[((size_t)ks * p.M + m) * r16 + j0 + jj], sum);
  }
}

// ---------------------------------------------------------------- weight tile
// Loads of kBatch consecutive blocks are issued together and the next batch is
// in flight while the current one is multiplied.
constexpr int kBatch = 4;

template <bool kXLds>
struct BlockLoads {
  u32x2 cw[kBatch];  // 8 code bytes per block (this lane's 16 elements)
  uint32_t c2[kBatch];
  float c1[kBatch];
  u32x4 x0[kBatch], x1[kBatch];  // only when X is read from global memory
};

struct WeightCtx {
  rsrc_t rc, r2, r1, rx;
  uint32_t code_off;   // byte offset of this lane's codes in block 0
  uint32_t blk0;       // block index of (row, block 0)
  uint32_t x_off;      // byte offset of this lane's X row at k = 16g
  const char* xs;      // X in LDS (bytes) or null
  int b_end;
};

template <bool kXLds>
__device__ __forceinline__ void load_blocks(const WeightCtx& c, BlockLoads<kXLds>& L, int b0) {
#pragma unroll
  for (int i = 0; i < kBatch; ++i) {
    const uint32_t b = (uint32_t)min(b0 + i, c.b_end - 1);
    L.cw[i] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(c.rc, c.code_off + 32 * b, 0, 0));
    L.c2[i] = __builtin_amdgcn_raw_buffer_load_b8(c.r2, c.blk0 + b, 0, 0);
    L.c1[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(c.r1, ((c.blk0 + b) >> 8) * 4, 0, 0));
    if (!kXLds) {
      L.x0[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(c.rx, c.x_off + 128 * b, 0, 0));
      L.x1[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(c.rx, c.x_off + 128 * b + 16, 0, 0));
    }
  }
}

template <bool kXLds>
__device__ __forceinline__ void mul_blocks(const WeightCtx& c, const BlockLoads<kXLds>& L, int b0, float mu,
                                           const char* lutb, uint32_t cb, f32x4& acc) {
#pragma unroll
  for (int i = 0; i < kBatch; ++i) {
    if (b0 + i >= c.b_end) break;
    const float chat = dequant_constant(L.c2[i], L.c1[i], mu);
    f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t w = L.cw[i][h];
      u32x4 whi, wlo;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t byte = (w >> (8 * q)) & 0xFFu;
        const uint2 e = *reinterpret_cast<const uint2*>(lutb + ((byte << 7) | cb));
        whi[q] = e.x;
        wlo[q] = e.y;
      }
      u32x4 xv;
      if (kXLds)
        xv = *reinterpret_cast<const u32x4*>(c.xs + c.x_off + 128 * (b0 + i) + 16 * h);
      else
        xv = h ? L.x1[i] : L.x0[i];
      const bf16x8 xa = as_bf16x8(xv);
      t = mfma16(xa, as_bf16x8(whi), t);
      t = mfma16(xa, as_bf16x8(wlo), t);
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[v] = __builtin_fmaf(chat, t[v], acc[v]);
  }
}

template <bool kXLds>
__device__ void weight_tile(const DecodeParams& p, int tile, const uint2* lut, const char* xs, float* red,
                            float* hs, float* bs, uint64_t ticket) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n0 = tile * kRows;
  const int nl = lane & 15, g = lane >> 4;
  const int nblk = p.K / 64;
  const float mu = *p.mean;
  const uint32_t cb = (uint32_t)(lane & 15) * 8u;  // this lane's table copy (bytes)
  const char* lutb = reinterpret_cast<const char*>(lut);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};

  // rows n0..n0+15 of B: issued now, parked in LDS after the weight stream
  constexpr int kBPer = 16 * 128 / kThreads;
  uint32_t bv[kBPer];
#pragma unroll
  for (int i = 0; i < kBPer; ++i) {
    const int e = threadIdx.x + i * kThreads;
    const int br = e / p.r, bc = e - br * p.r;
    bv[i] = (e < 16 * p.r && n0 + br < p.N) ? p.B[(size_t)(n0 + br) * p.r + bc] : 0u;
  }

  WeightCtx c;
  const uint32_t n_c2 = (uint32_t)p.N * nblk;
  c.rc = make_rsrc(p.codes, n_c2 * 32u);
  c.r2 = make_rsrc(p.c2, n_c2);
  c.r1 = make_rsrc(p.c1, ((n_c2 + 255u) / 256u) * 4u);
  c.rx = make_rsrc(p.X, (uint32_t)p.M * p.K * 2);
  const uint32_t row = (uint32_t)(n0 + nl);             // rows >= N read as zero codes
  c.code_off = row * (uint32_t)(p.K / 2) + 8u * g;
  c.blk0 = row * (uint32_t)nblk;
  c.x_off = ((uint32_t)min(nl, p.M - 1) * p.K + 16u * g) * 2u;
  c.xs = xs;
  const int per = (nblk + kWaves - 1) / kWaves;
  const int b_beg = wave * per;
  c.b_end = min(nblk, b_beg + per);
  if (b_beg < c.b_end) {
    BlockLoads<kXLds> La, Lb;
    load_blocks(c, La, b_beg);
    for (int b0 = b_beg; b0 < c.b_end; b0 += 2 * kBatch) {
      if (b0 + kBatch < c.b_end) load_blocks(c, Lb, b0 + kBatch);
      mul_blocks(c, La, b0, mu, lutb, cb, acc);
      if (b0 + 2 * kBatch < c.b_end) load_blocks(c, La, b0 + 2 * kBatch);
      if (b0 + kBatch < c.b_end) mul_blocks(c, Lb, b0 + kBatch, mu, lutb, cb, acc);
    }
  }
  // acc[v] = partial Y0[m = 4g + v][n0 + nl]
#pragma unroll
  for (int v = 0; v < 4; ++v) red[wave * 256 + (4 * g + v) * 16 + nl] = acc[v];
#pragma unroll
  for (int i = 0; i < kBPer; ++i) {
    const int e = threadIdx.x + i * kThreads;
    if (e < 16 * p.r) bs[e] = __uint_as_float(bv[i] << 16);
  }

  // wait until this launch's LoRA-down partials are published
  if (threadIdx.x == 0) {
    const uint64_t target = ((ticket >> 20) + 1) << 20;
    const uint64_t* hctr = reinterpret_cast<const uint64_t*>(p.ws);
    unsigned spins = 0;
    while (ld_ctr(hctr) < target) {
      __builtin_amdgcn_s_sleep(2);
      if (++spins > kSpinLimit) {
        __hip_atomic_store(reinterpret_cast<unsigned*>(p.ws + 128 * 9), 1u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
  }
  __syncthreads();
  {
    const int r16 = (p.r + 15) & ~15;
    for (int i = threadIdx.x; i < p.M * p.r; i += kThreads) {
      const int m = i / p.r, j = i - m * p.r;
      float part[kHSplit];
#pragma unroll
      for (int ks = 0; ks < kHSplit; ++ks) part[ks] = ld_shared_f32(&p.Hpart[((size_t)ks * p.M + m) * r16 + j]);
      float h = 0.f;
#pragma unroll
      for (int ks = 0; ks < kHSplit; ++ks) h += part[ks];
      hs[i] = h;
      if (tile == 0 && p.H) p.H[i] = h;
    }
  }
  __syncthreads();

  if (threadIdx.x < 256) {
    const int m = threadIdx.x >> 4, nn = threadIdx.x & 15;
    float y = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) y += red[w * 256 + threadIdx.x];
    const int n = n0 + nn;
    if (m < p.M && n < p.N) {
      const float* brow = bs + nn * p.r;
      const float* hrow = hs + m * p.r;
      float lora = 0.f;
      for (int j = 0; j < p.r; ++j) lora = __builtin_fmaf(hrow[j], brow[j], lora);
      y = __builtin_fmaf(p.scale, lora, y);
      p.Y[(size_t)m * p.N + n] = (uint16_t)(pack_bf16x2(y, 0.f) & 0xFFFFu);
    }
  }
}

// Two 512-thread workgroups per CU (4 waves per SIMD): at most 128 VGPRs.
template <bool kXLds>
__global__ void __launch_bounds__(kThreads, 4) qlora_decode_kernel(DecodeParams p) {
  __shared__ uint2 lut[256 * kLutCopies];       // 32 KiB
  __shared__ __attribute__((aligned(16))) char xs[kXLds ? kXLdsBytes : 16];
  __shared__ float red[kWaves * 256];           // 8 KiB
  __shared__ float hs[16 * 128];                // 8 KiB: H rows for the epilogue
  __shared__ float bs[16 * 128];                // 8 KiB: B rows of the tile
  __shared__ uint32_t words[16];
  const int tile = (int)blockIdx.x;

  if (tile < p.n_htiles) {
    lora_down_tile(p, tile, red);
    wait_stores();
    __syncthreads();
    if (threadIdx.x == 0)
      add_ctr(reinterpret_cast<uint64_t*>(p.ws), epoch_share((uint32_t)tile, (uint32_t)p.n_htiles));
    return;
  }

  // weight tile: take the epoch ticket now, use it at the wait
  const int wt = tile - p.n_htiles;
  uint64_t ticket = 0;
  if (threadIdx.x == 0) {
    const uint32_t nw = (uint32_t)p.n_wtiles;
    if (nw >= (uint32_t)kSlots) {
      const uint32_t s = (uint32_t)wt % kSlots;
      const uint32_t cnt = nw / kSlots + ((s < nw % kSlots) ? 1u : 0u);
      ticket = add_ctr(reinterpret_cast<uint64_t*>(p.ws + 128 * (1 + s)), epoch_share((uint32_t)wt / kSlots, cnt));
    } else {
      // fewer tiles than counters: this tile advances every counter it owns
      ticket = add_ctr(reinterpret_cast<uint64_t*>(p.ws + 128 * (1 + wt)), kEpoch);
      for (uint32_t s = (uint32_t)wt + nw; s < (uint32_t)kSlots; s += nw)
        add_ctr(reinterpret_cast<uint64_t*>(p.ws + 128 * (1 + s)), kEpoch);
    }
  }

  // pair table: entry for code byte e holds the hi and lo bf16 pairs of
  // (level[e & 15], level[e >> 4]), one copy per lane%16
  if (threadIdx.x < 16) words[threadIdx.x] = p.hilo.word[threadIdx.x];
  if (kXLds) {
    const int n16 = p.M * p.K / 8;  // 16-byte chunks of X
    for (int i = threadIdx.x; i < n16; i += kThreads)
      reinterpret_cast<u32x4*>(xs)[i] = *reinterpret_cast<const u32x4*>(p.X + 8 * i);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 256 * kLutCopies; i += kThreads) {
    const int e = i >> 4;
    const uint32_t w0 = words[e & 15], w1 = words[e >> 4];
    lut[i] = make_uint2((w0 & 0xFFFFu) | (w1 << 16), (w0 >> 16) | (w1 & 0xFFFF0000u));
  }
  __syncthreads();
  weight_tile<kXLds>(p, wt, lut, xs, red, hs, bs, ticket);
}

}  // namespace

size_t decode_workspace_bytes(int64_t M, int64_t r) {
  const int64_t r16 = (r + 15) & ~15;
  return kHpartOff + (size_t)(kHSplit * M * r16) * sizeof(float);
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
  p.ws = reinterpret_cast<char*>(a.workspace);
  p.Hpart = reinterpret_cast<float*>(p.ws + kHpartOff);
  p.H = a.H;
  const int64_t r16 = (a.r + 15) & ~15;
  p.n_htiles = (int)(r16 / kRows) * kHSplit;
  p.n_wtiles = (int)((a.N + kRows - 1) / kRows);
  p.hilo = nf4_hilo();
  const dim3 grid(p.n_htiles + p.n_wtiles);
  if ((size_t)a.M * a.K * 2 <= (size_t)kXLdsBytes)
    hipLaunchKernelGGL(qlora_decode_kernel<true>, grid, dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL(qlora_decode_kernel<false>, grid, dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace qlora
