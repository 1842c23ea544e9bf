// Fused QLoRA forward for 5 <= M <= 16 (decode), gfx950: the matrix-core
// path.  (M <= 4 takes the GEMV path; the launcher dispatches.)
//
// Y = bf16( X W_deq^T + s (X A^T) B^T )   (itwiki "QLoRA", section on the
// computation; minnong511 "quantization", y = W x + (alpha/r) B A x).
//
// At these M the layer is still bound by HBM bandwidth on the 4-bit weight.
// The pages describe the slow path as a separate dequantization kernel whose
// bf16 output makes a round trip through memory before the matrix product
// (irregular6612 "QLoRA - Efficient Finetuning of Quantized LLMs", the
// inference-speed discussion); here the packed codes are streamed once and
// expanded in registers straight into bf16 matrix-core operands.
//
//   * LoRA-down tiles: 16 rows of A times a quarter of K, partial sums of
//     H = X A^T, published as tagged words.
//   * Weight tiles: 16 output rows, all of K, split over the 8 waves.  Each
//     64-element NF4 block is one scaling unit: the levels enter bf16
//     16x16x32 MFMAs as bf16(level) and the block's fp32 constant c_hat
//     scales the block's partial product in fp32 afterwards, i.e. the weight
//     used is bf16(level) * c_hat rather than bf16(level * c_hat): the same
//     size of rounding, one place earlier.  A code byte indexes the pair
//     table of bf16 levels in LDS.  Each lane loads the X values of its own
//     MFMA operands (only lanes whose X row exists), so no wave waits for
//     another before its products.
#include <type_traits>

#include "decode_common.h"

namespace qlora {
namespace dec {
namespace {

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }

// Float f of the scratch space in the unused upper halves of the pair-table
// entries (bytes 128..255 of each 256-byte entry): 32 floats per entry,
// consecutive floats on consecutive banks.  Up to 256 * 32 floats.
__device__ __forceinline__ float* spare(char* lut, int f) {
  return reinterpret_cast<float*>(lut + ((f >> 5) << 8) + 128 + ((f & 31) << 2));
}
constexpr int kRedOff = 0;              // [kWaves][256] wave partials
constexpr int kHsOff = kWaves * 256;    // [16][128] H rows
static_assert(kHsOff + 16 * 128 <= 256 * 32, "scratch floats exceed the spare table halves");

// ---------------------------------------------------------------- LoRA-down tile
// Rows j0..j0+15 of A over a quarter of K; each wave takes a contiguous run of
// 32-wide steps and issues the loads of 8 steps at a time.  MFMA rows past M
// (lanes whose X row does not exist) carry zeros; their outputs are dropped.
constexpr int kHBatch = 8;

// ticket: thread 0's LoRA-down counter update (its epoch names this launch).
__device__ void lora_down_tile(const DecodeParams& p, int tile, float* red, uint32_t* tag_lds, uint64_t ticket) {
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
  const uint32_t x_off = ((uint32_t)jl * p.K + 8 * g) * 2;
  const bool xrow = jl < p.M;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  u32x4 xv[kHBatch];
#pragma unroll
  for (int i = 0; i < kHBatch; ++i) xv[i] = u32x4{0u, 0u, 0u, 0u};
  for (int s0 = s_beg; s0 < s_end; s0 += kHBatch) {
    u32x4 av[kHBatch];
#pragma unroll
    for (int i = 0; i < kHBatch; ++i) {
      const uint32_t k2 = (uint32_t)min(s0 + i, s_end - 1) * 64;   // 32 elements * 2 bytes
      if (xrow) xv[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, x_off + k2, 0, 0));
      av[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, a_off + k2, 0, 0));
    }
#pragma unroll
    for (int i = 0; i < kHBatch; ++i)
      if (s0 + i < s_end) acc = mfma16(as_bf16x8(xv[i]), as_bf16x8(av[i]), acc);
  }
  // acc[v] = partial H[m = 4g + v][j0 + jl]; reduce over the waves
#pragma unroll
  for (int v = 0; v < 4; ++v) red[wave * 256 + (4 * g + v) * 16 + jl] = acc[v];
  if (threadIdx.x == 0) *tag_lds = (uint32_t)(ticket >> 20) + 1u;
  __syncthreads();
  if (threadIdx.x < 256) {
    const int m = threadIdx.x >> 4, jj = threadIdx.x & 15;
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) sum += red[w * 256 + threadIdx.x];
    const int r16 = (p.r + 15) & ~15;
    if (m < p.M) st_tagged(&p.Hpart[((size_t)ks * p.M + m) * r16 + j0 + jj], *tag_lds, sum);
  }
}

// ---------------------------------------------------------------- weight tile
// Lane (nl, g) = (lane % 16, lane / 16) holds, per block, 8 code bytes of row
// n0 + nl (elements 16 g .. 16 g + 15 of the block: the MFMA B operand of the
// block's two 32-wide steps) and the matching X values of batch row m = nl
// (the A operand).  Loads of kBatch consecutive blocks are issued together
// and the next batch is in flight while the current one is multiplied.
constexpr int kBatch = 4;

template <bool kC2Vec>
struct Batch {
  u32x4 x0[kBatch], x1[kBatch];  // X for the block's two steps (lanes with nl < M)
  u32x2 cw[kBatch];              // 8 code bytes per block
  // c2 of the batch's blocks: one aligned dword (rows of c2 dword aligned),
  // else one byte load each
  typename std::conditional<kC2Vec, uint32_t, uint8_t[kBatch]>::type c2;
  float c1a, c1b;                // c1 of the batch's first and last block
};

struct Ctx {
  rsrc_t rc, r2, r1, rx;
  uint32_t code_off;   // byte offset of this lane's codes in block 0
  uint32_t blk0;       // block index of (row, block 0)
  uint32_t x_off;      // byte offset of this lane's X row at k = 16 g
  uint32_t n_c2;
  int b_end;
  bool xrow;
};

// X first (used first), then codes and constants.  A batch starts at a
// multiple of 4 blocks, so that with c2_vec its c2 bytes form one aligned
// dword.  Lanes without an X row load no X and keep the zeros they hold.
template <bool kC2Vec>
__device__ __forceinline__ void load_batch(const DecodeParams& p, const Ctx& c, Batch<kC2Vec>& L, int b0) {
  if (c.xrow) {
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const uint32_t b = (uint32_t)min(b0 + i, c.b_end - 1);
      L.x0[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(c.rx, c.x_off + 128 * b, 0, 0));
      L.x1[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(c.rx, c.x_off + 128 * b + 16, 0, 0));
    }
  }
#pragma unroll
  for (int i = 0; i < kBatch; ++i) {
    const uint32_t b = (uint32_t)min(b0 + i, c.b_end - 1);
    L.cw[i] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(c.rc, c.code_off + 32 * b, 0, 0));
  }
  if constexpr (kC2Vec) {
    L.c2 = __builtin_amdgcn_raw_buffer_load_b32(c.r2, c.blk0 + (uint32_t)b0, 0, 0);
  } else {
    // plain byte loads, which widen for free, on a clamped index
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const uint32_t blk = c.blk0 + (uint32_t)min(b0 + i, c.b_end - 1);
      L.c2[i] = p.c2[blk < c.n_c2 ? blk : c.n_c2 - 1u];
    }
  }
  L.c1a = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(c.r1, ((c.blk0 + b0) >> 8) * 4, 0, 0));
  L.c1b = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(c.r1, ((c.blk0 + b0 + kBatch - 1) >> 8) * 4, 0, 0));
}

template <bool kC2Vec>
__device__ __forceinline__ void mul_batch(const Ctx& c, const Batch<kC2Vec>& L, int b0, float mu, const char* lut,
                                          uint32_t lane4, f32x4& acc) {
#pragma unroll
  for (int i = 0; i < kBatch; ++i) {
    if (b0 + i >= c.b_end) break;
    const uint32_t blk = c.blk0 + (uint32_t)(b0 + i);
    const float c1 = ((blk >> 8) == ((c.blk0 + b0) >> 8)) ? L.c1a : L.c1b;
    float chat;
    if constexpr (kC2Vec)
      chat = i == 0 ? dequant_constant_byte<0>(L.c2, c1, mu)
           : i == 1 ? dequant_constant_byte<1>(L.c2, c1, mu)
           : i == 2 ? dequant_constant_byte<2>(L.c2, c1, mu)
                    : dequant_constant_byte<3>(L.c2, c1, mu);
    else
      chat = dequant_constant(L.c2[i], c1, mu);
    f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t w = L.cw[i][h];
      u32x4 wv;
      wv[0] = *reinterpret_cast<const uint32_t*>(lut + pair_addr<0>(w, lane4));
      wv[1] = *reinterpret_cast<const uint32_t*>(lut + pair_addr<1>(w, lane4));
      wv[2] = *reinterpret_cast<const uint32_t*>(lut + pair_addr<2>(w, lane4));
      wv[3] = *reinterpret_cast<const uint32_t*>(lut + pair_addr<3>(w, lane4));
      t = mfma16(as_bf16x8(h ? L.x1[i] : L.x0[i]), as_bf16x8(wv), t);
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[v] = __builtin_fmaf(chat, t[v], acc[v]);
  }
}

// kNB: batches per wave (the launcher's exact count), or 0 for any count.
template <bool kC2Vec, int kNB>
__device__ void weight_tile(const DecodeParams& p, int tile, char* lut, uint32_t* tag_lds) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n0 = tile * kRows;
  const int nl = lane & 15, g = lane >> 4;
  const int nblk = p.K / 64;
  const float mu = load_mean(p);
  // this launch's epoch: thread 0's counter update goes out first, and its
  // reply, which comes back ahead of every later load, is used only at the
  // end (no other thread reads the variable)
  uint64_t ticket;
  if (threadIdx.x == 0) ticket = take_weight_ticket(p, tile);

  Ctx c;
  const uint32_t n_c2 = (uint32_t)p.N * nblk;
  c.rc = make_rsrc(p.codes, n_c2 * 32u);
  c.r2 = make_rsrc(p.c2, n_c2);
  c.r1 = make_rsrc(p.c1, ((n_c2 + 255u) / 256u) * 4u);
  c.rx = make_rsrc(p.X, (uint32_t)p.M * p.K * 2);
  const uint32_t row = (uint32_t)(n0 + nl);             // rows >= N read as zero codes
  c.code_off = row * (uint32_t)(p.K / 2) + 8u * g;
  c.blk0 = row * (uint32_t)nblk;
  c.x_off = ((uint32_t)nl * p.K + 16u * g) * 2u;
  c.n_c2 = n_c2;
  c.xrow = nl < p.M;
  // each wave takes a run of whole batches (multiples of 4 blocks)
  const int per = ((nblk + kWaves - 1) / kWaves + kBatch - 1) / kBatch * kBatch;
  const int b_beg = min(nblk, wave * per);
  c.b_end = min(nblk, b_beg + per);

  Batch<kC2Vec> La = {}, Lb = {};
  const uint32_t lane4 = (uint32_t)(lane & 31) * 4u;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if constexpr (kNB > 0) {
    // A known batch count: every load is issued whatever the wave's share
    // (offsets are clamped, reads past the end return zero, multiplies past
    // the share are skipped), so each wait counts exactly the loads issued
    // after the one it waits for.  Two batches in flight.
    load_batch(p, c, La, b_beg);
    if constexpr (kNB > 1) load_batch(p, c, Lb, b_beg + kBatch);
    build_pair_table<kThreads>(p, lut);   // while the loads are in flight
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kNB; ++i) {
      Batch<kC2Vec>& cur = (i & 1) ? Lb : La;
      mul_batch(c, cur, b_beg + i * kBatch, mu, lut, lane4, acc);
      if (i + 2 < kNB) load_batch(p, c, cur, b_beg + (i + 2) * kBatch);
    }
  } else {
    const bool work = b_beg < c.b_end;
    if (work) {
      load_batch(p, c, La, b_beg);
      if (b_beg + kBatch < c.b_end) load_batch(p, c, Lb, b_beg + kBatch);
    }
    build_pair_table<kThreads>(p, lut);   // while the loads are in flight
    __syncthreads();
    if (work) {
      for (int b0 = b_beg; b0 < c.b_end; b0 += 2 * kBatch) {
        if (b0 != b_beg && b0 + kBatch < c.b_end) load_batch(p, c, Lb, b0 + kBatch);
        mul_batch(c, La, b0, mu, lut, lane4, acc);
        if (b0 + 2 * kBatch < c.b_end) load_batch(p, c, La, b0 + 2 * kBatch);
        if (b0 + kBatch < c.b_end) mul_batch(c, Lb, b0 + kBatch, mu, lut, lane4, acc);
      }
    }
  }
  // Epilogue.  The LoRA term s H B^T goes through the matrix cores too: wave
  // w < ceil(r / 32) takes j = 32 w .. 32 w + 31, with B[n0 + nl][j ..] read
  // straight as the B operand and s H[m][j ..] as the A operand, split into
  // bf16 high and low parts (two products: fp32 accuracy).  Its product
  // joins the wave's partial sums, and the 8 waves' sums meet in LDS.
  // B and this thread's LoRA-down partials are read right after the stream,
  // so their replies come back during the barrier.
  const int r16 = (p.r + 15) & ~15;
  const bool lwave = wave * 32 < p.r;
  const int jb = wave * 32 + 8 * g;                  // this lane's first j
  u32x4 bop = {0u, 0u, 0u, 0u};
  if (lwave && jb < p.r) {
    const rsrc_t rb = make_rsrc(p.B, (uint32_t)p.N * p.r * 2);   // rows past N read as 0
    const uint32_t off = ((uint32_t)(n0 + nl) * p.r + jb) * 2;
    if (p.b_vec) {   // r % 8 == 0: all 8 entries exist
      bop = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rb, off, 0, 0));
    } else {
      uint16_t e[8];
#pragma unroll
      for (int q = 0; q < 8; ++q)
        e[q] = jb + q < p.r ? (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(rb, off + 2 * q, 0, 0) : (uint16_t)0;
#pragma unroll
      for (int q = 0; q < 4; ++q) bop[q] = (uint32_t)e[2 * q] | ((uint32_t)e[2 * q + 1] << 16);
    }
  }
  constexpr int kHPer = 16 * 128 / kThreads;   // up to M*r = 2048 sums per tile
  const int mr = p.M * p.r;
  uint64_t hp[kHPer][kHSplit];
#pragma unroll
  for (int u = 0; u < kHPer; ++u) {
    const int i = threadIdx.x + u * kThreads;
    if (i < mr) {
      const int m = i / p.r, j = i - m * p.r;
#pragma unroll
      for (int ks = 0; ks < kHSplit; ++ks) hp[u][ks] = ld_tagged(&p.Hpart[((size_t)ks * p.M + m) * r16 + j]);
    }
  }
  if (threadIdx.x == 0) {
    // (the empty asm keeps the use of the reply here, at the end)
    asm volatile("" : "+v"(ticket));
    *tag_lds = (uint32_t)(ticket >> 20) + 1u;
  }
  __syncthreads();

  // this launch's LoRA-down partials (tag = epoch + 1), polled until present
  // or, past the deadline, computed here
  const uint32_t tag = *tag_lds;
  uint64_t deadline = 0;   // set at the first miss
#pragma unroll
  for (int u = 0; u < kHPer; ++u) {
    const int i = threadIdx.x + u * kThreads;
    if (i < mr) {
      const int m = i / p.r, j = i - m * p.r;
      float h = 0.f;
      bool got = true;
#pragma unroll
      for (int ks = 0; ks < kHSplit; ++ks) {
        float v = 0.f;
        got = got && poll_tagged(&p.Hpart[((size_t)ks * p.M + m) * r16 + j], hp[u][ks], tag, deadline, &v);
        h += v;
      }
      if (!got) h = lane_lora_down(p.X, p.A, p.K, m, j, p.ws);
      *spare(lut, kHsOff + m * 128 + j) = h;
      if (tile == 0 && p.H) p.H[i] = h;
    }
  }
  __syncthreads();

  if (lwave) {
    // A operand: s H[m = nl][jb .. jb + 7] as bf16 hi + lo (zeros past M or r)
    u32x4 ahi = {0u, 0u, 0u, 0u}, alo = {0u, 0u, 0u, 0u};
    if (nl < p.M) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float v[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int j = jb + 2 * q + e;
          v[e] = j < p.r ? p.scale * *spare(lut, kHsOff + nl * 128 + j) : 0.f;
        }
        const uint32_t hi = pack_bf16x2(v[0], v[1]);
        ahi[q] = hi;
        alo[q] = pack_bf16x2(v[0] - bf16_lo(hi), v[1] - bf16_hi(hi));
      }
    }
    acc = mfma16(as_bf16x8(ahi), as_bf16x8(bop), acc);
    acc = mfma16(as_bf16x8(alo), as_bf16x8(bop), acc);
  }
  // acc[v] = partial Y[m = 4g + v][n0 + nl]: the 8 waves' sums meet
#pragma unroll
  for (int v = 0; v < 4; ++v) *spare(lut, kRedOff + wave * 256 + (4 * g + v) * 16 + nl) = acc[v];
  __syncthreads();
  if ((int)threadIdx.x < 16 * p.M) {
    const int o = threadIdx.x, m = o >> 4, n = n0 + (o & 15);
    float y = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) y += *spare(lut, kRedOff + w * 256 + o);
    y *= p.inv_kappa;
    if (n < p.N) p.Y[(size_t)m * p.N + n] = (uint16_t)(pack_bf16x2(y, 0.f) & 0xFFFFu);
  }
}

template <bool kC2Vec, int kNB>
__global__ void __launch_bounds__(kThreads, 2) __attribute__((amdgpu_waves_per_eu(4))) qlora_decode_kernel(DecodeParams p) {
  // pair table; its entries' upper halves hold the tile's scratch floats
  __shared__ __attribute__((aligned(16))) char lut[256 * kPairStride];   // 64 KiB
  __shared__ uint32_t tag;
  const int tile = (int)blockIdx.x;
  QLORA_FETCH_ARGS(p);
  if (tile < p.n_htiles) {
    uint64_t hticket = 0;
    if (threadIdx.x == 0) hticket = take_down_ticket(p, tile);
    lora_down_tile(p, tile, reinterpret_cast<float*>(lut), &tag, hticket);
    return;
  }
  weight_tile<kC2Vec, kNB>(p, tile - p.n_htiles, lut, &tag);
}

typedef void (*DecodeKernel)(DecodeParams);
template <bool kC2Vec>
DecodeKernel decode_kernel(int nb) {
  switch (nb) {
    case 1: return qlora_decode_kernel<kC2Vec, 1>;
    case 2: return qlora_decode_kernel<kC2Vec, 2>;
    case 3: return qlora_decode_kernel<kC2Vec, 3>;
    case 4: return qlora_decode_kernel<kC2Vec, 4>;
    case 5: return qlora_decode_kernel<kC2Vec, 5>;
    case 6: return qlora_decode_kernel<kC2Vec, 6>;
    case 7: return qlora_decode_kernel<kC2Vec, 7>;
    case 8: return qlora_decode_kernel<kC2Vec, 8>;
    default: return qlora_decode_kernel<kC2Vec, 0>;
  }
}

}  // namespace

size_t decode_workspace_bytes(int64_t M, int64_t r) {
  const int64_t r16 = (r + 15) & ~15;
  return kHpartOff + (size_t)(kHSplit * M * r16) * sizeof(uint64_t);
}

hipError_t launch_decode_fwd(const FwdArgs& a, hipStream_t s) {
  DecodeParams p = decode_params(a);
  if (a.M <= 4) return launch_gemv_fwd(p, s);
  const int64_t r16 = (a.r + 15) & ~15;
  p.n_htiles = (int)(r16 / kRows) * kHSplit;
  // batches of kBatch blocks per wave (the weight tile's split of K)
  const int nblk = (int)(a.K / 64);
  const int per = ((nblk + kWaves - 1) / kWaves + kBatch - 1) / kBatch * kBatch;
  const int nb = per / kBatch;
  const DecodeKernel k = p.c2_vec ? decode_kernel<true>(nb) : decode_kernel<false>(nb);
  const dim3 grid(p.n_htiles + p.n_wtiles);
  hipLaunchKernelGGL(k, grid, dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace dec

size_t decode_workspace_bytes(int64_t M, int64_t r) { return dec::decode_workspace_bytes(M, r); }
size_t decode_wait_counter_offset() { return (size_t)dec::kGiveupCounter; }
hipError_t launch_decode_fwd(const FwdArgs& a, hipStream_t s) { return dec::launch_decode_fwd(a, s); }

}  // namespace qlora
