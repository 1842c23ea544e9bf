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
//     one scaling unit: the levels enter bf16 16x16x32 MFMAs as bf16(level)
//     and the block's fp32 constant c_hat scales the block's partial product
//     in fp32 afterwards, i.e. the weight used is bf16(level) * c_hat rather
//     than bf16(level * c_hat): the same size of rounding, one place earlier.
//     A byte of two codes indexes a table of bf16 pairs in LDS (32 copies, one
//     per lane%32, so lookups never conflict on a bank).  Loads use buffer
//     instructions with immediate offsets; rows past N read as zero.
//   * A weight tile then polls (bounded spin) until the LoRA-down partials of
//     this launch are present, sums them into H, adds s H B^T in fp32 and
//     stores bf16 Y.  Workgroups are dispatched in index order, so the
//     LoRA-down tiles are running or done before any weight tile waits.
//
// Launch epochs: every launch adds exactly 2^20 to each of the 9 counters,
// however many workgroups share a counter, so a workgroup's own counter
// update returns (epoch << 20) + something < 2^20, which names the launch
// (the same epoch on every counter, whatever mix of shapes and ranks, with or
// without adapter, used the workspace before).
// LoRA-down tiles store each partial as one 64-bit word (epoch tag, value),
// so a partial is valid exactly when its tag is this launch's; nothing has to
// be reset or waited for on the producer side.  Weight tiles spread their
// counter updates over 8 counters, issue them first and use the result only
// at the poll, so the update latency hides behind the weight stream.
#include "common.h"
#include "launch.h"

namespace qlora {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kRows = 16;          // output rows per weight tile
constexpr int kLutCopies = 32;     // pair table replicated per lane%32
constexpr int kHSplit = 4;         // K slices per LoRA-down row group
constexpr int kSlots = 8;          // weight-tile epoch counters
constexpr uint64_t kEpoch = uint64_t(1) << 20;
constexpr unsigned kSpinLimit = 1u << 20;  // ~50 ms per polled word, a safety net only
constexpr int kXLdsBytes = 16384;  // X staged in LDS when M*K*2 fits

// Workspace layout (bytes): [128*(1+s)] weight counter s (u64, s < 8),
// [128*9] timeout flag (u32), [128*(10+s)] LoRA-down counter s (u64, s < 8),
// [kHpartOff..] tagged partial sums (u64: tag << 32 | fp32 bits).  Counters
// sit 128 bytes apart so that their atomics do not queue on one cache line.
constexpr size_t kHpartOff = 4096;

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
  uint64_t* Hpart; // [kHSplit][M][r16] tagged partial sums (r16 = r rounded up to 16)
  char* ws;
  int n_htiles;
  int n_wtiles;
  int epi_group;   // threads per output in the epilogue (power of two, <= 32)
  int c2_vec;      // rows of c2 start 4-byte aligned (K % 256 == 0): dword c2 loads
  int b_vec;       // r % 8 == 0 and B 16-byte aligned: 16-byte B loads
  uint32_t hi[16]; // bf16(level) per code
};

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }

// Cross-workgroup data (H partials, counters) moves only through relaxed
// agent-scope atomics, which are coherent across the XCDs' separate L2 caches
// on their own; each partial carries its launch tag in the same 64-bit word,
// so no ordering between separate stores is needed and no L2
// write-back/invalidate fence is ever issued.
__device__ __forceinline__ void st_tagged(uint64_t* p, uint32_t tag, float v) {
  __hip_atomic_store(p, ((uint64_t)tag << 32) | __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_tagged(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_ctr(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t add_ctr(uint64_t* p, uint64_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// i-th of n equal integer shares of 2^20 (the shares add up to exactly 2^20)
__device__ __forceinline__ uint64_t epoch_share(uint32_t i, uint32_t n) {
  return kEpoch / n + ((i < kEpoch % n) ? 1u : 0u);
}

// Tile i of n takes its share of one launch epoch from a group of kSlots
// counters (byte offset base + 128 s): the tiles of counter s together add
// exactly 2^20.  With fewer tiles than counters a tile advances every counter
// it owns.  Returns the tile's own counter update.
// (One returning atomic on a computed address, no branch around it, so that
// nothing waits for its result before the result is used.)
__device__ __forceinline__ uint64_t take_slot_ticket(char* ws, int base, uint32_t i, uint32_t n) {
  const bool shared = n >= (uint32_t)kSlots;
  const uint32_t s = shared ? i % kSlots : i;
  const uint32_t cnt = n / kSlots + ((s < n % kSlots) ? 1u : 0u);
  const uint64_t share = shared ? epoch_share(i / kSlots, cnt) : kEpoch;
  const uint64_t ticket = add_ctr(reinterpret_cast<uint64_t*>(ws + base + 128 * s), share);
  if (!shared)
    for (uint32_t t = i + n; t < (uint32_t)kSlots; t += n)
      __hip_atomic_fetch_add(reinterpret_cast<uint64_t*>(ws + base + 128 * t), kEpoch, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
  return ticket;
}

constexpr int kWeightCtr = 128;        // weight counters at 128 (1 + s)
constexpr int kDownCtr = 128 * 10;     // LoRA-down counters at 128 (10 + s)

// Weight tile wt's ticket (one thread per tile).  Without an adapter there
// are no LoRA-down tiles: tile 0 advances their counters too, so that every
// launch moves every counter by one epoch.
__device__ __forceinline__ uint64_t take_weight_ticket(const DecodeParams& p, int wt) {
  const uint64_t ticket = take_slot_ticket(p.ws, kWeightCtr, (uint32_t)wt, (uint32_t)p.n_wtiles);
  if (p.n_htiles == 0 && wt == 0)
    for (int s = 0; s < kSlots; ++s) add_ctr(reinterpret_cast<uint64_t*>(p.ws + kDownCtr + 128 * s), kEpoch);
  return ticket;
}

__device__ __forceinline__ uint64_t take_down_ticket(const DecodeParams& p, int tile) {
  return take_slot_ticket(p.ws, kDownCtr, (uint32_t)tile, (uint32_t)p.n_htiles);
}

// ---------------------------------------------------------------- LoRA-down tile
// Rows j0..j0+15 of A over a quarter of K; each wave takes a contiguous run of
// 32-wide steps and issues the loads of 8 steps at a time.  MFMA rows past M
// carry copies of row M-1; their outputs are discarded.
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
// Loads of kBatch consecutive blocks are issued together and the next batch is
// in flight while the current one is multiplied.
constexpr int kBatch = 4;

template <bool kXLds>
struct BlockLoads {
  u32x2 cw[kBatch];  // 8 code bytes per block (this lane's 16 elements)
  uint32_t c2w;      // the 4 E4M3 constants of the batch's blocks, one byte each
  float c1a, c1b;    // second-level constants of the batch's first and last block
  u32x4 x0[kBatch], x1[kBatch];  // only when X is read from global memory
};

struct WeightCtx {
  rsrc_t rc, r2, r1, rx;
  uint32_t code_off;   // byte offset of this lane's codes in block 0
  uint32_t blk0;       // block index of (row, block 0)
  uint32_t x_off;      // byte offset of this lane's X row at k = 16g
  const char* xs;      // X in LDS (bytes) or null
  int b_end;
  int c2_vec;
};

// One batch = kBatch (= 4) consecutive blocks of this lane's row, starting at
// a multiple of 4 so that their c2 bytes form one aligned dword.  Few, wide
// loads keep the texture-address unit from backing up.
template <bool kXLds>
__device__ __forceinline__ void load_blocks(const WeightCtx& c, BlockLoads<kXLds>& L, int b0) {
#pragma unroll
  for (int i = 0; i < kBatch; ++i) {
    const uint32_t b = (uint32_t)min(b0 + i, c.b_end - 1);
    L.cw[i] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(c.rc, c.code_off + 32 * b, 0, 0));
    if (!kXLds) {
      L.x0[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(c.rx, c.x_off + 128 * b, 0, 0));
      L.x1[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(c.rx, c.x_off + 128 * b + 16, 0, 0));
    }
  }
  if (c.c2_vec) {
    L.c2w = __builtin_amdgcn_raw_buffer_load_b32(c.r2, c.blk0 + (uint32_t)b0, 0, 0);
  } else {
    L.c2w = 0u;
#pragma unroll
    for (int i = 0; i < kBatch; ++i)
      L.c2w |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(c.r2, c.blk0 + (uint32_t)b0 + i, 0, 0) << (8 * i);
  }
  L.c1a = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(c.r1, ((c.blk0 + b0) >> 8) * 4, 0, 0));
  L.c1b = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(c.r1, ((c.blk0 + b0 + kBatch - 1) >> 8) * 4, 0, 0));
}

template <bool kXLds>
__device__ __forceinline__ void mul_blocks(const WeightCtx& c, const BlockLoads<kXLds>& L, int b0, float mu,
                                           const char* lutb, uint32_t cb, f32x4& acc) {
#pragma unroll
  for (int i = 0; i < kBatch; ++i) {
    if (b0 + i >= c.b_end) break;
    const uint32_t blk = c.blk0 + (uint32_t)(b0 + i);
    const float c1 = ((blk >> 8) == ((c.blk0 + b0) >> 8)) ? L.c1a : L.c1b;
    const float chat = i == 0 ? dequant_constant_byte<0>(L.c2w, c1, mu)
                     : i == 1 ? dequant_constant_byte<1>(L.c2w, c1, mu)
                     : i == 2 ? dequant_constant_byte<2>(L.c2w, c1, mu)
                              : dequant_constant_byte<3>(L.c2w, c1, mu);
    f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t w = L.cw[i][h];
      u32x4 wv;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t byte = (w >> (8 * q)) & 0xFFu;
        wv[q] = *reinterpret_cast<const uint32_t*>(lutb + ((byte << 7) | cb));
      }
      u32x4 xv;
      if (kXLds)
        xv = *reinterpret_cast<const u32x4*>(c.xs + c.x_off + 128 * (b0 + i) + 16 * h);
      else
        xv = h ? L.x1[i] : L.x0[i];
      t = mfma16(as_bf16x8(xv), as_bf16x8(wv), t);
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[v] = __builtin_fmaf(chat, t[v], acc[v]);
  }
}

template <bool kXLds>
// ticket: thread 0's weight-counter update (its epoch names this launch).
__device__ void weight_tile(const DecodeParams& p, int tile, uint32_t* lut, char* xs, uint32_t* words, float* red,
                            float* hs, float* bs, uint32_t* tag_lds, uint64_t ticket) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n0 = tile * kRows;
  const int nl = lane & 15, g = lane >> 4;
  const int nblk = p.K / 64;
  const float mu = *p.mean;
  const uint32_t cb = (uint32_t)(lane & 31) * 4u;  // this lane's table copy (bytes)
  const char* lutb = reinterpret_cast<const char*>(lut);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};

  // rows n0..n0+15 of B (16 x r bf16, contiguous): issued now as 16-byte
  // chunks, parked in LDS after the weight stream (row stride r+1: no bank
  // conflicts when the 16 rows are read together)
  const int bs_ld = p.r + 1;
  const int rdiv = p.r > 0 ? p.r : 1;   // r = 0 (no adapter): every B/H loop is empty
  const int b_chunks = p.b_vec ? (16 * p.r) / 8 : 0;
  const rsrc_t rb = make_rsrc(p.B, (uint32_t)p.N * p.r * 2);   // rows past N read as 0
  u32x4 bchunk = {0u, 0u, 0u, 0u};
  if (threadIdx.x < b_chunks)
    bchunk = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rb, ((uint32_t)n0 * p.r + 8 * threadIdx.x) * 2, 0, 0));
  constexpr int kBPer = 16 * 128 / kThreads;   // element loads when B is not 16-byte friendly
  uint32_t bv[kBPer];
  if (!p.b_vec) {
#pragma unroll
    for (int i = 0; i < kBPer; ++i) {
      const int e = threadIdx.x + i * kThreads;
      const int br = e / rdiv, bc = e - br * p.r;
      bv[i] = (e < 16 * p.r && n0 + br < p.N) ? p.B[(size_t)(n0 + br) * p.r + bc] : 0u;
    }
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
  c.c2_vec = p.c2_vec;
  // each wave takes a run of whole batches (multiples of 4 blocks)
  const int per = ((nblk + kWaves - 1) / kWaves + kBatch - 1) / kBatch * kBatch;
  const int b_beg = min(nblk, wave * per);
  c.b_end = min(nblk, b_beg + per);

  // X (for staging) first, then the first two batches of weight loads: loads
  // complete in issue order, so staging X waits only for X, and the first
  // batch can be multiplied while the second is still arriving.
  constexpr int kXPer = kXLdsBytes / 16 / kThreads;
  u32x4 xv[kXPer];
  const int n16 = p.M * p.K / 8;  // 16-byte chunks of X
  if (kXLds) {
#pragma unroll
    for (int i = 0; i < kXPer; ++i) {
      const int j = threadIdx.x + i * kThreads;
      if (j < n16) xv[i] = *reinterpret_cast<const u32x4*>(p.X + 8 * j);
    }
  }
  BlockLoads<kXLds> La, Lb;
  const bool work = b_beg < c.b_end;
  if (work) {
    load_blocks(c, La, b_beg);
    if (b_beg + kBatch < c.b_end) load_blocks(c, Lb, b_beg + kBatch);
  }
  // pair table: entry for code byte e is bf16(level[e & 15]) | bf16(level[e >> 4]) << 16,
  // one copy per lane%32 (entry stride 128 bytes)
  if (threadIdx.x == 0) {
#pragma unroll
    for (int i = 0; i < 16; ++i) words[i] = p.hi[i];   // constant indices: scalar kernel-argument reads
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 256 * kLutCopies; i += kThreads) {
    const int e = i >> 5;
    lut[i] = words[e & 15] | (words[e >> 4] << 16);
  }
  if (kXLds) {
#pragma unroll
    for (int i = 0; i < kXPer; ++i) {
      const int j = threadIdx.x + i * kThreads;
      if (j < n16) reinterpret_cast<u32x4*>(xs)[j] = xv[i];
    }
  }
  __syncthreads();

  // LoRA-down partials this thread sums later: first read issued after the
  // first batch is multiplied, so it travels while the rest is computed
  constexpr int kHPer = 16 * 128 / kThreads;   // up to M*r = 2048 sums per tile
  const int r16 = (p.r + 15) & ~15;
  uint64_t hp[kHSplit];                         // early read of this thread's first sum
  bool hp_issued = false;
  auto issue_poll = [&]() {
    const int i = threadIdx.x;
    if (i < p.M * p.r) {
      const int m = i / p.r, j = i - m * p.r;
#pragma unroll
      for (int ks = 0; ks < kHSplit; ++ks) hp[ks] = ld_tagged(&p.Hpart[((size_t)ks * p.M + m) * r16 + j]);
    }
    hp_issued = true;
  };

  if (work) {
    for (int b0 = b_beg; b0 < c.b_end; b0 += 2 * kBatch) {
      if (b0 != b_beg && b0 + kBatch < c.b_end) load_blocks(c, Lb, b0 + kBatch);
      mul_blocks(c, La, b0, mu, lutb, cb, acc);
      if (!hp_issued) issue_poll();
      if (b0 + 2 * kBatch < c.b_end) load_blocks(c, La, b0 + 2 * kBatch);
      if (b0 + kBatch < c.b_end) mul_blocks(c, Lb, b0 + kBatch, mu, lutb, cb, acc);
    }
  }
  if (!hp_issued) issue_poll();
  // acc[v] = partial Y0[m = 4g + v][n0 + nl]
#pragma unroll
  for (int v = 0; v < 4; ++v) red[wave * 256 + (4 * g + v) * 16 + nl] = acc[v];
  if (threadIdx.x < b_chunks) {
    const int e0 = 8 * threadIdx.x, br = e0 / p.r, bc = e0 - br * p.r;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      bs[br * bs_ld + bc + 2 * q] = bf16_lo(bchunk[q]);
      bs[br * bs_ld + bc + 2 * q + 1] = bf16_hi(bchunk[q]);
    }
  }
  if (!p.b_vec) {
#pragma unroll
    for (int i = 0; i < kBPer; ++i) {
      const int e = threadIdx.x + i * kThreads;
      const int br = e / rdiv, bc = e - br * p.r;
      if (e < 16 * p.r) bs[br * bs_ld + bc] = __uint_as_float(bv[i] << 16);
    }
  }

  // collect this launch's LoRA-down partials (tag = epoch + 1), polling until
  // present; only thread 0 holds the counter update, so it shares the tag
  if (threadIdx.x == 0) *tag_lds = (uint32_t)(ticket >> 20) + 1u;
  __syncthreads();
  const uint32_t tag = *tag_lds;
#pragma unroll
  for (int u = 0; u < kHPer; ++u) {
    const int i = threadIdx.x + u * kThreads;
    if (i < p.M * p.r) {
      const int m = i / p.r, j = i - m * p.r;
      float h = 0.f;
#pragma unroll
      for (int ks = 0; ks < kHSplit; ++ks) {
        const uint64_t* src = &p.Hpart[((size_t)ks * p.M + m) * r16 + j];
        uint64_t v = u == 0 ? hp[ks] : ld_tagged(src);
        unsigned spins = 0;
        while ((uint32_t)(v >> 32) != tag) {   // not yet published: poll
          __builtin_amdgcn_s_sleep(2);
          if (++spins > kSpinLimit) {
            __hip_atomic_store(reinterpret_cast<unsigned*>(p.ws + 128 * 9), 1u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
            break;
          }
          v = ld_tagged(src);
        }
        h += __uint_as_float((uint32_t)v);
      }
      hs[i] = h;
      if (tile == 0 && p.H) p.H[i] = h;
    }
  }
  __syncthreads();

  // epilogue: output o = m*16 + nn gets G threads (G = 512 / (16 M), capped at
  // 32); each sums a share of the wave partials and of the r-long LoRA dot
  // product, then the G lanes combine with xor shuffles
  {
    const int G = p.epi_group;
    const int o = threadIdx.x / G, sub = threadIdx.x - o * G;
    const bool valid = o < 16 * p.M;
    float part = 0.f;
    if (valid) {
      const int m = o >> 4, nn = o & 15;
      for (int w = sub; w < kWaves; w += G) part += red[w * 256 + o];
      const float* brow = bs + nn * bs_ld;
      const float* hrow = hs + m * p.r;
      float lora = 0.f;
      for (int j = sub; j < p.r; j += G) lora = __builtin_fmaf(hrow[j], brow[j], lora);
      part = __builtin_fmaf(p.scale, lora, part);
    }
    for (int off = G >> 1; off >= 1; off >>= 1) part += __shfl_xor(part, off);
    if (valid && sub == 0) {
      const int m = o >> 4, n = n0 + (o & 15);
      if (n < p.N) p.Y[(size_t)m * p.N + n] = (uint16_t)(pack_bf16x2(part, 0.f) & 0xFFFFu);
    }
  }
}

template <bool kXLds>
__global__ void __launch_bounds__(kThreads, 4) qlora_decode_kernel(DecodeParams p) {
  __shared__ uint32_t lut[256 * kLutCopies];    // 32 KiB
  __shared__ __attribute__((aligned(16))) char xs[kXLds ? kXLdsBytes : 16];
  __shared__ float red[kWaves * 256];           // 8 KiB
  __shared__ float hs[16 * 128];                // 8 KiB: H rows for the epilogue
  __shared__ float bs[16 * 129];                // B rows of the tile, stride r+1
  __shared__ uint32_t words[16];
  const int tile = (int)blockIdx.x;

  if (tile < p.n_htiles) {
    __shared__ uint32_t htag;
    uint64_t hticket = 0;
    if (threadIdx.x == 0) hticket = take_down_ticket(p, tile);
    lora_down_tile(p, tile, red, &htag, hticket);
    return;
  }

  // weight tile: take the epoch ticket now, use it at the wait
  const int wt = tile - p.n_htiles;
  uint64_t ticket = 0;
  if (threadIdx.x == 0) ticket = take_weight_ticket(p, wt);

  __shared__ uint32_t wtag;
  weight_tile<kXLds>(p, wt, lut, xs, words, red, hs, bs, &wtag, ticket);
}

// ---------------------------------------------------------------- GEMV path (M <= 2)
// 16 output rows per workgroup.  Wave w takes rows 4 (w % 4) .. +3 of the
// tile over one half of K (w / 4).  Per row, lane l reads 16 bytes of codes
// (32 codes inside one NF4 block), so a load instruction covers 1 KB of one
// row.  Each wave loads the X values of its own pieces into registers, so no
// wave waits for another before its dot products: they run while the rest
// of the weight stream is still arriving.  A code byte indexes a table of
// bf16 level pairs in LDS (entry e at 256 e, one 4-byte copy per lane % 32:
// the address 256 byte + 4 (lane % 32) is one byte permute, and the lanes of
// a half-wave always hit distinct banks); v_dot2_f32_bf16 multiplies the
// pair with two X values in fp32.  The level enters as bf16(level) and the
// block's fp32 constant scales the block's sum afterwards, as in the
// matrix-core path above.  The two halves of K meet in LDS at the end.  The
// LoRA-down products come from one workgroup per row of A, each publishing
// H[m][j] as one tagged word.
constexpr int kGvRowsPerWave = 4;
constexpr int kGvStride = 256;   // bytes per pair-table entry

// bf16 pairs as the dot-product builtin takes them (raw 16-bit lanes)
typedef short s16x2 __attribute__((ext_vector_type(2)));

template <int M>
struct GvPiece {
  u32x4 x[M][4];               // the piece's 32 X values per batch row
  u32x4 w[kGvRowsPerWave];     // 16 bytes of codes per row
  uint8_t c2[kGvRowsPerWave];    // (bytes: widened where used, not ahead of a loop)
  float c1[kGvRowsPerWave];
};

// piece c of each of the wave's rows (c < K / 32), X first: it is used first
template <int M>
__device__ __forceinline__ void gv_load(const DecodeParams& p, const rsrc_t& rc, const rsrc_t& r2, const rsrc_t& r1,
                                        const rsrc_t& rx, const uint32_t (&row)[kGvRowsPerWave], uint32_t c,
                                        GvPiece<M>& L) {
  const uint32_t nblk = (uint32_t)p.K / 64, rb = (uint32_t)p.K / 2;
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      L.x[m][q] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, ((uint32_t)m * p.K + 32 * c) * 2 + 16 * q, 0, 0));
  // (constants through plain byte loads, which widen for free, on a row
  // clamped to N - 1; the buffer form's byte result costs a separate
  // widening instruction, which the compiler places early)
  const uint32_t last = (uint32_t)p.N - 1u, n_c2 = (uint32_t)p.N * nblk;
#pragma unroll
  for (int rr = 0; rr < kGvRowsPerWave; ++rr) {
    const uint32_t rowc = row[rr] < last ? row[rr] : last;
    const uint32_t blk = rowc * nblk + (c >> 1);
    L.w[rr] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rc, row[rr] * rb + 16 * c, 0, 0));
    L.c2[rr] = p.c2[blk < n_c2 ? blk : n_c2 - 1u];
    L.c1[rr] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r1, (blk >> 8) * 4, 0, 0));
  }
}

template <int M>
__device__ __forceinline__ void gv_mul(const GvPiece<M>& L, float mu, const char* lut, uint32_t lane4,
                                       float (&acc)[kGvRowsPerWave][M]) {
#pragma unroll
  for (int rr = 0; rr < kGvRowsPerWave; ++rr) {
    float part[M];
#pragma unroll
    for (int m = 0; m < M; ++m) part[m] = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t word = L.w[rr][q];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        // address bytes: [lane4, code byte b, 0, 0]
        const uint32_t a = __builtin_amdgcn_perm(word, lane4, 0x0c0c0000u | ((4u + b) << 8));
        const uint32_t wp = *reinterpret_cast<const uint32_t*>(lut + a);
#pragma unroll
        for (int m = 0; m < M; ++m) {
          // copy the vector element out first: a bit_cast applied to the
          // element expression itself reads element 0
          const uint32_t xp = L.x[m][q][b];
          part[m] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(s16x2, wp), __builtin_bit_cast(s16x2, xp),
                                                    part[m], false);
        }
      }
    }
    const float chat = dequant_constant(L.c2[rr], L.c1[rr], mu);
#pragma unroll
    for (int m = 0; m < M; ++m) acc[rr][m] = __builtin_fmaf(chat, part[m], acc[rr][m]);
  }
}

// Pair-table entry e = bf16(level[e & 15]) | bf16(level[e >> 4]) << 16 for a
// lane-varying e < 256: the 16 level words (scalar launch arguments) go into
// lanes 0..15 of one register and each half is fetched by a lane permute, so
// no memory is read.
__device__ __forceinline__ uint32_t pair_entry(const DecodeParams& p, uint32_t e) {
  int tab = 0;
#pragma unroll
  for (int k = 0; k < 16; ++k) asm volatile("v_writelane_b32 %0, %1, %2" : "+v"(tab) : "s"(p.hi[k]), "n"(k));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_ds_bpermute((int)((e & 15u) * 4u), tab);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_ds_bpermute((int)((e >> 4) * 4u), tab);
  return lo | (hi << 16);
}

// Lane exchanges without LDS: DPP within a row of 16 lanes, and gfx950's
// permlane swaps between rows (16) and halves (32) of the wave.
__device__ __forceinline__ float dpp_row_sum(float v) {   // every lane: its row's sum
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));    // quad_perm 1,0,3,2
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));    // quad_perm 2,3,0,1
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false));   // row_half_mirror
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, false));   // row_mirror
  return v;
}
// a + b after swapping a's upper 32 lanes with b's lower 32
__device__ __forceinline__ float swap32_add(float a, float b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// a + b after swapping a's odd 16-lane rows with b's even rows
__device__ __forceinline__ float swap16_add(float a, float b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float wave_sum(float v) {   // every lane: the wave's sum
  v = dpp_row_sum(v);
  v = swap16_add(v, v);
  return swap32_add(v, v);
}

// Sums of v[0..3] over the wave's 64 lanes: afterwards the lanes of row t
// (lanes 16 t .. 16 t + 15) hold the sum of v[t].  The swaps halve the values
// a lane carries, so 4 sums cost 2 + 1 swaps and one row reduction.
__device__ __forceinline__ float wave_sum4(const float (&v)[kGvRowsPerWave]) {
  // lower half: v0 (+ upper's v0), upper half: v2 (+ lower's v2); same for 1, 3
  const float a0 = swap32_add(v[0], v[2]), a1 = swap32_add(v[1], v[3]);
  // even rows keep a0, odd rows a1
  return dpp_row_sum(swap16_add(a0, a1));
}

// LoRA-down row j = tile: H[m][j] = sum_k X[m][k] A[j][k] for m < M, published
// as tagged words Hpart[m * r16 + j].
template <int M>
__device__ void gemv_down_tile(const DecodeParams& p, int j, float* red, uint32_t* tag_lds, uint64_t ticket) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const rsrc_t ra = make_rsrc(p.A + (size_t)j * p.K, (uint32_t)p.K * 2);
  const rsrc_t rx = make_rsrc(p.X, (uint32_t)M * p.K * 2);
  float acc[M];
#pragma unroll
  for (int m = 0; m < M; ++m) acc[m] = 0.f;
  for (int c = threadIdx.x; c < p.K / 8; c += kThreads) {   // 8 elements per chunk
    const u32x4 a = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, 16 * c, 0, 0));
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const u32x4 x = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, ((uint32_t)m * p.K + 8 * c) * 2, 0, 0));
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t aq = a[q], xq = x[q];
        acc[m] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(s16x2, aq), __builtin_bit_cast(s16x2, xq), acc[m],
                                                 false);
      }
    }
  }
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const float v = wave_sum(acc[m]);
    if (lane == 0) red[wave * M + m] = v;
  }
  if (threadIdx.x == 0) *tag_lds = (uint32_t)(ticket >> 20) + 1u;
  __syncthreads();
  if (threadIdx.x < M) {
    float h = 0.f;
    for (int w = 0; w < kWaves; ++w) h += red[w * M + threadIdx.x];
    const int r16 = (p.r + 15) & ~15;
    st_tagged(&p.Hpart[(size_t)threadIdx.x * r16 + j], *tag_lds, h);
  }
}

template <int M>
__device__ void gemv_tile(const DecodeParams& p, int tile, char* lut, float* red, uint32_t* tag_lds) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = wave & 3, half = wave >> 2;
  // (read ahead of the counter update: with no write before it, the
  // compiler may take it through the scalar cache)
  const float mu = *p.mean;
  // this launch's epoch: thread 0's counter update goes out first, and its
  // reply, which comes back ahead of every later load, is used only at the
  // end (no other thread reads the variable)
  uint64_t ticket;
  if (threadIdx.x == 0) ticket = take_weight_ticket(p, tile);

  uint32_t row[kGvRowsPerWave];
#pragma unroll
  for (int rr = 0; rr < kGvRowsPerWave; ++rr)
    row[rr] = (uint32_t)(tile * kRows + kGvRowsPerWave * grp + rr);
  const uint32_t n_c2 = (uint32_t)p.N * (uint32_t)(p.K / 64);
  const rsrc_t rc = make_rsrc(p.codes, n_c2 * 32u);   // rows >= N read as zero codes
  const rsrc_t r2 = make_rsrc(p.c2, n_c2);
  const rsrc_t r1 = make_rsrc(p.c1, ((n_c2 + 255u) / 256u) * 4u);
  const rsrc_t rx = make_rsrc(p.X, (uint32_t)M * p.K * 2);
  const int hp = p.K / 64;                 // pieces per row in each half of K
  const int npl = (hp + 63) / 64;          // pieces per lane
  const uint32_t c0 = (uint32_t)(half * hp + lane);
  // two pieces in flight at M = 1; at M = 2 one (registers)
  constexpr bool kTwo = M == 1;
  GvPiece<M> La, Lb;
  gv_load<M>(p, rc, r2, r1, rx, row, c0, La);
  if (kTwo && 1 < npl) gv_load<M>(p, rc, r2, r1, rx, row, c0 + 64, Lb);

  // pair table: entry e = bf16(level[e & 15]) | bf16(level[e >> 4]) << 16,
  // 32 copies; thread t writes 4 of the 8 16-byte pieces of entry t % 256,
  // in a per-entry rotated order (no bank conflicts between the 8 entries a
  // write instruction serves at once), while the loads are in flight.
  {
    const uint32_t e = threadIdx.x & 255, part = threadIdx.x >> 8;
    const uint32_t pv = pair_entry(p, e);
    u32x4* dst = reinterpret_cast<u32x4*>(lut + e * kGvStride);
#pragma unroll
    for (uint32_t i = 0; i < 4; ++i) dst[(4 * part + i + e) & 7] = u32x4{pv, pv, pv, pv};
  }
  __syncthreads();

  const uint32_t lane4 = (uint32_t)(lane & 31) * 4u;
  float acc[kGvRowsPerWave][M];
#pragma unroll
  for (int rr = 0; rr < kGvRowsPerWave; ++rr)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[rr][m] = 0.f;
  if constexpr (kTwo) {
    for (int i = 0; i < npl; i += 2) {
      if (i != 0 && i + 1 < npl) gv_load<M>(p, rc, r2, r1, rx, row, c0 + 64 * (i + 1), Lb);
      if (lane + 64 * i < hp) gv_mul<M>(La, mu, lut, lane4, acc);
      if (i + 2 < npl) gv_load<M>(p, rc, r2, r1, rx, row, c0 + 64 * (i + 2), La);
      if (i + 1 < npl && lane + 64 * (i + 1) < hp) gv_mul<M>(Lb, mu, lut, lane4, acc);
    }
  } else {
    for (int i = 0; i < npl; ++i) {
      if (i != 0) gv_load<M>(p, rc, r2, r1, rx, row, c0 + 64 * i, La);
      if (lane + 64 * i < hp) gv_mul<M>(La, mu, lut, lane4, acc);
    }
  }

  // Epilogue.  Waves of the first half of K reduce their sums and leave them
  // in LDS, and thread 0 publishes the launch tag there; waves of the second
  // half add s H B^T (H from this launch's tagged partials, tag = epoch + 1,
  // polled until present), their own sums and the first half's, and store.
  // The second half reads B and H before the barrier: the replies come back
  // while it waits.
  const bool lora = p.r > 0;
  uint32_t bv[kGvRowsPerWave][2];
  uint64_t hv[M][2];
  const int r16 = (p.r + 15) & ~15;
  if (half == 1 && lora) {
    const rsrc_t rbb = make_rsrc(p.B, (uint32_t)p.N * p.r * 2);   // rows past N read as 0
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int j = lane + 64 * h;
      if (j >= p.r) continue;
#pragma unroll
      for (int rr = 0; rr < kGvRowsPerWave; ++rr)
        bv[rr][h] = __builtin_amdgcn_raw_buffer_load_b16(rbb, (row[rr] * p.r + j) * 2, 0, 0);
#pragma unroll
      for (int m = 0; m < M; ++m) hv[m][h] = ld_tagged(&p.Hpart[(size_t)m * r16 + j]);
    }
  }
  const int rt = lane >> 4;   // this lane's row in the wave's group, if lane % 16 == 0
  if (half == 0) {
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float v[kGvRowsPerWave];
#pragma unroll
      for (int rr = 0; rr < kGvRowsPerWave; ++rr) v[rr] = acc[rr][m];
      const float t = wave_sum4(v);
      if ((lane & 15) == 0) red[(grp * kGvRowsPerWave + rt) * M + m] = t;
    }
    if (threadIdx.x == 0) {
      // (the empty asm keeps the use of the reply here, at the end)
      asm volatile("" : "+v"(ticket));
      *tag_lds = (uint32_t)(ticket >> 20) + 1u;
    }
  }
  __syncthreads();
  if (half == 0) return;

  if (lora) {
    const uint32_t tag = *tag_lds;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int j = lane + 64 * h;
      if (j >= p.r) continue;
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const uint64_t* src = &p.Hpart[(size_t)m * r16 + j];
        uint64_t v = hv[m][h];
        unsigned spins = 0;
        while ((uint32_t)(v >> 32) != tag) {   // not yet published: poll
          __builtin_amdgcn_s_sleep(1);
          if (++spins > kSpinLimit) {
            __hip_atomic_store(reinterpret_cast<unsigned*>(p.ws + 128 * 9), 1u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
            break;
          }
          v = ld_tagged(src);
        }
        const float hval = __uint_as_float((uint32_t)v);
        if (tile == 0 && grp == 0 && p.H) p.H[m * p.r + j] = hval;
        const float sh = p.scale * hval;
#pragma unroll
        for (int rr = 0; rr < kGvRowsPerWave; ++rr)
          acc[rr][m] = __builtin_fmaf(sh, __uint_as_float(bv[rr][h] << 16), acc[rr][m]);
      }
    }
  }
#pragma unroll
  for (int m = 0; m < M; ++m) {
    float v[kGvRowsPerWave];
#pragma unroll
    for (int rr = 0; rr < kGvRowsPerWave; ++rr) v[rr] = acc[rr][m];
    const float t = wave_sum4(v);
    if ((lane & 15) == 0 && row[0] + rt < (uint32_t)p.N) {
      const float y = t + red[(grp * kGvRowsPerWave + rt) * M + m];
      p.Y[(size_t)m * p.N + row[0] + rt] = (uint16_t)(pack_bf16x2(y, 0.f) & 0xFFFFu);
    }
  }
}

template <int M>
__global__ void __launch_bounds__(kThreads, 2) qlora_gemv_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(16))) char lut[256 * kGvStride];   // 64 KiB
  __shared__ float red[kRows * M];
  __shared__ uint32_t tag;
  const int tile = (int)blockIdx.x;
  // fetch the launch arguments both paths use in one round trip, ahead of
  // the branches (left alone, each branch would wait for its own fetch)
  asm volatile("" ::"s"(p.X), "s"(p.codes), "s"(p.c2), "s"(p.c1), "s"(p.mean), "s"(p.B), "s"(p.A), "s"(p.K),
               "s"(p.N), "s"(p.r), "s"(p.n_htiles), "s"(p.n_wtiles), "s"(p.ws));
  asm volatile("" ::"s"(p.hi[0]), "s"(p.hi[1]), "s"(p.hi[2]), "s"(p.hi[3]), "s"(p.hi[4]), "s"(p.hi[5]),
               "s"(p.hi[6]), "s"(p.hi[7]), "s"(p.hi[8]), "s"(p.hi[9]), "s"(p.hi[10]), "s"(p.hi[11]),
               "s"(p.hi[12]), "s"(p.hi[13]), "s"(p.hi[14]), "s"(p.hi[15]));
  if (tile < p.n_htiles) {
    uint64_t hticket = 0;
    if (threadIdx.x == 0) hticket = take_down_ticket(p, tile);
    gemv_down_tile<M>(p, tile, red, &tag, hticket);
    return;
  }
  gemv_tile<M>(p, tile - p.n_htiles, lut, red, &tag);
}

}  // namespace

size_t decode_workspace_bytes(int64_t M, int64_t r) {
  const int64_t r16 = (r + 15) & ~15;
  return kHpartOff + (size_t)(kHSplit * M * r16) * sizeof(uint64_t);
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
  p.Hpart = reinterpret_cast<uint64_t*>(p.ws + kHpartOff);
  p.H = a.H;
  const int64_t r16 = (a.r + 15) & ~15;
  const bool gemv = a.M <= 2;
  p.n_htiles = gemv ? (int)a.r : (int)(r16 / kRows) * kHSplit;
  p.n_wtiles = (int)((a.N + kRows - 1) / kRows);
  int G = kThreads / (16 * (int)a.M);
  G = G >= 32 ? 32 : (G >= 16 ? 16 : (G >= 8 ? 8 : (G >= 4 ? 4 : (G >= 2 ? 2 : 1))));
  p.epi_group = G;
  p.c2_vec = (a.K % 256 == 0) && (reinterpret_cast<uintptr_t>(a.w.c2) % 4 == 0);
  p.b_vec = (a.r % 8 == 0) && (reinterpret_cast<uintptr_t>(a.B) % 16 == 0);
  const Nf4HiLo& hl = nf4_hilo();
  for (int i = 0; i < 16; ++i) p.hi[i] = hl.word[i] & 0xFFFFu;
  const dim3 grid(p.n_htiles + p.n_wtiles);
  if (gemv && a.M == 1)
    hipLaunchKernelGGL(qlora_gemv_kernel<1>, grid, dim3(kThreads), 0, s, p);
  else if (gemv)
    hipLaunchKernelGGL(qlora_gemv_kernel<2>, grid, dim3(kThreads), 0, s, p);
  else if ((size_t)a.M * a.K * 2 <= (size_t)kXLdsBytes)
    hipLaunchKernelGGL(qlora_decode_kernel<true>, grid, dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL(qlora_decode_kernel<false>, grid, dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace qlora
