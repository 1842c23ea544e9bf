// Fused QLoRA forward for M <= 4 (decode), gfx950: the GEMV path.
//
// Y = bf16( X W_deq^T + s (X A^T) B^T )   (itwiki "QLoRA", section on the
// computation; minnong511 "quantization", y = W x + (alpha/r) B A x).
//
// At M <= 4 the layer is bound by HBM bandwidth on the 4-bit weight.  The
// pages describe the slow path as a separate dequantization kernel whose bf16
// output makes a round trip through memory before the matrix product
// (irregular6612 "QLoRA - Efficient Finetuning of Quantized LLMs", the
// inference-speed discussion); here the packed codes are streamed once and
// expanded in registers straight into bf16 dot products.
//
#include "decode_common.h"

namespace qlora {
namespace dec {
namespace {

// 16 output rows per workgroup.  Wave w takes rows 4 (w % 4) .. +3 of the
// tile over one half of K (w / 4).  (Layers that would need three or more
// rounds of workgroups take 32-row tiles instead: wave w, rows 4 w .. +3
// over all of K.)  Per row, lane l reads 16 bytes of codes
// (32 codes inside one NF4 block), so a load instruction covers 1 KB of one
// row.  Each wave loads the X values of its own pieces into registers, so no
// wave waits for another before its dot products: they run while the rest
// of the weight stream is still arriving.  A code byte indexes a table of
// bf16 level pairs in LDS (entry e at 256 e, one 4-byte copy per lane % 32:
// the address 256 byte + 4 (lane % 32) is one byte permute, and the lanes of
// a half-wave always hit distinct banks); v_dot2_f32_bf16 multiplies the
// pair with two X values in fp32.  Each 64-element NF4 block is one scaling
// unit: the level enters as bf16(level) and the block's fp32 constant c_hat
// scales the block's partial sum in fp32 afterwards, i.e. the weight used is
// bf16(level) * c_hat rather than bf16(level * c_hat): the same size of
// rounding, one place earlier.  The two halves of K meet in LDS at the end.  The
// LoRA-down products come from one workgroup per row of A, each publishing
// H[m][j] as one tagged word.
constexpr int kGvRowsPerWave = 4;

// kDw: the rows of c2 are dword aligned (K % 256 == 0, 4-byte aligned base):
// c2 comes as the dword holding the block's byte.
template <int M>
struct GvPiece {
  u32x4 x[M][4];               // the piece's 32 X values per batch row
  u32x4 w[kGvRowsPerWave];     // 16 bytes of codes per row
  uint32_t c2[kGvRowsPerWave];   // the c2 byte, or (kDw) the dword holding it
  float c1[kGvRowsPerWave];
};

// piece c of each of the wave's rows (c < K / 32), X first: it is used first
template <int M, bool kDw>
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
  // (a byte load's result needs a widening instruction, which the compiler
  // moves next to the load, where it waits for the reply: so c2 comes as a
  // dword when the rows allow, else through plain byte loads on a row
  // clamped to N - 1)
  const uint32_t last = (uint32_t)p.N - 1u, n_c2 = (uint32_t)p.N * nblk;
#pragma unroll
  for (int rr = 0; rr < kGvRowsPerWave; ++rr) {
    const uint32_t blk = row[rr] * nblk + (c >> 1);
    L.w[rr] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rc, row[rr] * rb + 16 * c, 0, 0));
    if constexpr (kDw) {
      L.c2[rr] = __builtin_amdgcn_raw_buffer_load_b32(r2, blk & ~3u, 0, 0);   // rows >= N read as 0
    } else {
      const uint32_t rowc = row[rr] < last ? row[rr] : last;
      const uint32_t bc = rowc * nblk + (c >> 1);
      L.c2[rr] = p.c2[bc < n_c2 ? bc : n_c2 - 1u];
    }
    L.c1[rr] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r1, (blk >> 8) * 4, 0, 0));
  }
}

// c2sh: with kDw, 8 x the byte's place in its dword (the same for the four
// rows: rows of c2 are dword aligned)
template <int M, bool kDw>
__device__ __forceinline__ void gv_mul(const GvPiece<M>& L, float mu, const char* lut, uint32_t lane4,
                                       uint32_t c2sh, float (&acc)[kGvRowsPerWave][M]) {
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
        const uint32_t a = b == 0 ? pair_addr<0>(word, lane4)
                         : b == 1 ? pair_addr<1>(word, lane4)
                         : b == 2 ? pair_addr<2>(word, lane4)
                                  : pair_addr<3>(word, lane4);
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
    // (the empty asm keeps the work on the loaded byte here, where it is
    // used; otherwise the compiler moves it next to the load, into a wait)
    uint32_t c2 = L.c2[rr];
    asm volatile("" : "+v"(c2));
    if constexpr (kDw) c2 >>= c2sh;
    const float chat = dequant_constant(c2, L.c1[rr], mu);
#pragma unroll
    for (int m = 0; m < M; ++m) acc[rr][m] = __builtin_fmaf(chat, part[m], acc[rr][m]);
  }
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
// as tagged words Hpart[c * gemv_hcopy_words(M, r) + m * r16 + j] in each
// copy c.
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
    const int r16 = (p.r + 15) & ~15, cw = gemv_hcopy_words(M, p.r);
#pragma unroll
    for (int c = 0; c < gemv_hcopies(M); ++c) st_tagged(&p.Hpart[(size_t)c * cw + threadIdx.x * r16 + j], *tag_lds, h);
  }
}

// kNPL: 16-byte pieces per lane and row (the launcher's exact count), or 0
// for any count (the launcher takes 0 whenever the rows of c2 are not dword
// aligned).
template <int M, int kNPL, bool kFull>
__device__ void gemv_tile(const DecodeParams& p, int tile, char* lut, float* red, uint32_t* tag_lds) {
  constexpr bool kDw = kNPL > 0;
  constexpr int kTileRows = kFull ? 2 * kRows : kRows;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // 16-row tiles: wave w takes rows 4 (w % 4) .. +3 over half w / 4 of K;
  // 32-row tiles (kFull): rows 4 w .. +3 over all of K
  const int grp = kFull ? wave : (wave & 3), half = kFull ? 0 : (wave >> 2);
  const bool finisher = kFull || half == 1;   // adds the LoRA term and stores
  // this launch's epoch: thread 0's counter update goes out first, and its
  // reply, which comes back ahead of every later load, is used only at the
  // end (no other thread reads the variable)
  uint64_t ticket;
  if (threadIdx.x == 0) ticket = take_weight_ticket(p, tile);

  uint32_t row[kGvRowsPerWave];
#pragma unroll
  for (int rr = 0; rr < kGvRowsPerWave; ++rr)
    row[rr] = (uint32_t)(tile * kTileRows + kGvRowsPerWave * grp + rr);
  const uint32_t n_c2 = (uint32_t)p.N * (uint32_t)(p.K / 64);
  const rsrc_t rc = make_rsrc(p.codes, n_c2 * 32u);   // rows >= N read as zero codes
  const rsrc_t r2 = make_rsrc(p.c2, n_c2);
  const rsrc_t r1 = make_rsrc(p.c1, ((n_c2 + 255u) / 256u) * 4u);
  const rsrc_t rx = make_rsrc(p.X, (uint32_t)M * p.K * 2);
  const int hp = kFull ? p.K / 32 : p.K / 64;   // pieces per row in the wave's range of K
  const int npl = (hp + 63) / 64;          // pieces per lane
  const uint32_t c0 = (uint32_t)(half * hp + lane);
  const uint32_t lane4 = (uint32_t)(lane & 31) * 4u;
  float acc[kGvRowsPerWave][M];
#pragma unroll
  for (int rr = 0; rr < kGvRowsPerWave; ++rr)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[rr][m] = 0.f;

  // LoRA operands of the second half's waves (see the epilogue): B[row][j]
  // for j = lane, lane + 64 and the first read of this launch's H partials
  const bool lora = p.r > 0;
  const int r16 = (p.r + 15) & ~15;
  const uint64_t* hcopy = p.Hpart + (size_t)((4 * tile + grp) % gemv_hcopies(M)) * gemv_hcopy_words(M, p.r);
  uint32_t bv[kGvRowsPerWave][2];
  uint64_t hv[M][2];
  auto load_b = [&]() {
    if (finisher && lora) {
      const uint32_t last = (uint32_t)p.N - 1u;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int j = lane + 64 * h;
        if (j >= p.r) continue;
        // plain 16-bit loads (they widen for free) on rows clamped to N - 1
#pragma unroll
        for (int rr = 0; rr < kGvRowsPerWave; ++rr)
          bv[rr][h] = p.B[(size_t)(row[rr] < last ? row[rr] : last) * p.r + j];
      }
    }
  };
  auto read_h = [&]() {
    if (finisher && lora) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int j = lane + 64 * h;
        if (j >= p.r) continue;
#pragma unroll
        for (int m = 0; m < M; ++m) hv[m][h] = ld_tagged(&hcopy[(size_t)m * r16 + j]);
      }
    }
  };

  if constexpr (kNPL > 0) {
    // A known piece count: every load is issued whatever the lane's share
    // (offsets of pieces past the row end stay in bounds or read zero; their
    // products are skipped), so each wait counts exactly the loads issued
    // after the one it waits for.  Two pieces in flight at M = 1, one at
    // M >= 2 (registers).
    constexpr int kDepth = M == 1 ? 2 : 1;
    GvPiece<M> L[kDepth];
#pragma unroll
    for (int i = 0; i < kDepth && i < kNPL; ++i) gv_load<M, kDw>(p, rc, r2, r1, rx, row, c0 + 64 * i, L[i]);
    // (the mean's pointer comes with the parameter block, after the loads)
    const float mu = load_mean(p);
    build_pair_table<kThreads>(p, lut);   // while the loads are in flight
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kNPL; ++i) {
      GvPiece<M>& cur = L[i % kDepth];
      if (M == 1 && i == kNPL - 1) {
        // B and the H partials are read once the last piece has arrived: by
        // then H has been published (read with the weight loads, the first
        // read comes back stale and the poll adds a round trip), and the
        // reads are in flight during the last dot products instead of after
        // them.  (At M >= 2 the registers that takes would spill.)
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
        load_b();
        read_h();
      }
      if (lane + 64 * i < hp) gv_mul<M, kDw>(cur, mu, lut, lane4, 8u * (((c0 + 64 * i) >> 1) & 3u), acc);
      if (i + kDepth < kNPL) gv_load<M, kDw>(p, rc, r2, r1, rx, row, c0 + 64 * (i + kDepth), cur);
    }
    if constexpr (M > 1) {
      load_b();
      read_h();
    }
  } else {
    // two pieces in flight at M = 1; at M >= 2 one (registers)
    constexpr bool kTwo = M == 1;
    GvPiece<M> La, Lb;
    gv_load<M, kDw>(p, rc, r2, r1, rx, row, c0, La);
    if (kTwo && 1 < npl) gv_load<M, kDw>(p, rc, r2, r1, rx, row, c0 + 64, Lb);
    const float mu = load_mean(p);
    build_pair_table<kThreads>(p, lut);   // while the loads are in flight
    __syncthreads();
    if constexpr (kTwo) {
      for (int i = 0; i < npl; i += 2) {
        if (i != 0 && i + 1 < npl) gv_load<M, kDw>(p, rc, r2, r1, rx, row, c0 + 64 * (i + 1), Lb);
        if (lane + 64 * i < hp) gv_mul<M, kDw>(La, mu, lut, lane4, 0u, acc);
        if (i + 2 < npl) gv_load<M, kDw>(p, rc, r2, r1, rx, row, c0 + 64 * (i + 2), La);
        if (i + 1 < npl && lane + 64 * (i + 1) < hp) gv_mul<M, kDw>(Lb, mu, lut, lane4, 0u, acc);
      }
    } else {
      for (int i = 0; i < npl; ++i) {
        if (i != 0) gv_load<M, kDw>(p, rc, r2, r1, rx, row, c0 + 64 * i, La);
        if (lane + 64 * i < hp) gv_mul<M, kDw>(La, mu, lut, lane4, 0u, acc);
      }
    }
    load_b();
    read_h();
  }

  // Epilogue.  Waves of the first half of K reduce their sums and leave them
  // in LDS, and thread 0 publishes the launch tag there; waves of the second
  // half add s H B^T (H from this launch's tagged partials, tag = epoch + 1,
  // polled until present), their own sums and the first half's, and store.
  const int rt = lane >> 4;   // this lane's row in the wave's group, if lane % 16 == 0
  if (!finisher) {
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float v[kGvRowsPerWave];
#pragma unroll
      for (int rr = 0; rr < kGvRowsPerWave; ++rr) v[rr] = acc[rr][m];
      const float t = wave_sum4(v);
      if ((lane & 15) == 0) red[(grp * kGvRowsPerWave + rt) * M + m] = t;
    }
  }
  if (threadIdx.x == 0) {
    // (the empty asm keeps the use of the reply here, at the end)
    asm volatile("" : "+v"(ticket));
    *tag_lds = (uint32_t)(ticket >> 20) + 1u;
  }
  __syncthreads();
  if (!finisher) return;

  if (lora) {
    const uint32_t tag = *tag_lds;
    uint64_t deadline = 0;   // set at the first miss
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int j = lane + 64 * h;
      if (j >= p.r) continue;
#pragma unroll
      for (int m = 0; m < M; ++m) {
        float hval;
        if (!poll_tagged(&hcopy[(size_t)m * r16 + j], hv[m][h], tag, deadline, &hval))
          hval = lane_lora_down(p.X, p.A, p.K, m, j, p.ws);
        if (tile == 0 && grp == 0 && p.H) p.H[m * p.r + j] = hval;
        const float sh = p.scale * hval;
#pragma unroll
        for (int rr = 0; rr < kGvRowsPerWave; ++rr) {
          uint32_t b = bv[rr][h];
          asm volatile("" : "+v"(b));   // (as for c2: the widening stays here)
          acc[rr][m] = __builtin_fmaf(sh, __uint_as_float(b << 16), acc[rr][m]);
        }
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
      const float y = (kFull ? t : t + red[(grp * kGvRowsPerWave + rt) * M + m]) * p.inv_kappa;
      p.Y[(size_t)m * p.N + row[0] + rt] = (uint16_t)(pack_bf16x2(y, 0.f) & 0xFFFFu);
    }
  }
}

// Two workgroups per CU (4 waves per SIMD) up to M = 3; at M = 4 the X
// registers need more, and one workgroup per CU runs faster than spilling.
//
// The pointers and sizes the first loads need come first in the argument
// list, ahead of the parameter block: they are preloaded into scalar
// registers at dispatch (this file is built with kernarg preloading; 14
// dwords fit beside the kernarg pointer), so the weight loads go out without
// waiting for a kernel-argument fetch; the rest of the block arrives while
// they are in flight, in the weight tiles and in the LoRA-down workgroups
// alike.  (The tile counts follow from N and r; K / 64 and r share a dword.
// Any early use of a field of the block waits for all of it: scalar loads
// complete out of order, so their only wait is for every one.)
template <int M, int kNPL, bool kFull>
__global__ void __launch_bounds__(kThreads, M <= 3 ? 4 : 2)
    qlora_gemv_kernel(const uint16_t* X, const uint8_t* codes, const uint8_t* c2, const float* c1, char* ws,
                      const uint16_t* A, int N, uint32_t kr, DecodeParams p) {
  __shared__ __attribute__((aligned(16))) char lut[256 * kPairStride];   // 64 KiB
  __shared__ float red[kRows * M];
  __shared__ uint32_t tag;
  const int tile = (int)blockIdx.x;
  p.X = X;
  p.codes = codes;
  p.c2 = c2;
  p.c1 = c1;
  p.ws = ws;
  p.A = A;
  p.K = (int)((kr & 0xFFFFFFu) << 6);   // kr = K / 64 | r << 24
  p.N = N;
  const int r = (int)(kr >> 24);
  p.r = r;
  p.n_htiles = r;                                                // one LoRA-down workgroup per row of A
  p.n_wtiles = (N + (kFull ? 2 * kRows : kRows) - 1) / (kFull ? 2 * kRows : kRows);   // the weight tiles
  if (tile < p.n_htiles) {
    uint64_t hticket = 0;
    if (threadIdx.x == 0) hticket = take_down_ticket(p, tile);
    gemv_down_tile<M>(p, tile, red, &tag, hticket);
    return;
  }
  gemv_tile<M, kNPL, kFull>(p, tile - p.n_htiles, lut, red, &tag);
}

typedef void (*GemvKernel)(const uint16_t*, const uint8_t*, const uint8_t*, const float*, char*, const uint16_t*, int,
                           uint32_t, DecodeParams);
template <int M>
GemvKernel gemv_kernel(int npl, bool full) {
  if (full) {   // 32-row tiles: whole pieces per lane over all of K (the launcher's condition)
    switch (npl) {
      case 1: return qlora_gemv_kernel<M, 1, true>;
      case 2: return qlora_gemv_kernel<M, 2, true>;
      case 3: return qlora_gemv_kernel<M, 3, true>;
      default: return qlora_gemv_kernel<M, 4, true>;
    }
  }
  switch (npl) {
    case 1: return qlora_gemv_kernel<M, 1, false>;
    case 2: return qlora_gemv_kernel<M, 2, false>;
    case 3: return qlora_gemv_kernel<M, 3, false>;
    case 4: return qlora_gemv_kernel<M, 4, false>;
    default: return qlora_gemv_kernel<M, 0, false>;
  }
}

}  // namespace

hipError_t launch_gemv_fwd(const DecodeParams& p0, hipStream_t s) {
  DecodeParams p = p0;
  p.n_htiles = p.r;   // one LoRA-down workgroup per row of A
  // 32-row tiles where 16-row tiles need three or more rounds of resident
  // workgroups (two per CU, one at M = 4) and 32-row tiles fewer, and every
  // lane takes whole pieces of all of K (K a multiple of 2048, at most 4
  // pieces, c2 rows dword-aligned).  The time steps with each round and
  // grows little with a workgroup's bytes: 22016 x 4096, M = 1, r = 64
  // 15.7 -> 13.8 us, 11008 x 4096 at M = 4 17.3 -> 16.3 us; from two rounds
  // to one it was a toss-up (4096^2 at M = 4 slower by 10 %).
  const int64_t slots = (p.M == 4 ? 1 : 2) * (int64_t)cu_count();
  const int64_t t16 = (p.N + kRows - 1) / kRows, t32 = (p.N + 2 * kRows - 1) / (2 * kRows);
  const int64_t rounds16 = (t16 + p.r + slots - 1) / slots, rounds32 = (t32 + p.r + slots - 1) / slots;
  const bool full = p.c2_vec && p.K % 2048 == 0 && p.K / 2048 <= 4 && rounds16 >= 3 && rounds32 < rounds16;
  if (full) p.n_wtiles = (int)t32;
  const int hp = full ? p.K / 32 : p.K / 64, npl = p.c2_vec ? (hp + 63) / 64 : 0;
  const GemvKernel k = p.M == 1 ? gemv_kernel<1>(npl, full)
                      : p.M == 2 ? gemv_kernel<2>(npl, full)
                      : p.M == 3 ? gemv_kernel<3>(npl, full)
                                 : gemv_kernel<4>(npl, full);
  const dim3 grid(p.n_htiles + p.n_wtiles);
  // K / 64 and r share a dword of the preloaded arguments (K < 2^30, r <= 128:
  // the decode path's own limits)
  const uint32_t kr = (uint32_t)(p.K >> 6) | ((uint32_t)p.r << 24);
  hipLaunchKernelGGL(k, grid, dim3(kThreads), 0, s, p.X, p.codes, p.c2, p.c1, p.ws, p.A, p.N, kr, p);
  return hipGetLastError();
}

}  // namespace dec
}  // namespace qlora
