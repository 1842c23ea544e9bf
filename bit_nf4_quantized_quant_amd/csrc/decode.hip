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
// Work split.  A workgroup takes 64 output rows (four 16-row MFMA groups)
// over one of S equal slices of K; its 8 waves split the slice's NF4 blocks
// (at most 4 each).  A wave holds the X values of its blocks in registers and
// uses each X fragment for all four row groups, so X crosses the L2 once per
// 64 weight rows and K slice (at M = 16 as many bytes as the codes) instead
// of once per 16 rows.  S is chosen so that the slices fill the chip.
//
// LoRA.  The workgroups also form H = X A^T, each from the X already in its
// registers: workgroup (g, s) computes the slice-s partial of columns
// j = g, g + G, ... of H (G = row groups), right after its X arrives, and
// publishes it as tagged words.  Slice s adds s H[:, J_s] B[:, J_s]^T for
// its share J_s of the r columns to its partial product, reading the S
// partials of those columns after its stream (they were published long
// before).  The slices then exchange their partial products: each owns
// 64 / S rows, publishes the other rows and sums the S partials of its own
// rows in slice order (so results do not depend on arrival order).
//
// Every wait is bounded (about 1 ms): a lane whose H partial or product
// partial does not arrive computes the value itself from X, A, B and the
// packed weight, and counts the fallback in the workspace's give-up counter.
//
// Each 64-element NF4 block is one scaling unit: the levels enter bf16
// 16x16x32 MFMAs as bf16(kappa level) and the block's fp32 constant c_hat
// scales the block's partial product in fp32 afterwards, i.e. the weight used
// is bf16(level) * c_hat rather than bf16(level * c_hat): the same size of
// rounding, one place earlier.  A code byte indexes the pair table of bf16
// levels in LDS.
#include <algorithm>

#include "decode_common.h"

namespace qlora {
namespace dec {
namespace {

constexpr int kTileRows = 64;                  // output rows per workgroup
constexpr int kGroups = kTileRows / 16;        // 16-row MFMA groups
constexpr int kMaxWaveBlocks = 4;              // NF4 blocks per wave (X held in registers)
constexpr int kMaxSlices = 16;
constexpr int kMaxHCols = 16;                  // LoRA-down columns per workgroup

__device__ __forceinline__ f32x4 mfma16(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                  0, 0);
}

__device__ __forceinline__ u32x4 ld128(const rsrc_t& rs, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
}

// LDS scratch in the pair table: the upper halves of its 256-byte entries
// (bytes 128..255, never read by the lookups) hold 8192 floats at any time;
// the lower halves hold 8192 more once the weight stream is over.
__device__ __forceinline__ float* spare(char* lut, int f) {
  return reinterpret_cast<float*>(lut + ((f >> 5) << 8) + 128 + ((f & 31) << 2));
}
__device__ __forceinline__ float* lower(char* lut, int f) {
  return reinterpret_cast<float*>(lut + ((f >> 5) << 8) + ((f & 31) << 2));
}
constexpr int kYredOff = 0;       // spare: [8 waves][1024] product wave partials (after the LoRA-up)
constexpr uint32_t kMissing = 0xFFFFFFFFu;   // a partial that never came (a NaN pattern)

// Up to 2 blocks per wave (slice rows of at most 512 bytes) the tile's
// packed codes are loaded a row at a time (consecutive lanes on consecutive
// 16-byte pieces: whole cache lines per load) and staged in the pair table's
// spare halves: byte b of row r in 128-byte piece 4 r + b / 128, its 32-byte
// quarters rotated by r % 4 so that the rows one MFMA operand read touches
// spread over the banks.  Longer slices load each MFMA operand straight from
// memory (16 rows x 8 bytes per load), which keeps the LDS at 72 KiB there
// too: two workgroups share a compute unit either way.
template <int kNB>
struct Stage {
  static constexpr bool kOn = kNB <= 2;
  static constexpr int kChunks = kOn ? 8 * kNB * 32 / 16 * kTileRows / kWaves / 64 : 1;   // 16-B loads per lane
  __device__ static __forceinline__ char* at(char* lut, int row, int b) {
    return lut + ((4 * row + (b >> 7)) << 8) + 128 + ((b & 127) ^ ((row & 3) << 5));
  }
};

// Y[m][row] * kappa computed by one lane from X, the packed weight, A and B,
// for an exchange whose partial never came; counted on the give-up counter.
// lev: the 16 levels bf16(kappa level[c]) as floats (LDS).
__device__ __attribute__((noinline)) float lane_output(const uint16_t* X, const uint8_t* codes, const uint8_t* c2,
                                                     const float* c1, float mu, const float* lev,
                                                     const uint16_t* A, const uint16_t* B, int K, int r, float scale,
                                                     int m, int row, char* ws) {
  __hip_atomic_fetch_add(reinterpret_cast<unsigned*>(ws + kGiveupCounter), 1u, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  const int nblk = K / 64;
  float y = 0.f;
  for (int b = 0; b < nblk; ++b) {
    const size_t flat = (size_t)row * nblk + b;
    const float chat = dequant_constant(c2[flat], c1[flat >> 8], mu);
    float part = 0.f;
    for (int k = 0; k < 64; ++k) {
      const uint32_t byte = codes[(size_t)row * (K / 2) + b * 32 + (k >> 1)];
      const uint32_t c = (k & 1) ? (byte >> 4) : (byte & 15u);
      part = __builtin_fmaf(__uint_as_float((uint32_t)X[(size_t)m * K + b * 64 + k] << 16), lev[c], part);
    }
    y = __builtin_fmaf(chat, part, y);
  }
  for (int j = 0; j < r; ++j) {
    float h = 0.f;   // H[m][j], here in plain fp32 multiply-adds
    for (int k = 0; k < K; ++k)
      h = __builtin_fmaf(__uint_as_float((uint32_t)X[(size_t)m * K + k] << 16),
                         __uint_as_float((uint32_t)A[(size_t)j * K + k] << 16), h);
    y = __builtin_fmaf(scale * h, __uint_as_float((uint32_t)B[(size_t)row * r + j] << 16), y);
  }
  return y;
}

// kNB: NF4 blocks per wave at most (the launcher's bound for this shape).
// kEarly: the pointers and sizes the first loads need come first in the
// argument list, ahead of the parameter block, and are preloaded into scalar
// registers at dispatch (this file is built with kernarg preloading), so the
// X, A and code loads go out without waiting for a kernel-argument fetch; the
// c2 pointer and the rest of the block arrive behind them.  kr = K / 64 |
// r << 24, msh = M | S << 8 | hcols << 16.  Otherwise the whole block is
// fetched first, in one round trip (the leading arguments unused): grids of
// more than one round of workgroups ran faster that way (11008 x 4096, M =
// 16: 21.8 against 22.4 us), those of one round slower (4096 x 4096, M = 16:
// 11.7 against 10.6 us).
template <int kNB, bool kEarly>
__global__ void __launch_bounds__(kThreads, 2)
    qlora_decode_kernel(const uint16_t* X, const uint16_t* A, const uint8_t* codes, const float* c1, char* ws,
                        int n_out, uint32_t kr, uint32_t msh, DecodeParams p) {
  // pair table (64 KiB); its spare halves hold the staged codes and then the
  // reductions
  __shared__ __attribute__((aligned(16))) char lut[256 * kPairStride];
  __shared__ float hbuf[2048];   // LoRA-down wave partials, then the H partials read back
  __shared__ float lev[16];
  __shared__ uint32_t tag_lds;
  if constexpr (kEarly) {
    p.X = X;
    p.A = A;
    p.codes = codes;
    p.c1 = c1;
    p.ws = ws;
    p.N = n_out;
    p.K = (int)((kr & 0xFFFFFFu) << 6);
    p.r = (int)(kr >> 24);
    p.M = (int)(msh & 0xFFu);
    p.S = (int)((msh >> 8) & 0xFFu);
    p.hcols = (int)(msh >> 16);
    p.G = (n_out + kTileRows - 1) / kTileRows;
    p.n_htiles = 0;
    p.n_wtiles = p.G * p.S;
  } else {
    QLORA_FETCH_ARGS(p);
    asm volatile("" ::"s"(p.G), "s"(p.S), "s"(p.hcols), "s"(p.Ypart), "s"(p.Hpart));
  }
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nl = lane & 15, g4 = lane >> 4;
  const int S = p.S;
  const int bid = (int)blockIdx.x;
  // workgroup -> (row group g, slice s): a row group's slices are adjacent
  const int g = __builtin_amdgcn_readfirstlane(bid / S), s = bid - g * S;
  const int n0 = g * kTileRows;
  const int K = p.K, N = p.N, M = p.M, r = p.r;
  const int nblk = K >> 6;
  float mu = 0.f;
  if constexpr (!kEarly) mu = load_mean(p);
  // this launch's epoch: wave 0 reads this workgroup's counter ahead of
  // every other load, and only then does thread 0 add the workgroup's share
  // (a read after it could see the launch's last share and the next epoch);
  // the tag, epoch + 1, reaches the other waves through LDS
  uint32_t epoch = 0;
  if (wave == 0) epoch = slot_epoch(p.ws, kWeightCtr, (uint32_t)bid);
  if (threadIdx.x == 0) (void)take_weight_ticket(p, bid);

  // this wave's blocks: the slice [sb0, sb1) split over the 8 waves
  const int sb0 = s * nblk / S, sb1 = (s + 1) * nblk / S;
  const int len = sb1 - sb0, per = len >> 3, rem = len & 7;
  const int wb0 = sb0 + wave * per + min(wave, rem);
  const int nbw = per + (wave < rem ? 1 : 0);
  int blk[kNB];   // clamped: every load is issued whatever the wave's share
#pragma unroll
  for (int i = 0; i < kNB; ++i) blk[i] = min(wb0 + min(i, max(nbw - 1, 0)), nblk - 1);

  const rsrc_t rx = make_rsrc(p.X, (uint32_t)M * K * 2);         // rows >= M read as zero
  const rsrc_t ra = make_rsrc(p.A, (uint32_t)r * K * 2);         // rows >= r read as zero
  const rsrc_t rc = make_rsrc(p.codes, (uint32_t)N * (K / 2));   // rows >= N read as zero
  const rsrc_t r2 = make_rsrc(p.c2, (uint32_t)N * nblk);
  const rsrc_t r1 = make_rsrc(p.c1, (uint32_t)((N * nblk + 255) / 256) * 4u);

  // LoRA-down columns of this workgroup: j = g hc + c, c < count (<= 16)
  const int hc = p.hcols;
  const int count = r > 0 ? max(0, min(hc, r - g * hc)) : 0;
  const uint32_t jrow = nl < count ? (uint32_t)(g * hc + nl) : (uint32_t)r;   // r: reads zero

  // Loads: X, then (workgroups that produce H) A, the LoRA-down operands,
  // then codes and the block constants.  Lane (nl, g4) holds, per block,
  // elements 16 g4 .. 16 g4 + 15: the MFMA operands of the block's two
  // 32-wide steps (X row nl as the A operand, weight row or A row nl as the
  // B operand).
  u32x4 x[kNB][2];
#pragma unroll
  for (int i = 0; i < kNB; ++i) {
    const uint32_t kb = (uint32_t)blk[i] * 128u + 32u * g4;
    x[i][0] = ld128(rx, (uint32_t)nl * K * 2 + kb);
    x[i][1] = ld128(rx, (uint32_t)nl * K * 2 + kb + 16);
  }
  u32x4 a[kNB][2];
  if (count > 0) {
#pragma unroll
    for (int i = 0; i < kNB; ++i) {
      const uint32_t kb = (uint32_t)blk[i] * 128u + 32u * g4;
      a[i][0] = ld128(ra, jrow * (uint32_t)K * 2 + kb);
      a[i][1] = ld128(ra, jrow * (uint32_t)K * 2 + kb + 16);
    }
  }
  // The tile's codes, row by row: wave w loads rows 8 w .. 8 w + 7 of the
  // slice, consecutive lanes on consecutive 16-byte pieces of a row (whole
  // cache lines per load), for the LDS stage.  Pieces past the wave's rows
  // repeat its last piece.
  const int rowp = 2 * len;                    // 16-byte pieces per row of the slice
  const int wpieces = 8 * rowp;                // the wave's pieces
  u32x4 cv[Stage<kNB>::kChunks];
  uint32_t cdst[Stage<kNB>::kChunks];
  u32x2 cwd[Stage<kNB>::kOn ? 1 : kNB][kGroups];   // longer slices: the operands themselves
  if constexpr (Stage<kNB>::kOn) {
#pragma unroll
    for (int u = 0; u < Stage<kNB>::kChunks; ++u) {
      const int idx = min(u * 64 + lane, wpieces - 1);
      const int rr = idx / rowp, cc = idx - rr * rowp;
      const uint32_t row = (uint32_t)(n0 + 8 * wave + rr);
      cv[u] = ld128(rc, row * (uint32_t)(K / 2) + (uint32_t)sb0 * 32u + (uint32_t)cc * 16u);
      cdst[u] = (uint32_t)(Stage<kNB>::at(lut, 8 * wave + rr, cc * 16) - lut);
    }
  } else {
#pragma unroll
    for (int q = 0; q < kGroups; ++q) {
      const uint32_t row = (uint32_t)(n0 + 16 * q + nl);
#pragma unroll
      for (int i = 0; i < kNB; ++i)
        cwd[i][q] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                                                  rc, row * (uint32_t)(K / 2) + (uint32_t)blk[i] * 32u + 8u * g4, 0, 0));
    }
  }
  // (nothing below moves above the code loads: the c2 pointer comes with the
  // parameter block, and waiting for it there would hold them back)
  if constexpr (kEarly) __builtin_amdgcn_sched_barrier(0);
  // Block constants with one lane per tile row (row n0 + lane): the c2 byte
  // of each of the wave's blocks, and c1 of its first and last block (a run
  // of <= 4 blocks crosses at most one 256-block boundary of the flattened
  // constant index).  They reach the MFMA layout by lane permutes.
  const uint32_t f0 = (uint32_t)(n0 + lane) * (uint32_t)nblk + (uint32_t)blk[0];
  uint32_t c2r[kNB];
#pragma unroll
  for (int i = 0; i < kNB; ++i) c2r[i] = __builtin_amdgcn_raw_buffer_load_b8(r2, f0 + (uint32_t)i, 0, 0);
  const float c1a = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r1, (f0 >> 8) * 4u, 0, 0));
  const float c1b = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r1, ((f0 + kNB - 1) >> 8) * 4u, 0, 0));
  // (the mean's pointer comes with the parameter block, after the loads)
  if constexpr (kEarly) mu = load_mean(p);
  build_pair_table<kThreads>(p, lut);   // while the loads are in flight
  if (threadIdx.x < 16) {
    uint32_t hv = 0;
#pragma unroll
    for (int c = 0; c < 16; ++c) hv = (int)threadIdx.x == c ? p.hi[c] : hv;
    lev[threadIdx.x] = __uint_as_float(hv << 16);
  }

  // LoRA-down: this wave's part of H_s[m][j] for the workgroup's columns
  if (count > 0) {
    f32x4 th = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < kNB; ++i) {
      if (i < nbw) {
        th = mfma16(x[i][0], a[i][0], th);
        th = mfma16(x[i][1], a[i][1], th);
      }
    }
    // th[v] = partial H[m = 4 g4 + v][column nl]
#pragma unroll
    for (int v = 0; v < 4; ++v) hbuf[wave * 256 + (4 * g4 + v) * 16 + nl] = th[v];
  }
  if (threadIdx.x == 0) {
    asm volatile("" : "+v"(epoch));   // (keeps the use of the counter's value, and its wait, here)
    tag_lds = epoch + 1u;
  }
  __syncthreads();
  const uint32_t tag = tag_lds;
  if (count > 0 && threadIdx.x < 256) {
    const int m = threadIdx.x >> 4, col = threadIdx.x & 15;
    if (m < M && col < count) {
      float h = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) h += hbuf[w * 256 + threadIdx.x];
      st_tagged(&p.Hpart[((size_t)s * M + m) * r + g * hc + col], tag, h);
    }
  }
  // codes into the stage
  if constexpr (Stage<kNB>::kOn) {
#pragma unroll
    for (int u = 0; u < Stage<kNB>::kChunks; ++u) *reinterpret_cast<u32x4*>(lut + cdst[u]) = cv[u];
    __syncthreads();
  }

  // The weight stream: per block and row group, two MFMAs on bf16 levels and
  // the block constant applied to their sum in fp32.
  const uint32_t lane4 = (uint32_t)(lane & 31) * 4u;
  f32x4 acc[kGroups];
#pragma unroll
  for (int q = 0; q < kGroups; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < kNB; ++i) {
    if (i >= nbw) break;
    // this row lane's c_hat of block i, then the MFMA layout's: row 16 q + nl
    uint32_t c2 = c2r[i];
    asm volatile("" : "+v"(c2));   // (keeps any widening here, not next to the load)
    const float chat_row = dequant_constant(c2, ((f0 + i) >> 8) == (f0 >> 8) ? c1a : c1b, mu);
#pragma unroll
    for (int q = 0; q < kGroups; ++q) {
      const float chat = __int_as_float(__builtin_amdgcn_ds_bpermute(4 * (16 * q + nl), __float_as_int(chat_row)));
      // 8 code bytes of row 16 q + nl: elements 16 g4 .. 16 g4 + 15 of the block
      u32x2 cw;
      if constexpr (Stage<kNB>::kOn)
        cw = *reinterpret_cast<const u32x2*>(Stage<kNB>::at(lut, 16 * q + nl, (blk[i] - sb0) * 32 + 8 * g4));
      else
        cw = cwd[i][q];
      f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t w = cw[h];
        u32x4 wv;
        wv[0] = *reinterpret_cast<const uint32_t*>(lut + pair_addr<0>(w, lane4));
        wv[1] = *reinterpret_cast<const uint32_t*>(lut + pair_addr<1>(w, lane4));
        wv[2] = *reinterpret_cast<const uint32_t*>(lut + pair_addr<2>(w, lane4));
        wv[3] = *reinterpret_cast<const uint32_t*>(lut + pair_addr<3>(w, lane4));
        t = mfma16(x[i][h], wv, t);
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[q][v] = __builtin_fmaf(chat, t[v], acc[q][v]);
    }
  }

  // LoRA-up of this slice's columns J_s = [jl, jl + nj): read the S partials
  // of H[:, J_s] (thread: one (slice, m, j) word each, up to 4) and the
  // wave's B operands, all issued before any wait.
  const int jl = s * r / S, nj = (s + 1) * r / S - jl;
  const int nsteps = (nj + 31) >> 5;
  const int nwords = S * M * nj;   // <= M r <= 2048
  uint64_t hw[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int idx = threadIdx.x + u * kThreads;
    if (idx < nwords) {
      const int sp = idx / (M * nj), rest = idx - sp * (M * nj);
      const int m = rest / nj, jj = rest - m * nj;
      hw[u] = ld_tagged(&p.Hpart[((size_t)sp * M + m) * r + jl + jj]);
    }
  }
  // B operands: items (row group q, 32-wide step st) with q = wave % 4 and
  // st = wave / 4 + 2 u
  const int qb = wave & 3;
  u32x4 bop[2];
  {
    const rsrc_t rb = make_rsrc(p.B, (uint32_t)N * r * 2);   // rows past N read as zero
    const uint32_t brow = (uint32_t)(n0 + 16 * qb + nl);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      bop[u] = u32x4{0u, 0u, 0u, 0u};
      const int jj0 = 32 * ((wave >> 2) + 2 * u) + 8 * g4;
      if (jj0 < nj) {
        const uint32_t off = (brow * (uint32_t)r + (uint32_t)(jl + jj0)) * 2u;
        if (p.b_vec && (jl % 8) == 0 && (nj % 8) == 0) {
          bop[u] = ld128(rb, off);
        } else {
          uint32_t e[8];
#pragma unroll
          for (int q = 0; q < 8; ++q)
            e[q] = jj0 + q < nj ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rb, off + 2 * q, 0, 0) : 0u;
#pragma unroll
          for (int q = 0; q < 4; ++q) bop[u][q] = e[2 * q] | (e[2 * q + 1] << 16);
        }
      }
    }
  }
  // partials, polled, into LDS (a missing one as kMissing)
  {
    uint64_t deadline = 0;   // set at the first miss
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int idx = threadIdx.x + u * kThreads;
      if (idx < nwords) {
        const int sp = idx / (M * nj), rest = idx - sp * (M * nj);
        const int m = rest / nj, jj = rest - m * nj;
        float v;
        if (!poll_tagged(&p.Hpart[((size_t)sp * M + m) * r + jl + jj], hw[u], tag, deadline, &v))
          v = __uint_as_float(kMissing);
        hbuf[idx] = v;
      }
    }
  }
  __syncthreads();   // every wave's stream is over: the table's lower halves are free
  // H[m][j] for j in J_s: the S partials in slice order (or, if one is
  // missing, computed here), scaled by s into the lower halves
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int idx = threadIdx.x + u * kThreads;
    if (idx < M * nj) {
      const int m = idx / nj, jj = idx - m * nj;
      float h = 0.f;
      bool missing = false;
      for (int sp = 0; sp < S; ++sp) {
        const float v = hbuf[sp * M * nj + idx];
        missing = missing || __float_as_uint(v) == kMissing;
        h += v;
      }
      if (missing) h = lane_lora_down(p.X, p.A, K, m, jl + jj, p.ws);
      if (g == 0 && p.H) p.H[(size_t)m * r + jl + jj] = h;
      *lower(lut, m * 128 + jj) = p.scale * h;
    }
  }
  __syncthreads();
  if (nj > 0) {
    // A operand: s H[m = nl][jl + jj0 .. + 7] as bf16 high + low parts (two
    // products: fp32 accuracy); zero past M or nj
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int st = (wave >> 2) + 2 * u;
      if (st >= nsteps) break;
      const int jj0 = 32 * st + 8 * g4;
      u32x4 ahi = {0u, 0u, 0u, 0u}, alo = {0u, 0u, 0u, 0u};
      if (nl < M) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float v[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int jj = jj0 + 2 * q + e;
            v[e] = jj < nj ? *lower(lut, nl * 128 + jj) : 0.f;
          }
          const uint32_t hi = pack_bf16x2(v[0], v[1]);
          ahi[q] = hi;
          alo[q] = pack_bf16x2(v[0] - bf16_lo(hi), v[1] - bf16_hi(hi));
        }
      }
#pragma unroll
      for (int q = 0; q < kGroups; ++q) {
        if (q == qb) {
          acc[q] = mfma16(ahi, bop[u], acc[q]);
          acc[q] = mfma16(alo, bop[u], acc[q]);
        }
      }
    }
  }
  // acc[q][v] = partial Y[m = 4 g4 + v][row 16 q + nl]: the waves' sums meet
#pragma unroll
  for (int q = 0; q < kGroups; ++q)
#pragma unroll
    for (int v = 0; v < 4; ++v) *spare(lut, kYredOff + wave * 1024 + q * 256 + (4 * g4 + v) * 16 + nl) = acc[q][v];
  __syncthreads();

  // Exchange.  Output o = 256 q + 16 m + nl (row rt = 16 q + nl of the
  // tile); the thread holds o = t and t + 512.  Slice s owns rows
  // [os(s), os(s + 1)), os(s) = 64 s / S: it publishes the other rows'
  // partials and sums its own.  Layout per (row group, owner, source slice):
  // RS = ceil(64 / S) rows of M words.
  const int RS = (kTileRows + S - 1) / S;
  const size_t ybase = (size_t)g * S * S * RS * M;
  float own[2];
  bool owns[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int o = threadIdx.x + u * kThreads;
    const int q = o >> 8, m = (o >> 4) & 15, rt = 16 * q + (o & 15);
    float y = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) y += *spare(lut, kYredOff + w * 1024 + o);
    own[u] = y;
    owns[u] = false;
    if (m >= M || n0 + rt >= N) continue;
    const int owner = (rt * S + S - 1) / kTileRows;
    if (owner != s) {
      const int lr = rt - owner * kTileRows / S;
      st_tagged(&p.Ypart[ybase + ((size_t)(owner * S + s) * RS + lr) * M + m], tag, y);
    } else {
      owns[u] = true;
    }
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    if (!owns[u]) continue;
    const int o = threadIdx.x + u * kThreads;
    const int q = o >> 8, m = (o >> 4) & 15, rt = 16 * q + (o & 15);
    const int lr = rt - s * kTileRows / S;
    const uint64_t* src = &p.Ypart[ybase + ((size_t)(s * S) * RS + lr) * M + m];   // + sp RS M
    const size_t step = (size_t)RS * M;
    uint64_t wv[kMaxSlices];
#pragma unroll
    for (int sp = 0; sp < kMaxSlices; ++sp)
      if (sp < S && sp != s) wv[sp] = ld_tagged(src + sp * step);
    uint64_t deadline = 0;
    float y = 0.f;
    bool ok = true;
#pragma unroll
    for (int sp = 0; sp < kMaxSlices; ++sp) {
      if (sp >= S) break;
      float v = own[u];
      if (sp != s) ok = ok && poll_tagged(src + sp * step, wv[sp], tag, deadline, &v);
      y += v;
    }
    if (!ok)
      y = lane_output(p.X, p.codes, p.c2, p.c1, mu, lev, p.A, p.B, K, r, p.scale, m, n0 + rt, p.ws);
    y *= p.inv_kappa;
    p.Y[(size_t)m * N + n0 + rt] = (uint16_t)(pack_bf16x2(y, 0.f) & 0xFFFFu);
  }
}

typedef void (*DecodeKernel)(const uint16_t*, const uint16_t*, const uint8_t*, const float*, char*, int, uint32_t,
                             uint32_t, DecodeParams);
DecodeKernel decode_kernel(int nb, bool early) {
  if (early) {
    switch (nb) {
      case 1: return qlora_decode_kernel<1, true>;
      case 2: return qlora_decode_kernel<2, true>;
      case 3: return qlora_decode_kernel<3, true>;
      default: return qlora_decode_kernel<4, true>;
    }
  }
  switch (nb) {
    case 1: return qlora_decode_kernel<1, false>;
    case 2: return qlora_decode_kernel<2, false>;
    case 3: return qlora_decode_kernel<3, false>;
    default: return qlora_decode_kernel<4, false>;
  }
}

}  // namespace

// Slices of K: the count that minimises the heaviest compute unit's share
// (workgroups per unit, rounded up, times blocks per workgroup), keeping
// every wave within kMaxWaveBlocks blocks and, where K allows, every wave
// busy (slices of at least 8 blocks); the fewest slices among equals.
int decode_slices(int64_t N, int64_t K) {
  const int64_t G = (N + kTileRows - 1) / kTileRows, nblk = K / 64, cus = cu_count();
  const int64_t most = std::max<int64_t>(1, std::min<int64_t>(kMaxSlices, nblk / kWaves));
  int best = 0;
  int64_t best_cost = 0;
  for (int S = 1; S <= most; ++S) {
    const int64_t slice = (nblk + S - 1) / S;
    if (slice > (int64_t)kWaves * kMaxWaveBlocks) continue;
    const int64_t cost = (G * S + cus - 1) / cus * slice;
    if (best == 0 || cost < best_cost) {
      best = S;
      best_cost = cost;
    }
  }
  if (best == 0) return kMaxSlices;
  // Past one round of resident workgroups (two per CU) the model undercounts
  // the slices' exchange: there the fewest slices that give every CU a
  // workgroup measured faster (M = 16: 22016 x 4096 S = 8 -> 2, 62.1 -> 31.7
  // us; 12288 x 4096, M = 12, r = 32, 4 -> 2, 21.0 -> 19.6; 11008 x 4096 4 ->
  // 2, 21.9 -> 21.6, at M = 8 19.1 -> 19.4).  Within one round the model's
  // choice stays (4096 x 11008: S = 6 instead of 8 was 21.2 -> 24.3 us).
  if (G * best > 2 * cus) {
    int64_t fill = std::max<int64_t>((cus + G - 1) / G, (nblk + kWaves * kMaxWaveBlocks - 1) / (kWaves * kMaxWaveBlocks));
    fill = std::min<int64_t>(std::max<int64_t>(fill, 1), most);
    if ((nblk + fill - 1) / fill <= (int64_t)kWaves * kMaxWaveBlocks) return (int)fill;
  }
  return best;
}

// LoRA-down columns per producing workgroup: as few as the row groups allow,
// and enough that every producer (workgroups g < ceil(r / hcols) of every
// slice) lies among the first cu_count() workgroups, which are resident
// from the start: a consumer never waits for a workgroup that is waiting
// for a free compute unit.
int decode_hcols(int64_t N, int64_t r, int S) {
  if (r == 0) return 1;
  const int64_t G = (N + kTileRows - 1) / kTileRows, cus = cu_count();
  int64_t hc = std::max<int64_t>(1, (r + G - 1) / G);
  // producers: row groups g < P = ceil(r / hc) of every slice, workgroups below P S
  while (hc < kMaxHCols && (r + hc - 1) / hc * S > cus) ++hc;
  return (int)hc;
}

bool decode_supported(int64_t N, int64_t K, int64_t r) {
  const int64_t nblk = K / 64;
  const int S = decode_slices(N, K);
  return (nblk + S - 1) / S <= (int64_t)kWaves * kMaxWaveBlocks && decode_hcols(N, r, S) <= kMaxHCols;
}

size_t decode_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t r) {
  if (M <= 4) return kHpartOff + (size_t)gemv_hcopies((int)M) * gemv_hcopy_words((int)M, (int)r) * sizeof(uint64_t);   // the GEMV path
  const int64_t S = decode_slices(N, K), G = (N + kTileRows - 1) / kTileRows;
  const int64_t RS = (kTileRows + S - 1) / S;
  const size_t hpart = ((size_t)(S * M * r) * sizeof(uint64_t) + 255) & ~(size_t)255;
  const size_t ypart = S > 1 ? (size_t)(G * S * S * RS * M) * sizeof(uint64_t) : 0;
  return kHpartOff + hpart + ypart;
}

hipError_t launch_decode_fwd(const FwdArgs& a, hipStream_t s) {
  DecodeParams p = decode_params(a);
  if (a.M <= 4) return launch_gemv_fwd(p, s);
  const int S = decode_slices(a.N, a.K);
  p.G = (int)((a.N + kTileRows - 1) / kTileRows);
  p.S = S;
  p.hcols = decode_hcols(a.N, a.r, S);
  p.n_htiles = 0;
  p.n_wtiles = p.G * S;
  const size_t hpart = ((size_t)(S * a.M * a.r) * sizeof(uint64_t) + 255) & ~(size_t)255;
  p.Ypart = reinterpret_cast<uint64_t*>(p.ws + kHpartOff + hpart);
  const int64_t nblk = a.K / 64, slice = (nblk + S - 1) / S;
  const int nb = (int)((slice + kWaves - 1) / kWaves);
  // K / 64 (< 2^24), r (<= 128), M (<= 16), S (<= 16) and hcols (<= 16) packed
  // into two preloaded dwords
  const uint32_t kr = (uint32_t)(a.K >> 6) | ((uint32_t)a.r << 24);
  const uint32_t msh = (uint32_t)a.M | ((uint32_t)S << 8) | ((uint32_t)p.hcols << 16);
  const bool early = p.n_wtiles <= 2 * (int64_t)cu_count();   // one round of resident workgroups
  hipLaunchKernelGGL(decode_kernel(nb, early), dim3(p.n_wtiles), dim3(kThreads), 0, s, p.X, p.A, p.codes, p.c1,
                     p.ws, p.N, kr, msh, p);
  return hipGetLastError();
}

}  // namespace dec

size_t decode_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t r) {
  return dec::decode_workspace_bytes(M, N, K, r);
}
bool decode_supported(int64_t M, int64_t N, int64_t K, int64_t r) {
  // (the GEMV passes K / 64 in 24 bits: K < 2^30)
  return M <= 4 ? K < (int64_t(1) << 30) : dec::decode_supported(N, K, r);
}
size_t decode_wait_counter_offset() { return (size_t)dec::kGiveupCounter; }
hipError_t launch_decode_fwd(const FwdArgs& a, hipStream_t s) { return dec::launch_decode_fwd(a, s); }

}  // namespace qlora
