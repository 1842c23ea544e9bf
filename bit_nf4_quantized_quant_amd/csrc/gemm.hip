// LDS-tiled bf16 MFMA engine with operand loaders that dequantize NF4 on the
// way into LDS (gfx950).  Serves the forward at M > 16 and every product of
// the backward.
//
// itwiki "QLoRA", section on the computation: the layer output is
// X doubleDequant(c1, c2, W) + X L1 L2 with bf16 compute; weights are
// dequantized again for every forward and backward product and only the
// input and the LoRA factors receive gradients.  minnong511 "quantization":
// y = W x + (alpha/r) B A x; backward updates A and B only.
//
// The engine computes C[i][j] = sum_k Aop[i][k] * Bop[j][k] for a BM x BN
// output tile, double-buffered in LDS with one barrier per 64-wide reduction
// step.  2 x WN waves each own (BM/2) x (BN/WN) of the tile as 32x32x16 MFMA
// accumulators: 4 waves for 128 x 128 tiles, 8 waves (two per SIMD, so one
// wave's dequantization overlaps the other's MFMAs) for 256 x 256 tiles.
// The two products with the weight (forward Y and backward dX) keep their
// operands in fragment-major tiles (below), or the weight in its own [n][k]
// layout read by transposing LDS reads, with loads two steps ahead; the
// skinny LoRA products stage [rows][64 + 8] bf16 tiles (reduction
// contiguous, 16-byte pad so that 16-byte fragment reads of eight
// consecutive rows hit distinct banks).
//
// Loaders turn every source layout into that LDS form:
//   XRows     bf16 [rows][red] (X, dY) into fragment-major tiles
//   WRows     NF4 codes [rows][K/2] -> bf16 W_deq rows (forward), bit-exact
//   WNat      NF4 codes [n][K/2] -> bf16 W_deq in its own layout (dX)
//   RowsBf16  bf16 [rows][red] (A, B, and the bf16 H^T, dH^T)
//   ColsBf16  bf16 [red][rows] (transposed operands of the LoRA gradients)
// A transposed source is read as 4 x 8 patches (4 rows of 8 contiguous
// elements) and written to LDS as 8 rows of 4 reduction elements.
#include <algorithm>
#include <map>
#include <mutex>
#include <type_traits>
#include <utility>

#include "common.h"
#include "launch.h"

namespace qlora {
namespace {

constexpr int BK = 64;
constexpr int PITCH = BK + 8;  // bf16 elements per LDS row
constexpr int NT = 256;        // threads per workgroup

typedef uint16_t lds_t;

__device__ __forceinline__ void st_lds16(lds_t* p, const u32x4& v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ void st_lds8(lds_t* p, const u32x2& v) { *reinterpret_cast<u32x2*>(p) = v; }
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// Byte b of w (b a constant): one instruction each.
__device__ __forceinline__ uint32_t byte_of(uint32_t w, int b) {
  return __builtin_amdgcn_perm(0u, w, 0x0C0C0C00u | (uint32_t)b);   // v_perm_b32: byte b, zeros above
}

// 64-bit integer minimum (integer instructions only)
__device__ __forceinline__ int64_t lmin(int64_t a, int64_t b) { return a < b ? a : b; }

__device__ __forceinline__ uint32_t lo16(uint32_t a, uint32_t b) { return (a & 0xFFFFu) | (b << 16); }
__device__ __forceinline__ uint32_t hi16(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xFFFF0000u); }

// ---------------------------------------------------------------- loaders

// bf16 source, rows contiguous in the reduction index.
template <int R, int T = NT>
struct RowsBf16 {
  static constexpr int kChunks = R * BK / 8 / T;  // 16-byte chunks per thread
  const uint16_t* src;
  int64_t ld;       // elements between rows
  int rows;         // valid rows from row0
  int red;          // valid reduction length
  int64_t row0;
  bool vec;         // ld % 8 == 0 and 16-byte aligned base
  u32x4 reg[kChunks];

  __device__ __forceinline__ void load(int kt) {
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const int idx = threadIdx.x + c * T;
      const int rr = idx >> 3, ch = idx & 7;
      const int k = kt * BK + ch * 8;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (rr < rows) {
        const uint16_t* p = src + (row0 + rr) * ld + k;
        if (vec && k + 8 <= red) {
          v = ld16(p);
        } else {
          uint32_t e[8];
#pragma unroll
          for (int q = 0; q < 8; ++q) e[q] = (k + q < red) ? p[q] : 0u;
          v = u32x4{e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16)};
        }
      }
      reg[c] = v;
    }
  }
  __device__ __forceinline__ void store(lds_t* t) const {
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const int idx = threadIdx.x + c * T;
      st_lds16(t + (idx >> 3) * PITCH + (idx & 7) * 8, reg[c]);
    }
  }
};

// bf16 source stored [red][rows]: tile row i is source column col0 + i.
template <int R, int T = NT>
struct ColsBf16 {
  static constexpr int kPatches = 2 * R;  // (BK/4) x (R/8) patches of 4 red x 8 cols
  static constexpr int kPer = (kPatches + T - 1) / T;
  const uint16_t* src;
  int64_t ld;    // elements between source rows (reduction steps)
  int cols;      // valid tile rows (source columns) from col0
  int red;       // valid reduction length
  int64_t col0;
  bool vec;
  u32x4 reg[kPer][4];

  __device__ __forceinline__ void load(int kt) {
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int pid = threadIdx.x + u * T;
      if (pid >= kPatches) break;
      const int pr = pid % (BK / 4), pc = pid / (BK / 4);
      const int c = pc * 8;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int k = kt * BK + pr * 4 + q;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (k < red) {
          const uint16_t* p = src + (int64_t)k * ld + col0 + c;
          if (vec && c + 8 <= cols) {
            v = ld16(p);
          } else {
            uint32_t e[8];
#pragma unroll
            for (int z = 0; z < 8; ++z) e[z] = (c + z < cols) ? p[z] : 0u;
            v = u32x4{e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16)};
          }
        }
        reg[u][q] = v;
      }
    }
  }
  __device__ __forceinline__ void store(lds_t* t) const {
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int pid = threadIdx.x + u * T;
      if (pid >= kPatches) break;
      const int pr = pid % (BK / 4), pc = pid / (BK / 4);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        // columns 2w (low halves) and 2w+1 (high halves)
        const u32x2 a = {lo16(reg[u][0][w], reg[u][1][w]), lo16(reg[u][2][w], reg[u][3][w])};
        const u32x2 b = {hi16(reg[u][0][w], reg[u][1][w]), hi16(reg[u][2][w], reg[u][3][w])};
        st_lds8(t + (pc * 8 + 2 * w) * PITCH + pr * 4, a);
        st_lds8(t + (pc * 8 + 2 * w + 1) * PITCH + pr * 4, b);
      }
    }
  }
};

// NF4 weight rows [n][k]: tile row i = weight row n0 + i, reduction = k.  One
// 64-wide reduction step is exactly one NF4 block per row, so every thread
// needs a single constant: thread t dequantizes half a block (32 codes) of row
// t/2 (for R = 128) to bf16( fp32(level * c_hat) ).
template <int R, int T = NT>
struct Nf4Rows {
  static constexpr int kUnits = R * 2 / T;  // half-blocks per thread
  const uint8_t* codes;
  const uint8_t* c2;
  const float* c1;
  float mean;
  int64_t K;
  int rows;
  int64_t row0;
  const float* lut;  // 16 levels in LDS
  u32x4 q[kUnits];
  float chat[kUnits];

  __device__ __forceinline__ void load(int kt) {
#pragma unroll
    for (int u = 0; u < kUnits; ++u) {
      const int idx = threadIdx.x + u * T;
      const int rr = idx >> 1, h = idx & 1;
      if (rr < rows) {
        const int64_t n = row0 + rr;
        q[u] = ld16(codes + n * (K / 2) + kt * 32 + h * 16);
        const int64_t bi = n * (K / 64) + kt;
        chat[u] = dequant_constant(c2[bi], c1[bi >> 8], mean);
      } else {
        q[u] = u32x4{0u, 0u, 0u, 0u};
        chat[u] = 0.f;
      }
    }
  }
  __device__ __forceinline__ void store(lds_t* t) const {
#pragma unroll
    for (int u = 0; u < kUnits; ++u) {
      const int idx = threadIdx.x + u * T;
      const int rr = idx >> 1, h = idx & 1;
      lds_t* dst = t + rr * PITCH + h * 32;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t word = q[u][w];
        u32x4 o;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const float lo = __fmul_rn(lut[(word >> (8 * b)) & 15u], chat[u]);
          const float hi = __fmul_rn(lut[(word >> (8 * b + 4)) & 15u], chat[u]);
          o[b] = pack_bf16x2(lo, hi);
        }
        st_lds16(dst + w * 8, o);
      }
    }
  }
};

// ---------------------------------------------------------------- branch-free loaders

// Loaders of the main products read through buffer resources based at the
// tile's first row, so offsets stay 32-bit for any tensor and the loops carry
// no bounds branches: tile rows past the valid ones repeat the last valid row
// (their outputs are never stored) and reads past a resource's end return 0.
// (Arguments are wave-uniform; readfirstlane states it so that the resource
// lives in scalar registers.)
__device__ __forceinline__ rsrc_t tile_rsrc(const void* base, int64_t off_bytes, int64_t total_bytes) {
  const int64_t rem = total_bytes - off_bytes;
  const uint64_t a = reinterpret_cast<uint64_t>(static_cast<const char*>(base) + off_bytes);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const uint32_t n = __builtin_amdgcn_readfirstlane((uint32_t)lmin(rem, 0xFFFFFFFFll));
  return make_rsrc(reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo), n);
}

// Fragment-major LDS tiles (the pipelined products): an R x 64 operand tile
// is a set of 1 KB blocks, block (s, g) for 16-deep sub-step s (0..3) and
// row group g (32 rows).  A block holds the 64 bf16x8 operands that the lanes
// of a 32x32x16 MFMA take: lane l's operand (row 32 g + l % 32, reduction
// 16 s + 8 h .. +7 with h = l / 32) sits in 16-byte slot
// 32 h + (l % 32 + 2 s + h) % 32.  A fragment read is two contiguous
// (rotated) 512-byte halves; the rotation also spreads the writes over all
// banks when 8 lanes store the 8 chunks of one row (the coalesced order of the
// global loads) or 2 lanes per row store one chunk each.  No padding is
// needed.
template <int R>
__device__ __forceinline__ int frag_slot(int row, int c8) {   // c8: 8-element chunk 0..7 of the step
  const int s = c8 >> 1, half = c8 & 1;
  const int pos = 32 * half + (((row & 31) + 2 * s + half) & 31);
  return ((s * (R / 32) + (row >> 5)) * 64 + pos) * 8;   // in bf16 elements
}
// the slot lane l reads in sub-step s
__device__ __forceinline__ int frag_read_slot(int lane, int s) {
  return 32 * (lane >> 5) + (((lane & 31) + 2 * s + (lane >> 5)) & 31);
}

// bf16 rows [rows][ld], reduction contiguous (X, dY).  kVec: ld % 8 == 0, so a
// row's 8-element chunks are 16-byte aligned.  A reduction tail past the row
// end reads the next row (or zero past the tensor): finite values that the
// other operand's zeros cancel.  kDepth: steps in flight in registers.
// kChecked: the step offset goes in the per-lane offset, which the buffer
// range check covers, so a tail past the tensor's end reads 0.
template <int R, int T, bool kVec, int kDepth = 2, bool kChecked = false>
struct XRows {
  static constexpr int kChunks = R * BK / 8 / T;   // 16-byte chunks per thread: chunk c is
  static_assert(kChunks % 4 == 0, "whole chunks per quarter step");   // row (tid + c T) / 8, part (tid + c T) % 8
  rsrc_t rs;
  uint32_t off[kChunks];
  u32x4 reg[kDepth][kChunks];

  __device__ __forceinline__ void init(const uint16_t* src, int64_t ld, int64_t total_rows, int64_t row0) {
    const int rows = (int)lmin(R, total_rows - row0);
    rs = tile_rsrc(src, row0 * ld * 2, total_rows * ld * 2);
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const int idx = threadIdx.x + c * T;
      off[c] = (uint32_t)(((int64_t)min(idx >> 3, rows - 1) * ld + (idx & 7) * 8) * 2);
    }
  }
  template <int S>
  __device__ __forceinline__ void load(int kt) {
    const int sof = kChecked ? 0 : kt * BK * 2;
    const uint32_t vof = kChecked ? (uint32_t)(kt * BK * 2) : 0u;
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      if (kVec) {
        reg[S][c] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off[c] + vof, sof, 0));
      } else {
        uint32_t e[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) e[q] = __builtin_amdgcn_raw_buffer_load_b16(rs, off[c] + vof + 2 * q, sof, 0);
        reg[S][c] = u32x4{e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16)};
      }
    }
  }
  template <int S, int P>
  __device__ __forceinline__ void prep() {}
  // quarter P of the next step (register slot S when two steps are in flight)
  template <int S, int P>
  __device__ __forceinline__ void store_part(lds_t* t) const {
    constexpr int s = kDepth == 2 ? S : 0;
#pragma unroll
    for (int c = P; c < kChunks; c += 4) {
      const int idx = threadIdx.x + c * T;
      st_lds16(t + frag_slot<R>(idx >> 3, idx & 7), reg[s][c]);
    }
  }
  // pipeline hooks: step kt0 into LDS buffer t (and the following step in flight)
  __device__ __forceinline__ void prologue(int kt0, int last, lds_t* t) {
    load<0>(kt0);
    store_part<0, 0>(t);
    store_part<0, 1>(t);
    store_part<0, 2>(t);
    store_part<0, 3>(t);
    if (kDepth == 2) load<kDepth - 1>(min(kt0 + 1, last));
  }
  // at the start of step kt: issue the loads of the step kDepth ahead into slot S
  template <int S>
  __device__ __forceinline__ void ahead(int kt, int last) {
    load<kDepth == 2 ? S : 0>(min(kt + kDepth, last));
  }
};

// Eight codes (one dword of packed nibbles) to eight bf16 weights,
// bf16( fp32(level * c_hat) ), bit-exact with W_deq, in two halves: fetch8
// issues one pair-table read per code byte (the table's byte address is the
// whole LDS address), finish8 scales and rounds.  A product step issues the
// reads of a sub-step before its matrix-core instructions and the rest after
// them (the compiler schedules within that).
struct Levels8 {
  float2 v[4];
};
__device__ __forceinline__ Levels8 fetch8(uint32_t word, const float2* lut2) {
  Levels8 l;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const uint32_t off = ((word >> (8 * b)) & 0xFFu) * 8u;
    l.v[b] = *reinterpret_cast<const float2*>(reinterpret_cast<const char*>(lut2) + off);
  }
  return l;
}
__device__ __forceinline__ u32x4 finish8(const Levels8& l, float chat) {
  u32x4 o;
#pragma unroll
  for (int b = 0; b < 4; ++b) o[b] = pack_bf16x2(__fmul_rn(l.v[b].x, chat), __fmul_rn(l.v[b].y, chat));
  return o;
}

// NF4 weight rows [n][k] (forward): unit u of a thread is half a block (32
// codes, one constant) of row (tid + u T) / 2, expanded to
// bf16( fp32(level * c_hat) ), bit-exact with W_deq.
template <int R, int T>
struct WRows {
  static constexpr int kUnits = R * 2 / T;
  rsrc_t rc, r2, r1;
  uint32_t coff[kUnits];   // code bytes of this half-block at kt = 0 (tile-relative)
  uint32_t boff[kUnits];   // its block index at kt = 0 (tile-relative)
  uint32_t bglob[kUnits];  // its global block index at kt = 0
  float mean;
  const float2* lut2;
  u32x4 q[2][kUnits];      // two steps in flight
  uint32_t c2v[2][kUnits];
  float c1v[2][kUnits];
  float chat[kUnits];      // constants of the step being stored
  Levels8 lv[kUnits];      // levels of the chunk being stored

  __device__ __forceinline__ void init(const uint8_t* codes, const uint8_t* c2, const float* c1, float mu,
                                       int64_t N, int64_t K, int64_t row0, const float2* lut2_) {
    const int rows = (int)lmin(R, N - row0);
    const int64_t nb = K / BK;
    rc = tile_rsrc(codes, row0 * (K / 2), N * (K / 2));
    r2 = tile_rsrc(c2, row0 * nb, N * nb);
    r1 = tile_rsrc(c1, 0, ((N * nb + 255) / 256) * 4);
    mean = mu;
    lut2 = lut2_;
#pragma unroll
    for (int u = 0; u < kUnits; ++u) {
      const int idx = threadIdx.x + u * T;
      const int rr = min(idx >> 1, rows - 1), h = idx & 1;
      coff[u] = (uint32_t)(rr * (K / 2) + h * 16);
      boff[u] = (uint32_t)(rr * nb);
      bglob[u] = (uint32_t)((row0 + rr) * nb);
    }
  }
  template <int S>
  __device__ __forceinline__ void load(int kt) {
#pragma unroll
    for (int u = 0; u < kUnits; ++u) {
      q[S][u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rc, coff[u], kt * 32, 0));
      c2v[S][u] = __builtin_amdgcn_raw_buffer_load_b8(r2, boff[u], kt, 0);
      c1v[S][u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r1, ((bglob[u] + kt) >> 8) * 4, 0, 0));
    }
  }
  // chunk P (8 codes) of every unit of the step held in slot S
  template <int S, int P>
  __device__ __forceinline__ void store_part(lds_t* t) {
#pragma unroll
    for (int u = 0; u < kUnits; ++u) store_unit<S, P>(t, u);
  }
  template <int S, int P>
  __device__ __forceinline__ void prep() {
#pragma unroll
    for (int u = 0; u < kUnits; ++u) lv[u] = fetch8(q[S][u][P], lut2);
  }
  template <int S, int P>
  __device__ __forceinline__ void store_unit(lds_t* t, int u) {
    if (P == 0) chat[u] = dequant_constant(c2v[S][u], c1v[S][u], mean);
    const int idx = threadIdx.x + u * T;
    const int row = idx >> 1, h = idx & 1;
    st_lds16(t + frag_slot<R>(row, 4 * h + P), finish8(lv[u], chat[u]));
  }
  __device__ __forceinline__ void prologue(int kt0, int last, lds_t* t) {
    load<0>(kt0);
    prep<0, 0>();
    store_part<0, 0>(t);
    prep<0, 1>();
    store_part<0, 1>(t);
    prep<0, 2>();
    store_part<0, 2>(t);
    prep<0, 3>();
    store_part<0, 3>(t);
    load<1>(min(kt0 + 1, last));
  }
  template <int S>
  __device__ __forceinline__ void ahead(int kt, int last) {
    load<S>(min(kt + 2, last));
  }
};

// NF4 weight as the reduction-side operand of dX = dY W_deq: a step is 64
// weight rows n (the reduction) by BN columns k (the output), expanded to
// bf16( fp32(level * c_hat) ) (bit-exact with W_deq) into LDS in the
// weight's own layout, [64 n][BN k] at a row stride of kRowBytes.  Unit c of
// row n is 32 consecutive codes (one 16-byte load, one block constant) and
// 64 bytes of LDS, whose four 16-byte pieces sit in the order P ^ swz(n, c).
// A 16-byte store is served 8 lanes (128 bytes) at a time: with rows 64
// (mod 128) bytes apart, the piece order puts each such group of lanes on 8
// different 16-byte bank groups, and a transposing read (4 rows x 64 bytes
// per half wave) still covers each row's unit whole.  Rows past N get
// c_hat = 0, so they add nothing; step offsets go in the per-lane offset,
// which the buffer range check covers, so codes past the tensor read 0.
template <int BN, int T>
struct WNat {
  static_assert(BN == 128 || BN == 256, "tile widths with a conflict-free piece order");
  static constexpr int kRowBytes = BN * 2 + 64;
  static constexpr int kUnits = 64 * (BN / 32) / T;
  static_assert(kUnits >= 1 && 64 * (BN / 32) % T == 0, "whole units per thread");
  __host__ __device__ static constexpr int swz(int n, int c) {
    return BN == 256 ? ((c >> 1) & 3) : (((c >> 1) & 1) | ((n & 1) << 1));
  }
  rsrc_t rc, r2, r1;
  uint32_t coff[kUnits];   // code bytes of the unit at step 0 (tile-relative)
  uint32_t boff[kUnits];   // its block index at step 0 (tile-relative)
  uint32_t bglob[kUnits];  // its global block index at step 0
  uint32_t soff[kUnits];   // its LDS byte offset in a tile
  int sw[kUnits];          // its piece order
  uint32_t rstep, bstep;   // code bytes and blocks per 64 rows
  int64_t N;
  float mean;
  const float2* lut2;
  u32x4 q[2][kUnits];
  uint32_t c2v[2][kUnits];
  float c1v[2][kUnits];
  int lim[2];              // rows of the step held in each slot that exist
  float chat[kUnits];
  Levels8 lv[kUnits];      // levels of the chunk being stored

  __device__ __forceinline__ void init(const uint8_t* codes, const uint8_t* c2, const float* c1, float mu,
                                       int64_t N_, int64_t K, int64_t k0, const float2* lut2_) {
    const int64_t nb = K / BK;
    N = N_;
    rc = tile_rsrc(codes, k0 / 2, N * (K / 2));
    r2 = tile_rsrc(c2, k0 / BK, N * nb);
    r1 = tile_rsrc(c1, 0, ((N * nb + 255) / 256) * 4);
    rstep = (uint32_t)(64 * (K / 2));
    bstep = (uint32_t)(64 * nb);
    mean = mu;
    lut2 = lut2_;
#pragma unroll
    for (int u = 0; u < kUnits; ++u) {
      const int idx = threadIdx.x + u * T;
      const int n = idx / (BN / 32), c = idx % (BN / 32);
      coff[u] = (uint32_t)(n * (K / 2) + c * 16);
      boff[u] = (uint32_t)(n * nb + c / 2);
      bglob[u] = (uint32_t)(n * nb + k0 / BK + c / 2);
      soff[u] = (uint32_t)(n * kRowBytes + c * 64);
      sw[u] = swz(n, c);
    }
  }
  template <int S>
  __device__ __forceinline__ void load(int kt) {
    lim[S] = (int)lmin(64, N - (int64_t)kt * 64);
#pragma unroll
    for (int u = 0; u < kUnits; ++u) {
      q[S][u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rc, coff[u] + kt * rstep, 0, 0));
      c2v[S][u] = __builtin_amdgcn_raw_buffer_load_b8(r2, boff[u] + kt * bstep, 0, 0);
      c1v[S][u] = __uint_as_float(
          __builtin_amdgcn_raw_buffer_load_b32(r1, ((bglob[u] + (uint32_t)kt * bstep) >> 8) * 4, 0, 0));
    }
  }
  template <int S, int P>
  __device__ __forceinline__ void prep() {
#pragma unroll
    for (int u = 0; u < kUnits; ++u) lv[u] = fetch8(q[S][u][P], lut2);
  }
  template <int S, int P>
  __device__ __forceinline__ void store_part(lds_t* t) {
#pragma unroll
    for (int u = 0; u < kUnits; ++u) {
      const int n = (threadIdx.x + u * T) / (BN / 32);
      if (P == 0) chat[u] = n < lim[S] ? dequant_constant(c2v[S][u], c1v[S][u], mean) : 0.f;
      st_lds16(reinterpret_cast<lds_t*>(reinterpret_cast<char*>(t) + soff[u] + 16 * (P ^ sw[u])),
               finish8(lv[u], chat[u]));
    }
  }
  __device__ __forceinline__ void prologue(int kt0, int last, lds_t* t) {
    load<0>(kt0);
    prep<0, 0>();
    store_part<0, 0>(t);
    prep<0, 1>();
    store_part<0, 1>(t);
    prep<0, 2>();
    store_part<0, 2>(t);
    prep<0, 3>();
    store_part<0, 3>(t);
    load<1>(min(kt0 + 1, last));
  }
  template <int S>
  __device__ __forceinline__ void ahead(int kt, int last) {
    load<S>(min(kt + 2, last));
  }
};

// ---------------------------------------------------------------- engine

// A BM x BN tile computed by 2 x WN waves, each (BM/2) x (BN/WN) as 32x32 MFMA tiles.
template <int BM, int BN, int WN = 2>
struct Acc {
  static constexpr int TM = BM / 2 / 32, TN = BN / WN / 32;
  f32x16 c[TM][TN];
};

template <int BM, int BN, int WN>
__device__ __forceinline__ void mma_tile(const lds_t* sa, const lds_t* sb, Acc<BM, BN, WN>& acc) {
  constexpr int TM = Acc<BM, BN, WN>::TM, TN = Acc<BM, BN, WN>::TN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int r = lane & 31, kq = (lane >> 5) * 8;
  // big wave tiles keep their accumulators in the 256 AGPRs; load fragments
  // one 16-deep step at a time so they fit the VGPRs next to the prefetch
#pragma unroll(TM * TN >= 16 ? 1 : 4)
  for (int kk = 0; kk < BK; kk += 16) {
    bf16x8 fa[TM], fb[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
      fa[i] = __builtin_bit_cast(bf16x8, ld16(sa + (wm * (BM / 2) + i * 32 + r) * PITCH + kk + kq));
#pragma unroll
    for (int j = 0; j < TN; ++j)
      fb[j] = __builtin_bit_cast(bf16x8, ld16(sb + (wn * (BN / WN) + j * 32 + r) * PITCH + kk + kq));
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc.c[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j], fa[i], acc.c[i][j], 0, 0, 0);
  }
}

template <int BM, int BN, int WN, class LA, class LB>
__device__ __forceinline__ void run_phase(LA& la, LB& lb, int kt0, int kt1, lds_t* sa, lds_t* sb, Acc<BM, BN, WN>& acc) {
  if (kt0 >= kt1) return;
  constexpr int SA = BM * PITCH, SB = BN * PITCH;
  la.load(kt0);
  lb.load(kt0);
  la.store(sa);
  lb.store(sb);
  __syncthreads();
  // the last step is peeled so that the loop body has no branches
  int kt = kt0;
  for (; kt + 1 < kt1; ++kt) {
    const int cur = (kt - kt0) & 1;
    la.load(kt + 1);
    lb.load(kt + 1);
    mma_tile<BM, BN, WN>(sa + cur * SA, sb + cur * SB, acc);
    la.store(sa + (cur ^ 1) * SA);
    lb.store(sb + (cur ^ 1) * SB);
    __syncthreads();
  }
  const int cur = (kt - kt0) & 1;
  mma_tile<BM, BN, WN>(sa + cur * SA, sb + cur * SB, acc);
}


// One 64-deep step on LDS buffers (sa, sb), with the expansion of the next
// step (register slot S -> LDS buffers da, db) spread over its four 16-deep
// sub-steps, so that the dequantization VALU work issues between MFMAs.
template <int BM, int BN, int WN, int S, class LA, class LB>
__device__ __forceinline__ void mma_step_store(const lds_t* sa, const lds_t* sb, Acc<BM, BN, WN>& acc, LA& la,
                                               LB& lb, lds_t* da, lds_t* db) {
  constexpr int TM = Acc<BM, BN, WN>::TM, TN = Acc<BM, BN, WN>::TN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN;
  // fragments of sub-step P+1 are read while sub-step P multiplies
  bf16x8 fa[2][TM], fb[2][TN];
  auto read = [&](int buf, int ps) {   // fragment-major tiles: one contiguous 1 KB per fragment
#pragma unroll
    for (int i = 0; i < TM; ++i)
      fa[buf][i] = __builtin_bit_cast(
          bf16x8, ld16(sa + ((ps * (BM / 32) + (wm * (BM / 2) + i * 32) / 32) * 64 + frag_read_slot(lane, ps)) * 8));
#pragma unroll
    for (int j = 0; j < TN; ++j)
      fb[buf][j] = __builtin_bit_cast(
          bf16x8, ld16(sb + ((ps * (BN / 32) + (wn * (BN / WN) + j * 32) / 32) * 64 + frag_read_slot(lane, ps)) * 8));
  };
  auto sub = [&](auto P) {
    constexpr int p = decltype(P)::value;
    if (p < 3) read((p + 1) & 1, p + 1);
    la.template prep<S, p>();
    lb.template prep<S, p>();
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc.c[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[p & 1][j], fa[p & 1][i], acc.c[i][j], 0, 0, 0);
    la.template store_part<S, p>(da);
    lb.template store_part<S, p>(db);
  };
  read(0, 0);
  sub(std::integral_constant<int, 0>{});
  sub(std::integral_constant<int, 1>{});
  sub(std::integral_constant<int, 2>{});
  sub(std::integral_constant<int, 3>{});
}

// The step of mma_step_store with the B operand in the weight's own layout
// (WNat): a 32x32x16 B fragment (operand rows = 32 output columns k, 16 of
// the reduction n) is two gfx950 transposing reads.  In each 16-lane group
// the transposing read hands lane i element e of source lane 4 e + i / 4's
// 8 bytes, element i % 4; so with source lane j pointing at row n + j / 4,
// columns k + 4 (j % 4) .. + 3, lane i receives rows n .. n + 3 of column
// k + i.  Lanes 16 G .. 16 G + 15 take columns 16 (G % 2) + i of the
// fragment and reduction elements 8 (G / 2) .. + 7 of the sub-step.
typedef short s16x4 __attribute__((ext_vector_type(4)));
template <int BNT>
__device__ __forceinline__ bf16x8 frag_tr(const lds_t* sb, int row0, int ps) {
  using W = WNat<BNT, 128>;
  const int lane = threadIdx.x & 63;
  const int G = (lane >> 4) & 3, i = lane & 15;
  const int n = 16 * ps + 8 * (G >> 1) + (i >> 2);   // (n + 4 has the same piece order)
  const int c = row0 >> 5;                            // the unit (row0 is a multiple of 32)
  const int piece = 2 * (G & 1) + ((i >> 1) & 1);
  const char* base = reinterpret_cast<const char*>(sb) + n * W::kRowBytes + c * 64 +
                     16 * (piece ^ W::swz(n, c)) + 8 * (i & 1);
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(base));
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(base + 4 * W::kRowBytes));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

template <int BM, int BN, int WN, int S, class LA, class LB>
__device__ __forceinline__ void mma_step_store_tr(const lds_t* sa, const lds_t* sb, Acc<BM, BN, WN>& acc, LA& la,
                                                  LB& lb, lds_t* da, lds_t* db) {
  constexpr int TM = Acc<BM, BN, WN>::TM, TN = Acc<BM, BN, WN>::TN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN;
  bf16x8 fa[2][TM], fb[2][TN];
  auto read = [&](int buf, int ps) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
      fa[buf][i] = __builtin_bit_cast(
          bf16x8, ld16(sa + ((ps * (BM / 32) + (wm * (BM / 2) + i * 32) / 32) * 64 + frag_read_slot(lane, ps)) * 8));
#pragma unroll
    for (int j = 0; j < TN; ++j) fb[buf][j] = frag_tr<BN>(sb, wn * (BN / WN) + j * 32, ps);
  };
  auto sub = [&](auto P) {
    constexpr int p = decltype(P)::value;
    if (p < 3) read((p + 1) & 1, p + 1);
    la.template prep<S, p>();
    lb.template prep<S, p>();
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc.c[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[p & 1][j], fa[p & 1][i], acc.c[i][j], 0, 0, 0);
    la.template store_part<S, p>(da);
    lb.template store_part<S, p>(db);
  };
  read(0, 0);
  sub(std::integral_constant<int, 0>{});
  sub(std::integral_constant<int, 1>{});
  sub(std::integral_constant<int, 2>{});
  sub(std::integral_constant<int, 3>{});
}

// run_pipelined with the B operand in the weight's own layout (SB bytes per
// buffer: 64 rows of WNat<BN>::kRowBytes).
template <int BM, int BN, int WN, class LA, class LB>
__device__ __forceinline__ void run_pipelined_tr(LA& la, LB& lb, int kt0, int kt1, lds_t* sa, lds_t* sb,
                                                 Acc<BM, BN, WN>& acc) {
  if (kt0 >= kt1) return;
  constexpr int SA = BM * BK, SB = 64 * WNat<BN, 128>::kRowBytes / 2;
  const int last = kt1 - 1;
  la.prologue(kt0, last, sa);
  lb.prologue(kt0, last, sb);
  __syncthreads();
  for (int kt = kt0;; kt += 2) {
    la.template ahead<0>(kt, last);
    lb.template ahead<0>(kt, last);
    mma_step_store_tr<BM, BN, WN, 1>(sa, sb, acc, la, lb, sa + SA, sb + SB);
    __syncthreads();
    if (kt + 1 > last) break;
    la.template ahead<1>(kt + 1, last);
    lb.template ahead<1>(kt + 1, last);
    mma_step_store_tr<BM, BN, WN, 0>(sa + SA, sb + SB, acc, la, lb, sa, sb);
    __syncthreads();
    if (kt + 2 > last) break;
  }
}

// The X/W product over steps [kt0, kt1) on fragment-major tiles (SA, SB bf16
// elements per buffer): LDS double buffer, and global loads
// two steps ahead in two register slots, so the loads of step kt+2 travel
// while step kt is multiplied and step kt+1 is expanded.  Loads past the end
// repeat the last step (harmless) and the final expansion lands in the
// buffer nobody reads, which keeps the loop free of branches.
template <int BM, int BN, int WN, class LA, class LB>
__device__ __forceinline__ void run_pipelined(LA& la, LB& lb, int kt0, int kt1, lds_t* sa, lds_t* sb,
                                              Acc<BM, BN, WN>& acc) {
  if (kt0 >= kt1) return;
  constexpr int SA = BM * BK, SB = BN * BK;
  const int last = kt1 - 1;
  la.prologue(kt0, last, sa);
  lb.prologue(kt0, last, sb);
  __syncthreads();
  for (int kt = kt0;; kt += 2) {
    // step kt in buffer 0; register slot 1 holds step kt+1; slot 0 is free
    la.template ahead<0>(kt, last);
    lb.template ahead<0>(kt, last);
    mma_step_store<BM, BN, WN, 1>(sa, sb, acc, la, lb, sa + SA, sb + SB);
    __syncthreads();
    if (kt + 1 > last) break;
    // step kt+1 in buffer 1; slot 0 holds step kt+2; slot 1 is free
    la.template ahead<1>(kt + 1, last);
    lb.template ahead<1>(kt + 1, last);
    mma_step_store<BM, BN, WN, 0>(sa + SA, sb + SB, acc, la, lb, sa, sb);
    __syncthreads();
    if (kt + 2 > last) break;
  }
}

// The products run with the weight-side fragment as the MFMA's first operand,
// so a 32x32 accumulator holds the transposed tile: lane l has output row
// l % 32 and, in register group g (values 4 g .. 4 g + 3), the four
// consecutive output columns 8 g + 4 (l / 32) .. + 3, which leave as one
// 8-byte (bf16) or 16-byte (fp32) store.
template <int BM, int BN, int WN, class F>
__device__ __forceinline__ void for_each_out4(const Acc<BM, BN, WN>& acc, F f) {
  constexpr int TM = Acc<BM, BN, WN>::TM, TN = Acc<BM, BN, WN>::TN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int row = wm * (BM / 2) + i * 32 + (lane & 31);
        const int col = wn * (BN / WN) + j * 32 + 8 * g + 4 * (lane >> 5);
        f(row, col, f32x4{acc.c[i][j][4 * g], acc.c[i][j][4 * g + 1], acc.c[i][j][4 * g + 2], acc.c[i][j][4 * g + 3]});
      }
}

// Four consecutive outputs (row m, columns n .. n + 3) of a row-major matrix
// with row stride ld: one vector store when `vec` (the four are 8- or 16-byte
// aligned whenever n % 4 == 0) and all four are inside [M, N), else one store
// per element inside the extent.
__device__ __forceinline__ void store4_bf16(uint16_t* base, int64_t ld, int64_t m, int64_t n, int64_t M, int64_t N,
                                            const f32x4& v, bool vec) {
  if (m >= M) return;
  uint16_t* q = base + m * ld + n;
  if (vec && n + 3 < N) {
    *reinterpret_cast<u32x2*>(q) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    return;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (n + e < N) q[e] = (uint16_t)(pack_bf16x2(v[e], 0.f) & 0xFFFFu);
}
__device__ __forceinline__ void store4_f32(float* base, int64_t ld, int64_t m, int64_t n, int64_t M, int64_t N,
                                           const f32x4& v, bool vec) {
  if (m >= M) return;
  float* q = base + m * ld + n;
  if (vec && n + 3 < N) {
    *reinterpret_cast<f32x4*>(q) = v;
    return;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (n + e < N) q[e] = v[e];
}

template <int BM, int BN, int WN>
__device__ __forceinline__ void zero(Acc<BM, BN, WN>& acc) {
#pragma unroll
  for (int i = 0; i < Acc<BM, BN, WN>::TM; ++i)
#pragma unroll
    for (int j = 0; j < Acc<BM, BN, WN>::TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc.c[i][j][v] = 0.f;
}

__device__ __forceinline__ void load_lut(float* lut, const Nf4Table& tab) {
  if (threadIdx.x < 16) lut[threadIdx.x] = tab.level[threadIdx.x];
}

// The pair table of the weight loaders: entry b = (level[b & 15], level[b >> 4]),
// the two levels of code byte b (element 2i in the low nibble), so one 8-byte
// LDS read serves two codes.  Built from the 16-entry table after a barrier.
__device__ __forceinline__ void load_lut2(float2* lut2, float* lut, const Nf4Table& tab) {
  load_lut(lut, tab);
  __syncthreads();
  for (int b = threadIdx.x; b < 256; b += blockDim.x) lut2[b] = make_float2(lut[b & 15], lut[b >> 4]);
}

__device__ __forceinline__ uint16_t to_bf16(float f) { return (uint16_t)(pack_bf16x2(f, 0.f) & 0xFFFFu); }

// LoRA term appended to a tile's accumulators straight from global memory:
// acc[i][j] += sum_k Aop(i, k) * Bop(j, k) over k < kr (kr <= 128), with the
// operands small and cache-resident.  fa(row, k0) / fb(row, k0) return the
// 8 bf16 values at k0 .. k0+7 of one operand row (zeros past the extents).
template <int BM, int BN, int WN, class FA, class FB>
__device__ __forceinline__ void lora_tail(Acc<BM, BN, WN>& acc, int kr, FA fa, FB fb) {
  constexpr int TM = Acc<BM, BN, WN>::TM, TN = Acc<BM, BN, WN>::TN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int r = lane & 31, kq = (lane >> 5) * 8;
#pragma unroll 1
  for (int kk = 0; kk < kr; kk += 16) {
    bf16x8 a[TM], b[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) a[i] = __builtin_bit_cast(bf16x8, fa(wm * (BM / 2) + i * 32 + r, kk + kq));
#pragma unroll
    for (int j = 0; j < TN; ++j) b[j] = __builtin_bit_cast(bf16x8, fb(wn * (BN / WN) + j * 32 + r, kk + kq));
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc.c[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[j], a[i], acc.c[i][j], 0, 0, 0);
  }
}

// 8 fp32 values of row `row` (k0 .. k0+7, zero past rows/kr), scaled, as bf16x8 bits
__device__ __forceinline__ u32x4 frag_f32_row(const float* src, int64_t ld, int64_t row, int64_t rows, int k0,
                                              int kr, float scale) {
  float f[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) f[q] = (row < rows && k0 + q < kr) ? src[row * ld + k0 + q] * scale : 0.f;
  return u32x4{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7])};
}

// 8 bf16 values of row `row` of a row-major bf16 matrix (k0 .. k0+7)
__device__ __forceinline__ u32x4 frag_bf16_row(const uint16_t* src, int64_t ld, int64_t row, int64_t rows, int k0,
                                               int kr, bool vec) {
  if (row < rows && vec && k0 + 8 <= kr) return ld16(src + row * ld + k0);
  uint32_t e[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) e[q] = (row < rows && k0 + q < kr) ? src[row * ld + k0 + q] : 0u;
  return u32x4{e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16)};
}

// 8 bf16 values of column `col` of a row-major bf16 matrix [kr][ld] (rows k0 .. k0+7)
__device__ __forceinline__ u32x4 frag_bf16_col(const uint16_t* src, int64_t ld, int64_t col, int64_t cols, int k0,
                                               int kr) {
  uint32_t e[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) e[q] = (col < cols && k0 + q < kr) ? src[(int64_t)(k0 + q) * ld + col] : 0u;
  return u32x4{e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16)};
}

// ---------------------------------------------------------------- kernels

// A workgroup-uniform value computed with vector instructions (integer
// division has no scalar form) moved back to a scalar register, so that the
// step counters derived from it stay scalar: a buffer load's scalar offset
// that lives in a vector register costs a loop around every load.
// (Through an asm operand: the readfirstlane builtin is folded away when the
// compiler knows the value is uniform, leaving it in the vector register.)
__device__ __forceinline__ int uniform(int v) {
  int r;
  asm volatile("s_mov_b32 %0, %1" : "=s"(r) : "s"(v));
  return r;
}

// Tile order.  Workgroups are dispatched round-robin over the 8 XCDs, each
// with its own L2.  Workgroup L runs on XCD L % 8; give XCD x a contiguous
// range of logical tiles (a bijection of [0, T)), and walk logical tiles in
// grouped-raster order (gm row tiles by every column tile), so the CUs of one
// XCD work on a compact block of tiles and share X and W slices in their L2.
__device__ __forceinline__ int xcd_logical(int L, int T) {
  const int x = L & 7, j = L >> 3;
  const int q = T >> 3, rem = T & 7;
  return x * q + min(x, rem) + j;
}
// (per lane: the tile may differ across a wave)
__device__ __forceinline__ void group_tile_lane(int logical, int mtiles, int ntiles, int gm, int& mi, int& ni) {
  const int per_group = gm * ntiles;
  const int group = logical / per_group;
  const int first_m = group * gm;
  const int gm_eff = min(gm, mtiles - first_m);
  const int in_group = logical - group * per_group;
  mi = first_m + in_group % gm_eff;
  ni = in_group / gm_eff;
}
// (workgroup-uniform `logical`)
__device__ __forceinline__ void group_tile(int logical, int mtiles, int ntiles, int gm, int& mi, int& ni) {
  group_tile_lane(logical, mtiles, ntiles, gm, mi, ni);
  mi = uniform(mi);
  ni = uniform(ni);
}
__device__ __forceinline__ void tile_of(int L, int mtiles, int ntiles, int gm, int& mi, int& ni) {
  group_tile(xcd_logical(L, mtiles * ntiles), mtiles, ntiles, gm, mi, ni);
}

// dynamic LDS of the pipelined products (fragment-major tiles, two buffers)
__host__ __device__ constexpr size_t frag_lds_bytes(int bm, int bn) {
  return (size_t)2 * (bm + bn) * BK * sizeof(lds_t);
}

// Forward, M > 16: Y = bf16( X W_deq^T + (s H) B^T ).  Phase 1 streams X and
// the NF4 weight over K; phase 2 appends the LoRA product as r more reduction
// steps with s*H (bf16) against B.
struct FwdGemmParams {
  const uint16_t* X;
  int64_t M, N, K;
  int r;
  const uint8_t* codes;
  const uint8_t* c2;
  const float* c1;
  const float* mean;
  const float* H;
  const uint16_t* B;
  bool b_vec;
  float scale;
  uint16_t* Y;
  int64_t ldy;          // elements between rows of Y (N, or more for a column range)
  bool y_vec;           // Y 8-byte aligned and ldy % 4 == 0: four outputs per store
  float* part;          // split-K partials [splits][M][N] (splits > 1, ldy = N)
  int splits, steps_per_split;
  int mtiles, ntiles, gm;
  Nf4Table tab;
  // stream-K (fwd_gemm_sk_kernel): sk_w workgroups share the tiles' 64-deep
  // steps; partial tiles go to slots of slot_rows x BN fp32 values in `part`
  int sk_w;
  int slot_rows;
};

template <int BM, int BN, int WN>
__global__ void __launch_bounds__(128 * WN) fwd_gemm_kernel(FwdGemmParams p) {
  constexpr int T = 128 * WN;
  extern __shared__ __attribute__((aligned(16))) lds_t smem[];
  __shared__ float lut[16];
  __shared__ float2 lut2[256];
  lds_t* sa = smem;
  lds_t* sb = smem + 2 * BM * BK;   // fragment-major tiles, double-buffered
  load_lut2(lut2, lut, p.tab);
  const int tiles = p.mtiles * p.ntiles;
  const int split = uniform((int)blockIdx.x / tiles);
  int mi, ni;
  tile_of((int)blockIdx.x - split * tiles, p.mtiles, p.ntiles, p.gm, mi, ni);
  const int64_t m0 = (int64_t)mi * BM, n0 = (int64_t)ni * BN;
  const int ksteps = (int)(p.K / BK);
  const int kt0 = split * p.steps_per_split, kt1 = min(ksteps, kt0 + p.steps_per_split);
  Acc<BM, BN, WN> acc;
  zero(acc);
  __syncthreads();
  {
    XRows<BM, T, true, (WN == 4 ? 2 : 1)> la;
    la.init(p.X, p.K, p.M, m0);
    WRows<BN, T> lb;
    lb.init(p.codes, p.c2, p.c1, *p.mean, p.N, p.K, n0, lut2);
    run_pipelined<BM, BN, WN>(la, lb, kt0, kt1, sa, sb, acc);
  }
  if (split == 0)
    lora_tail<BM, BN, WN>(
        acc, p.r,
        [&](int i, int k0) { return frag_f32_row(p.H, p.r, m0 + i, p.M, k0, p.r, p.scale); },
        [&](int j, int k0) { return frag_bf16_row(p.B, p.r, n0 + j, p.N, k0, p.r, p.b_vec); });
  if (p.splits == 1) {
    for_each_out4(acc, [&](int i, int j, const f32x4& v) {
      store4_bf16(p.Y, p.ldy, m0 + i, n0 + j, p.M, p.N, v, p.y_vec);
    });
  } else {
    float* out = p.part + (int64_t)split * p.M * p.N;
    for_each_out4(acc, [&](int i, int j, const f32x4& v) {
      store4_f32(out, p.N, m0 + i, n0 + j, p.M, p.N, v, (p.N & 3) == 0);
    });
  }
}

// Stream-K order of the forward product.  The steps of all tiles, tile after
// tile (logical tile order, ksteps steps each: U = tiles x ksteps), are cut
// into sk_w ranges [floor(l U / sk_w), floor((l + 1) U / sk_w)), one per
// workgroup (l: its XCD-contiguous logical index), so every workgroup runs the
// same number of steps give or take one, in one round of resident
// workgroups, where split-K's fixed pieces leave the last round part empty.
// A workgroup takes the pieces of its range tile by tile: a whole tile is
// stored as bf16 at once; a piece of a tile goes, as fp32, to slot l + t (t:
// the logical tile), which no other piece uses, and reduce_streamk_kernel sums
// a tile's pieces in step order.  The LoRA term rides on the piece that holds
// the tile's first step.
__host__ __device__ __forceinline__ int64_t sk_owner(int64_t x, int64_t units, int w) {
  return ((x + 1) * w - 1) / units;   // the range holding step x
}

template <int BM, int BN, int WN>
__global__ void __launch_bounds__(128 * WN, 2) fwd_gemm_sk_kernel(FwdGemmParams p) {
  constexpr int T = 128 * WN;
  extern __shared__ __attribute__((aligned(16))) lds_t smem[];
  __shared__ float lut[16];
  __shared__ float2 lut2[256];
  lds_t* sa = smem;
  lds_t* sb = smem + 2 * BM * BK;
  load_lut2(lut2, lut, p.tab);
  const int tiles = p.mtiles * p.ntiles;
  const int ksteps = (int)(p.K / BK);
  const int64_t units = (int64_t)tiles * ksteps;
  const int l = xcd_logical((int)blockIdx.x, p.sk_w);
  const int64_t end = (int64_t)(l + 1) * units / p.sk_w;
  for (int64_t pos = (int64_t)l * units / p.sk_w; pos < end;) {
    const int t = uniform((int)(pos / ksteps));
    const int kt0 = uniform((int)(pos - (int64_t)t * ksteps));
    const int kt1 = uniform((int)min<int64_t>(ksteps, kt0 + (end - pos)));
    int mi, ni;
    group_tile(t, p.mtiles, p.ntiles, p.gm, mi, ni);
    const int64_t m0 = (int64_t)mi * BM, n0 = (int64_t)ni * BN;
    Acc<BM, BN, WN> acc;
    zero(acc);
    __syncthreads();   // the previous piece's last reads of the LDS tiles are done
    {
      XRows<BM, T, true, (WN == 4 ? 2 : 1)> la;
      la.init(p.X, p.K, p.M, m0);
      WRows<BN, T> lb;
      lb.init(p.codes, p.c2, p.c1, *p.mean, p.N, p.K, n0, lut2);
      run_pipelined<BM, BN, WN>(la, lb, kt0, kt1, sa, sb, acc);
    }
    if (kt0 == 0)
      lora_tail<BM, BN, WN>(
          acc, p.r,
          [&](int i, int k0) { return frag_f32_row(p.H, p.r, m0 + i, p.M, k0, p.r, p.scale); },
          [&](int j, int k0) { return frag_bf16_row(p.B, p.r, n0 + j, p.N, k0, p.r, p.b_vec); });
    if (kt0 == 0 && kt1 == ksteps) {
      for_each_out4(acc, [&](int i, int j, const f32x4& v) {
        store4_bf16(p.Y, p.ldy, m0 + i, n0 + j, p.M, p.N, v, p.y_vec);
      });
    } else {
      float* out = p.part + (int64_t)(l + t) * p.slot_rows * BN;
      for_each_out4(acc, [&](int i, int j, const f32x4& v) {
        store4_f32(out, BN, i, j, p.slot_rows, BN, v, true);
      });
    }
    pos += kt1 - kt0;
  }
}

// Sum of the stream-K pieces of the tiles that more than one workgroup
// shared: Y[m0 + i][n0 + j] = bf16(sum over the ranges l_first .. l_last
// holding the tile's steps, in that order, of slot l + t).  One thread per
// four columns of a slot row; tiles stored whole by one workgroup are skipped.
__global__ void __launch_bounds__(256) reduce_streamk_kernel(const float* __restrict__ part, int tiles,
                                                             int ksteps, int w, int mtiles, int ntiles, int gm,
                                                             int slot_rows, int64_t M, int64_t N,
                                                             uint16_t* __restrict__ Y, int64_t ldy, bool y_vec) {
  constexpr int BN = 128;
  const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_tile = (int64_t)slot_rows * (BN / 4);
  if (q >= (int64_t)tiles * per_tile) return;
  const int t = (int)(q / per_tile);
  const int i = (int)((q - t * per_tile) / (BN / 4)), j = 4 * (int)(q % (BN / 4));
  const int64_t units = (int64_t)tiles * ksteps;
  const int l0 = (int)sk_owner((int64_t)t * ksteps, units, w);
  const int l1 = (int)sk_owner((int64_t)(t + 1) * ksteps - 1, units, w);
  if (l0 == l1) return;
  int mi, ni;
  group_tile_lane(t, mtiles, ntiles, gm, mi, ni);
  if ((int64_t)mi * 128 + i >= M) return;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int l = l0; l <= l1; ++l) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(part + ((int64_t)(l + t) * slot_rows + i) * BN + j);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += v[e];
  }
  store4_bf16(Y, ldy, (int64_t)mi * 128 + i, (int64_t)ni * BN + j, M, N, acc, y_vec);
}

// Generic bf16 x bf16 product with fp32 output (split-K partials or final):
// out[split][i][j] = scale * sum_{k in split} Aop[i][k] Bop[j][k].
template <int BM, int BN, class LA, class LB>
struct SkinnyParams {
  LA la;
  LB lb;
  int64_t rows, cols;   // output extent
  int ksteps;           // total 64-wide reduction steps
  int steps_per_split;
  float* out;           // [splits][rows][cols]
};

template <int BM, int BN, class LA, class LB>
__global__ void __launch_bounds__(NT) skinny_kernel(SkinnyParams<BM, BN, LA, LB> p) {
  __shared__ __attribute__((aligned(16))) lds_t sa[2 * BM * PITCH];
  __shared__ __attribute__((aligned(16))) lds_t sb[2 * BN * PITCH];
  const int64_t i0 = (int64_t)blockIdx.y * BM, j0 = (int64_t)blockIdx.x * BN;
  LA la = p.la;
  LB lb = p.lb;
  la.row_origin(i0, p.rows);
  lb.row_origin(j0, p.cols);
  Acc<BM, BN, 2> acc;
  zero(acc);
  const int kt0 = blockIdx.z * p.steps_per_split;
  const int kt1 = min(p.ksteps, kt0 + p.steps_per_split);
  run_phase<BM, BN, 2>(la, lb, kt0, kt1, sa, sb, acc);
  float* out = p.out + (int64_t)blockIdx.z * p.rows * p.cols;
  for_each_out4(acc, [&](int i, int j, const f32x4& v) {
    store4_f32(out, p.cols, i0 + i, j0 + j, p.rows, p.cols, v, (p.cols & 3) == 0);
  });
}

// Sum split-K partials: out = scale * sum_s part[s]; bf16 or fp32 output.
// Four consecutive values per thread (16-byte partial loads) when count % 4
// == 0 and the outputs allow 8-byte (bf16) or 16-byte (fp32) stores; the
// split order is fixed, so the sums are deterministic.
__global__ void __launch_bounds__(256) reduce_splits_kernel(const float* __restrict__ part, int splits,
                                                            int64_t count, float scale,
                                                            uint16_t* __restrict__ out_bf16,
                                                            float* __restrict__ out_f32) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const bool vec = (count & 3) == 0 && (reinterpret_cast<uintptr_t>(out_bf16) & 7) == 0 &&
                   (reinterpret_cast<uintptr_t>(out_f32) & 15) == 0;
  if (vec) {
    const int64_t n4 = count >> 2;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
      for (int k = 0; k < splits; ++k) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(part + (int64_t)k * count + 4 * i);
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[q] += v[q];
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] *= scale;
      if (out_bf16)
        *reinterpret_cast<u32x2*>(out_bf16 + 4 * i) = u32x2{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
      if (out_f32) *reinterpret_cast<f32x4*>(out_f32 + 4 * i) = acc;
    }
    return;
  }
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride) {
    float s = 0.f;
#pragma unroll 4
    for (int k = 0; k < splits; ++k) s += part[(int64_t)k * count + i];
    s *= scale;
    if (out_bf16) out_bf16[i] = to_bf16(s);
    if (out_f32) out_f32[i] = s;
  }
}

// Split-K partials of a column range of the output: out[i][j] (row stride
// ld) = bf16(sum_s part[s][i][j]) for part [splits][rows][cols], the split
// order fixed.  Four columns per thread when cols % 4 == 0 and the output
// rows allow 8-byte stores.
__global__ void __launch_bounds__(256) reduce_splits_cols_kernel(const float* __restrict__ part, int splits,
                                                                 int64_t rows, int64_t cols,
                                                                 uint16_t* __restrict__ out, int64_t ld) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t count = rows * cols;
  const bool vec = (cols & 3) == 0 && (ld & 3) == 0 && (reinterpret_cast<uintptr_t>(out) & 7) == 0;
  if (vec) {
    for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < count / 4; q += stride) {
      const int64_t i = (4 * q) / cols, j = 4 * q - i * cols;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int k = 0; k < splits; ++k) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(part + (int64_t)k * count + 4 * q);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] += v[e];
      }
      *reinterpret_cast<u32x2*>(out + i * ld + j) = u32x2{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
    }
    return;
  }
  for (int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; o < count; o += stride) {
    float acc = 0.f;
    for (int k = 0; k < splits; ++k) acc += part[(int64_t)k * count + o];
    const int64_t i = o / cols;
    out[i * ld + (o - i * cols)] = to_bf16(acc);
  }
}

// out[c][r] = bf16(src[r][c]) for an fp32 src [rows][cols] (out row length
// rows), and, with lo_out, lo_out[c][r] = bf16(src[r][c] - out[c][r]): the
// pair carries each value to about 2^-17 relative, so the LoRA factors'
// gradients see H and dH at fp32-like precision through bf16 matrix cores.
// The reduction index m ends up contiguous, for 16-byte vector loads.  16 x 64
// tiles through LDS (one workgroup per 16 rows, so a 4096-row source fills
// the chip); each thread stores pairs of consecutive rows (4 bytes).
__device__ __forceinline__ void store_pair_t(uint16_t* __restrict__ out, int64_t rows, int64_t r, int64_t c,
                                             uint32_t v) {
  if (r + 1 < rows && (rows & 1) == 0)
    *reinterpret_cast<uint32_t*>(out + c * rows + r) = v;
  else {
    out[c * rows + r] = (uint16_t)(v & 0xFFFFu);
    if (r + 1 < rows) out[c * rows + r + 1] = (uint16_t)(v >> 16);
  }
}

__global__ void __launch_bounds__(256) f32_to_bf16_t_kernel(const float* __restrict__ src, int64_t rows,
                                                            int64_t cols, uint16_t* __restrict__ out,
                                                            uint16_t* __restrict__ lo_out) {
  __shared__ float t[16][65];
  const int64_t r0 = (int64_t)blockIdx.x * 16, c0 = (int64_t)blockIdx.y * 64;
  const int tc = threadIdx.x & 63, tr = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t r = r0 + tr + 4 * i, c = c0 + tc;
    t[tr + 4 * i][tc] = (r < rows && c < cols) ? src[r * cols + c] : 0.f;
  }
  __syncthreads();
  const int pr = threadIdx.x & 7, pc = threadIdx.x >> 3;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int cc = pc + 32 * i;
    const int64_t c = c0 + cc, r = r0 + 2 * pr;
    if (c >= cols || r >= rows) continue;
    const float x0 = t[2 * pr][cc], x1 = t[2 * pr + 1][cc];
    const uint32_t v = pack_bf16x2(x0, x1);
    store_pair_t(out, rows, r, c, v);
    // x - bf16(x) is exact in fp32 (the rounding error of a rounding to 8 bits)
    if (lo_out) store_pair_t(lo_out, rows, r, c, pack_bf16x2(x0 - bf16_lo(v), x1 - bf16_hi(v)));
  }
}

// The single pass's partials to the gradients in one launch: the first
// hb = ceil(M/16) ceil(r/64) workgroups form dH = s sum_g part_h[g] on 16 x 64
// tiles (four consecutive values per thread, 16-byte loads), store it (fp32
// [M][r], for the dX product) and its bf16 hi and lo transposes [r][M] (the
// dA product's operand, as f32_to_bf16_t_kernel writes them); the rest form
// dB = bf16(s sum_g part_b[g]), four values per thread.  The sums run over
// the partials in index order, as reduce_splits_kernel's do, so the results
// are those of the three launches this replaces.  r % 8 == 0.
__global__ void __launch_bounds__(256) lora_finish_kernel(const float* __restrict__ part_h, int gn,
                                                          const float* __restrict__ part_b, int gm, int64_t M,
                                                          int64_t N, int r, float scale, float* __restrict__ dH,
                                                          uint16_t* __restrict__ dHt, uint16_t* __restrict__ dB) {
  const int64_t cb = (r + 63) / 64, hb = ((M + 15) / 16) * cb;
  const int64_t bid = blockIdx.x;
  if (bid < hb) {
    __shared__ float t[16][65];
    const int64_t r0 = (bid / cb) * 16, c0 = (bid % cb) * 64;
    const int tr = threadIdx.x >> 4, tc = 4 * (threadIdx.x & 15);   // row, first of four columns
    const int64_t row = r0 + tr, col = c0 + tc;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (row < M && col < r) {
      const float* q = part_h + row * r + col;
#pragma unroll 4
      for (int g = 0; g < gn; ++g) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(q + (int64_t)g * M * r);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] += v[e];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] *= scale;
      *reinterpret_cast<f32x4*>(dH + row * r + col) = acc;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) t[tr][tc + e] = acc[e];
    __syncthreads();
    const int pr = threadIdx.x & 7, pc = threadIdx.x >> 3;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int cc = pc + 32 * i;
      const int64_t c = c0 + cc, rr = r0 + 2 * pr;
      if (c >= r || rr >= M) continue;
      const float x0 = t[2 * pr][cc], x1 = t[2 * pr + 1][cc];
      const uint32_t v = pack_bf16x2(x0, x1);
      store_pair_t(dHt, M, rr, c, v);
      store_pair_t(dHt + (int64_t)r * M, M, rr, c, pack_bf16x2(x0 - bf16_lo(v), x1 - bf16_hi(v)));
    }
    return;
  }
  const int64_t count = N * r;
  const int64_t q = (bid - hb) * 256 + threadIdx.x;
  if (4 * q >= count) return;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int g = 0; g < gm; ++g) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(part_b + (int64_t)g * count + 4 * q);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += v[e];
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) acc[e] *= scale;
  *reinterpret_cast<u32x2*>(dB + 4 * q) = u32x2{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
}

// Gradient of a LoRA factor from a product whose small operand came as hi
// and lo bf16 halves: part[s] holds the product against [hi; lo], so
// out[i][j] = bf16(scale * sum_s (part[s][i*pitch + j] + part[s][i*pitch + j + lo_off])).
__global__ void __launch_bounds__(256) reduce_hilo_kernel(const float* __restrict__ part, int splits,
                                                          int64_t split_stride, int64_t rows, int64_t cols,
                                                          int64_t pitch, int64_t lo_off, float scale,
                                                          uint16_t* __restrict__ out) {
  const int64_t count = rows * cols;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; o < count; o += stride) {
    const int64_t i = o / cols, j = o - i * cols;
    const float* p = part + i * pitch + j;
    float hi = 0.f, lo = 0.f;
    for (int k = 0; k < splits; ++k) {
      hi += p[(int64_t)k * split_stride];
      lo += p[(int64_t)k * split_stride + lo_off];
    }
    out[o] = to_bf16(scale * (hi + lo));
  }
}

// ---------------------------------------------------------------- LoRA gradients in one pass over dY

// itwiki "QLoRA", section on the computation: the output gradient dY reaches
// the adapter through dH = s dY B (then dA = dH^T X) and dB = s dY^T H.  One
// launch reads every element of dY once and forms both products from the same
// LDS tile: workgroup (gm, gn) owns a run of 64-row tiles of dY and the C
// 128-column chunks [n0, n0 + 128 C).  Per (tile, chunk) step the 8 waves
//   - waves 0-3: dH[64 rows x 64 j] += dY tile . B chunk (rows read as they
//     lie), a partial over this workgroup's columns, stored after the tile's
//     last chunk into part_h[gn];
//   - all waves: dB[128 n x 64 j] += dY^T . H for the tile (gfx950
//     transposing LDS reads; H as bf16 hi and lo halves, both accumulated,
//     fp32-like), kept in registers across the workgroup's tiles and stored
//     at the end into part_b[gm].
// Two small reductions (over gn and gm, in fixed order) finish dH and dB.
// The B chunk, transposed to [j][n], stays in LDS for the whole workgroup;
// each tile's rows of H come in as fp32 and enter LDS as H^T hi and lo.
// Ranks up to 64 (multiples of 8) are padded to 64 with zeros.
struct LgParams {
  const uint16_t* dY;   // [M][N]
  const uint16_t* B;    // [N][r]
  const float* H;       // [M][r] fp32 (split into bf16 hi and lo halves on the way into LDS)
  int64_t M, N;
  int r;
  int gm;               // workgroups along M
  int mtiles;           // 64-row tiles of M
  float* part_h;        // [gn][M][r]
  float* part_b;        // [gm][N][r]
};

// A [64][128] bf16 tile in 256-byte rows of 16 pieces (8 elements each).
// Piece p of row m sits at slot p ^ f(m), f mixing the row's low four bits,
// so that the 16 rows of one piece (a row-wise fragment read) and 4 adjacent
// rows of 4 adjacent pieces (a transposing read) each cover all 16 slots.
__device__ __forceinline__ int dy_slot(int m, int piece) {
  const int i = m & 15;
  return piece ^ (((i & 3) << 2) | ((i >> 2) & 3));
}
// Rows m0 .. m0 + 31 of the tile, columns 16 ps + 8 (lane / 32) .. + 7:
// the operand of a product that reduces over the tile's columns.
__device__ __forceinline__ bf16x8 dy_frag_rows(const char* t, int m0, int ps) {
  const int lane = threadIdx.x & 63;
  const int m = m0 + (lane & 31);
  return __builtin_bit_cast(bf16x8, ld16(t + m * 256 + 16 * dy_slot(m, 2 * ps + (lane >> 5))));
}
// Columns n0 .. n0 + 31 of the tile, rows 16 ps + 8 (lane / 32) .. + 7: the
// operand of a product that reduces over the tile's rows, two transposing
// reads (lane i of each 16-lane group receives 4 rows of column i; see
// frag_tr).
__device__ __forceinline__ bf16x8 dy_frag_cols(const char* t, int n0, int ps) {
  const int lane = threadIdx.x & 63;
  const int G = (lane >> 4) & 3, i = lane & 15;
  const int m = 16 * ps + 8 * (G >> 1) + (i >> 2);
  const int pc = (n0 >> 3) + 2 * (G & 1) + ((i >> 1) & 1);
  const char* a0 = t + m * 256 + 16 * dy_slot(m, pc) + 8 * (i & 1);
  const char* a1 = t + (m + 4) * 256 + 16 * dy_slot(m + 4, pc) + 8 * (i & 1);
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(a0));
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(a1));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}
// B chunk in LDS as [64 j][128 C n]; piece p of row j at slot p ^ (j & 15).
template <int C>
__device__ __forceinline__ int bt_off(int j, int piece) {
  return j * (256 * C) + 16 * (piece ^ (j & 15));
}
// H^T tile in LDS as [hi, lo][64 j][64 m]; piece p of row j at p ^ ((j / 2) & 7).
__device__ __forceinline__ int ht_off(int hl, int j, int piece) {
  return hl * 8192 + j * 128 + 16 * (piece ^ ((j >> 1) & 7));
}

__host__ __device__ constexpr size_t lg_lds_bytes(int C) { return (size_t)2 * 16384 + 2 * 16384 + (size_t)16384 * C; }

template <int C>
__global__ void __launch_bounds__(512) lora_grads_kernel(LgParams p) {
  static_assert(C == 2 || C == 4, "an even number of chunks keeps the register slot of a step a constant");
  extern __shared__ __attribute__((aligned(16))) char lg_smem[];
  char* sdy = lg_smem;            // 2 x 16 KB: dY tiles
  char* sht = lg_smem + 32768;    // 2 x 16 KB: H^T hi/lo tiles
  char* sbt = lg_smem + 65536;    // 16 C KB: the B chunk, transposed
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int gm = uniform((int)blockIdx.x % p.gm), gn = uniform((int)blockIdx.x / p.gm);
  const int t0 = (int)((int64_t)gm * p.mtiles / p.gm), t1 = (int)((int64_t)(gm + 1) * p.mtiles / p.gm);
  const int ntiles = t1 - t0;
  const int64_t m0 = (int64_t)t0 * 64, n0 = (int64_t)gn * 128 * C;
  const int r = p.r;

  // The B chunk, transposed: 4 rows n x 8 columns j per patch, written as
  // 8 rows j of 4 columns n.  Rows past N read 0 (resource end); columns
  // past r are 0.
  {
    const rsrc_t rb = make_rsrc(p.B, (uint32_t)(p.N * r * 2));
#pragma unroll
    for (int u = 0; u < C / 2; ++u) {
      const int q = tid + 512 * u;
      const int j0 = 8 * (q & 7), nl = 4 * (q >> 3);
      u32x4 v[4];
#pragma unroll
      for (int z = 0; z < 4; ++z) {
        const int64_t n = n0 + nl + z;
        v[z] = j0 < r && n < p.N
                   ? __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rb, (uint32_t)(n * r + j0) * 2, 0, 0))
                   : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const u32x2 a = {lo16(v[0][w], v[1][w]), lo16(v[2][w], v[3][w])};
        const u32x2 b = {hi16(v[0][w], v[1][w]), hi16(v[2][w], v[3][w])};
        *reinterpret_cast<u32x2*>(sbt + bt_off<C>(j0 + 2 * w, nl >> 3) + 2 * (nl & 7)) = a;
        *reinterpret_cast<u32x2*>(sbt + bt_off<C>(j0 + 2 * w + 1, nl >> 3) + 2 * (nl & 7)) = b;
      }
    }
  }

  // dY tile pieces (row q / 16, piece q % 16 of q = tid + 512 u) through a
  // resource based at the workgroup's first row: rows past M read 0.  A
  // chunk's columns past N read the next row, finite values that the zero
  // columns of the B chunk cancel; their dB rows are not stored.
  const rsrc_t rdy = tile_rsrc(p.dY, m0 * p.N * 2, p.M * p.N * 2);
  uint32_t dyo[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int q = tid + 512 * u;
    dyo[u] = (uint32_t)(((q >> 4) * p.N + n0 + 8 * (q & 15)) * 2);
  }
  // H rows of a tile: thread tid loads H[m][j0 .. j0 + 7], m = tid % 64,
  // j0 = 8 (tid / 64), and stores their bf16 hi and lo halves into the H^T
  // tile (as f32_to_bf16_t_kernel rounds them); columns j >= r and rows past
  // M read 0.
  const rsrc_t rh = make_rsrc(p.H, (uint32_t)(p.M * r * 4));
  const int hm = tid & 63, hj0 = 8 * (tid >> 6);
  const bool h_ok = hj0 < r;
  const uint32_t hoff = (uint32_t)(((m0 + hm) * r + hj0) * 4);

  // C steps in flight: step (t, c) sits in register slot c.  Steps past the
  // last tile load through an offset past every resource's end (zeros, no
  // memory traffic) and store into the idle LDS buffer, so the loop carries
  // no branches around its loads.
  u32x4 ydr[C][2];
  f32x4 hrow[2];
  auto load = [&](auto CC, int t) {
    constexpr int c = decltype(CC)::value;
    const bool live = t < ntiles;
    const uint32_t so = (uint32_t)((64 * (int64_t)t * p.N + 128 * c) * 2);
#pragma unroll
    for (int u = 0; u < 2; ++u)
      ydr[c][u] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(rdy, live ? dyo[u] + so : 0xFFFFFFF0u, 0, 0));
    if (c == 0) {
#pragma unroll
      for (int u = 0; u < 2; ++u)
        hrow[u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                rh, live && h_ok ? hoff + (uint32_t)(t * 256 * r) + 16 * u : 0xFFFFFFF0u,
                                                0, 0));
    }
  };
  auto store = [&](auto CC, int t) {
    constexpr int c = decltype(CC)::value;
    char* ty = sdy + (c & 1) * 16384;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int q = tid + 512 * u;
      st_lds16(reinterpret_cast<lds_t*>(ty + (q >> 4) * 256 + 16 * dy_slot(q >> 4, q & 15)), ydr[c][u]);
    }
    if (c == 0) {
      char* th = sht + (t & 1) * 16384;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = hrow[e >> 2][e & 3];
        const uint32_t hi = pack_bf16x2(x, 0.f) & 0xFFFFu;
        const uint32_t lo = pack_bf16x2(x - __uint_as_float(hi << 16), 0.f) & 0xFFFFu;
        *reinterpret_cast<uint16_t*>(th + ht_off(0, hj0 + e, hm >> 3) + 2 * (hm & 7)) = (uint16_t)hi;
        *reinterpret_cast<uint16_t*>(th + ht_off(1, hj0 + e, hm >> 3) + 2 * (hm & 7)) = (uint16_t)lo;
      }
    }
  };

  f32x16 acc_h = {};
  f32x16 acc_b[C];
#pragma unroll
  for (int c = 0; c < C; ++c) acc_b[c] = f32x16{};
  bf16x8 hf[4], lf[4];
  const int mh = wave & 1, jt = wave >> 1;    // dH: rows 32 mh.., columns 32 jt.. (waves 0-3)
  const int nt = wave >> 1, jb = wave & 1;    // dB: chunk columns 32 nt.., columns 32 jb..

  load(std::integral_constant<int, 0>{}, 0);
  load(std::integral_constant<int, 1>{}, 0);
  if constexpr (C == 4) {
    load(std::integral_constant<int, 2>{}, 0);
    load(std::integral_constant<int, 3>{}, 0);
  }
  store(std::integral_constant<int, 0>{}, 0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    auto step = [&](auto CC) {
      constexpr int c = decltype(CC)::value;
      const char* ty = sdy + (c & 1) * 16384;
      load(std::integral_constant<int, c>{}, t + 1);
      if (c == 0) {
        const char* th = sht + (t & 1) * 16384;
        const int j = 32 * jb + (lane & 31);
#pragma unroll
        for (int ps = 0; ps < 4; ++ps) {
          hf[ps] = __builtin_bit_cast(bf16x8, ld16(th + ht_off(0, j, 2 * ps + (lane >> 5))));
          lf[ps] = __builtin_bit_cast(bf16x8, ld16(th + ht_off(1, j, 2 * ps + (lane >> 5))));
        }
      }
      if (wave < 4) {
        const int j = 32 * jt + (lane & 31);
#pragma unroll
        for (int ps = 0; ps < 8; ++ps) {
          const bf16x8 a = dy_frag_rows(ty, 32 * mh, ps);
          const bf16x8 b = __builtin_bit_cast(bf16x8, ld16(sbt + bt_off<C>(j, 16 * c + 2 * ps + (lane >> 5))));
          acc_h = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, acc_h, 0, 0, 0);
        }
      }
#pragma unroll
      for (int ps = 0; ps < 4; ++ps) {
        const bf16x8 a = dy_frag_cols(ty, 32 * nt, ps);
        acc_b[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hf[ps], a, acc_b[c], 0, 0, 0);
        acc_b[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lf[ps], a, acc_b[c], 0, 0, 0);
      }
      if (c == C - 1 && wave < 4) {
        // this tile's dH over the workgroup's columns
        float* out = p.part_h + (int64_t)gn * p.M * r;
        const int64_t m = m0 + 64 * (int64_t)t + 32 * mh + (lane & 31);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int j = 32 * jt + 8 * g + 4 * (lane >> 5);
          if (m < p.M && j < r)
            *reinterpret_cast<f32x4*>(out + m * r + j) =
                f32x4{acc_h[4 * g], acc_h[4 * g + 1], acc_h[4 * g + 2], acc_h[4 * g + 3]};
        }
        acc_h = f32x16{};
      }
      store(std::integral_constant<int, (c + 1) % C>{}, c + 1 < C ? t : t + 1);
      __syncthreads();
    };
    step(std::integral_constant<int, 0>{});
    step(std::integral_constant<int, 1>{});
    if constexpr (C == 4) {
      step(std::integral_constant<int, 2>{});
      step(std::integral_constant<int, 3>{});
    }
  }

  // dB over this workgroup's rows
  float* out = p.part_b + (int64_t)gm * p.N * r;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int64_t n = n0 + 128 * c + 32 * nt + (lane & 31);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int j = 32 * jb + 8 * g + 4 * (lane >> 5);
      if (n < p.N && j < r)
        *reinterpret_cast<f32x4*>(out + n * r + j) =
            f32x4{acc_b[c][4 * g], acc_b[c][4 * g + 1], acc_b[c][4 * g + 2], acc_b[c][4 * g + 3]};
    }
  }
}

// dX = dY W_deq + dH A (bf16 output, split-K partials when splits > 1).
struct DxParams {
  const uint16_t* dY;
  int64_t M, N, K;
  int r;
  const uint8_t* codes;
  const uint8_t* c2;
  const float* c1;
  const float* mean;
  const float* dH;
  const uint16_t* A;
  uint16_t* dX;
  float* part;          // split-K partials [splits][M][K] (splits > 1)
  int splits, steps_per_split;
  int mtiles, ntiles, gm;
  Nf4Table tab;
};

// dX = dY W_deq + dH A (bf16 output), one product on the pipelined engine:
// rows of dY (reduction n contiguous, zero past the tensor) against the
// weight's codes expanded per step into its own [n][k] layout (WNat), which
// the matrix cores take through transposing LDS reads; r more reduction
// steps append dH against A.  No expanded copy of the weight is written:
// the codes are the only weight bytes read.  kVecY: N % 8 == 0 (16-byte rows
// of dY).
template <int BM, int BN, int WN, bool kVecY>
__global__ void __launch_bounds__(128 * WN) dxr_gemm_kernel(DxParams p) {
  constexpr int T = 128 * WN;
  extern __shared__ __attribute__((aligned(16))) lds_t smem[];
  __shared__ float lut[16];
  __shared__ float2 lut2[256];
  lds_t* sa = smem;
  lds_t* sb = smem + 2 * BM * BK;   // A fragment-major, B in the weight's layout; both double-buffered
  load_lut2(lut2, lut, p.tab);
  const int tiles = p.mtiles * p.ntiles;
  const int split = uniform((int)blockIdx.x / tiles);
  int mi, ki;
  tile_of((int)blockIdx.x - split * tiles, p.mtiles, p.ntiles, p.gm, mi, ki);
  const int64_t m0 = (int64_t)mi * BM, k0 = (int64_t)ki * BN;
  const int nsteps = (int)((p.N + BK - 1) / BK);
  const int nt0 = split * p.steps_per_split, nt1 = min(nsteps, nt0 + p.steps_per_split);
  Acc<BM, BN, WN> acc;
  zero(acc);
  __syncthreads();
  {
    XRows<BM, T, kVecY, (WN == 4 && kVecY ? 2 : 1), true> la;
    la.init(p.dY, p.N, p.M, m0);
    WNat<BN, T> lb;
    lb.init(p.codes, p.c2, p.c1, *p.mean, p.N, p.K, k0, lut2);
    run_pipelined_tr<BM, BN, WN>(la, lb, nt0, nt1, sa, sb, acc);
  }
  if (split == 0)
    lora_tail<BM, BN, WN>(
        acc, p.r,
        [&](int i, int kk) { return frag_f32_row(p.dH, p.r, m0 + i, p.M, kk, p.r, 1.0f); },
        [&](int j, int kk) { return frag_bf16_col(p.A, p.K, k0 + j, p.K, kk, p.r); });
  // (dX is 16-byte aligned and K % 64 == 0: every group of four is aligned)
  if (p.splits == 1) {
    for_each_out4(acc, [&](int i, int j, const f32x4& v) {
      store4_bf16(p.dX, p.K, m0 + i, k0 + j, p.M, p.K, v, true);
    });
  } else {
    float* out = p.part + (int64_t)split * p.M * p.K;
    for_each_out4(acc, [&](int i, int j, const f32x4& v) {
      store4_f32(out, p.K, m0 + i, k0 + j, p.M, p.K, v, true);
    });
  }
}

__host__ __device__ constexpr size_t dxr_lds_bytes(int bm, int bn) {
  return (size_t)2 * bm * BK * sizeof(lds_t) + (size_t)2 * 64 * (bn * 2 + 64);
}

// Skinny-product loaders with a per-tile origin, built on the loaders above.
template <int R>
struct SRowsBf16 : RowsBf16<R, NT> {
  __device__ __forceinline__ void row_origin(int64_t o, int64_t total) {
    this->row0 = o;
    this->rows = (int)lmin(R, total - o);
  }
};
template <int R>
struct SColsBf16 : ColsBf16<R, NT> {
  __device__ __forceinline__ void row_origin(int64_t o, int64_t total) {
    this->col0 = o;
    this->cols = (int)lmin(R, total - o);
  }
};
unsigned cdiv(int64_t a, int64_t b) { return (unsigned)((a + b - 1) / b); }

template <int BM, int BN, class LA, class LB>
hipError_t launch_skinny(const LA& la, const LB& lb, int64_t rows, int64_t cols, int64_t red, int splits,
                         float* out, hipStream_t s) {
  SkinnyParams<BM, BN, LA, LB> p{la, lb, rows, cols, 0, 0, out};
  p.ksteps = (int)((red + BK - 1) / BK);
  p.steps_per_split = (p.ksteps + splits - 1) / splits;
  // splits that receive no steps (and an empty reduction) still write zeros
  dim3 grid(cdiv(cols, BN), cdiv(rows, BM), (unsigned)splits);
  if (grid.x == 0 || grid.y == 0) return hipSuccess;
  hipLaunchKernelGGL((skinny_kernel<BM, BN, LA, LB>), grid, dim3(NT), 0, s, p);
  return hipGetLastError();
}

// Split-K of a skinny product: double the splits while the workgroups number
// under 512 and every split keeps at least min_steps of the 64-deep steps, at
// most 64.  The LoRA-down H = X A^T and dH = s dY B (r <= 128 columns, few
// tiles) go down to 2 steps per split: their partials are small, and more
// workgroups beat the prologue each one pays (3-5 us less at M = 64..512 on
// the Llama MLP shapes than with 8 steps).
int pick_splits(int64_t tiles, int64_t ksteps, int64_t min_steps) {
  int s = 1;
  while (tiles * s < 512 && s * 2 * min_steps <= ksteps && s < 64) s *= 2;
  return s;
}
constexpr int64_t kLoraMinSteps = 2;

}  // namespace

// ------------------------------------------------------------------ host side

// H = X A^T as fp32 [M, r] (single split: written directly).
hipError_t launch_lora_down(const uint16_t* X, int64_t M, int64_t K, const uint16_t* A, int64_t r,
                            float* H, float* scratch, hipStream_t s) {
  SRowsBf16<128> la;
  la.src = X; la.ld = K; la.red = (int)K; la.vec = true;
  SRowsBf16<64> lb;
  lb.src = A; lb.ld = K; lb.red = (int)K; lb.vec = true;
  const int64_t ksteps = K / BK;
  const int splits = pick_splits((int64_t)cdiv(M, 128) * cdiv(r, 64), ksteps, kLoraMinSteps);
  float* out = splits == 1 ? H : scratch;
  hipError_t e = launch_skinny<128, 64>(la, lb, M, r, K, splits, out, s);
  if (e != hipSuccess || splits == 1) return e;
  hipLaunchKernelGGL(reduce_splits_kernel, dim3(cdiv(M * r, 256)), dim3(256), 0, s, scratch, splits,
                     (int64_t)(M * r), 1.0f, (uint16_t*)nullptr, H);
  return hipGetLastError();
}

size_t lora_down_scratch_bytes(int64_t M, int64_t K, int64_t r) {
  const int splits = pick_splits((int64_t)cdiv(M, 128) * cdiv(r, 64), K / BK, kLoraMinSteps);
  return splits == 1 ? 0 : (size_t)splits * M * r * sizeof(float);
}

// Launch a tiled kernel with dynamic LDS (its limit raised once per device).
template <class Kern, class P>
hipError_t launch_tiled(Kern kern, int threads, size_t lds, int mtiles, int ntiles, int splits, P& p,
                        hipStream_t s) {
  hipError_t e = ensure_lds_limit(reinterpret_cast<const void*>(kern), lds);
  if (e != hipSuccess) return e;
  p.mtiles = mtiles;
  p.ntiles = ntiles;
  p.gm = mtiles >= 8 ? mtiles / 8 : 1;
  hipLaunchKernelGGL(kern, dim3((unsigned)(mtiles * ntiles * splits)), dim3(threads), lds, s, p);
  return hipGetLastError();
}

// Tile size and split-K for an M x N output over `steps` 64-deep steps:
// 256 x 256 tiles (8 waves, one workgroup per CU) when they alone give every
// CU a tile, else 128 x 128 tiles (4 waves, two workgroups per CU), split
// along the reduction until about 512 workgroups run, keeping at least 8
// steps per split.
struct GemmPlan {
  int tile, mtiles, ntiles, splits, steps_per_split;
};

GemmPlan gemm_plan(int64_t M, int64_t N, int64_t steps) {
  GemmPlan g;
  const int64_t t256 = cdiv(M, 256) * cdiv(N, 256);
  g.tile = (M >= 256 && t256 >= 256) ? 256 : 128;
  g.mtiles = (int)cdiv(M, g.tile);
  g.ntiles = (int)cdiv(N, g.tile);
  const int64_t tiles = (int64_t)g.mtiles * g.ntiles;
  int sp = 1;
  if (g.tile == 128)
    while (tiles * sp < 512 && steps / (sp * 2) >= 8 && sp < 16) sp *= 2;
  g.steps_per_split = std::max(1, (int)cdiv(steps, sp));   // an empty reduction is one empty split
  g.splits = std::max(1, (int)cdiv(steps, g.steps_per_split));
  return g;
}

// Large layers run on 256 x 256 tiles, one workgroup per CU.  When their
// count leaves the last round of workgroups partly empty, the columns of
// whole rounds stay on one launch and the remaining columns (at least a whole
// 256 block of them) run as a second launch: 256 x 256 tiles split in two
// along the reduction when twice their count fits one round (a split step
// costs what a 256 step costs, against a 128 x 128 step at about 60 % of it
// for a quarter of the work), else 128 x 128 tiles, two per CU.
struct FwdTail {
  int64_t n_main = 0;   // columns of the main launch; 0: no separate tail
  bool split256 = false;
  size_t scratch = 0;   // fp32 partials of the split tail
};
static FwdTail fwd_tail(const GemmPlan& g, int64_t M, int64_t N, int64_t ksteps) {
  FwdTail t;
  if (g.tile != 256 || g.splits != 1) return t;
  const int64_t cus = cu_count();
  const int64_t tiles = (int64_t)g.mtiles * g.ntiles, rounds = tiles / cus;
  const int64_t n_main = rounds * cus / g.mtiles * 256;   // 256-wide column tiles of whole rounds
  if (tiles % cus == 0 || rounds < 1 || n_main <= 0 || n_main >= N) return t;
  const int64_t nn = N - n_main;
  if (cdiv(M, 128) * cdiv(nn, 128) > 2 * cus) return t;
  t.n_main = n_main;
  t.split256 = ksteps >= 2 && 2 * (int64_t)g.mtiles * cdiv(nn, 256) <= cus;
  t.scratch = t.split256 ? (size_t)2 * M * nn * sizeof(float) : 0;
  return t;
}

// Stream-K (fwd_gemm_sk_kernel) on the 128 x 128 tiles where split-K (more
// than one piece per tile: partials are written either way) would need more
// than one round of resident workgroups (two per CU), and every range keeps
// at least 32 steps.  Measured on MI355X, forward with r = 64: M = 384 and
// 512 on 11008 x 4096 and M = 512 on 12288 x 4096 (32-48 steps per range)
// 5-8 % faster; M = 256 on 11008 x 4096 (21.5 steps) 4 % slower, since a
// step with two workgroups on every CU costs more than one in split-K's
// lightly loaded second round; M = 1024 (no split: stream-K adds the
// partials) 9 % slower.
struct SkPlan {
  bool on = false;
  int w = 0, slot_rows = 0;
  size_t scratch = 0;   // fp32 pieces: w + tiles - 1 slots of slot_rows x 128
};
static SkPlan sk_plan(const GemmPlan& g, int64_t M, int64_t ksteps) {
  SkPlan k;
  const int64_t slots = 2 * (int64_t)cu_count();
  const int64_t tiles = (int64_t)g.mtiles * g.ntiles;
  if (g.tile != 128 || g.splits < 2 || tiles * g.splits <= slots || tiles * ksteps < 32 * slots) return k;
  k.on = true;
  k.w = (int)slots;
  k.slot_rows = (int)std::min<int64_t>(M, 128);
  k.scratch = (size_t)(k.w + tiles - 1) * k.slot_rows * 128 * sizeof(float);
  return k;
}

size_t gemm_fwd_scratch_bytes(int64_t M, int64_t N, int64_t K) {
  const GemmPlan g = gemm_plan(M, N, K / BK);
  const SkPlan k = sk_plan(g, M, K / BK);
  if (k.on) return k.scratch;
  const size_t split = g.splits > 1 ? (size_t)g.splits * M * N * sizeof(float) : 0;
  return std::max(split, fwd_tail(g, M, N, K / BK).scratch);
}

// Compute units of the current device (cached per device; thread-safe).
int cu_count() {
  static std::mutex mu;
  static std::map<int, int> cus;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cus.find(dev);
  if (it != cus.end()) return it->second;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  cus[dev] = n;
  return n;
}

// Raises `kernel`'s dynamic-LDS limit to at least `bytes` on the current
// device, once per (device, kernel, size) (thread-safe).
hipError_t ensure_lds_limit(const void* kernel, size_t bytes) {
  static std::mutex mu;
  static std::map<std::pair<int, const void*>, size_t> raised;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  size_t& have = raised[{dev, kernel}];
  if (have >= bytes) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == hipSuccess) have = bytes;
  return e;
}

// The forward product over output columns [n0, n0 + nn) of the layer (rows n0..
// of the weight), with the given tile size and split.
static FwdGemmParams fwd_params(const FwdArgs& a, int64_t n0, int64_t nn, float* scratch) {
  const int64_t nblk = a.K / BK;
  FwdGemmParams p;
  p.X = a.X;
  p.M = a.M;
  p.N = nn;
  p.K = a.K;
  p.r = (int)a.r;
  p.codes = a.w.codes + n0 * (a.K / 2);
  p.c2 = a.w.c2 + n0 * nblk;
  p.c1 = a.w.c1 + n0 * nblk / 256;   // (n0 * nblk is a multiple of 256)
  p.mean = a.w.mean;
  p.H = a.H;
  p.B = a.B + n0 * a.r;
  p.b_vec = (a.r % 8) == 0 && (reinterpret_cast<uintptr_t>(p.B) % 16) == 0;
  p.scale = a.scale;
  p.Y = a.Y + n0;
  p.ldy = a.N;
  p.y_vec = (reinterpret_cast<uintptr_t>(p.Y) % 8) == 0 && (a.N % 4) == 0;
  p.part = scratch;
  p.tab = code_table(a.w.table);
  p.sk_w = 0;
  p.slot_rows = 0;
  return p;
}

hipError_t launch_fwd_cols(const FwdArgs& a, int64_t n0, int64_t nn, int tile, int splits, int steps_per_split,
                           float* scratch, hipStream_t s) {
  FwdGemmParams p = fwd_params(a, n0, nn, scratch);
  p.splits = splits;
  p.steps_per_split = steps_per_split;
  const int mtiles = (int)cdiv(a.M, tile), ntiles = (int)cdiv(nn, tile);
  if (tile == 256)
    return launch_tiled(fwd_gemm_kernel<256, 256, 4>, 512, frag_lds_bytes(256, 256), mtiles, ntiles, splits, p, s);
  return launch_tiled(fwd_gemm_kernel<128, 128, 2>, 256, frag_lds_bytes(128, 128), mtiles, ntiles, splits, p, s);
}

// The stream-K product and the sum of its shared tiles.
static hipError_t launch_fwd_sk(const FwdArgs& a, const GemmPlan& g, const SkPlan& k, float* scratch,
                                hipStream_t s) {
  FwdGemmParams p = fwd_params(a, 0, a.N, scratch);
  p.splits = 1;
  p.steps_per_split = (int)(a.K / BK);
  p.sk_w = k.w;
  p.slot_rows = k.slot_rows;
  p.mtiles = g.mtiles;
  p.ntiles = g.ntiles;
  p.gm = g.mtiles >= 8 ? g.mtiles / 8 : 1;
  const size_t lds = frag_lds_bytes(128, 128);
  void (*kern)(FwdGemmParams) = fwd_gemm_sk_kernel<128, 128, 2>;
  hipError_t e = ensure_lds_limit(reinterpret_cast<const void*>(kern), lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)k.w), dim3(256), lds, s, p);
  const int tiles = g.mtiles * g.ntiles;
  const int64_t threads = (int64_t)tiles * k.slot_rows * 32;
  hipLaunchKernelGGL(reduce_streamk_kernel, dim3((unsigned)cdiv(threads, 256)), dim3(256), 0, s, scratch, tiles,
                     (int)(a.K / BK), k.w, g.mtiles, g.ntiles, p.gm, k.slot_rows, a.M, a.N, a.Y, a.N, p.y_vec);
  return hipGetLastError();
}

hipError_t launch_gemm_fwd(const FwdArgs& a, float* scratch, hipStream_t s) {
  const GemmPlan g = gemm_plan(a.M, a.N, a.K / BK);
  hipError_t e;
  const FwdTail t = fwd_tail(g, a.M, a.N, a.K / BK);
  if (t.n_main > 0) {
    if ((e = launch_fwd_cols(a, 0, t.n_main, 256, 1, g.steps_per_split, scratch, s)) != hipSuccess) return e;
    const int64_t nn = a.N - t.n_main;
    const int ksteps = (int)(a.K / BK);
    if (!t.split256) return launch_fwd_cols(a, t.n_main, nn, 128, 1, ksteps, scratch, s);
    const int half = (ksteps + 1) / 2;
    if ((e = launch_fwd_cols(a, t.n_main, nn, 256, (int)cdiv(ksteps, half), half, scratch, s)) != hipSuccess)
      return e;
    hipLaunchKernelGGL(reduce_splits_cols_kernel, dim3((unsigned)std::min<int64_t>(cdiv(a.M * nn, 1024), 4096)),
                       dim3(256), 0, s, scratch, (int)cdiv(ksteps, half), a.M, nn, a.Y + t.n_main, a.N);
    return hipGetLastError();
  }
  const SkPlan k = sk_plan(g, a.M, a.K / BK);
  if (k.on) return launch_fwd_sk(a, g, k, scratch, s);
  if ((e = launch_fwd_cols(a, 0, a.N, g.tile, g.splits, g.steps_per_split, scratch, s)) != hipSuccess) return e;
  if (g.splits == 1) return e;
  hipLaunchKernelGGL(reduce_splits_kernel, dim3((unsigned)std::min<int64_t>(cdiv(a.M * a.N, 256), 4096)),
                     dim3(256), 0, s, scratch, g.splits, (int64_t)(a.M * a.N), 1.0f, a.Y, (float*)nullptr);
  return hipGetLastError();
}

// The single-pass LoRA-gradient launch: C chunks of 128 columns per
// workgroup (4, or 2 for N <= 256), gn workgroups along N and as many along M
// as keep the launch within one workgroup per CU (at least one 64-row tile
// each).  It takes ranks that are multiples of 8 up to 64 and M, N multiples
// of 8 (16-byte rows of H^T, dY and B); other layers form dH and dB as two
// separate products, each reading dY.
struct LgPlan {
  bool ok;
  int C, gn, gm, mtiles;
  size_t part_h, part_b;   // partial bytes
};
static LgPlan lg_plan(int64_t M, int64_t N, int64_t r) {
  LgPlan g{};
  g.ok = M > 0 && N > 0 && r > 0 && r <= 64 && r % 8 == 0 && M % 8 == 0 && N % 8 == 0;
  if (!g.ok) return g;
  g.C = N > 256 ? 4 : 2;
  g.gn = (int)cdiv(N, 128 * g.C);
  g.mtiles = (int)cdiv(M, 64);
  g.gm = (int)std::max<int64_t>(1, std::min<int64_t>(g.mtiles, cu_count() / g.gn));
  // 32-bit buffer offsets: a workgroup's rows of dY, B and H^T
  const int64_t rows = 64 * cdiv(g.mtiles, g.gm);
  g.ok = rows * N * 2 < (1ll << 31) && N * r * 2 < (1ll << 31) && M * r * 4 < (1ll << 31);
  g.part_h = (size_t)g.gn * M * r * sizeof(float);
  g.part_b = (size_t)g.gm * N * r * sizeof(float);
  return g;
}

// Backward workspace: H (if recomputed), dH, their bf16 transposes and
// split-K partials (or the single-pass launch's partials of dH and dB).
struct BwdPlan {
  int s_dh, s_db, s_da;
  size_t off_H, off_dH, off_Ht, off_dHt, off_part, bytes;
};

// Split-K of a 128 x 128 skinny product: as many splits as keep all its
// workgroups in one round (two per CU at 74 KB of LDS each), at least 1, at
// most 64 and no more than the reduction's steps.  (A second, partly empty
// round cost the 65B-scale layer's dB product 6 us.)
static int one_round_splits(int64_t tiles, int64_t ksteps) {
  const int64_t slots = 2 * (int64_t)cu_count();
  return (int)std::max<int64_t>(1, std::min<int64_t>({64, slots / std::max<int64_t>(tiles, 1), ksteps}));
}

static BwdPlan bwd_plan(int64_t M, int64_t N, int64_t K, int64_t r) {
  BwdPlan b;
  b.s_dh = pick_splits((int64_t)cdiv(M, 128) * cdiv(r, 64), (N + BK - 1) / BK, kLoraMinSteps);
  b.s_db = one_round_splits((int64_t)cdiv(N, 128) * cdiv(2 * r, 128), (M + BK - 1) / BK);
  b.s_da = one_round_splits((int64_t)cdiv(2 * r, 128) * cdiv(K, 128), (M + BK - 1) / BK);
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  b.off_H = 0;
  b.off_dH = al((size_t)M * r * 4);
  b.off_Ht = b.off_dH + al((size_t)M * r * 4);     // bf16 hi/lo of H^T and dH^T [2r][M]
  b.off_dHt = b.off_Ht + al((size_t)M * r * 4);
  b.off_part = b.off_dHt + al((size_t)M * r * 4);
  size_t part = std::max({(size_t)b.s_dh * M * r, (size_t)b.s_db * N * 2 * r, (size_t)b.s_da * 2 * r * K}) * 4;
  part = std::max(part, lora_down_scratch_bytes(M, K, r));
  const LgPlan lg = lg_plan(M, N, r);
  if (lg.ok) part = std::max(part, al(lg.part_h) + lg.part_b);
  const GemmPlan g = gemm_plan(M, K, (N + BK - 1) / BK);
  if (g.splits > 1) part = std::max(part, (size_t)g.splits * M * K * sizeof(float));
  b.bytes = b.off_part + al(part);
  return b;
}

size_t gemm_bwd_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t r) {
  return bwd_plan(M, N, K, r).bytes;
}

hipError_t launch_linear_bwd(const BwdArgs& a, hipStream_t s) {
  const BwdPlan plan = bwd_plan(a.M, a.N, a.K, a.r);
  char* ws = reinterpret_cast<char*>(a.workspace);
  float* H = const_cast<float*>(a.H);
  float* dH = reinterpret_cast<float*>(ws + plan.off_dH);
  float* part = reinterpret_cast<float*>(ws + plan.off_part);
  hipError_t e;
  if (a.r > 0) {  // no adapter (r = 0): only the input gradient
    if (a.M > 0 && !H) {
      H = reinterpret_cast<float*>(ws + plan.off_H);
      if ((e = launch_lora_down(a.X, a.M, a.K, a.A, a.r, H, part, s)) != hipSuccess) return e;
    }
    const bool n_vec = (a.N % 8) == 0;
    const bool r_vec = (a.r % 8) == 0 && (reinterpret_cast<uintptr_t>(a.B) % 16) == 0;
    const bool m_vec = (a.M % 8) == 0;
    uint16_t* Ht = reinterpret_cast<uint16_t*>(ws + plan.off_Ht);
    uint16_t* dHt = reinterpret_cast<uint16_t*>(ws + plan.off_dHt);
    const dim3 tgrid(cdiv(a.M, 16), cdiv(a.r, 64));
    const LgPlan lg = lg_plan(a.M, a.N, a.r);
    const bool one_pass = lg.ok && (reinterpret_cast<uintptr_t>(a.dY) % 16) == 0 &&
                          (reinterpret_cast<uintptr_t>(a.B) % 16) == 0 && (reinterpret_cast<uintptr_t>(H) % 16) == 0;
    // H^T as bf16 hi/lo for the separate dB product (the single pass splits H itself)
    if (a.M > 0 && !one_pass)
      hipLaunchKernelGGL(f32_to_bf16_t_kernel, tgrid, dim3(256), 0, s, H, a.M, a.r, Ht, Ht + a.r * a.M);
    if (one_pass) {
      // dH and dB from one read of dY, then their reductions
      LgParams q;
      q.dY = a.dY;
      q.B = a.B;
      q.H = H;
      q.M = a.M;
      q.N = a.N;
      q.r = (int)a.r;
      q.gm = lg.gm;
      q.mtiles = lg.mtiles;
      q.part_h = part;
      q.part_b = reinterpret_cast<float*>(reinterpret_cast<char*>(part) + ((lg.part_h + 255) & ~(size_t)255));
      const auto kern = lg.C == 4 ? lora_grads_kernel<4> : lora_grads_kernel<2>;
      if ((e = ensure_lds_limit(reinterpret_cast<const void*>(kern), lg_lds_bytes(lg.C))) != hipSuccess) return e;
      hipLaunchKernelGGL(kern, dim3((unsigned)(lg.gm * lg.gn)), dim3(512), lg_lds_bytes(lg.C), s, q);
      const int64_t hb = (int64_t)cdiv(a.M, 16) * cdiv(a.r, 64), bb = cdiv(a.N * a.r, 1024);
      hipLaunchKernelGGL(lora_finish_kernel, dim3((unsigned)(hb + bb)), dim3(256), 0, s, q.part_h, lg.gn, q.part_b,
                         lg.gm, a.M, a.N, (int)a.r, a.scale, dH, dHt, a.dB);
    }
    // dH = s dY B : rows m, cols j, reduction n
    if (a.M > 0 && !one_pass) {
      SRowsBf16<128> la;
      la.src = a.dY; la.ld = a.N; la.red = (int)a.N; la.vec = n_vec;
      SColsBf16<64> lb;
      lb.src = a.B; lb.ld = a.r; lb.red = (int)a.N; lb.vec = r_vec;
      if ((e = launch_skinny<128, 64>(la, lb, a.M, a.r, a.N, plan.s_dh, part, s)) != hipSuccess) return e;
      hipLaunchKernelGGL(reduce_splits_kernel, dim3(cdiv(a.M * a.r, 256)), dim3(256), 0, s, part, plan.s_dh,
                         (int64_t)(a.M * a.r), a.scale, (uint16_t*)nullptr, dH);
      hipLaunchKernelGGL(f32_to_bf16_t_kernel, tgrid, dim3(256), 0, s, dH, a.M, a.r, dHt, dHt + a.r * a.M);
    }
    // dB = s dY^T H : rows n, cols j, reduction m; H as [hi; lo] (2r columns)
    if (a.N > 0 && !one_pass) {
      SColsBf16<128> la;
      la.src = a.dY; la.ld = a.N; la.red = (int)a.M; la.vec = n_vec;
      SRowsBf16<128> lb;
      lb.src = Ht; lb.ld = a.M; lb.red = (int)a.M; lb.vec = m_vec;
      if ((e = launch_skinny<128, 128>(la, lb, a.N, 2 * a.r, a.M, plan.s_db, part, s)) != hipSuccess) return e;
      hipLaunchKernelGGL(reduce_hilo_kernel, dim3(cdiv(a.N * a.r, 256)), dim3(256), 0, s, part, plan.s_db,
                         (int64_t)(a.N * 2 * a.r), a.N, a.r, 2 * a.r, a.r, a.scale, a.dB);
    }
    // dA = dH^T X : rows j, cols k, reduction m; dH^T as [hi; lo] (2r rows)
    {
      SRowsBf16<128> la;
      la.src = dHt; la.ld = a.M; la.red = (int)a.M; la.vec = m_vec;
      SColsBf16<128> lb;
      lb.src = a.X; lb.ld = a.K; lb.red = (int)a.M; lb.vec = true;
      if ((e = launch_skinny<128, 128>(la, lb, 2 * a.r, a.K, a.M, plan.s_da, part, s)) != hipSuccess) return e;
      hipLaunchKernelGGL(reduce_hilo_kernel, dim3(cdiv(a.r * a.K, 256)), dim3(256), 0, s, part, plan.s_da,
                         (int64_t)(2 * a.r * a.K), a.r, a.K, a.K, a.r * a.K, 1.0f, a.dA);
    }
  }
  // dX = dY W_deq + dH A
  if (a.dX && a.M > 0) {
    DxParams p;
    p.dY = a.dY;
    p.M = a.M;
    p.N = a.N;
    p.K = a.K;
    p.r = (int)a.r;
    p.codes = a.w.codes;
    p.c2 = a.w.c2;
    p.c1 = a.w.c1;
    p.mean = a.w.mean;
    p.dH = dH;
    p.A = a.A;
    p.dX = a.dX;
    const GemmPlan g = gemm_plan(a.M, a.K, (a.N + BK - 1) / BK);
    p.part = part;
    p.splits = g.splits;
    p.steps_per_split = g.steps_per_split;
    p.tab = code_table(a.w.table);
    const bool vy = (a.N % 8) == 0;
    if (g.tile == 256)
      e = launch_tiled(vy ? dxr_gemm_kernel<256, 256, 4, true> : dxr_gemm_kernel<256, 256, 4, false>, 512,
                       dxr_lds_bytes(256, 256), g.mtiles, g.ntiles, g.splits, p, s);
    else
      e = launch_tiled(vy ? dxr_gemm_kernel<128, 128, 2, true> : dxr_gemm_kernel<128, 128, 2, false>, 256,
                       dxr_lds_bytes(128, 128), g.mtiles, g.ntiles, g.splits, p, s);
    if (e != hipSuccess) return e;
    if (g.splits > 1)
      hipLaunchKernelGGL(reduce_splits_kernel, dim3((unsigned)std::min<int64_t>(cdiv(a.M * a.K, 256), 4096)),
                         dim3(256), 0, s, part, g.splits, (int64_t)(a.M * a.K), 1.0f, a.dX, (float*)nullptr);
  }
  return hipGetLastError();
}

}  // namespace qlora
