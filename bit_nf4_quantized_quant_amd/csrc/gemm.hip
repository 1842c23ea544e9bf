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
// The forward product keeps its operands in fragment-major tiles (below)
// with loads two steps ahead; the backward's products stage [rows][64 + 8]
// bf16 tiles (reduction contiguous, 16-byte pad so that 16-byte fragment
// reads of eight consecutive rows hit distinct banks).
//
// Loaders turn every source layout into that LDS form:
//   RowsBf16  bf16 [rows][red] (X, dY, A, B, and the bf16 H^T, dH^T)
//   Nf4Rows   NF4 codes [rows][K/2] -> bf16 W_deq, bit-exact with the spec
//   Nf4Cols   NF4 codes read as [red = n][rows = k]: the transposed weight for dX
//   ColsBf16  bf16 [red][rows] (transposed operands of the LoRA gradients)
// A transposed source is read as 4 x 8 patches (4 rows of 8 contiguous
// elements) and written to LDS as 8 rows of 4 reduction elements.
#include <algorithm>
#include <type_traits>

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
template <int R, int T, bool kVec, int kDepth = 2>
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
    const int sof = kt * BK * 2;
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      if (kVec) {
        reg[S][c] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off[c], sof, 0));
      } else {
        uint32_t e[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) e[q] = __builtin_amdgcn_raw_buffer_load_b16(rs, off[c] + 2 * q, sof, 0);
        reg[S][c] = u32x4{e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16)};
      }
    }
  }
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
  const float* lut;
  u32x4 q[2][kUnits];      // two steps in flight
  uint32_t c2v[2][kUnits];
  float c1v[2][kUnits];
  float chat[kUnits];      // constants of the step being stored

  __device__ __forceinline__ void init(const uint8_t* codes, const uint8_t* c2, const float* c1, float mu,
                                       int64_t N, int64_t K, int64_t row0, const float* lut_) {
    const int rows = (int)lmin(R, N - row0);
    const int64_t nb = K / BK;
    rc = tile_rsrc(codes, row0 * (K / 2), N * (K / 2));
    r2 = tile_rsrc(c2, row0 * nb, N * nb);
    r1 = tile_rsrc(c1, 0, ((N * nb + 255) / 256) * 4);
    mean = mu;
    lut = lut_;
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
  // chunk P (8 codes) of every unit of the step held in slot S; the level
  // table lives in static LDS, so a code's byte address (code * 4) is its
  // whole ds_read address
  template <int S, int P>
  __device__ __forceinline__ void store_part(lds_t* t) {
#pragma unroll
    for (int u = 0; u < kUnits; ++u) store_unit<S, P>(t, u);
  }
  template <int S, int P>
  __device__ __forceinline__ void store_unit(lds_t* t, int u) {
    if (P == 0) chat[u] = dequant_constant(c2v[S][u], c1v[S][u], mean);
    const int idx = threadIdx.x + u * T;
    const int row = idx >> 1, h = idx & 1;
    const uint32_t word = q[S][u][P];
    const uint32_t lo4 = (word << 2) & 0x3C3C3C3Cu;   // 4 * low nibble of each byte
    const uint32_t hi4 = (word >> 2) & 0x3C3C3C3Cu;   // 4 * high nibble of each byte
    u32x4 o;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const uint32_t al = byte_of(lo4, b), ah = byte_of(hi4, b);
      const float lo = __fmul_rn(*reinterpret_cast<const float*>(reinterpret_cast<const char*>(lut) + al), chat[u]);
      const float hi = __fmul_rn(*reinterpret_cast<const float*>(reinterpret_cast<const char*>(lut) + ah), chat[u]);
      o[b] = pack_bf16x2(lo, hi);
    }
    st_lds16(t + frag_slot<R>(row, 4 * h + P), o);
  }
  __device__ __forceinline__ void prologue(int kt0, int last, lds_t* t) {
    load<0>(kt0);
    store_part<0, 0>(t);
    store_part<0, 1>(t);
    store_part<0, 2>(t);
    store_part<0, 3>(t);
    load<1>(min(kt0 + 1, last));
  }
  template <int S>
  __device__ __forceinline__ void ahead(int kt, int last) {
    load<S>(min(kt + 2, last));
  }
};

// NF4 weight read transposed: tile row i = weight column k0 + i, reduction =
// weight row n.  A thread takes patches of 4 rows (n) x 8 columns (k); the 8
// columns lie in one block of each row, so a patch needs 4 constants.
template <int R, int T = NT>
struct Nf4Cols {
  static constexpr int kPatches = 2 * R;
  static constexpr int kPer = (kPatches + T - 1) / T;
  const uint8_t* codes;
  const uint8_t* c2;
  const float* c1;
  float mean;
  int64_t N, K;
  int64_t col0;
  const float* lut;
  uint32_t word[kPer][4];
  float chat[kPer][4];

  __device__ __forceinline__ void load(int kt) {
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int pid = threadIdx.x + u * T;
      if (pid >= kPatches) break;
      const int pr = pid % (BK / 4), pc = pid / (BK / 4);
      const int64_t k = col0 + pc * 8;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t n = (int64_t)kt * BK + pr * 4 + q;
        if (n < N && k < K) {
          word[u][q] = *reinterpret_cast<const uint32_t*>(codes + n * (K / 2) + k / 2);
          const int64_t bi = n * (K / 64) + k / 64;
          chat[u][q] = dequant_constant(c2[bi], c1[bi >> 8], mean);
        } else {
          word[u][q] = 0u;
          chat[u][q] = 0.f;
        }
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
      for (int z = 0; z < 8; ++z) {
        float v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = __fmul_rn(lut[(word[u][q] >> (4 * z)) & 15u], chat[u][q]);
        st_lds8(t + (pc * 8 + z) * PITCH + pr * 4, u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])});
      }
    }
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
        acc.c[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc.c[i][j], 0, 0, 0);
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
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc.c[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[p & 1][i], fb[p & 1][j], acc.c[i][j], 0, 0, 0);
    la.template store_part<S, p>(da);
    lb.template store_part<S, p>(db);
  };
  read(0, 0);
  sub(std::integral_constant<int, 0>{});
  sub(std::integral_constant<int, 1>{});
  sub(std::integral_constant<int, 2>{});
  sub(std::integral_constant<int, 3>{});
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

// Lane l of a 32x32 accumulator holds column l%32 and rows 8*(v/4) + 4*(l/32) + v%4.
template <int BM, int BN, int WN, class F>
__device__ __forceinline__ void for_each_out(const Acc<BM, BN, WN>& acc, F f) {
  constexpr int TM = Acc<BM, BN, WN>::TM, TN = Acc<BM, BN, WN>::TN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = wm * (BM / 2) + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        const int col = wn * (BN / WN) + j * 32 + (lane & 31);
        f(row, col, acc.c[i][j][v]);
      }
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
        acc.c[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc.c[i][j], 0, 0, 0);
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
__device__ __forceinline__ void tile_of(int L, int mtiles, int ntiles, int gm, int& mi, int& ni) {
  const int T = mtiles * ntiles;
  const int x = L & 7, j = L >> 3;
  const int q = T >> 3, rem = T & 7;
  const int logical = x * q + min(x, rem) + j;
  const int per_group = gm * ntiles;
  const int group = logical / per_group;
  const int first_m = group * gm;
  const int gm_eff = min(gm, mtiles - first_m);
  const int in_group = logical - group * per_group;
  mi = uniform(first_m + in_group % gm_eff);
  ni = uniform(in_group / gm_eff);
}

// dynamic LDS of the pipelined products (fragment-major tiles, two buffers)
__host__ __device__ constexpr size_t frag_lds_bytes(int bm, int bn) {
  return (size_t)2 * (bm + bn) * BK * sizeof(lds_t);
}

__host__ __device__ constexpr size_t gemm_lds_bytes(int bm, int bn) {
  return (size_t)2 * (bm + bn) * PITCH * sizeof(lds_t) + 16 * sizeof(float);
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
  float* part;          // split-K partials [splits][M][N] (splits > 1, ldy = N)
  int splits, steps_per_split;
  int mtiles, ntiles, gm;
  Nf4Table tab;
};

template <int BM, int BN, int WN>
__global__ void __launch_bounds__(128 * WN) fwd_gemm_kernel(FwdGemmParams p) {
  constexpr int T = 128 * WN;
  extern __shared__ __attribute__((aligned(16))) lds_t smem[];
  __shared__ float lut[16];
  lds_t* sa = smem;
  lds_t* sb = smem + 2 * BM * BK;   // fragment-major tiles, double-buffered
  load_lut(lut, p.tab);
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
    lb.init(p.codes, p.c2, p.c1, *p.mean, p.N, p.K, n0, lut);
    run_pipelined<BM, BN, WN>(la, lb, kt0, kt1, sa, sb, acc);
  }
  if (split == 0)
    lora_tail<BM, BN, WN>(
        acc, p.r,
        [&](int i, int k0) { return frag_f32_row(p.H, p.r, m0 + i, p.M, k0, p.r, p.scale); },
        [&](int j, int k0) { return frag_bf16_row(p.B, p.r, n0 + j, p.N, k0, p.r, p.b_vec); });
  if (p.splits == 1) {
    for_each_out(acc, [&](int i, int j, float v) {
      const int64_t m = m0 + i, n = n0 + j;
      if (m < p.M && n < p.N) p.Y[m * p.ldy + n] = to_bf16(v);
    });
  } else {
    float* out = p.part + (int64_t)split * p.M * p.N;
    for_each_out(acc, [&](int i, int j, float v) {
      const int64_t m = m0 + i, n = n0 + j;
      if (m < p.M && n < p.N) out[m * p.N + n] = v;
    });
  }
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
  for_each_out(acc, [&](int i, int j, float v) {
    const int64_t a = i0 + i, b = j0 + j;
    if (a < p.rows && b < p.cols) out[a * p.cols + b] = v;
  });
}

// Sum split-K partials: out = scale * sum_s part[s]; bf16 or fp32 output.
__global__ void __launch_bounds__(256) reduce_splits_kernel(const float* __restrict__ part, int splits,
                                                            int64_t count, float scale,
                                                            uint16_t* __restrict__ out_bf16,
                                                            float* __restrict__ out_f32) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride) {
    float s = 0.f;
    for (int k = 0; k < splits; ++k) s += part[(int64_t)k * count + i];
    s *= scale;
    if (out_bf16) out_bf16[i] = to_bf16(s);
    if (out_f32) out_f32[i] = s;
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

// dX = dY W_deq + dH A (bf16 output).  Phase 1 contracts over n with the
// transposed NF4 weight; phase 2 appends r steps of dH against A^T.
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

template <int BM, int BN, int WN>
__global__ void __launch_bounds__(128 * WN) dx_gemm_kernel(DxParams p) {
  constexpr int T = 128 * WN;
  extern __shared__ __attribute__((aligned(16))) lds_t smem[];
  lds_t* sa = smem;
  lds_t* sb = smem + 2 * BM * PITCH;
  float* lut = reinterpret_cast<float*>(sb + 2 * BN * PITCH);
  load_lut(lut, p.tab);
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
    RowsBf16<BM, T> la{p.dY, p.N, (int)lmin(BM, p.M - m0), (int)p.N, m0, (p.N % 8) == 0};
    Nf4Cols<BN, T> lb{p.codes, p.c2, p.c1, *p.mean, p.N, p.K, k0, lut};
    run_phase<BM, BN, WN>(la, lb, nt0, nt1, sa, sb, acc);
  }
  if (split == 0)
    lora_tail<BM, BN, WN>(
        acc, p.r,
        [&](int i, int kk) { return frag_f32_row(p.dH, p.r, m0 + i, p.M, kk, p.r, 1.0f); },
        [&](int j, int kk) { return frag_bf16_col(p.A, p.K, k0 + j, p.K, kk, p.r); });
  if (p.splits == 1) {
    for_each_out(acc, [&](int i, int j, float v) {
      const int64_t m = m0 + i, k = k0 + j;
      if (m < p.M && k < p.K) p.dX[m * p.K + k] = to_bf16(v);
    });
  } else {
    float* out = p.part + (int64_t)split * p.M * p.K;
    for_each_out(acc, [&](int i, int j, float v) {
      const int64_t m = m0 + i, k = k0 + j;
      if (m < p.M && k < p.K) out[m * p.K + k] = v;
    });
  }
}

// ---------------------------------------------------------------- dX at large M
// At large M the backward's dX = dY W_deq is a dense, compute-bound product
// whose reduction runs over the weight's rows n.  The weight is then expanded
// once per call into a scratch W_deq^T, bf16 [K][ldt] (ldt = N rounded up to
// 64, zero past N), and the product runs on the pipelined bf16 engine with
// both operands stored along the reduction.  The expansion moves 2.5 bytes
// per weight (codes in, bf16 out), a few percent of the product's time at
// M >= 512; below that the fused dx_gemm_kernel reads the codes directly.
constexpr int64_t kDxtMinM = 512;
constexpr int kDtN = 128, kDtK = 256;   // tile of the transposing expansion (n x k)

// W_deq^T tile: thread t takes rows n0 + 2 (t % 64) + {0, 1} and the 32
// columns k0 + 32 (t / 64) .. +31 (half a block of each row, so one constant
// per row): one 16-byte code load per row, 8 threads covering 128
// contiguous code bytes of a row.  It expands them to bf16 (fp32 level *
// c_hat, bit-exact with W_deq) and stores (n, n+1) pairs per column into an
// LDS tile [k][n]; the tile leaves as 256-byte rows of the output.
__global__ void __launch_bounds__(512) nf4_dequant_t_kernel(const uint8_t* __restrict__ codes,
                                                            const uint8_t* __restrict__ c2,
                                                            const float* __restrict__ c1,
                                                            const float* __restrict__ mean, int64_t N, int64_t K,
                                                            int64_t ldt, uint16_t* __restrict__ out, Nf4Table tab) {
  __shared__ float lut[16];
  __shared__ __attribute__((aligned(16))) uint32_t t[kDtK * kDtN / 2];   // [k][n pair], 64 KiB
  load_lut(lut, tab);
  const int64_t ntiles = (ldt + kDtN - 1) / kDtN;
  const int64_t n0 = (int64_t)(blockIdx.x % ntiles) * kDtN, k0 = (int64_t)(blockIdx.x / ntiles) * kDtK;
  const int np = threadIdx.x & 63, kg = threadIdx.x >> 6;
  const int64_t kc = k0 + 32 * kg;
  const float mu = *mean;
  u32x4 w[2];
  float chat[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int64_t n = n0 + 2 * np + h;
    if (n < N && kc < K) {
      w[h] = ld16(codes + n * (K / 2) + kc / 2);
      const int64_t bi = n * (K / 64) + kc / 64;
      chat[h] = dequant_constant(c2[bi], c1[bi >> 8], mu);
    } else {   // rows past N (and columns past K) expand to zero
      w[h] = u32x4{0u, 0u, 0u, 0u};
      chat[h] = 0.f;
    }
  }
  __syncthreads();   // the level table
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    const float lo = __fmul_rn(lut[(w[0][e >> 3] >> (4 * (e & 7))) & 15u], chat[0]);
    const float hi = __fmul_rn(lut[(w[1][e >> 3] >> (4 * (e & 7))) & 15u], chat[1]);
    t[(32 * kg + e) * (kDtN / 2) + np] = pack_bf16x2(lo, hi);
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kDtK * kDtN / 8 / 512; ++i) {
    const int c = threadIdx.x + i * 512, kr = c >> 4, j = c & 15;
    const int64_t k = k0 + kr, n = n0 + 8 * j;
    if (k < K && n < ldt)
      *reinterpret_cast<u32x4*>(out + k * ldt + n) = *reinterpret_cast<const u32x4*>(&t[kr * (kDtN / 2) + 4 * j]);
  }
}

struct DxtParams {
  const uint16_t* dY;
  const uint16_t* wt;   // W_deq^T [K][ldt]
  int64_t M, N, K, ldt;
  int r;
  const float* dH;
  const uint16_t* A;
  uint16_t* dX;
  float* part;          // split-K partials [splits][M][K] (splits > 1)
  int splits, steps_per_split;
  int mtiles, ntiles, gm;
};

// dX = dY W_deq + dH A on the pipelined engine: rows of dY (reduction n
// contiguous; past N they meet W_deq^T's zero columns) against rows of
// W_deq^T.  kVecY: N % 8 == 0 (16-byte rows of dY).
template <int BM, int BN, int WN, bool kVecY>
__global__ void __launch_bounds__(128 * WN) dxt_gemm_kernel(DxtParams p) {
  constexpr int T = 128 * WN;
  extern __shared__ __attribute__((aligned(16))) lds_t smem[];
  lds_t* sa = smem;
  lds_t* sb = smem + 2 * BM * BK;   // fragment-major tiles, double-buffered
  const int tiles = p.mtiles * p.ntiles;
  const int split = uniform((int)blockIdx.x / tiles);
  int mi, ki;
  tile_of((int)blockIdx.x - split * tiles, p.mtiles, p.ntiles, p.gm, mi, ki);
  const int64_t m0 = (int64_t)mi * BM, k0 = (int64_t)ki * BN;
  const int nsteps = (int)(p.ldt / BK);
  const int nt0 = split * p.steps_per_split, nt1 = min(nsteps, nt0 + p.steps_per_split);
  Acc<BM, BN, WN> acc;
  zero(acc);
  __syncthreads();
  {
    XRows<BM, T, kVecY, (WN == 4 && kVecY ? 2 : 1)> la;
    la.init(p.dY, p.N, p.M, m0);
    XRows<BN, T, true, (WN == 4 ? 2 : 1)> lb;
    lb.init(p.wt, p.ldt, p.K, k0);
    run_pipelined<BM, BN, WN>(la, lb, nt0, nt1, sa, sb, acc);
  }
  if (split == 0)
    lora_tail<BM, BN, WN>(
        acc, p.r,
        [&](int i, int kk) { return frag_f32_row(p.dH, p.r, m0 + i, p.M, kk, p.r, 1.0f); },
        [&](int j, int kk) { return frag_bf16_col(p.A, p.K, k0 + j, p.K, kk, p.r); });
  if (p.splits == 1) {
    for_each_out(acc, [&](int i, int j, float v) {
      const int64_t m = m0 + i, k = k0 + j;
      if (m < p.M && k < p.K) p.dX[m * p.K + k] = to_bf16(v);
    });
  } else {
    float* out = p.part + (int64_t)split * p.M * p.K;
    for_each_out(acc, [&](int i, int j, float v) {
      const int64_t m = m0 + i, k = k0 + j;
      if (m < p.M && k < p.K) out[m * p.K + k] = v;
    });
  }
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

int pick_splits(int64_t tiles, int64_t ksteps) {
  int s = 1;
  while (tiles * s < 512 && s * 2 <= ksteps && s < 64) s *= 2;
  return s;
}

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
  const int splits = pick_splits((int64_t)cdiv(M, 128) * cdiv(r, 64), ksteps);
  float* out = splits == 1 ? H : scratch;
  hipError_t e = launch_skinny<128, 64>(la, lb, M, r, K, splits, out, s);
  if (e != hipSuccess || splits == 1) return e;
  hipLaunchKernelGGL(reduce_splits_kernel, dim3(cdiv(M * r, 256)), dim3(256), 0, s, scratch, splits,
                     (int64_t)(M * r), 1.0f, (uint16_t*)nullptr, H);
  return hipGetLastError();
}

size_t lora_down_scratch_bytes(int64_t M, int64_t K, int64_t r) {
  const int splits = pick_splits((int64_t)cdiv(M, 128) * cdiv(r, 64), K / BK);
  return splits == 1 ? 0 : (size_t)splits * M * r * sizeof(float);
}

// Launch a tiled kernel with dynamic LDS (raising the per-kernel limit once).
template <class Kern, class P>
hipError_t launch_tiled(Kern kern, int threads, size_t lds, int mtiles, int ntiles, int splits, P& p,
                        hipStream_t s) {
  // the LDS limit is raised once per kernel (several kernels can share this
  // instantiation: remember which ones; setting it twice is harmless)
  static const void* done[8] = {};
  const void* kp = reinterpret_cast<const void*>(kern);
  bool seen = false;
  for (const void* d : done) seen = seen || d == kp;
  if (!seen) {
    hipError_t e = hipFuncSetAttribute(kp, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    for (const void*& d : done)
      if (!d) {
        d = kp;
        break;
      }
  }
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

size_t gemm_fwd_scratch_bytes(int64_t M, int64_t N, int64_t K) {
  const GemmPlan g = gemm_plan(M, N, K / BK);
  return g.splits > 1 ? (size_t)g.splits * M * N * sizeof(float) : 0;
}

// Compute units of the current device (cached per device).
int cu_count() {
  static int cus[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

// The forward product over output columns [n0, n0 + nn) of the layer (rows n0..
// of the weight), with the given tile size and split.
hipError_t launch_fwd_cols(const FwdArgs& a, int64_t n0, int64_t nn, int tile, int splits, int steps_per_split,
                           float* scratch, hipStream_t s) {
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
  p.part = scratch;
  p.splits = splits;
  p.steps_per_split = steps_per_split;
  p.tab = code_table(a.w.table);
  const int mtiles = (int)cdiv(a.M, tile), ntiles = (int)cdiv(nn, tile);
  if (tile == 256)
    return launch_tiled(fwd_gemm_kernel<256, 256, 4>, 512, frag_lds_bytes(256, 256), mtiles, ntiles, splits, p, s);
  return launch_tiled(fwd_gemm_kernel<128, 128, 2>, 256, frag_lds_bytes(128, 128), mtiles, ntiles, splits, p, s);
}

// Large layers run on 256 x 256 tiles, one workgroup per CU.  When their
// count leaves the last round of workgroups partly empty, the columns of
// whole rounds stay on 256 x 256 tiles and the remaining columns (at least
// a whole 256 block of them) run as a second launch on 128 x 128 tiles, two
// per CU, whose single round takes a fraction of a 256 round.
hipError_t launch_gemm_fwd(const FwdArgs& a, float* scratch, hipStream_t s) {
  const GemmPlan g = gemm_plan(a.M, a.N, a.K / BK);
  hipError_t e;
  if (g.tile == 256 && g.splits == 1) {
    const int64_t cus = cu_count();
    const int64_t tiles = (int64_t)g.mtiles * g.ntiles, rounds = tiles / cus;
    const int64_t nt_main = rounds * cus / g.mtiles;         // 256-wide column tiles of whole rounds
    const int64_t n_main = nt_main * 256;
    const int64_t tail_tiles = cdiv(a.M, 128) * cdiv(a.N - n_main, 128);
    if (tiles % cus != 0 && rounds >= 1 && n_main > 0 && n_main < a.N && tail_tiles <= 2 * cus) {
      if ((e = launch_fwd_cols(a, 0, n_main, 256, 1, g.steps_per_split, scratch, s)) != hipSuccess) return e;
      return launch_fwd_cols(a, n_main, a.N - n_main, 128, 1, (int)(a.K / BK), scratch, s);
    }
  }
  if ((e = launch_fwd_cols(a, 0, a.N, g.tile, g.splits, g.steps_per_split, scratch, s)) != hipSuccess) return e;
  if (g.splits == 1) return e;
  hipLaunchKernelGGL(reduce_splits_kernel, dim3((unsigned)std::min<int64_t>(cdiv(a.M * a.N, 256), 4096)),
                     dim3(256), 0, s, scratch, g.splits, (int64_t)(a.M * a.N), 1.0f, a.Y, (float*)nullptr);
  return hipGetLastError();
}

// Backward workspace: H (if recomputed), dH, their bf16 transposes, split-K
// partials and, at large M, the expanded W_deq^T.
struct BwdPlan {
  int s_dh, s_db, s_da;
  bool dxt;        // dX through the expanded W_deq^T
  int64_t ldt;     // its row length (N rounded up to 64)
  size_t off_H, off_dH, off_Ht, off_dHt, off_part, off_wt, bytes;
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
  b.s_dh = pick_splits((int64_t)cdiv(M, 128) * cdiv(r, 64), (N + BK - 1) / BK);
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
  b.dxt = M >= kDxtMinM && N > 0;
  b.ldt = (N + 63) / 64 * 64;
  const GemmPlan g = gemm_plan(M, K, b.dxt ? b.ldt / BK : (N + BK - 1) / BK);
  if (g.splits > 1) part = std::max(part, (size_t)g.splits * M * K * sizeof(float));
  b.off_wt = b.off_part + al(part);
  b.bytes = b.off_wt + (b.dxt ? al((size_t)b.ldt * K * 2) : 0);
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
    if (a.M > 0) hipLaunchKernelGGL(f32_to_bf16_t_kernel, tgrid, dim3(256), 0, s, H, a.M, a.r, Ht, Ht + a.r * a.M);
    // dH = s dY B : rows m, cols j, reduction n
    if (a.M > 0) {
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
    if (a.N > 0) {
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
  if (a.dX && a.M > 0 && plan.dxt) {
    uint16_t* wt = reinterpret_cast<uint16_t*>(ws + plan.off_wt);
    hipLaunchKernelGGL(nf4_dequant_t_kernel, dim3(cdiv(plan.ldt, kDtN) * cdiv(a.K, kDtK)), dim3(512), 0, s,
                       a.w.codes, a.w.c2, a.w.c1, a.w.mean, a.N, a.K, plan.ldt, wt, code_table(a.w.table));
    DxtParams p;
    p.dY = a.dY;
    p.wt = wt;
    p.M = a.M;
    p.N = a.N;
    p.K = a.K;
    p.ldt = plan.ldt;
    p.r = (int)a.r;
    p.dH = dH;
    p.A = a.A;
    p.dX = a.dX;
    const GemmPlan g = gemm_plan(a.M, a.K, plan.ldt / BK);
    p.part = part;
    p.splits = g.splits;
    p.steps_per_split = g.steps_per_split;
    const bool vy = (a.N % 8) == 0;
    if (g.tile == 256)
      e = launch_tiled(vy ? dxt_gemm_kernel<256, 256, 4, true> : dxt_gemm_kernel<256, 256, 4, false>, 512,
                       frag_lds_bytes(256, 256), g.mtiles, g.ntiles, g.splits, p, s);
    else
      e = launch_tiled(vy ? dxt_gemm_kernel<128, 128, 2, true> : dxt_gemm_kernel<128, 128, 2, false>, 256,
                       frag_lds_bytes(128, 128), g.mtiles, g.ntiles, g.splits, p, s);
    if (e != hipSuccess) return e;
    if (g.splits > 1)
      hipLaunchKernelGGL(reduce_splits_kernel, dim3((unsigned)std::min<int64_t>(cdiv(a.M * a.K, 256), 4096)),
                         dim3(256), 0, s, part, g.splits, (int64_t)(a.M * a.K), 1.0f, a.dX, (float*)nullptr);
  } else if (a.dX && a.M > 0) {
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
    if (g.tile == 256)
      e = launch_tiled(dx_gemm_kernel<256, 256, 4>, 512, gemm_lds_bytes(256, 256), g.mtiles, g.ntiles, g.splits,
                       p, s);
    else
      e = launch_tiled(dx_gemm_kernel<128, 128, 2>, 256, gemm_lds_bytes(128, 128), g.mtiles, g.ntiles, g.splits,
                       p, s);
    if (e != hipSuccess) return e;
    if (g.splits > 1)
      hipLaunchKernelGGL(reduce_splits_kernel, dim3((unsigned)std::min<int64_t>(cdiv(a.M * a.K, 256), 4096)),
                         dim3(256), 0, s, part, g.splits, (int64_t)(a.M * a.K), 1.0f, a.dX, (float*)nullptr);
  }
  return hipGetLastError();
}

}  // namespace qlora
