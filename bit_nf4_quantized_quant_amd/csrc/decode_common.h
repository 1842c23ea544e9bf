// Shared pieces of the fused decode-size QLoRA forward kernels (gfx950): the
// launch parameters, the cross-workgroup hand-off of the LoRA-down products,
// the pair table of bf16 NF4 levels and lane reductions.
//
// Y = bf16( X W_deq^T + s (X A^T) B^T )   (itwiki "QLoRA", section on the
// computation; minnong511 "quantization", y = W x + (alpha/r) B A x).
//
// One launch does everything.  Workgroups publish partial results (parts of
// H = X A^T, and on the matrix-core path partial products of K slices) as
// tagged words, and other workgroups of the same launch read them after
// their own weight stream, polling (bounded spin) until the words carry this
// launch's tag.  Workgroups are dispatched in index order on this hardware
// and every producer publishes without waiting for anyone, so the words are
// normally there; nothing depends on that for correctness: a wait that
// reaches its deadline (about 1 ms) gives up, the waiting lane computes the
// value itself from the layer's inputs, and a give-up counter in the
// workspace records it for the caller.
//
// Launch epochs: every launch adds exactly 2^20 to each of the counters of a
// group, however many workgroups share a counter, so a workgroup's own
// counter update returns (epoch << 20) + something < 2^20, which names the
// launch (the same epoch on every counter, whatever mix of shapes, with or
// without adapter, used the workspace before).  Producers store each
// partial as one 64-bit word (epoch tag, value), so a partial is valid
// exactly when its tag is this launch's; nothing has to be reset or waited
// for on the producer side.  A workgroup's counter update goes out ahead of
// its weight loads, so its latency hides behind them.
//
// Workspace layout (bytes): [128*(1+s)] weight counter s (u64, s < 8),
// [128*9] give-up counter (u32), [128*(10+s)] LoRA-down counter s (u64, s < 8),
// [kHpartOff..] tagged partial sums (u64: tag << 32 | fp32 bits) of H, then
// (matrix-core path) of the K slices' products.  Counters sit 128 bytes
// apart so that their atomics do not queue on one cache line.
#pragma once

#include "common.h"
#include "launch.h"

namespace qlora {
namespace dec {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kRows = 16;          // output rows per GEMV weight tile
constexpr int kSlots = 8;          // weight-tile epoch counters
constexpr uint64_t kEpoch = uint64_t(1) << 20;
// Deadline of a weight tile's wait for the LoRA-down products, in ticks of
// the 100 MHz real-time counter (1 ms; the products normally arrive within a
// few microseconds of the launch).
constexpr uint64_t kWaitTicks = 100000;
constexpr size_t kHpartOff = 4096;
constexpr int kGiveupCounter = 128 * 9;

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
  uint64_t* Hpart; // tagged partial sums of H: GEMV [M][r16] (r16 = r rounded up to 16),
                   // matrix-core path [S][M][r] (per K slice)
  uint64_t* Ypart; // matrix-core path: tagged partial products exchanged between K slices
  char* ws;
  int n_htiles;    // GEMV: LoRA-down workgroups ahead of the weight tiles
  int n_wtiles;    // workgroups that take a weight ticket
  int G;           // matrix-core path: 64-row groups of N
  int S;           // matrix-core path: K slices
  int hcols;       // matrix-core path: LoRA-down columns per producing workgroup
  int c2_vec;      // rows of c2 start 4-byte aligned (K % 256 == 0): dword c2 loads
  int b_vec;       // r % 8 == 0 and B 16-byte aligned: 16-byte B loads
  uint32_t hi[16]; // bf16(kappa * level) per code
  float inv_kappa; // 1 / kappa: scales the block sums back at the output
};

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

// This launch's epoch as workgroup i sees it without waiting on an atomic:
// its counter's value shifted by 20.  Every launch adds exactly 2^20 to each
// counter in shares, so while a launch runs each counter lies within
// [epoch 2^20, (epoch + 1) 2^20) until its last share is added: a workgroup
// reads its counter before adding its own share.
__device__ __forceinline__ uint32_t slot_epoch(char* ws, int base, uint32_t i) {
  return (uint32_t)(ld_ctr(reinterpret_cast<const uint64_t*>(ws + base + 128 * (i % kSlots))) >> 20);
}

__device__ __forceinline__ uint64_t take_down_ticket(const DecodeParams& p, int tile) {
  return take_slot_ticket(p.ws, kDownCtr, (uint32_t)tile, (uint32_t)p.n_htiles);
}

// The GEMV's LoRA-down workgroups publish H in gemv_hcopies(M) copies, each
// gemv_hcopy_words(M, r) words long, and a weight wave reads copy
// (4 tile + its row group) % gemv_hcopies(M): every weight wave reads all of
// H, and with one copy their reads, which go to the coherence point, queue on
// the same few lines (M = 1 on 4096 x 4096: 5.50 -> 5.36-5.40 us with eight
// copies; M = 3 8.0 -> 7.85 us).  At M = 4 the weight workgroups run one per
// CU, so the last of them wait for the LoRA-down workgroups' CUs, and the
// extra stores cost more than they save (9.08 -> 9.25 us): one copy there.
__host__ __device__ constexpr int gemv_hcopies(int M) { return M <= 3 ? 8 : 1; }
__host__ __device__ constexpr int gemv_hcopy_words(int M, int r) {
  return (((M * ((r + 15) & ~15) * 8 + 255) & ~255) + 256) / 8;
}

// s_waitcnt operand that waits for every vector memory load and for nothing
// else (gfx9 encoding: vmcnt in bits 3:0 and 15:14 = 0, expcnt in 6:4 and
// lgkmcnt in 11:8 at their maxima).
constexpr int kWaitVm0 = 0x0F70;

__device__ __forceinline__ uint64_t realtime() { return __builtin_amdgcn_s_memrealtime(); }

// A workgroup-uniform value moved to a scalar register (integer division runs
// on the vector unit), so that offsets derived from it stay scalar.
__device__ __forceinline__ int uniform_int(int v) {
  int r;
  asm volatile("s_mov_b32 %0, %1" : "=s"(r) : "s"(v));
  return r;
}

// Polls a tagged partial until it carries `tag` (first: the word already
// read) and stores its value in *out.  The lane's deadline (0 = not yet set)
// is set at its first miss; returns false, leaving *out alone, once the
// real-time counter passes it.
// (The poll count is bounded too, at kMaxPolls reads per word, each at
// least one memory round trip.)
constexpr unsigned kMaxPolls = 1u << 16;
__device__ __forceinline__ bool poll_tagged(const uint64_t* src, uint64_t first, uint32_t tag, uint64_t& deadline,
                                            float* out) {
  uint64_t v = first;
  unsigned polls = 0;
  while ((uint32_t)(v >> 32) != tag) {
    const uint64_t now = realtime();
    if (deadline == 0)
      deadline = now + kWaitTicks;
    else if (now > deadline || ++polls > kMaxPolls)
      return false;
    __builtin_amdgcn_s_sleep(1);
    v = ld_tagged(src);
  }
  *out = __uint_as_float((uint32_t)v);
  return true;
}

// H[m][j] = sum_k X[m][k] A[j][k] by one lane, for a wait that gave up: the
// same fp32 sums of bf16 pair products the LoRA-down tiles form (in another
// order), and one count on the workspace's give-up counter.
__device__ __attribute__((noinline)) float lane_lora_down(const uint16_t* X, const uint16_t* A, int K, int m, int j,
                                                        char* ws) {
  __hip_atomic_fetch_add(reinterpret_cast<unsigned*>(ws + kGiveupCounter), 1u, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  const rsrc_t rx = make_rsrc(X + (size_t)m * K, (uint32_t)K * 2);
  const rsrc_t ra = make_rsrc(A + (size_t)j * K, (uint32_t)K * 2);
  float acc = 0.f;
  for (int k = 0; k < K; k += 8) {
    const u32x4 x = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, (uint32_t)k * 2, 0, 0));
    const u32x4 a = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, (uint32_t)k * 2, 0, 0));
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t xq = x[q], aq = a[q];
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(short __attribute__((ext_vector_type(2))), aq),
                                            __builtin_bit_cast(short __attribute__((ext_vector_type(2))), xq), acc,
                                            false);
    }
  }
  return acc;
}

// The weight's mean (read-only during a launch) through the scalar cache: a
// read in the constant address space is a scalar load, counted apart from
// the vector loads, so no wait for it lands behind the weight stream.
__device__ __forceinline__ float load_mean(const DecodeParams& p) {
  return *reinterpret_cast<const __attribute__((address_space(4))) float*>(
      reinterpret_cast<uintptr_t>(p.mean));
}

// bf16 pairs as the dot-product builtin takes them (raw 16-bit lanes)
typedef short s16x2 __attribute__((ext_vector_type(2)));

// Pair table in LDS: entry e (code byte e) = bf16(level[e & 15]) |
// bf16(level[e >> 4]) << 16 at byte 256 e, 32 copies (one per lane % 32), so
// that the address 256 byte + 4 (lane % 32) is one byte permute and the
// lanes of a half-wave always hit distinct banks.
constexpr int kPairStride = 256;

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

// Address of code byte b (0..3) of `word` in the pair table, for the lane
// whose copy offset is lane4 = 4 (lane % 32): bytes [lane4, byte b, 0, 0].
template <int b>
__device__ __forceinline__ uint32_t pair_addr(uint32_t word, uint32_t lane4) {
  return __builtin_amdgcn_perm(word, lane4, 0x0c0c0000u | ((4u + b) << 8));
}

// Builds the table: thread t of `nthreads` (a multiple of 256) writes its
// share of entry t % 256's eight 16-byte pieces, in a per-entry rotated order
// (no bank conflicts between the 8 entries a write instruction serves).
template <int nthreads>
__device__ __forceinline__ void build_pair_table(const DecodeParams& p, char* lut) {
  constexpr uint32_t per = 8 / (nthreads / 256);
  const uint32_t e = threadIdx.x & 255, part = threadIdx.x >> 8;
  const uint32_t pv = pair_entry(p, e);
  u32x4* dst = reinterpret_cast<u32x4*>(lut + e * kPairStride);
#pragma unroll
  for (uint32_t i = 0; i < per; ++i) dst[(per * part + i + e) & 7] = u32x4{pv, pv, pv, pv};
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

// The launch arguments both paths of a kernel use, fetched in one round trip
// ahead of the first branch (left alone, each branch waits for its own).
#define QLORA_FETCH_ARGS(p)                                                                              \
  do {                                                                                                   \
    asm volatile("" ::"s"((p).X), "s"((p).codes), "s"((p).c2), "s"((p).c1), "s"((p).mean), "s"((p).B),  \
                 "s"((p).A), "s"((p).K), "s"((p).N), "s"((p).M), "s"((p).r), "s"((p).n_htiles),          \
                 "s"((p).n_wtiles), "s"((p).ws));                                                        \
    asm volatile("" ::"s"((p).hi[0]), "s"((p).hi[1]), "s"((p).hi[2]), "s"((p).hi[3]), "s"((p).hi[4]),    \
                 "s"((p).hi[5]), "s"((p).hi[6]), "s"((p).hi[7]), "s"((p).hi[8]), "s"((p).hi[9]),        \
                 "s"((p).hi[10]), "s"((p).hi[11]), "s"((p).hi[12]), "s"((p).hi[13]), "s"((p).hi[14]),   \
                 "s"((p).hi[15]));                                                                       \
  } while (0)

// Host side: the parameters every decode path shares (the LoRA-down tile
// count is set by the path).
inline DecodeParams decode_params(const FwdArgs& a) {
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
  // the main product comes out kappa times too large; so does the LoRA term
  // with scale * kappa, and the sum is multiplied by 1 / kappa at the output
  const DecodeLevels& dl = decode_levels(a.w.table);
  p.scale = a.scale * dl.kappa;
  p.inv_kappa = 1.0f / dl.kappa;
  p.Y = a.Y;
  p.ws = reinterpret_cast<char*>(a.workspace);
  p.Hpart = reinterpret_cast<uint64_t*>(p.ws + kHpartOff);
  p.Ypart = nullptr;
  p.H = a.H;
  p.n_htiles = 0;
  p.G = 0;
  p.S = 1;
  p.hcols = 1;
  p.n_wtiles = (int)((a.N + kRows - 1) / kRows);
  p.c2_vec = (a.K % 256 == 0) && (reinterpret_cast<uintptr_t>(a.w.c2) % 4 == 0);
  p.b_vec = (a.r % 8 == 0) && (reinterpret_cast<uintptr_t>(a.B) % 16 == 0);
  for (int i = 0; i < 16; ++i) p.hi[i] = dl.bf16[i];
  return p;
}

hipError_t launch_gemv_fwd(const DecodeParams& p, hipStream_t s);

}  // namespace dec
}  // namespace qlora
