// C ABI of libqlora.so: argument validation on the host, then kernel launches
// on the caller's stream.  Every check runs before the first HIP call, so a
// rejected call touches neither the device nor the stream.
#include <algorithm>
#include <cstring>
#include <map>
#include <mutex>

#include "qlora.h"
#include "launch.h"
#include "nf4_table.h"

namespace qlora {
size_t decode_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t r);
bool decode_supported(int64_t M, int64_t N, int64_t K, int64_t r);
size_t decode_wait_counter_offset();
hipError_t launch_decode_fwd(const FwdArgs& a, hipStream_t s);
hipError_t launch_gemm_fwd(const FwdArgs& a, float* scratch, hipStream_t s);
size_t gemm_fwd_scratch_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_lora_down(const uint16_t* X, int64_t M, int64_t K, const uint16_t* A, int64_t r, float* H,
                            float* scratch, hipStream_t s);
size_t lora_down_scratch_bytes(int64_t M, int64_t K, int64_t r);
size_t gemm_bwd_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t r);
}  // namespace qlora

using namespace qlora;

namespace {

constexpr int64_t kMaxDim = int64_t(1) << 31;       // every extent must fit a 32-bit grid index
constexpr int64_t kMaxElems = int64_t(1) << 40;     // elements of any one tensor
constexpr int64_t kDecodeMaxM = 16;
constexpr int64_t kMaxRowLen = int64_t(1) << 23;        // K, N: 256 rows of a tile within 4 GiB
constexpr int64_t kMaxWeightBytes = int64_t(1) << 32;   // packed codes of one weight
constexpr int64_t kMaxGridRows = int64_t(65535) * 128;  // M, N: 128-row tiles along a grid's y axis

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int status_of(hipError_t e) { return e == hipSuccess ? QLORA_OK : QLORA_EHIP; }

size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

// Shape checks shared by forward and backward.
int check_layer(int64_t M, int64_t N, int64_t K, int64_t r) {
  if (M < 0 || N < 0 || K < 0 || r < 0) return QLORA_EINVAL;
  if (K % 64 != 0) return QLORA_ESHAPE;
  if (r > 128) return QLORA_ESHAPE;
  if (M >= kMaxDim || N >= kMaxDim || K >= kMaxDim) return QLORA_ESHAPE;
  if (M * K >= kMaxElems || N * K >= kMaxElems || M * N >= kMaxElems) return QLORA_ESHAPE;
  // the products address a tile's rows and the packed weight with 32-bit offsets
  if (K >= kMaxRowLen || N >= kMaxRowLen || N * K / 2 >= kMaxWeightBytes) return QLORA_ESHAPE;
  // the LoRA products launch 128-row tiles of M and of N along a grid's y axis
  if (M > kMaxGridRows || N > kMaxGridRows) return QLORA_ESHAPE;
  return QLORA_OK;
}

bool table_ok(int table) { return table >= 0 && table < kCodeTables; }

int check_weight(const uint8_t* codes, const uint8_t* c2, const float* c1, const float* mean) {
  if (!codes || !c2 || !c1 || !mean) return QLORA_EINVAL;
  if (!aligned(codes, 16) || !aligned(c1, 4) || !aligned(mean, 4)) return QLORA_EINVAL;
  return QLORA_OK;
}

// Forward workspace: the decode kernel keeps its launch counters in the first
// kFwdReserved bytes whatever M is, so one workspace can serve both paths.
constexpr size_t kFwdReserved = 4096;

bool use_decode(int64_t M, int64_t N, int64_t K, int64_t r) {
  // the decode kernels address the codes with 32-bit byte offsets
  return M <= kDecodeMaxM && N * K / 2 < (int64_t(1) << 31) && decode_supported(M, N, K, r);
}

size_t fwd_ws(int64_t M, int64_t N, int64_t K, int64_t r) {
  if (use_decode(M, N, K, r)) return round256(decode_workspace_bytes(M, N, K, r));
  // H, then one scratch region used first by the LoRA-down split-K partials
  // and then by the main product's split-K partials
  const size_t scratch = std::max(lora_down_scratch_bytes(M, K, r), gemm_fwd_scratch_bytes(M, N, K));
  return kFwdReserved + round256((size_t)M * r * sizeof(float)) + round256(scratch);
}

// Checks of the forward's arguments other than its workspace.
int check_fwd(const uint16_t* X, int64_t M, int64_t N, int64_t K, const uint8_t* codes, const uint8_t* c2,
              const float* c1, const float* mean, int table, const uint16_t* A, const uint16_t* B, int64_t r,
              const uint16_t* Y, const float* H_out) {
  int st = check_layer(M, N, K, r);
  if (!st && !table_ok(table)) st = QLORA_EINVAL;
  if (st) return st;
  if (K == 0) return QLORA_ESHAPE;
  if (M == 0 || N == 0) return QLORA_OK;
  if ((st = check_weight(codes, c2, c1, mean))) return st;
  if (!X || !Y) return QLORA_EINVAL;
  if (r > 0 && (!A || !B)) return QLORA_EINVAL;
  if (!aligned(X, 16) || !aligned(A, 16) || !aligned(B, 2) || !aligned(Y, 2)) return QLORA_EINVAL;
  if (H_out && !aligned(H_out, 4)) return QLORA_EINVAL;
  return QLORA_OK;
}

// The forward's launches over a workspace of at least fwd_ws(M, N, K, r) bytes.
int launch_fwd(const uint16_t* X, int64_t M, int64_t N, int64_t K, const uint8_t* codes, const uint8_t* c2,
               const float* c1, const float* mean, int table, const uint16_t* A, const uint16_t* B, int64_t r,
               float alpha, uint16_t* Y, float* H_out, void* workspace, hipStream_t s) {
  FwdArgs a;
  a.X = X;
  a.M = M;
  a.N = N;
  a.K = K;
  a.r = r;
  a.w = Nf4Weight{codes, c2, c1, mean, table};
  a.A = A;
  a.B = B;
  a.scale = r > 0 ? alpha / (float)r : 0.f;
  a.Y = Y;
  a.H = r > 0 ? H_out : nullptr;
  a.workspace = workspace;
  if (use_decode(M, N, K, r)) return status_of(launch_decode_fwd(a, s));
  char* ws = reinterpret_cast<char*>(workspace) + kFwdReserved;
  float* scratch = reinterpret_cast<float*>(ws + round256((size_t)M * r * sizeof(float)));
  if (r > 0) {
    float* H = H_out ? H_out : reinterpret_cast<float*>(ws);
    a.H = H;
    if (launch_lora_down(X, M, K, A, r, H, scratch, s) != hipSuccess) return QLORA_EHIP;
  }
  return status_of(launch_gemm_fwd(a, scratch, s));
}

// The no-allocation forward's scratch: a file-scope device array, one copy
// per GPU, zero at load (the decode launch counters start consistent) and
// kept between calls.  Host code uses it only through the device address
// hipGetSymbolAddress gives for the current device, taken once per device.
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
static_assert(kNoAllocScratchBytes == QLORA_NOALLOC_SCRATCH_BYTES, "header and library disagree");
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

hipError_t noalloc_scratch(void** out) {
  static std::mutex mu;
  static std::map<int, void*> ptrs;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  auto it = ptrs.find(dev);
  if (it == ptrs.end()) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) return e != hipSuccess ? e : hipErrorInvalidSymbol;
    it = ptrs.emplace(dev, ptr).first;
  }
  *out = it->second;
  return hipSuccess;
}

}  // namespace

extern "C" {

const char* qlora_status_str(int status) {
  switch (status) {
    case QLORA_OK: return "QLORA_OK";
    case QLORA_EINVAL: return "QLORA_EINVAL: null, negative, misaligned argument or workspace too small";
    case QLORA_ESHAPE: return "QLORA_ESHAPE: unsupported shape (K % 64, r above 128, size limit)";
    case QLORA_EHIP: return "QLORA_EHIP: the HIP runtime rejected a kernel launch";
    default: return "QLORA: unknown status";
  }
}

int qlora_nf4_sizes(int64_t N, int64_t K, int64_t* code_bytes, int64_t* n_c2, int64_t* n_c1) {
  if (N < 0 || K < 0) return QLORA_EINVAL;
  if (K % 64 != 0) return QLORA_ESHAPE;
  if (N >= kMaxDim || K >= kMaxDim || N * K >= kMaxElems) return QLORA_ESHAPE;
  const int64_t p = N * K;
  if (code_bytes) *code_bytes = p / 2;
  if (n_c2) *n_c2 = p / 64;
  if (n_c1) *n_c1 = (p / 64 + 255) / 256;
  return QLORA_OK;
}

int qlora_nf4_levels(int table, float* levels16) {
  if (!levels16 || !table_ok(table)) return QLORA_EINVAL;
  std::memcpy(levels16, code_table(table).level, 16 * sizeof(float));
  return QLORA_OK;
}

int qlora_nf4_quantize(const float* W, int64_t N, int64_t K, int table, uint8_t* codes, float* absmax,
                       void* stream) {
  int st = qlora_nf4_sizes(N, K, nullptr, nullptr, nullptr);
  if (st) return st;
  if (!table_ok(table)) return QLORA_EINVAL;
  if (N * K == 0) return QLORA_OK;
  if (!W || !codes || !absmax) return QLORA_EINVAL;
  if (!aligned(W, 16) || !aligned(codes, 16) || !aligned(absmax, 4)) return QLORA_EINVAL;
  return status_of(launch_nf4_quantize(W, N, K, table, codes, absmax, (hipStream_t)stream));
}

int qlora_nf4_quantize_bf16(const uint16_t* W, int64_t N, int64_t K, int table, uint8_t* codes, float* absmax,
                            void* stream) {
  int st = qlora_nf4_sizes(N, K, nullptr, nullptr, nullptr);
  if (st) return st;
  if (!table_ok(table)) return QLORA_EINVAL;
  if (N * K == 0) return QLORA_OK;
  if (!W || !codes || !absmax) return QLORA_EINVAL;
  if (!aligned(W, 8) || !aligned(codes, 16) || !aligned(absmax, 4)) return QLORA_EINVAL;
  return status_of(launch_nf4_quantize_bf16(W, N, K, table, codes, absmax, (hipStream_t)stream));
}

size_t qlora_double_quant_workspace(int64_t n_c2) {
  (void)n_c2;
  return double_quant_workspace_bytes();
}

int qlora_double_quant(const float* absmax, int64_t n_c2, uint8_t* c2, float* c1, float* mean, void* workspace,
                       size_t workspace_bytes, void* stream) {
  if (n_c2 < 0) return QLORA_EINVAL;
  if (n_c2 >= kMaxElems / 64) return QLORA_ESHAPE;
  if (n_c2 == 0) return QLORA_OK;
  if (!absmax || !c2 || !c1 || !mean || !workspace) return QLORA_EINVAL;
  if (!aligned(absmax, 4) || !aligned(c1, 4) || !aligned(mean, 4) || !aligned(workspace, 8)) return QLORA_EINVAL;
  if (workspace_bytes < double_quant_workspace_bytes()) return QLORA_EINVAL;
  return status_of(launch_double_quant(absmax, n_c2, c2, c1, mean, workspace, (hipStream_t)stream));
}

int qlora_nf4_dequant(const uint8_t* codes, const uint8_t* c2, const float* c1, const float* mean, int table,
                      int64_t N, int64_t K, uint16_t* W_bf16, void* stream) {
  int st = qlora_nf4_sizes(N, K, nullptr, nullptr, nullptr);
  if (st) return st;
  if (!table_ok(table)) return QLORA_EINVAL;
  if (N * K == 0) return QLORA_OK;
  if ((st = check_weight(codes, c2, c1, mean))) return st;
  if (!W_bf16 || !aligned(W_bf16, 16)) return QLORA_EINVAL;
  return status_of(launch_nf4_dequant(codes, c2, c1, mean, table, N, K, W_bf16, (hipStream_t)stream));
}

int qlora_merge(const uint8_t* codes, const uint8_t* c2, const float* c1, const float* mean, int table, int64_t N,
                int64_t K, const uint16_t* A, const uint16_t* B, int64_t r, float alpha, uint16_t* W_out,
                void* stream) {
  int st = qlora_nf4_sizes(N, K, nullptr, nullptr, nullptr);
  if (st) return st;
  if (!table_ok(table)) return QLORA_EINVAL;
  if (r < 0) return QLORA_EINVAL;
  if (r > 128) return QLORA_ESHAPE;
  if (N * K == 0) return QLORA_OK;
  if ((st = check_weight(codes, c2, c1, mean))) return st;
  if (!W_out || !aligned(W_out, 16)) return QLORA_EINVAL;
  if (r > 0 && (!A || !B || !aligned(A, 2) || !aligned(B, 2))) return QLORA_EINVAL;
  const float s = r > 0 ? alpha / (float)r : 0.f;
  return status_of(launch_nf4_merge(codes, c2, c1, mean, table, N, K, A, B, r, s, W_out, (hipStream_t)stream));
}

size_t qlora_linear_fwd_workspace(int64_t M, int64_t N, int64_t K, int64_t r) {
  if (check_layer(M, N, K, r)) return 0;
  return fwd_ws(M, N, K, r);
}

int qlora_linear_fwd(const uint16_t* X, int64_t M, int64_t N, int64_t K, const uint8_t* codes, const uint8_t* c2,
                     const float* c1, const float* mean, int table, const uint16_t* A, const uint16_t* B,
                     int64_t r, float alpha, uint16_t* Y, float* H_out, void* workspace, size_t workspace_bytes,
                     void* stream) {
  int st = check_fwd(X, M, N, K, codes, c2, c1, mean, table, A, B, r, Y, H_out);
  if (st != QLORA_OK) return st;
  if (M == 0 || N == 0) return QLORA_OK;
  if (!workspace || !aligned(workspace, 256)) return QLORA_EINVAL;
  if (workspace_bytes < fwd_ws(M, N, K, r)) return QLORA_EINVAL;
  return launch_fwd(X, M, N, K, codes, c2, c1, mean, table, A, B, r, alpha, Y, H_out, workspace,
                    (hipStream_t)stream);
}

int qlora_linear_fwd_noalloc(const uint16_t* X, int64_t M, int64_t N, int64_t K, const uint8_t* codes,
                             const uint8_t* c2, const float* c1, const float* mean, int table, const uint16_t* A,
                             const uint16_t* B, int64_t r, float alpha, uint16_t* Y, float* H_out, void* stream) {
  int st = check_fwd(X, M, N, K, codes, c2, c1, mean, table, A, B, r, Y, H_out);
  if (st != QLORA_OK) return st;
  if (M == 0 || N == 0) return QLORA_OK;
  if (fwd_ws(M, N, K, r) > kNoAllocScratchBytes) return QLORA_ESHAPE;
  void* ws = nullptr;
  if (noalloc_scratch(&ws) != hipSuccess) return QLORA_EHIP;
  return launch_fwd(X, M, N, K, codes, c2, c1, mean, table, A, B, r, alpha, Y, H_out, ws, (hipStream_t)stream);
}

size_t qlora_linear_fwd_wait_counter_offset(void) { return decode_wait_counter_offset(); }

size_t qlora_linear_bwd_workspace(int64_t M, int64_t N, int64_t K, int64_t r) {
  if (check_layer(M, N, K, r)) return 0;
  return gemm_bwd_workspace_bytes(M, N, K, r);
}

int qlora_linear_bwd(const uint16_t* dY, const uint16_t* X, int64_t M, int64_t N, int64_t K, const uint8_t* codes,
                     const uint8_t* c2, const float* c1, const float* mean, int table, const uint16_t* A,
                     const uint16_t* B, int64_t r, float alpha, const float* H, uint16_t* dX, uint16_t* dA,
                     uint16_t* dB, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_layer(M, N, K, r);
  if (!st && !table_ok(table)) st = QLORA_EINVAL;
  if (st) return st;
  if (K == 0) return QLORA_ESHAPE;
  if ((st = check_weight(codes, c2, c1, mean))) return st;
  if (!workspace) return QLORA_EINVAL;
  // pointers to empty tensors may be NULL (dY, B, dB when N == 0; dY, X when M == 0)
  if (r > 0 && (!A || !dA || (N > 0 && (!B || !dB)))) return QLORA_EINVAL;
  if (M > 0 && (!X || (N > 0 && !dY))) return QLORA_EINVAL;
  if (!aligned(dY, 16) || !aligned(X, 16) || !aligned(A, 16) || !aligned(B, 2) || !aligned(dA, 16) ||
      !aligned(dB, 2) || !aligned(workspace, 256))
    return QLORA_EINVAL;
  if (H && !aligned(H, 4)) return QLORA_EINVAL;
  if (dX && !aligned(dX, 16)) return QLORA_EINVAL;
  if (workspace_bytes < gemm_bwd_workspace_bytes(M, N, K, r)) return QLORA_EINVAL;
  // N == 0 still runs: the sums over N are empty, so dX and dA are written as zeros
  if (r == 0 && (M == 0 || !dX)) return QLORA_OK;  // no adapter and no input gradient to write

  BwdArgs a;
  a.dY = dY;
  a.X = X;
  a.M = M;
  a.N = N;
  a.K = K;
  a.r = r;
  a.w = Nf4Weight{codes, c2, c1, mean, table};
  a.A = A;
  a.B = B;
  a.scale = r > 0 ? alpha / (float)r : 0.f;
  a.H = H;
  a.dX = dX;
  a.dA = dA;
  a.dB = dB;
  a.workspace = workspace;
  return status_of(launch_linear_bwd(a, (hipStream_t)stream));
}

}  // extern "C"
