/*
 * qlora.h -- C ABI of libqlora.so: the QLoRA NF4 quantized linear layer on one
 * AMD MI355X (gfx950).
 *
 * The layer (itwiki "QLoRA", section on the computation; minnong511
 * "quantization", the boxed y = W x + (alpha/r) B A x equation):
 *
 *     Y = X * W_deq^T + s * (X * A^T) * B^T,      s = alpha / r
 *     W_deq = doubleDequant(c1, c2, W_nf4)        (bf16)
 *
 * with X [M,K], W [N,K] (out x in), A [r,K], B [N,r] (kdkrkwhr "LoRA vs
 * Q-LoRA", section 1: B is d x r, A is r x k).  The frozen base weight is kept
 * as 4-bit NormalFloat codes in blocks of 64 with one absmax constant per block
 * (itwiki "QLoRA", NF4 section); the constants are double-quantized: centred
 * on their tensor mean and stored as E4M3 bytes in blocks of 256, one fp32
 * scale per block (itwiki "QLoRA", double quantization section).
 *
 * Conventions shared by every entry point
 *   - Tensor arguments are DEVICE pointers to row-major, contiguous storage.
 *     bf16 values are passed as uint16_t bit patterns.  Sizes are element
 *     counts (int64_t).
 *   - The caller allocates and owns every buffer (inputs, outputs and the
 *     workspaces sized by the *_workspace helpers).  The library never
 *     allocates, frees or synchronizes; it validates arguments on the host and
 *     queues kernels on `stream` (a hipStream_t; NULL = the null stream).
 *   - Return value: QLORA_OK or an error code.  Every argument and shape check
 *     runs before the first launch, so on QLORA_EINVAL or QLORA_ESHAPE nothing
 *     has been queued.  QLORA_EHIP reports a launch the HIP runtime refused;
 *     kernels of the same call queued before it may already be on the stream,
 *     and the call's outputs are then unspecified.  Faults inside kernels
 *     surface at the caller's next synchronization, as for any HIP kernel.
 *   - Inputs must be finite; non-finite inputs give unspecified results.
 *   - Zero-sized problems (N, M or K equal to 0, as allowed per entry point)
 *     are accepted; they queue nothing except where an output is a sum over
 *     the empty extent (the backward's gradients), which is then written as 0.
 *   - Alignment: pointers to fp32/bf16 matrices and to the packed codes must be
 *     16-byte aligned; absmax, c1, mean and H need 4-byte alignment; c2 and B
 *     need only their natural alignment.
 *   - Calls may be made from several host threads at once (the library's only
 *     host-side state, per-device caches of the CU count and of raised kernel
 *     LDS limits, is guarded by a mutex).  The forward keeps launch counters
 *     in its workspace between calls; two calls that share a workspace must
 *     not run concurrently on the device.
 *
 * Storage of one quantized weight W [N,K] (P = N*K, K % 64 == 0):
 *   codes  uint8 [N, K/2]       code of element 2i in the low nibble of byte i,
 *                               element 2i+1 in the high nibble
 *   absmax float [P/64]         first-level constants (input to double quant)
 *   c2     uint8 [P/64]         E4M3 (OCP e4m3fn) code of (absmax - mean)/c1
 *   c1     float [ceil(P/16384)] second-level fp32 constant per 256 c2 values
 *   mean   float [1]            tensor mean of absmax (device memory)
 * Block b covers elements [64b, 64b+64) of row-major W, so every block lies in
 * one row; c2[b] belongs to c1[b / 256].
 */
#ifndef QLORA_H
#define QLORA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QLORA_OK 0
#define QLORA_EINVAL 1  /* null pointer, negative size, misaligned pointer, workspace too small */
#define QLORA_ESHAPE 2  /* K % 64 != 0, r above 128, sizes past the supported range */
#define QLORA_EHIP 3    /* the HIP runtime rejected a launch (hipGetLastError) */

/*
 * Code tables (the `table` argument): the 16 levels a 4-bit code stands for,
 * ascending.  The quantizer picks the nearest level, the lowest code on a
 * tie; an all-zero block stores code 7 (the zero level of NF4 and FP4; the
 * uniform grid has no zero).  The weight's codes, the quantizer and every
 * consumer must use the same table.
 *   QLORA_TABLE_NF4       4-bit NormalFloat (itwiki "QLoRA", NF4 section)
 *   QLORA_TABLE_UNIFORM4  16 evenly spaced levels on [-1, 1], fp32(-1 + i*(2/15))
 *                         (the comparison grid of the same section's example)
 *   QLORA_TABLE_FP4       4-bit float, 2 exponent and 1 mantissa bits (0, 0.5,
 *                         1, 1.5, 2, 3, 4, 6 and negatives) divided by 6; codes
 *                         7 and 8 are both zero.  The pages name FP4 without
 *                         giving its grid; this grid is the library's reading.
 * Any other value is rejected with QLORA_EINVAL.
 */
#define QLORA_TABLE_NF4 0
#define QLORA_TABLE_UNIFORM4 1
#define QLORA_TABLE_FP4 2

/* Human-readable name of a status code (static string). */
const char* qlora_status_str(int status);

/*
 * Host-only.  Storage sizes of a quantized [N,K] weight: packed code bytes,
 * number of c2 bytes (= absmax floats) and number of c1 floats.  Any output
 * pointer may be NULL.  Returns QLORA_ESHAPE if K % 64 != 0.
 */
int qlora_nf4_sizes(int64_t N, int64_t K, int64_t* code_bytes, int64_t* n_c2, int64_t* n_c1);

/*
 * Host-only.  Copies the 16 levels of code table `table` (fp32, ascending,
 * code i -> levels[i]) into host memory `levels16`.  QLORA_TABLE_NF4's levels
 * come from the quantile construction on the itwiki "QLoRA" page (NF4 section): standard
 * normal quantiles at 8 probabilities spaced evenly from 0.5 (excluded) to the
 * offset 0.9677083 for the positive half, 7 for the negative half, an exact 0,
 * normalized by the largest magnitude.
 */
int qlora_nf4_levels(int table, float* levels16);

/*
 * Blockwise NF4 quantization (itwiki "QLoRA", NF4 section; minnong511
 * "quantization", block-wise quantization).
 *   W      in   fp32 [N,K]      weights (16-B aligned)
 *   table  in   code table (QLORA_TABLE_*; NF4 is the method's)
 *   codes  out  uint8 [N,K/2]   packed codes (16-B aligned)
 *   absmax out  fp32 [N*K/64]   max |w| of each 64-element block
 * Each element becomes the index of the level nearest to fp32(w / absmax)
 * (IEEE division; an exact tie goes to the lower level); a block with absmax
 * 0 stores code 7 (the zero level).  N >= 0; K >= 0 with K % 64 == 0.
 */
int qlora_nf4_quantize(const float* W, int64_t N, int64_t K, int table, uint8_t* codes, float* absmax,
                       void* stream);

/*
 * The same quantization of bf16 weights (minnong511 "quantization", the QLoRA
 * pipeline: the base model's FP16/BF16 weights are what gets quantized to 4
 * bits).  Each bf16 value is widened exactly to fp32 and quantized as in
 * qlora_nf4_quantize, so the codes and absmax equal those of the widened
 * fp32 weights bit for bit.
 *   W      in   bf16 [N,K]      weights as uint16 bit patterns (8-B aligned)
 *   table  in   code table (QLORA_TABLE_*)
 *   codes  out  uint8 [N,K/2]   packed codes (16-B aligned)
 *   absmax out  fp32 [N*K/64]   max |w| of each 64-element block
 * Same shapes, status codes and stream behaviour as qlora_nf4_quantize.
 */
int qlora_nf4_quantize_bf16(const uint16_t* W, int64_t N, int64_t K, int table, uint8_t* codes, float* absmax,
                            void* stream);

/* Workspace bytes needed by qlora_double_quant for n_c2 constants. */
size_t qlora_double_quant_workspace(int64_t n_c2);

/*
 * Double quantization of the absmax constants (itwiki "QLoRA", double
 * quantization section).
 *   absmax    in   fp32 [n_c2]
 *   c2        out  uint8 [n_c2]          E4M3 codes
 *   c1        out  fp32 [ceil(n_c2/256)]  per-256 scale amax/448
 *   mean      out  fp32 [1]              the exact mean of absmax rounded once to fp32
 *   workspace      scratch of qlora_double_quant_workspace(n_c2) bytes (8-B aligned),
 *                  contents on entry do not matter
 * With x = fp32(absmax - mean): c1_b = fp32(max_b |x| / 448); c2 = e4m3(fp32(x / c1_b)),
 * round to nearest even, saturating at +-448; a block whose c1 is 0 stores 0.
 */
int qlora_double_quant(const float* absmax, int64_t n_c2, uint8_t* c2, float* c1, float* mean,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * Standalone dequantization to bf16 (itwiki "QLoRA", section on the
 * computation: doubleDequant; irregular6612 "QLoRA - Efficient Finetuning of
 * Quantized LLMs": the base weight is dequantized to bf16 before merging).
 *   table  in   the code table the codes were made with (QLORA_TABLE_*)
 *   W_bf16 out  bf16 [N,K]:  W_deq = bf16( fp32( L[code] * c_hat ) ),
 *   c_hat = fp32( fp32( e4m3(c2) * c1 ) + mean )   (no fused multiply-add).
 */
int qlora_nf4_dequant(const uint8_t* codes, const uint8_t* c2, const float* c1, const float* mean, int table,
                      int64_t N, int64_t K, uint16_t* W_bf16, void* stream);

/*
 * Merge of the adapter into the dequantized base weight (irregular6612
 * "QLoRA - Efficient Finetuning of Quantized LLMs": after training the
 * adapter is folded into the bf16 base weight; minnong511 "quantization":
 * W' = W + (alpha/r) B A).
 *   codes, c2, c1, mean, table   the quantized weight [N,K], as for qlora_nf4_dequant
 *   A      in   bf16 [r,K]
 *   B      in   bf16 [N,r]
 *   W_out  out  bf16 [N,K] (16-B aligned):
 *          W' = bf16( W_deq + s * sum_j B[n][j] A[j][k] ),  s = fp32(alpha / r),
 *          computed in fp64: the sum over j in ascending order (each product
 *          exact, one rounding per addition), times s (one rounding), plus
 *          W_deq (one rounding), one rounding to bf16 (nearest, ties to even).
 * 0 <= r <= 128 (r = 0 gives W_deq); A and B may be NULL when r = 0.
 * Same shape rules, status codes and stream behaviour as qlora_nf4_dequant.
 */
int qlora_merge(const uint8_t* codes, const uint8_t* c2, const float* c1, const float* mean, int table,
                int64_t N, int64_t K, const uint16_t* A, const uint16_t* B, int64_t r, float alpha, uint16_t* W_out,
                void* stream);

/*
 * Workspace bytes needed by qlora_linear_fwd: at M <= 16 the decode kernels'
 * launch counters and tagged partials (under 70 KiB at M <= 4, about
 * 8 S N M bytes for S slices of K above); at larger M, H (4 M r bytes) and
 * fp32 partials of the LoRA-down and of the main product where it splits
 * its reduction (at mid-size M: split-K, splits x 4 M N bytes, or stream-K
 * pieces of 64 KiB each, 2 x CUs + tiles - 1 of them, e.g. 56 MB for
 * N = 11008 at M = 512; and the 256-tile tail of a large layer: 8 M x tail
 * columns, e.g. 50 MB for N = 22016, K = 8192 at M = 4096).
 */
size_t qlora_linear_fwd_workspace(int64_t M, int64_t N, int64_t K, int64_t r);

/*
 * Forward of the QLoRA linear (itwiki "QLoRA", section on the computation;
 * minnong511 "quantization", y = W x + (alpha/r) B A x).
 *   X      in   bf16 [M,K]       activations (16-B aligned)
 *   codes, c2, c1, mean          the quantized weight W [N,K] (see above)
 *   table                        its code table (QLORA_TABLE_*)
 *   A      in   bf16 [r,K]       LoRA down factor (16-B aligned)
 *   B      in   bf16 [N,r]       LoRA up factor
 *   r, alpha                     rank (0..128) and LoRA alpha; s = alpha / r in fp32.
 *                                r = 0 is a layer without adapter: Y = bf16(X W_deq^T);
 *                                A, B and H_out may then be NULL and are not accessed
 *   Y      out  bf16 [M,N]       Y = bf16( X W_deq^T + s H B^T ), fp32 accumulation
 *   H_out  out  fp32 [M,r]       H = X A^T (may be NULL; keep it for the backward)
 *   workspace                    qlora_linear_fwd_workspace(M,N,K,r) bytes,
 *                                256-B aligned, zero-filled once before its first
 *                                use.  The library keeps launch counters in it
 *                                between calls (any shapes may share one workspace
 *                                as long as it is large enough); do not modify it
 *                                (except the wait counter below), and zero it again
 *                                after a call that faulted.  Its contents after a
 *                                call are not zero.
 * Requires K % 64 == 0; M and N at most 65535 * 128.
 */
int qlora_linear_fwd(const uint16_t* X, int64_t M, int64_t N, int64_t K, const uint8_t* codes,
                     const uint8_t* c2, const float* c1, const float* mean, int table, const uint16_t* A,
                     const uint16_t* B, int64_t r, float alpha, uint16_t* Y, float* H_out,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Size of the no-allocation forward's scratch, per GPU (16 MiB). */
#define QLORA_NOALLOC_SCRATCH_BYTES (16u << 20)

/*
 * qlora_linear_fwd without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  It allocates nothing: its scratch (the
 * decode path's launch counters and H partials, the tiled path's H and
 * split-K partials) is a static device array of QLORA_NOALLOC_SCRATCH_BYTES
 * inside the library, one copy per GPU, held until the process ends; its
 * device address is looked up once per device, on the first call made with
 * that device current.  Arguments, results and status codes are those of
 * qlora_linear_fwd; a shape whose forward workspace
 * (qlora_linear_fwd_workspace) exceeds QLORA_NOALLOC_SCRATCH_BYTES is
 * rejected with QLORA_ESHAPE.  For M <= 4 the forward needs under 70 KiB;
 * for 5 <= M <= 16 about 8 S N M bytes, S the K slices of that path (1 to
 * 16): 2 MiB at M = 16 with N = K = 4096, 22 MiB (rejected here) for the
 * 22016 x 8192 layer; M = 64 with N = K = 4096, r = 64 needs 8 MiB.
 * Every call on one GPU shares that GPU's scratch:
 * calls that overlap on one GPU (concurrent streams, or host threads that
 * use the same device) race and must not be made.  The scratch keeps the
 * last call's contents; nothing in it needs clearing between calls.
 */
int qlora_linear_fwd_noalloc(const uint16_t* X, int64_t M, int64_t N, int64_t K, const uint8_t* codes,
                             const uint8_t* c2, const float* c1, const float* mean, int table, const uint16_t* A,
                             const uint16_t* B, int64_t r, float alpha, uint16_t* Y, float* H_out, void* stream);

/*
 * Byte offset, inside the forward workspace, of a uint32 counter.  For
 * M <= 16 the workgroups of one launch hand partial results to each other
 * (parts of H = X A^T and, for 5 <= M <= 16, partial products of slices of
 * K) and wait, up to about 1 ms, for the ones they need; a wait that reaches
 * that deadline gives up, the waiting lane computes the value itself from
 * the layer's inputs (Y and H_out stay correct), and the counter goes up by
 * one per value so computed.  A nonzero count therefore means a launch ran
 * that slow fallback, e.g. because other work held the compute units.  The
 * library never resets the counter; the caller may zero these 4 bytes
 * between calls (read them after synchronizing the stream).
 */
size_t qlora_linear_fwd_wait_counter_offset(void);

/*
 * Workspace bytes needed by qlora_linear_bwd: H (when recomputed), dH and
 * their bf16 transposes (16 M r bytes) and fp32 partials of the LoRA
 * gradients and of dX, which grow with M r, N r and r K (and with M K only
 * when dX splits its reduction, at small M).  Where dH and dB come from one
 * pass over dY (M, N and r multiples of 8, r <= 64), their partials take
 * 4 r (gn M + gm N) bytes, gn = N / 512 column blocks and gm = CUs / gn row
 * blocks.  Nothing of the weight's size: dX expands the codes on chip.  E.g.
 * 74 MiB for N = 22016, K = 8192 at M = 4096, r = 64; 2 MiB for
 * N = K = 4096 at M = 1.
 */
size_t qlora_linear_bwd_workspace(int64_t M, int64_t N, int64_t K, int64_t r);

/*
 * Backward of the QLoRA linear for the input and the LoRA factors; the NF4
 * weight is frozen and gets no gradient (itwiki "QLoRA", section on the
 * computation; minnong511 "quantization", backward: W not updated, A and B
 * get gradients).  With H = X A^T and s = alpha / r:
 *   dH = s dY B      dB = s dY^T H      dA = dH^T X      dX = dY W_deq + dH A
 *   dY  in   bf16 [M,N];  X in bf16 [M,K]
 *   codes, c2, c1, mean, table   the quantized weight, as for the forward
 *   H   in   fp32 [M,r] from the forward, or NULL to recompute it
 *   dX  out  bf16 [M,K] (may be NULL to skip the input gradient)
 *   dA  out  bf16 [r,K];  dB out bf16 [N,r]
 *   r = 0 (no adapter): only dX = dY W_deq; A, B, H, dA, dB may be NULL
 *   Empty sums give zeros: M = 0 writes dA = dB = 0; N = 0 writes dX = dA = 0
 *   workspace  qlora_linear_bwd_workspace(M,N,K,r) bytes, 256-B aligned
 *              (contents on entry do not matter)
 * Requires K % 64 == 0; M and N at most 65535 * 128.
 */
int qlora_linear_bwd(const uint16_t* dY, const uint16_t* X, int64_t M, int64_t N, int64_t K,
                     const uint8_t* codes, const uint8_t* c2, const float* c1, const float* mean, int table,
                     const uint16_t* A, const uint16_t* B, int64_t r, float alpha, const float* H,
                     uint16_t* dX, uint16_t* dA, uint16_t* dB, void* workspace,
                     size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QLORA_H */
