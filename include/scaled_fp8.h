/*
 * scaled_fp8.h — C ABI of the MI355X (gfx950) scaled FP8 linear-layer library
 * (libscaled_fp8.so).
 *
 * What it computes.  The FP8 linear layer of "Training and inference of large
 * language models using 8-bit floating point" (paper review page, section
 * "Proposed method"): each tensor gets a power-of-two scale derived from its
 * maximum absolute value (amax) through log2(format max / amax) with a
 * configurable margin; tensors are scaled before the cast to FP8 (E4M3 for
 * weights and activations, E5M2 for gradients) and the matrix product is
 * unscaled afterwards.  From "Per-Tensor and Per-Block Scaling Strategies for
 * Effective FP8 Training" (summary page, "Key Questions Answered"): delayed
 * scaling takes the scale from amaxes observed over past iterations, and
 * per-block (MXFP8) scaling gives every block of a tensor its own scale.
 *
 * Readings of what the pages leave open, applied by every entry point:
 *   - FP8 formats are OCP OFP8 E4M3 (max 448, no Inf) and E5M2 (max 57344);
 *   - the cast rounds to nearest, ties to even (subnormals included), and
 *     saturates: |v| > max and +-Inf give +-max; NaN gives 0x7F | sign; the
 *     sign of zero is kept;
 *   - bias = floor(log2(fmax / amax)) - margin, computed with exact integer
 *     exponent arithmetic, clamped to [-126, 126]; amax 0, Inf or NaN gives
 *     bias 0; the scale applied before the cast is 2^bias;
 *   - MX blocks are 1 x 32 along the contiguous (K) axis; the block exponent
 *     follows the same rule with margin 0, clamped to [-127, 127], stored as
 *     the E8M0 code 127 - e (0xFF for a block holding a NaN);
 *   - the GEMM accumulates in fp32 and multiplies by 2^-(bias_a + bias_b)
 *     before the single rounding to the output type (bf16 RNE or fp32).
 *
 * Conventions for every call.
 *   - Return value: FP8_OK (0) or a negative FP8_ERR_* code.  All argument
 *     checks run on the host before any HIP call, so a rejected call has no
 *     effect on the device and touches no HIP state.
 *   - Every pointer except the stream is DEVICE memory owned by the caller.
 *     The library allocates nothing, frees nothing, keeps no state between
 *     calls and is thread-safe; work is enqueued asynchronously on `stream`
 *     (0 = the default stream) and the library never synchronizes.
 *   - Scalars that flow between calls (amax, bias, scale) live in device
 *     memory, so a whole linear layer can be enqueued with no host round trip.
 *   - Matrices are row-major with a leading dimension `ld*` in ELEMENTS of
 *     their own type (bytes for FP8 codes and E8M0 scales); ld >= cols.
 *   - Output scalars such as `amax_out` are overwritten, not accumulated.
 *   - Launch failures are reported as FP8_ERR_LAUNCH from hipGetLastError.
 *   - Calls that write overlapping buffers on different streams race; the
 *     caller orders them.
 */
#ifndef SCALED_FP8_H
#define SCALED_FP8_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* FP8 element formats (OCP OFP8). */
enum { FP8_E4M3 = 0, FP8_E5M2 = 1 };
/* High-precision data types for inputs and GEMM outputs. */
enum { FP8_DT_BF16 = 0, FP8_DT_F32 = 1 };
/* MX block-exponent rules (see mx_quantize_rule). */
enum { MX_RULE_FMAX = 0, MX_RULE_OCP = 1 };

/* Status codes. */
enum {
  FP8_OK = 0,
  FP8_ERR_NULL = -1,        /* a required pointer is NULL */
  FP8_ERR_SHAPE = -2,       /* negative size, ld < cols, K % 16 (GEMM) or
                               cols % 32 / rows % 32 / K % 32 (MX) violated,
                               bad window */
  FP8_ERR_ALIGN = -3,       /* GEMM operand base or leading dimension not a
                               multiple of 16 bytes (required by 16-byte loads) */
  FP8_ERR_DTYPE = -4,       /* unknown FP8_DT_* value */
  FP8_ERR_FORMAT = -5,      /* unknown FP8_E* or MX_RULE_* value */
  FP8_ERR_LAUNCH = -6,      /* hipGetLastError reported a launch failure */
  FP8_ERR_UNSUPPORTED = -7  /* valid but not implemented combination */
};

/* Human-readable name of a status code (static storage, never NULL). */
const char* fp8_status_string(int status);

/* Library ABI version (increases when a signature changes or an entry point
 * is added): 4. */
int fp8_abi_version(void);

/*
 * fp8_amax — per-tensor maximum absolute value ("Proposed method": the scale
 * is based on each tensor's maximum absolute value).
 *   x        [rows x cols] of `dtype`, leading dimension ld (elements).
 *   amax_out one float: max |x| over the tensor, exact (no rounding); NaN if
 *            any element is NaN, +Inf if any is infinite, 0 for an empty
 *            tensor.  Overwritten.
 * Any alignment is accepted (16-byte aligned rows take the vector path).
 */
int fp8_amax(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld,
             float* amax_out, hipStream_t stream);

/*
 * fp8_amax_scale — current scaling in one launch: fp8_amax followed by
 * fp8_compute_scale ("Proposed method": the bias comes from log2 of the ratio
 * of the format maximum to the tensor's largest magnitude, with a margin),
 * fused so that the scale is ready after a single pass over x.
 *   x, dtype, rows, cols, ld   as fp8_amax;
 *   fmt, margin                as fp8_compute_scale;
 *   amax_out, bias_out         required, overwritten: exactly fp8_amax's amax
 *                              and fp8_compute_scale's bias of it;
 *   scale_out, scale_inv_out   optional (NULL = skip);
 *   workspace                  FP8_AMAX_SCALE_WORKSPACE_BYTES of caller-owned
 *                              device memory, 4-byte aligned, ZERO before the
 *                              first use; every call leaves it zero again (its
 *                              first 8 bytes hold a ticket and a running
 *                              maximum during the call).  Calls sharing a
 *                              workspace must not overlap (order them on one
 *                              stream).
 * One kernel: each workgroup reduces its share, folds it into the running
 * maximum with an atomic max and takes a ticket; the workgroup that takes the
 * last ticket writes the outputs and clears the workspace.  No zero-fill
 * launch and no separate scale launch; the state is the same for any size.
 */
#define FP8_AMAX_SCALE_WORKSPACE_BYTES 256
int fp8_amax_scale(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld,
                   int fmt, int margin, float* amax_out, int32_t* bias_out,
                   float* scale_out, float* scale_inv_out, void* workspace,
                   hipStream_t stream);

/*
 * fp8_amax_scale_noalloc — fp8_amax_scale without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops).  The reduction state lives in a static array of
 * FP8_AMAX_SCALE_WORKSPACE_BYTES inside the library, one copy per GPU, held
 * until the process ends; it is cleared the first time a GPU uses it (a small
 * kernel on `stream`) and every call leaves it zero again.  Every call on one
 * GPU shares that array: calls that overlap on the same GPU (different
 * streams, host threads) race and give wrong results; order them.  The state
 * does not grow with the tensor (a ticket and a running maximum), so no
 * input is too large for it; arguments and results are those of
 * fp8_amax_scale.  Allocates nothing (no hipMalloc, no library allocation);
 * FP8_ERR_LAUNCH if the array's device address cannot be obtained.
 */
int fp8_amax_scale_noalloc(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld,
                           int fmt, int margin, float* amax_out, int32_t* bias_out,
                           float* scale_out, float* scale_inv_out, hipStream_t stream);

/*
 * fp8_compute_scale — exponent bias from an amax ("Proposed method": log2 of
 * the ratio of the format maximum to the tensor amplitude, with a margin).
 *   amax      one float (device), e.g. from fp8_amax.
 *   fmt       FP8_E4M3 or FP8_E5M2 (selects fmax = 448 or 57344).
 *   margin    integer subtracted from floor(log2(fmax / amax)).
 *   bias_out  one int32: the bias (scale before the cast = 2^bias).
 *   scale_out, scale_inv_out  optional floats 2^bias and 2^-bias (NULL = skip).
 */
int fp8_compute_scale(const float* amax, int fmt, int margin, int32_t* bias_out,
                      float* scale_out, float* scale_inv_out, hipStream_t stream);

/*
 * Delayed-scaling history ("Per-Tensor and Per-Block Scaling Strategies ...",
 * "Key Questions Answered" / "Key Actionable Insights": the scale comes from
 * the largest amax seen over past iterations).  State lives in caller-owned
 * device memory: `hist` holds `window` floats (1 <= window <= 4096) and
 * `state` two int32 {count, head}: count = valid entries (saturates at
 * window), head = next slot to overwrite.  Checkpointing the layer's scaling
 * state means copying these window*4 + 8 bytes.
 *
 * fp8_history_init  zeroes hist and sets {count, head} = {0, 0}.
 * fp8_history_push  stores *amax at hist[head] and advances the ring.
 * fp8_compute_scale_delayed  bias from the maximum over the `count` valid
 *   entries (0 when count == 0, giving bias 0), by the rule of
 *   fp8_compute_scale.  The window holds earlier steps only; for the first
 *   step the caller pushes that step's own amax first (fp8_amax, then
 *   fp8_history_push), so the first step is current-scaled.
 */
int fp8_history_init(float* hist, int32_t* state, int window, hipStream_t stream);
int fp8_history_push(float* hist, int32_t* state, int window, const float* amax,
                     hipStream_t stream);
int fp8_compute_scale_delayed(const float* hist, const int32_t* state, int window,
                              int fmt, int margin, int32_t* bias_out,
                              float* scale_out, float* scale_inv_out,
                              hipStream_t stream);

/*
 * fp8_quantize — per-tensor scaled cast ("Proposed method": scale the input,
 * then cast to FP8).  q[r, c] = sat_RNE_fmt(x[r, c] * 2^(*bias)).
 *   x        [rows x cols] of `dtype`, leading dimension ld.
 *   bias     one int32 (device), e.g. from fp8_compute_scale[_delayed].
 *   q        [rows x cols] FP8 codes, leading dimension ldq (bytes).
 *   qT       optional [cols x rows] transposed copy, leading dimension ldqT
 *            (NULL = none; ldqT ignored).  Lets a GEMM that contracts over
 *            `rows` read this operand with K contiguous.
 *   amax_out optional: max |x| of the INPUT, fused into the same pass (the
 *            amax a delayed-scaling history records for this step).
 * Any alignment is accepted (aligned rows take the vector path).
 */
int fp8_quantize(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld,
                 int fmt, const int32_t* bias, uint8_t* q, int64_t ldq,
                 uint8_t* qT, int64_t ldqT, float* amax_out, hipStream_t stream);

/*
 * fp8_quantize_sat — fp8_quantize that also counts the elements the cast
 * saturates.  "Per-Tensor and Per-Block Scaling Strategies for Effective FP8
 * Training" (summary page, "Key Questions Answered"): a delayed scale comes
 * from earlier iterations' maxima, so a step whose amax jumps above them
 * has values the format cannot hold, which the cast clamps to +-max.
 *   sat_out  one uint64 (device, required): the number of elements with
 *            |x * 2^(*bias)| > fmax (+-Inf included, NaN not), exact;
 *            overwritten.
 * Every other argument, check and result is that of fp8_quantize (q, qT and
 * amax_out are bit-identical to its outputs).
 */
int fp8_quantize_sat(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld,
                     int fmt, const int32_t* bias, uint8_t* q, int64_t ldq,
                     uint8_t* qT, int64_t ldqT, float* amax_out, uint64_t* sat_out,
                     hipStream_t stream);

/*
 * fp8_quantize_delayed — one step of delayed scaling in one launch: the bias
 * from the window of earlier steps' amaxes ("Per-Tensor and Per-Block
 * Scaling Strategies ...", "Key Questions Answered": the scale follows the
 * largest amax over past iterations), the cast with it, and the push of this
 * step's amax into the window.  Results equal, bit for bit, the sequence
 *   fp8_compute_scale_delayed(hist, state, window, fmt, margin, bias_out)
 *   fp8_quantize_sat(x, ..., bias_out, q, ldq, qT, ldqT, amax_out, sat)
 *   fp8_history_push(hist, state, window, amax_out)
 * including the window and state it leaves behind.
 *   x, dtype, rows, cols, ld, fmt, q, ldq, qT, ldqT   as fp8_quantize (x and
 *                                  q may be NULL when rows * cols == 0);
 *   margin, hist, state, window    as fp8_compute_scale_delayed / the
 *                                  history calls (the window must not be
 *                                  empty for a delayed scale: the first step
 *                                  pushes its own amax beforehand, as in the
 *                                  sequence; an empty window gives bias 0);
 *   bias_out, amax_out             required, overwritten: the bias used and
 *                                  max |x| (the amax pushed);
 *   sat_out                        optional (NULL = skip): saturated count
 *                                  as in fp8_quantize_sat;
 *   workspace                      FP8_AMAX_SCALE_WORKSPACE_BYTES of
 *                                  caller-owned device memory, 8-byte
 *                                  aligned, ZERO before the first use and
 *                                  left zero by every call (its first 16
 *                                  bytes hold a ticket, a running maximum
 *                                  and a 64-bit count during the call).
 *                                  Calls sharing a workspace, or a history,
 *                                  must not overlap (order them on one
 *                                  stream).
 * One kernel: each workgroup takes the bias from the window, casts its
 * share and folds its maximum and count into the workspace; the last to
 * finish writes the outputs and pushes the amax.  With a transposed copy of
 * an input other than 16-byte aligned bf16 rows the step runs as the three
 * calls above (the workspace is then not touched).
 */
int fp8_quantize_delayed(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld,
                         int fmt, int margin, float* hist, int32_t* state, int window,
                         uint8_t* q, int64_t ldq, uint8_t* qT, int64_t ldqT,
                         int32_t* bias_out, float* amax_out, uint64_t* sat_out,
                         void* workspace, hipStream_t stream);

/*
 * mx_quantize — per-block (MXFP8-style) cast ("Key Questions Answered": a
 * tensor is split into blocks with a scale each).  Blocks are 1 x 32 along
 * cols (the GEMM's K axis); cols % 32 == 0 is required.
 *   q        [rows x cols] FP8 codes (fmt), leading dimension ldq (bytes).
 *   scales   [rows x cols/32] E8M0 codes, leading dimension ld_scales (bytes):
 *            code = 127 - e_b with e_b = floor(log2(fmax / block_amax)) in
 *            [-127, 127]; 127 for an all-zero or infinite block; 0xFF for a
 *            block holding a NaN.  q = sat_RNE(x * 2^e_b).
 */
int mx_quantize(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld,
                int fmt, uint8_t* q, int64_t ldq, uint8_t* scales,
                int64_t ld_scales, hipStream_t stream);

/*
 * mx_quantize_t — per-block cast with the blocks along ROWS, written
 * transposed ("Key Questions Answered": per-block scaling; the backward
 * products contract over the token axis, so their MX operands need blocks
 * along it).  Blocks are 32 x 1 (32 consecutive rows of one column); the
 * result equals mx_quantize of x^T:
 *   qT       [cols x rows] FP8 codes (fmt), leading dimension ldqT (bytes):
 *            qT[c, r] = sat_RNE(x[r, c] * 2^e_b) for the block b of rows
 *            32 floor(r/32) .. +31 in column c.
 *   scalesT  [cols x rows/32] E8M0 codes, leading dimension ld_scales, by the
 *            rule of mx_quantize.
 * rows % 32 == 0 is required; any alignment is accepted.
 */
int mx_quantize_t(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld,
                  int fmt, uint8_t* qT, int64_t ldqT, uint8_t* scalesT,
                  int64_t ld_scales, hipStream_t stream);

/*
 * mx_quantize_rule / mx_quantize_t_rule — mx_quantize / mx_quantize_t with a
 * choice of block-exponent rule.  The summary page ("Key Questions
 * Answered") names MXFP8 block scaling but not how a block's scale is
 * chosen; MX_RULE_OCP is the shared-scale rule of the OCP Microscaling (MX)
 * specification that MXFP8 belongs to:
 *   rule = MX_RULE_FMAX  e_b = floor(log2(fmax / block_amax)), exactly what
 *                        mx_quantize / mx_quantize_t compute: the block
 *                        maximum never exceeds the format maximum;
 *   rule = MX_RULE_OCP   e_b = emax - floor(log2(block_amax)), emax being the
 *                        exponent of the format's largest binade (8 for
 *                        E4M3, 15 for E5M2): the block maximum lands in that
 *                        binade and, when its significand exceeds 1.75 (the
 *                        format maximum's), saturates to +-fmax.  It equals
 *                        FMAX's e_b, or FMAX's e_b + 1 when the significand
 *                        of block_amax is above 1.75.
 * Both clamp e_b to [-127, 127] and share the zero, Inf and NaN conventions,
 * layouts and argument rules of mx_quantize / mx_quantize_t; an unknown rule
 * returns FP8_ERR_FORMAT.  The GEMM reads either rule's scales unchanged.
 */
int mx_quantize_rule(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld,
                     int fmt, int rule, uint8_t* q, int64_t ldq, uint8_t* scales,
                     int64_t ld_scales, hipStream_t stream);
int mx_quantize_t_rule(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld,
                       int fmt, int rule, uint8_t* qT, int64_t ldqT, uint8_t* scalesT,
                       int64_t ld_scales, hipStream_t stream);

/*
 * fp8_scaled_gemm — per-tensor scaled FP8 GEMM with unscale ("Proposed
 * method": matrix multiplication on the FP8 operands, unscaled afterwards).
 *   C[m, n] = 2^-(*bias_a + *bias_b) * sum_k opA[m, k] * opB[n, k]
 * with fp32 accumulation and one rounding to out_dtype.
 *   opA is [M x K]: A stored [M x K] (trans_a = 0) or [K x M] (trans_a = 1).
 *   opB is [N x K]: B stored [N x K] (trans_b = 0) or [K x N] (trans_b = 1).
 *   The forward layer Y = X W^T is trans_a = trans_b = 0 (W stored [out x in]);
 *   dX = dY W is trans_b = 1; dW = dY^T X is trans_a = trans_b = 1.
 *   fmt_a, fmt_b  E4M3 or E5M2 independently (E5M2 gradients x E4M3).
 *   C        [M x N] of out_dtype (bf16 or fp32), leading dimension ldc.
 *   out_amax optional: max |C| over the STORED (rounded) output, for the next
 *            layer's scale; overwritten.
 * Requirements: K % 16 == 0; A, B 16-byte aligned with lda, ldb multiples of
 * 16; a transposed operand's M (or N) a multiple of 16.  K == 0 gives C = 0.
 */
int fp8_scaled_gemm(int64_t M, int64_t N, int64_t K,
                    const uint8_t* A, int fmt_a, int trans_a, int64_t lda,
                    const int32_t* bias_a,
                    const uint8_t* B, int fmt_b, int trans_b, int64_t ldb,
                    const int32_t* bias_b,
                    void* C, int out_dtype, int64_t ldc, float* out_amax,
                    hipStream_t stream);

/*
 * mx_scaled_gemm — block-scaled FP8 GEMM ("Key Questions Answered": per-block
 * scaling; the product consumes the per-block scales).
 *   C[m, n] = sum_j 2^(sa[m, j] - 127) * 2^(sb[n, j] - 127)
 *                   * sum_{k in block j} A[m, k] * B[n, k]
 * A [M x K] and B [N x K] FP8 codes (K contiguous, both), A_scales [M x K/32]
 * and B_scales [N x K/32] E8M0 codes (as written by mx_quantize), fp32
 * accumulation, C [M x N] bf16 or fp32, optional fused out_amax as above.
 * Requirements: K % 32 == 0; A, B 16-byte aligned with lda, ldb multiples of
 * 16.  Scales may have any alignment; with 4-byte aligned scale rows and
 * K >= 512 the product runs the faster kernel (the bytes after a scale
 * row's K/32 codes are never read).
 */
int mx_scaled_gemm(int64_t M, int64_t N, int64_t K,
                   const uint8_t* A, int fmt_a, int64_t lda,
                   const uint8_t* A_scales, int64_t lds_a,
                   const uint8_t* B, int fmt_b, int64_t ldb,
                   const uint8_t* B_scales, int64_t lds_b,
                   void* C, int out_dtype, int64_t ldc, float* out_amax,
                   hipStream_t stream);

/*
 * Packed E8M0 scale layout for the block-scaled GEMM.  The per-block scales of
 * "Key Questions Answered" (summary page) are the same codes as mx_quantize
 * writes; only their order in memory changes, so that the GEMM copies whole
 * cache lines of them (a row-major [rows x K/32] matrix hands it 16 bytes per
 * row, one cache line per row per 4 K-stages).
 *
 * Layout: rows are grouped in tiles of 256, K-blocks in groups of 16 (512 K
 * elements); each (tile t, group g) is one 4096-byte block holding, for
 * r = 0..255, the 16 codes of row 256 t + r, blocks 16 g .. 16 g + 15.  The
 * code of (row, block j) sits at byte
 *     ((row / 256) * G + j / 16) * 4096 + (row % 256) * 16 + j % 16,
 * with G = ceil(kblocks / 16).  Positions past the matrix (rows >= rows,
 * j >= kblocks) hold 127 (scale 1).
 */

/* Size in bytes of the packed layout of a [rows x kblocks] E8M0 matrix:
 * ceil(rows / 256) * ceil(kblocks / 16) * 4096 (FP8_ERR_SHAPE if negative).
 * Host-only; no HIP call. */
int64_t mx_packed_scales_bytes(int64_t rows, int64_t kblocks);

/*
 * mx_pack_scales — rewrite row-major E8M0 codes scales [rows x kblocks]
 * (leading dimension ld_scales bytes, any alignment) into the packed layout
 * above.  packed: mx_packed_scales_bytes(rows, kblocks) bytes, 16-byte
 * aligned (else FP8_ERR_ALIGN).  Every byte of `packed` is written, padding
 * included.
 */
int mx_pack_scales(const uint8_t* scales, int64_t rows, int64_t kblocks, int64_t ld_scales,
                   uint8_t* packed, hipStream_t stream);

/*
 * mx_quantize_packed — mx_quantize_rule writing its E8M0 codes straight into
 * the packed layout (no separate mx_pack_scales pass).  q as for mx_quantize;
 * packed: mx_packed_scales_bytes(rows, cols / 32) bytes, 16-byte aligned
 * (else FP8_ERR_ALIGN); every byte is written (127 past the matrix).  The
 * codes equal mx_pack_scales applied to mx_quantize_rule's, bit for bit.
 */
int mx_quantize_packed(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld,
                       int fmt, int rule, uint8_t* q, int64_t ldq, uint8_t* packed,
                       hipStream_t stream);

/*
 * mx_quantize_t_packed — mx_quantize_t_rule (the MX cast of x^T: blocks of 32
 * rows, qT [cols x rows]) writing the E8M0 codes of qT, a [cols x rows/32]
 * matrix, in the packed layout: mx_packed_scales_bytes(cols, rows / 32)
 * bytes, 16-byte aligned (else FP8_ERR_ALIGN); every byte is written (127
 * past the matrix).  Equal to mx_pack_scales of mx_quantize_t_rule's codes.
 */
int mx_quantize_t_packed(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld,
                         int fmt, int rule, uint8_t* qT, int64_t ldqT, uint8_t* packed,
                         hipStream_t stream);

/*
 * mx_scaled_gemm_packed — mx_scaled_gemm with both scale operands in the
 * packed layout (A_packed from mx_pack_scales of A's [M x K/32] codes or from
 * mx_quantize_packed / mx_quantize_t_packed, B_packed likewise for B's
 * [N x K/32] codes).  Same result as mx_scaled_gemm on the row-major codes,
 * bit for bit where that call runs the same kernel (4-byte aligned scale
 * rows, K >= 512); this call runs it for every K.
 * Requirements: those of mx_scaled_gemm, plus K > 0 (else
 * FP8_ERR_UNSUPPORTED) and 16-byte aligned packed buffers (FP8_ERR_ALIGN).
 */
int mx_scaled_gemm_packed(int64_t M, int64_t N, int64_t K,
                          const uint8_t* A, int fmt_a, int64_t lda, const uint8_t* A_packed,
                          const uint8_t* B, int fmt_b, int64_t ldb, const uint8_t* B_packed,
                          void* C, int out_dtype, int64_t ldc, float* out_amax,
                          hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SCALED_FP8_H */
