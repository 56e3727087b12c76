/* rmsnorm_mi355x.h -- C ABI of the row-wise normalisation library for MI355X
 * (gfx950): RMSNorm and its variants, and LayerNorm.
 *
 * The operation ("Pre-built kernel library guide" (FlyDSL), section 1.2 RMSNorm):
 * for every row i of a row-major [M, N] array,
 *     rstd_i = 1 / sqrt(mean_j(x_ij^2) + eps)
 *     y_ij   = x_ij * rstd_i * gamma_j
 * with fp32 accumulation and one round-to-nearest-even rounding at each store.
 *
 * Conventions shared by every call:
 *   - All data pointers are DEVICE pointers owned by the caller; arrays are
 *     contiguous and row-major ("contiguous 2-D ... row-major rows", FlyDSL guide
 *     section 2.2). The library never allocates, frees or synchronises.
 *   - Work is enqueued on the caller's stream and runs asynchronously; the call
 *     returns once the kernels are launched. The stream (0 for the null
 *     stream) must belong to the current HIP device, whose memory the pointers
 *     refer to.
 *   - Type codes (rmsn_dtype): activations x, r/h, y, dy, dx share x_dtype in
 *     {RMSN_F32, RMSN_F16, RMSN_BF16}; gamma_dtype is x_dtype or RMSN_F32 (fp32
 *     weights with 16-bit activations, FlyDSL guide section 1.2); rstd and
 *     dgamma are always fp32.
 *   - Shapes: M >= 0 rows, 1 <= N <= RMSN_MAX_N columns (else RMSN_ERR_SHAPE).
 *     M == 0 is a no-op returning RMSN_OK
 *     (pointers are not inspected). Every pointer must be aligned to its element
 *     size; 16-byte-aligned rows (base aligned and N * element size a multiple
 *     of 16) take the vectorised path, anything else a scalar path.
 *   - Errors: argument errors are detected on the host before any HIP call and
 *     returned as negative rmsn_status codes; nothing is enqueued then. A
 *     failed launch returns RMSN_ERR_HIP and rmsnorm_last_hip_error() gives the
 *     hipError_t (an error left on the calling thread by an earlier, unrelated
 *     HIP call is cleared before the launch and never reported as the
 *     library's). Faults during execution surface at the caller's next
 *     synchronisation, as for any asynchronous HIP work.
 *   - Input domain: every finite input and every finite eps >= 0. The kernels
 *     accumulate in fp32; a row whose fp32 statistics leave the range where
 *     they are exact to rounding -- q = mean(x^2) + eps outside
 *     [2^-100, FLT_MAX], which takes |x| beyond about 1.8e19, or squares that
 *     underflow when eps is below 2^-100, or an eps near the fp32 maximum --
 *     is recomputed in fp64 by the same launch, so results match the fp64
 *     definition over the whole domain (LayerNorm: the same test on its
 *     centred sum of squares). eps = 0 with an all-zero row is the
 *     definition's 0/0: rstd = +inf and y = NaN, as in fp64; quantised codes
 *     of such a row are unspecified. An element whose exact result is beyond
 *     the output type's range rounds to +-inf (fp16, bf16, fp32) or saturates
 *     (fp8, fp4). Inputs holding inf or NaN give unspecified results.
 *   - Thread safety: besides the per-thread last HIP error the calls keep only
 *     per-device facts queried on first use (compute-unit count, LDS size per
 *     workgroup, kernels' dynamic-LDS limits), set idempotently through
 *     atomics; concurrent calls on different buffers are safe.
 */
#ifndef RMSNORM_MI355X_H
#define RMSNORM_MI355X_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Largest row length N accepted (2^31 - 2^20). */
#define RMSN_MAX_N 2146435072

/* Size of the fixed device buffer behind rmsnorm_bwd_noalloc (32 MiB per GPU). */
#define RMSN_NOALLOC_SCRATCH_BYTES (32u * 1024u * 1024u)

typedef enum {
  RMSN_F32 = 0,
  RMSN_F16 = 1,
  RMSN_BF16 = 2
} rmsn_dtype;

typedef enum {
  RMSN_OK = 0,
  RMSN_ERR_NULL = -1,       /* a required pointer is null */
  RMSN_ERR_SHAPE = -2,      /* M < 0, N < 1, M * N too large to index, or a
                               call's own shape rule (MX: N % 32; QK: strides) */
  RMSN_ERR_DTYPE = -3,      /* unsupported x_dtype / gamma_dtype pair */
  RMSN_ERR_WORKSPACE = -4,  /* backward workspace null or too small */
  RMSN_ERR_OVERLAP = -5,    /* buffers overlap in a way the call forbids */
  RMSN_ERR_ALIGN = -6,      /* a pointer is not aligned to its element size (or
                               to what a call requires, e.g. MX inputs: 16 B) */
  RMSN_ERR_EPS = -7,        /* eps negative or not finite */
  RMSN_ERR_MODE = -8,       /* unknown quantisation mode */
  RMSN_ERR_SCRATCH = -9,    /* rmsnorm_bwd_noalloc: the shape needs more than
                               RMSN_NOALLOC_SCRATCH_BYTES of workspace */
  RMSN_ERR_HIP = -100       /* a kernel launch failed; see rmsnorm_last_hip_error */
} rmsn_status;

/* Forward RMSNorm (FlyDSL guide section 1.2, build_rmsnorm_module with
 * store_rstd and weight_dtype_str).
 *   x      [M, N] x_dtype, read.
 *   gamma  [N] gamma_dtype, read.
 *   y      [M, N] x_dtype, written. y == x (exact in-place) is allowed; any
 *          other overlap with x, gamma or rstd is RMSN_ERR_OVERLAP.
 *   rstd   [M] fp32, written with 1/sqrt(mean(x^2)+eps) per row; may be NULL.
 *   eps    finite, >= 0; added to the mean square inside the square root.
 * Rows with N <= 8192 stay in registers, longer rows are cached in LDS (or
 * re-read when a row exceeds the LDS cache). */
int rmsnorm_fwd(const void* x, const void* gamma, void* y, float* rstd,
                int64_t M, int64_t N, float eps, int x_dtype, int gamma_dtype,
                hipStream_t stream);

/* Fused residual add + forward RMSNorm ("TIRx kernels", FlashInfer ports,
 * flashinfer.norm fused_add_rmsnorm; FlyDSL guide section 1.2 fused-add
 * wrappers). The pages name the operation without defining it; this library
 * reads it as
 *     h_ij = round_x_dtype(x_ij + r_ij)     (sum in fp32, one rounding)
 *     residual <- h  (in place),   y = RMSNorm(h)   (of the rounded h)
 *   x         [M, N] x_dtype, read. x == residual (exact) is allowed.
 *   residual  [M, N] x_dtype, read as r and overwritten with h.
 *   gamma, rstd, eps as in rmsnorm_fwd.
 *   y         [M, N] x_dtype, written; may equal x exactly, must not overlap
 *             residual, gamma or rstd. */
int rmsnorm_fused_add_fwd(const void* x, void* residual, const void* gamma, void* y,
                          float* rstd, int64_t M, int64_t N, float eps, int x_dtype,
                          int gamma_dtype, hipStream_t stream);

/* Output modes of rmsnorm_quant_fwd. */
typedef enum {
  RMSN_QUANT_FP8_TENSOR = 1, /* fp8 e4m3, one caller scale for the whole tensor, read */
  RMSN_QUANT_FP8_ROW = 2,    /* fp8 e4m3, one scale per row, computed and written */
  RMSN_QUANT_MXFP8 = 3,      /* MX: e4m3 elements, E8M0 scale per 32 elements, written */
  RMSN_QUANT_MXFP4 = 4       /* MX: e2m1 elements, E8M0 scale per 32 elements, written */
} rmsn_quant_mode;

/* Forward RMSNorm (optionally after the fused residual add) with a
 * quantised output. The pages name these variants ("TIRx kernels", FlashInfer
 * ports, flashinfer.norm: rmsnorm_quant, fused_add_rmsnorm_quant,
 * rmsnorm_fp4quant, add_rmsnorm_fp4quant) without defining them; the FlyDSL
 * guide uses e4m3fn (OCP, not fnuz) on gfx950 (section 3b, FlashAttention
 * fp8) and per-32 E8M0 block scales with fp4 / fp8 elements (section 3.1,
 * Preshuffle GEMM, its MX paragraph). Readings taken:
 *   The RMSNorm value y (fp32, never rounded to the activation type) is
 *   divided by a scale s and rounded to the element format, nearest-even,
 *   saturated at its largest value: fp8 e4m3 "fn" (1 sign, 4 exponent bits,
 *   bias 7, 3 fraction bits, no infinity, max 448) or fp4 e2m1 (1 sign, 2
 *   exponent bits, bias 1, 1 fraction bit: 0, 0.5, 1, 1.5, 2, 3, 4, 6).
 *   RMSN_QUANT_FP8_TENSOR: s = scale[0] (fp32, read on the device; positive
 *     and finite).
 *   RMSN_QUANT_FP8_ROW: s_i = amax_i / 448 with amax_i = max_j |y_ij|,
 *     written to scale[i] (fp32, [M]); each row's largest element maps to
 *     +-448; a zero row gets s = 0 and zero codes.
 *   RMSN_QUANT_MXFP8 / RMSN_QUANT_MXFP4 (OCP Microscaling layout): each block
 *     of 32 consecutive row elements has s = 2^(c - 127) with the E8M0 code
 *     c = clamp(floor(log2 amax) - emax + 127, 0, 254), amax the block's
 *     max |y| and emax 8 (e4m3) or 2 (e2m1); codes are written to scale
 *     (uint8, [M, N / 32], row-major). A zero block gets c = 0 and zero
 *     elements. N must be a multiple of 32 (else RMSN_ERR_SHAPE), and x,
 *     residual and gamma 16-byte aligned, q aligned to 8 / 4 (MXFP8 with
 *     16-bit / fp32 activations) or 4 / 2 (MXFP4) bytes (else RMSN_ERR_ALIGN).
 *   x, residual, gamma, rstd, eps as in rmsnorm_fwd / rmsnorm_fused_add_fwd;
 *             residual may be NULL (plain forward) or is read as r and
 *             overwritten with h = round(x + r), and h is normalised.
 *   q         the element codes, written; overlaps nothing else. fp8 modes:
 *             [M, N] bytes. MXFP4: [M, N / 2] bytes, element 2k in the low
 *             nibble of byte k, element 2k + 1 in the high nibble.
 * The kernel scales in fp32 (y / s as x * gamma * (rstd / s), or y * 2^(127 - c)
 * exactly for MX), so a code may be one step from the exactly rounded one
 * where y / s lies within fp32 rounding of a tie, and an MX block whose amax
 * lies within fp32 rounding of a power of two may take the neighbouring code.
 * Rows holding inf or NaN give unspecified codes. */
int rmsnorm_quant_fwd(const void* x, void* residual, const void* gamma, void* q,
                      void* scale, int quant_mode, float* rstd, int64_t M, int64_t N,
                      float eps, int x_dtype, int gamma_dtype, hipStream_t stream);

/* Per-head RMSNorm of q and k, in place, in one launch (QK-norm; the
 * "TIRx kernels" page lists flashinfer.norm's qk_rmsnorm among its FlashInfer
 * ports without a definition). Reading taken: q is [tokens, q_heads,
 * head_dim] and k [tokens, k_heads, head_dim]; every head vector is one
 * RMSNorm row of head_dim elements (as in rmsnorm_fwd) with its tensor's
 * gamma[head_dim], overwritten by its normalised value.
 *   q, k       head h of token t starts at element t * stride + h * head_dim
 *              (heads contiguous, tokens q_stride / k_stride elements apart,
 *              stride >= heads * head_dim). k may be NULL with k_heads == 0.
 *              q and k may interleave inside one buffer (a fused QKV
 *              projection) provided their per-token windows are disjoint and
 *              share one stride; any other overlap is RMSN_ERR_OVERLAP.
 *              Elements between windows are not touched.
 *   q_gamma, k_gamma  [head_dim] gamma_dtype, read.
 *   tokens >= 0, q_heads >= 1, k_heads >= 0, 1 <= head_dim <= 8192, and
 *   tokens * (q_heads + k_heads) below 2^31 (else RMSN_ERR_SHAPE). */
int rmsnorm_qk_fwd(void* q, void* k, const void* q_gamma, const void* k_gamma,
                   int64_t tokens, int64_t q_heads, int64_t k_heads, int64_t head_dim,
                   int64_t q_stride, int64_t k_stride, float eps, int x_dtype,
                   int gamma_dtype, hipStream_t stream);

/* Bytes of device workspace rmsnorm_bwd (and rmsnorm_fused_add_bwd) needs
 * for an [M, N] problem, whatever the dtypes: the fp32 dgamma partials,
 * G x N (rounded up to 256 bytes) with G = max(min(M, T), ceil(M / 64))
 * partial rows, T = 256 for N <= 32768 and ceil(2^22 / N) above (such rows
 * take the two-pass tier, which runs column tiles x G workgroups), and for
 * N > 8192 a 16-byte record per row (rows longer than the one-pass kernel
 * holds keep their row dots there; rows of up to 4096 16-byte units --
 * 32768 16-bit / 16384 fp32 elements, 24576 for 16-bit LayerNorm with fp32
 * gamma -- stay
 * one-pass and leave it unused). Pure host
 * function; returns 0 for M <= 0, N <= 0 or N > RMSN_MAX_N. */
size_t rmsnorm_bwd_workspace_size(int64_t M, int64_t N);

/* Backward RMSNorm (FlyDSL guide section 1.2, "Backward": inputs x, gamma, dy
 * and the saved rstd, no eps since the forward baked it into rstd). With
 * rho_i = rstd[i] and c_i = (1/N) sum_j dy_ij gamma_j x_ij:
 *     dx_ij     = rho_i * (gamma_j dy_ij - x_ij rho_i^2 c_i)
 *     dgamma_j  = sum_i dy_ij x_ij rho_i          (fp32, OVERWRITTEN)
 * dgamma is reduced in two stages (per-workgroup fp32 partials in the
 * workspace, then a fixed-order column sum) with no atomics, so repeated calls
 * with the same inputs give bit-identical dx and dgamma.
 *   dy, x     [M, N] x_dtype, read.
 *   rstd      [M] fp32, read.
 *   gamma     [N] gamma_dtype, read.
 *   dx        [M, N] x_dtype, written; may equal dy or x exactly.
 *   dgamma    [N] fp32, written.
 *   workspace at least rmsnorm_bwd_workspace_size(M, N) bytes of device
 *             memory, 16-byte aligned, disjoint from every other buffer; its
 *             contents on entry are ignored.
 * The workgroup partition depends only on M and N, which fixes the summation
 * order. A row whose fp32 row dot overflows (a product dy x or dy x gamma beyond the
 * fp32 range) is recomputed in fp64 in the same launch. Outside that, the
 * fp32 formula needs gamma_j dy_ij within the fp32 range, and rstd as the
 * forward produced it (positive, finite); a row with rstd = +inf (the 0/0 of
 * the forward) gives NaN, as in fp64. */
int rmsnorm_bwd(const void* dy, const void* x, const float* rstd, const void* gamma,
                void* dx, float* dgamma, void* workspace, size_t workspace_bytes,
                int64_t M, int64_t N, int x_dtype, int gamma_dtype, hipStream_t stream);

/* rmsnorm_bwd for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation, kernels and results bit for bit, with the workspace taken
 * from a fixed device array of RMSN_NOALLOC_SCRATCH_BYTES that the library
 * holds on every GPU it runs on until the process ends. The first call on a
 * device looks up that device's copy of the array (hipGetSymbolAddress),
 * which is when the HIP runtime may load the library's code for the device
 * and reserve the array; no call allocates or frees memory itself, and every
 * later call leaves device memory as it finds it. Arguments as in
 * rmsnorm_bwd; the stream must belong to the current device.
 *   Limit: rmsnorm_bwd_workspace_size(M, N) <= RMSN_NOALLOC_SCRATCH_BYTES,
 *   else RMSN_ERR_SCRATCH before any HIP call (e.g. 8192 x 8192 needs 8 MiB;
 *   N = 8192 fits up to M = 65536).
 *   Calls that overlap in time on one GPU (several streams or threads) share
 *   the array and race: serialise them. Nothing in it needs clearing between
 *   calls (each call writes what it reads). */
int rmsnorm_bwd_noalloc(const void* dy, const void* x, const float* rstd, const void* gamma,
                        void* dx, float* dgamma, int64_t M, int64_t N, int x_dtype,
                        int gamma_dtype, hipStream_t stream);

/* Backward of the fused residual add + RMSNorm (rmsnorm_fused_add_fwd): with
 * h the saved sum (the residual buffer after the forward) and rstd its saved
 * rstd, the gradient of h is the norm's backward over h plus the gradient
 * that reaches h through the residual stream:
 *     dh_ij = rho_i (gamma_j dy_ij - h_ij rho_i^2 c_i) + dresidual_ij
 * summed in fp32 and rounded once; dh is the gradient of both x and the old
 * residual. dgamma and the workspace are as in rmsnorm_bwd (same size
 * function). The pages list the fused add among the FlashInfer ports of the
 * "TIRx kernels" page and FlyDSL's fused-add training wrappers without a
 * formula; this is the derivative of the forward reading above.
 *   dy, h      [M, N] x_dtype, read.
 *   dresidual  [M, N] x_dtype, read; may be NULL (then dh is rmsnorm_bwd's dx).
 *   dh         [M, N] x_dtype, written; may equal dy, h or dresidual exactly. */
int rmsnorm_fused_add_bwd(const void* dy, const void* h, const float* rstd,
                          const void* gamma, const void* dresidual, void* dh,
                          float* dgamma, void* workspace, size_t workspace_bytes,
                          int64_t M, int64_t N, int x_dtype, int gamma_dtype,
                          hipStream_t stream);

/* LayerNorm forward ("Pre-built kernel library guide" (FlyDSL), section 1.1,
 * build_layernorm_module: Input, Gamma, Beta, Output): for every row i,
 *     mean_i = (1/N) sum_j x_ij,   var_i = (1/N) sum_j (x_ij - mean_i)^2,
 *     rstd_i = 1 / sqrt(var_i + eps),
 *     y_ij   = (x_ij - mean_i) * rstd_i * gamma_j + beta_j
 * with fp32 arithmetic: the mean from one row reduction, the variance from a
 * second one over the centred values (no E[x^2] - mean^2 cancellation), and
 * (x - mean) * rstd * gamma + beta with one fused multiply-add, rounded once.
 *   x          [M, N] x_dtype, read.
 *   gamma      [N] gamma_dtype, read;  beta [N] gamma_dtype, read, or NULL (0).
 *   y          [M, N] x_dtype, written; may equal x exactly.
 *   mean, rstd [M] fp32 each, written when not NULL (for the backward).
 * Shapes, dtypes, alignment and errors as for rmsnorm_fwd. */
int layernorm_fwd(const void* x, const void* gamma, const void* beta, void* y, float* mean,
                  float* rstd, int64_t M, int64_t N, float eps, int x_dtype,
                  int gamma_dtype, hipStream_t stream);

/* Bytes of device workspace layernorm_bwd needs: two fp32 partial arrays
 * (dgamma, dbeta) of G rows each, G as for rmsnorm_bwd_workspace_size, and,
 * for rows longer than 8192, a 16-byte record per row. 0 for M <= 0, N <= 0
 * or N > RMSN_MAX_N. */
size_t layernorm_bwd_workspace_size(int64_t M, int64_t N);

/* LayerNorm backward. The pages give only the forward (FlyDSL guide, section
 * 1.1); this is its derivative with the saved per-row mean and rstd (the
 * forward's outputs, eps already inside rstd):
 *     xhat_ij = (x_ij - mean_i) rstd_i
 *     c1_i = (1/N) sum_j gamma_j dy_ij,   c2_i = (1/N) sum_j gamma_j dy_ij xhat_ij
 *     dx_ij = rstd_i (gamma_j dy_ij - c1_i - xhat_ij c2_i)
 *     dgamma_j = sum_i dy_ij xhat_ij,     dbeta_j = sum_i dy_ij
 * fp32 arithmetic with the row dots accumulated in double; dgamma and dbeta
 * (fp32, OVERWRITTEN) are reduced in two fixed-order stages as in
 * rmsnorm_bwd, so repeated calls give bit-identical results.
 *   dy, x      [M, N] x_dtype, read.    mean, rstd [M] fp32, read.
 *   gamma      [N] gamma_dtype, read.
 *   dx         [M, N] x_dtype, written; may equal dy or x exactly.
 *   dgamma     [N] fp32, written.   dbeta [N] fp32, written, or NULL (skipped).
 *   workspace  at least layernorm_bwd_workspace_size(M, N) bytes, 16-byte
 *              aligned, disjoint from every other buffer.
 * Domain: with the forward's mean and rstd, |xhat| <= sqrt(N), so the fp32
 * dots hold for every finite x; the row dots need sum_j |gamma_j dy_ij|
 * within the fp32 range (a gradient near the fp32 maximum is outside). */
int layernorm_bwd(const void* dy, const void* x, const float* mean, const float* rstd,
                  const void* gamma, void* dx, float* dgamma, float* dbeta, void* workspace,
                  size_t workspace_bytes, int64_t M, int64_t N, int x_dtype, int gamma_dtype,
                  hipStream_t stream);

/* Static English description of a status code ("unknown status" otherwise). */
const char* rmsnorm_status_string(int status);

/* hipError_t (as int) of the last failed launch on the calling thread, or 0. */
int rmsnorm_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* RMSNORM_MI355X_H */
