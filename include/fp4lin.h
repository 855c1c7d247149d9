/*
 * fp4lin.h - C ABI of the MI355X (gfx950) FP4 quantized linear-layer forward
 *
 *      Y = dequant(Aq . Wq) + dA . W
 *
 * The method is the forward pass of the FP4 linear layer described on the pages about
 * "Optimizing Large Language Model Training Using FP4 Quantization":
 *   - QbitAI report, quantization-format paragraph: E2M1 (1 sign, 2 exponent, 1 mantissa
 *     bit);
 *   - QbitAI report, granularity paragraph: W quantized per output channel (column), A per
 *     token (row), chosen so the GEMM needs no extra transpose;
 *   - QbitAI report, forward-quantization paragraph: at the start of each forward, W and A
 *     of every linear layer are scaled into the FP4 range (scale+shift, per-layer ranges)
 *     and rounded to the nearest FP4 value by table lookup;
 *   - QbitAI report, outlier paragraph, and the paper abstract: outliers of A are found by
 *     a quantile search, clamped to a threshold (A_clamped), and compensated by the sparse
 *     matrix dA that is non-zero only where clamping happened.
 *
 * Readings fixed by this library where the pages are silent (the CPU oracle takes the
 * same ones):
 *   - scale: r = fl32(6 / amax) per row of A_clamped and per column of W, dequantization
 *     scale s = fl32(amax / 6); a vector with amax < 2^-120 gets r = s = 0;
 *   - rounding: nearest E2M1 value, ties to the even code, saturation at 6, sign copied;
 *   - threshold: T = the (k+1)-th smallest |a| over all M*K entries, k = floor(q*(M*K-1))
 *     in IEEE double; an outlier is |a| > T strictly; delta = fl32(a - copysign(T, a));
 *   - product: acc = sum_k value(Aq) * value(Wq), exact in fp32 for K <= 65536;
 *     Y_main = fl32(fl32(acc * sA[m]) * sW[n]);
 *   - compensation uses the original W: Y = Y_main + sum over row m's dA entries of
 *     delta * W[k][n], accumulated in fp32 in ascending k.
 *
 * Layouts (all row-major, dense, base pointers 16-byte aligned):
 *   A   M x K activations (tokens x in-features), fp32 or bf16
 *   W   K x N weights (in x out), same dtype as A
 *   Aq  M x K/2 bytes: code of A[m][k] in byte (m, k/2), low nibble for even k
 *   Wq  N x K/2 bytes: code of W[k][n] in byte (n, k/2), low nibble for even k
 *       (K-contiguous per output channel: both GEMM operands are K-contiguous)
 *   sA  fp32[M], sW fp32[N]
 *   dA  COO sorted by (row, col): coo_row/coo_col int32[nnz], coo_val fp32[nnz],
 *       row_ptr int32[M+1] (CSR row offsets of the same list)
 *   Y   M x N, fp32 or bf16 (bf16 = round-to-nearest-even of the fp32 result)
 *
 * Ownership and threading: the caller owns every buffer (device memory unless stated).
 * The library never allocates, frees or synchronizes, and never copies device data to
 * the host: each call only validates its arguments on the host and enqueues kernels on
 * the caller's HIP stream (hipStream_t passed as void*, NULL = default stream); results
 * are ready when that stream reaches them.  The only global state is a per-device cache of
 * the device's properties (gfx950 or not, compute-unit count), filled on first use under a
 * lock: calls on different streams are independent as long as their buffers do not overlap.
 *
 * Errors: every argument check runs on the host before the first HIP call and returns a
 * status; nothing is enqueued then.  FP4_ERR_DEVICE: the current device is not gfx950.
 * FP4_ERR_HIP: a launch failed (the stream may hold part of the work).  Inputs must be
 * finite; NaN or Inf give unspecified codes and outputs.
 */
#ifndef FP4LIN_H
#define FP4LIN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t fp4_status;
enum {
    FP4_OK = 0,
    FP4_ERR_NULL = 1,      /* a required pointer is NULL */
    FP4_ERR_SHAPE = 2,     /* a size is out of range (see each call) */
    FP4_ERR_DTYPE = 3,     /* unknown dtype or axis code */
    FP4_ERR_QUANTILE = 4,  /* q is NaN or outside [0, 1] */
    FP4_ERR_CAPACITY = 5,  /* COO capacity below fp4_outlier_capacity() */
    FP4_ERR_WORKSPACE = 6, /* workspace smaller than the size query returns */
    FP4_ERR_DEVICE = 7,    /* current HIP device is not gfx950 */
    FP4_ERR_HIP = 8,       /* a HIP runtime call or launch failed */
    FP4_ERR_ALIGN = 9,     /* a pointer is not 16-byte aligned */
    FP4_ERR_SCRATCH = 10   /* the problem needs more than the no-alloc entry point's fixed scratch */
};
enum { FP4_F32 = 0, FP4_BF16 = 1 };          /* element types of A, W, X, Y */
/* Output type of fp4_gemm only (no compensation term): the exact accumulator in two bytes.
 * Element (m, n) is the int16 4*acc (acc is a multiple of 1/4), except in escaped blocks:
 * aligned 128-row x 64-column blocks (rows 128i.., columns 64j..), each lying in an aligned
 * 128 x 128 block that holds some |acc| > 8191.75, and covering every such element.  There
 * every element is -32768 and the workspace holds fl(fl(acc*sA)*sW) as fp32 at element
 * (m, n) (those blocks are recomputed by a second kernel).  This is how the GEMM hands its
 * result to the compensation pass inside fp4_gemm and fp4_linear_forward, where the escaped
 * blocks are instead written straight to Y. */
enum { FP4_Q16 = 2 };
enum { FP4_PER_ROW = 0, FP4_PER_COL = 1 };   /* token-wise (A) / channel-wise (W) */

/* Limits shared by all calls: 32 <= K <= 65536 and K % 32 == 0 (contraction length:
 * two codes per byte, 16-byte vector lanes, and the fp32 accumulator stays exact);
 * 1 <= M and M * K < 2^32; 1 <= N and N % 8 == 0.  The product (fp4_gemm,
 * fp4_linear_forward) also needs N * K < 2^32 and, when it adds the compensation term,
 * K * N * sizeof(W element) < 2^31.  The outlier calls need the capacity bound
 * M*K - 1 - floor(q * (M*K - 1)) <= 2^29 (int32 COO offsets); a smaller q is rejected with
 * FP4_ERR_QUANTILE. */

/* Quantize one matrix X (R x C) to E2M1 codes and fp32 scales.
 * QbitAI report, granularity and forward-quantization paragraphs.
 *   axis FP4_PER_ROW: one scale per row (token-wise, as for A); needs C % 32 == 0,
 *                     32 <= C <= 65536; codes R x C/2, scales fp32[R].
 *   axis FP4_PER_COL: one scale per column (channel-wise, as for W with R = K, C = N);
 *                     needs R % 32 == 0, 32 <= R <= 65536, C % 8 == 0; codes C x R/2
 *                     (transposed: R-contiguous per column), scales fp32[C].  The scales
 *                     buffer also serves as the column-maximum scratch during the call.
 *   clamp_T: NULL, or a device fp32[1] holding T: each |x| > T is replaced by
 *            copysign(T, x) before scaling (the clamp of the outlier paragraph).
 * Returns FP4_OK or FP4_ERR_{NULL,SHAPE,DTYPE,ALIGN,DEVICE,HIP}. */
fp4_status fp4_quantize(const void *X, int32_t x_dtype, int64_t R, int64_t C, int32_t axis,
                        const float *clamp_T, uint8_t *codes, float *scales, void *stream);

/* Host-only: the largest possible nnz of dA for an M x K input and quantile q,
 * M*K - 1 - floor(q * (M*K - 1)); -1 if the arguments are invalid. */
int64_t fp4_outlier_capacity(int64_t M, int64_t K, double q);

/* Host-only: workspace bytes fp4_outlier_clamp needs for an M x K input of a_dtype
 * (0 if the arguments are invalid). */
size_t fp4_outlier_workspace_bytes(int64_t M, int64_t K, int32_t a_dtype, double q);

/* Outlier clamping and compensation (QbitAI report, outlier paragraph; abstract):
 * T = quantile q of |A| over the whole tensor; dA = A - clamp(A, -T, T) in COO order.
 *   T        device fp32[1] (out)
 *   coo_row, coo_col, coo_val  device arrays of `capacity` entries (out; the first *nnz
 *            are written).  capacity >= fp4_outlier_capacity(M, K, q) is required.
 *   row_ptr  device int32[M+1] (out), nnz  device int64[1] (out)
 *   workspace device scratch of at least fp4_outlier_workspace_bytes() bytes.
 * Returns FP4_OK or FP4_ERR_{NULL,SHAPE,DTYPE,QUANTILE,CAPACITY,WORKSPACE,ALIGN,DEVICE,HIP}. */
fp4_status fp4_outlier_clamp(const void *A, int32_t a_dtype, int64_t M, int64_t K, double q,
                             float *T, int32_t *coo_row, int32_t *coo_col, float *coo_val,
                             int64_t capacity, int32_t *row_ptr, int64_t *nnz, void *workspace,
                             size_t ws_bytes, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): fp4_outlier_clamp without a workspace argument.
 * The scratch is a fixed array of FP4_NOALLOC_SCRATCH_BYTES (64 MiB) that the library holds on
 * each GPU it runs on until the process ends.
 * A problem whose scratch (fp4_outlier_workspace_bytes) exceeds it is rejected with
 * FP4_ERR_SCRATCH before anything is enqueued; e.g. a bf16 16384 x 13824 input at q = 0.99
 * needs 38 MB.  Outputs, results and the other statuses are those of fp4_outlier_clamp; the
 * call allocates, frees and memsets nothing (the scratch is cleared by a fill kernel).  Every
 * call on one GPU shares that GPU's array: calls that overlap in time on one GPU (different
 * streams, or host threads) race and must be serialized by the caller; calls on one stream
 * are ordered. */
#define FP4_NOALLOC_SCRATCH_BYTES (64u << 20)
fp4_status fp4_outlier_clamp_noalloc(const void *A, int32_t a_dtype, int64_t M, int64_t K, double q,
                                     float *T, int32_t *coo_row, int32_t *coo_col, float *coo_val,
                                     int64_t capacity, int32_t *row_ptr, int64_t *nnz, void *stream);

/* Host-only: workspace bytes fp4_gemm needs: with the compensation term, one byte per
 * 128 x 64 output block (the map of escaped blocks) for a bf16 Y (the two-byte hand-over
 * goes through Y itself), plus M * N * 2 for an fp32 Y (the hand-over); for y_dtype FP4_Q16
 * (no compensation term) M * N * 4 (the fp32 escapes) plus the map; else 0 (also 0 for
 * invalid arguments).  Each part is rounded up to 256 bytes. */
size_t fp4_gemm_workspace_bytes(int64_t M, int64_t N, int32_t y_dtype, int32_t with_comp);

/* The FP4 GEMM with dequantization, plus the sparse compensation term (QbitAI report,
 * GEMM-kernel paragraph: the product of the two FP4 operands, here on CDNA4 FP4 matrix
 * cores with fp32 accumulation; granularity paragraph: sA and sW factor out of the K-sum;
 * outlier paragraph: the product of dA with the weights is added back).
 *   Aq M x K/2, sA fp32[M], Wq N x K/2, sW fp32[N] (as produced by fp4_quantize)
 *   row_ptr, coo_col, coo_val: dA as produced by fp4_outlier_clamp (CSR row offsets and
 *            the column/value lists sorted by (row, col)), or all three NULL for no
 *            compensation term; W (K x N, w_dtype) is then unused and may be NULL.
 *   capacity the number of entries the dA lists were sized for (fp4_outlier_capacity),
 *            or 0 if unknown; it only picks the shape of the compensation kernel.
 *   Y        M x N of y_dtype (out); FP4_Q16 (int16 elements) only without dA
 *   acc_out  NULL, or device fp32[M*N] receiving the raw accumulator acc (a check aid).
 *   workspace, ws_bytes: device scratch of at least fp4_gemm_workspace_bytes() bytes
 *            (may be NULL when that is 0).  With dA the GEMM hands its accumulator to the
 *            compensation pass as FP4_Q16 elements (in Y for a bf16 Y, in the workspace for
 *            an fp32 Y) with the map of escaped blocks in the workspace; the pass rebuilds
 *            Y_main = fl(fl(acc*sA)*sW) bit for bit from them, and the escaped blocks are
 *            recomputed from the codes and written with the same arithmetic.
 * Kernels run on the stream in order: the GEMM; then, for FP4_Q16, the escape kernel; with
 * dA, the compensation pass and the escape kernel.
 * Returns FP4_OK or FP4_ERR_{NULL,SHAPE,DTYPE,WORKSPACE,ALIGN,DEVICE,HIP}. */
fp4_status fp4_gemm(const uint8_t *Aq, const float *sA, const uint8_t *Wq, const float *sW,
                    int64_t M, int64_t N, int64_t K, const int32_t *row_ptr,
                    const int32_t *coo_col, const float *coo_val, int64_t capacity, const void *W,
                    int32_t w_dtype, void *Y, int32_t y_dtype, float *acc_out, void *workspace,
                    size_t ws_bytes, void *stream);

/* FP8 (E4M3) gradient codec: the single-GPU quantize/dequantize half of the FP8 gradient
 * communication that the QbitAI report and the paper abstract pair with FP4 training (the
 * pages give no scaling rule).  Readings: one per-tensor scale from amax = max |x|,
 * multiplier r = fl(448 / amax), dequantization scale s = fl(amax / 448) (both 0 when
 * amax < 2^-120); code = E4M3(fl(x * r)), nearest with ties to the even mantissa,
 * saturating at 448 (never NaN), sign kept; dequantization fl(value(code) * s).
 *   fp4_fp8_quantize:   X n elements of x_dtype (in); codes u8[n] (out); scale device
 *                       fp32[1] (out, s); workspace >= fp4_fp8_workspace_bytes() bytes.
 *   fp4_fp8_dequantize: codes u8[n] and scale fp32[1] (in); Y n elements of y_dtype
 *                       (out; bf16 = round-to-nearest-even of the fp32 value).
 * 1 <= n <= 2^40; X, codes, Y and workspace 16-byte aligned.
 * Return FP4_OK or FP4_ERR_{NULL,SHAPE,DTYPE,WORKSPACE,ALIGN,DEVICE,HIP}. */
size_t fp4_fp8_workspace_bytes(void);
fp4_status fp4_fp8_quantize(const void *X, int32_t x_dtype, int64_t n, uint8_t *codes, float *scale,
                            void *workspace, size_t ws_bytes, void *stream);
fp4_status fp4_fp8_dequantize(const uint8_t *codes, int64_t n, const float *scale, void *Y,
                              int32_t y_dtype, void *stream);

/* FP4-on-FP8 emulation of the product (the pages' own execution mode: the QbitAI report's
 * format paragraph and the topaibox summary's simulation section hold FP4 values in FP8 and
 * multiply them on FP8 matrix cores).  Aq and Wq (as for fp4_gemm) are expanded to E4M3
 * bytes, which represent every E2M1 value exactly, into the workspace (M*K + N*K bytes,
 * fp4_gemm_fp8emu_workspace_bytes), then multiplied on the E4M3 MFMA with fp32
 * accumulation.  acc and Y are bit-identical to fp4_gemm without a compensation term; the
 * matrix cores run at half the FP4 rate on twice the operand bytes.  Needs M*K and N*K
 * below 2^31 besides fp4_gemm's limits.
 * Returns FP4_OK or FP4_ERR_{NULL,SHAPE,DTYPE,WORKSPACE,ALIGN,DEVICE,HIP}. */
size_t fp4_gemm_fp8emu_workspace_bytes(int64_t M, int64_t N, int64_t K);
fp4_status fp4_gemm_fp8emu(const uint8_t *Aq, const float *sA, const uint8_t *Wq, const float *sW,
                           int64_t M, int64_t N, int64_t K, void *Y, int32_t y_dtype,
                           float *acc_out, void *workspace, size_t ws_bytes, void *stream);

/* Byte offsets of the intermediates inside the fp4_linear_forward workspace, so a caller
 * can read T, the COO list, the codes and the scales after a forward. */
struct fp4_ws_layout {
    size_t total;                 /* bytes needed */
    size_t T;                     /* fp32[1] */
    size_t nnz;                   /* int64[1] */
    size_t row_ptr;               /* int32[M+1] */
    size_t coo_row, coo_col, coo_val; /* capacity entries each */
    size_t Aq, sA, Wq, sW;        /* codes and scales */
    size_t handoff;               /* the GEMM's hand-over to the compensation pass (the int16
                                     accumulators for an fp32 Y, nothing for a bf16 Y, which
                                     holds them itself; see FP4_Q16) and the map of escaped
                                     blocks.  It is the last region of the workspace: every
                                     other offset is the same for both Y types. */
    size_t scratch;               /* internal */
    int64_t capacity;             /* fp4_outlier_capacity(M, K, q) */
};

/* Host-only: workspace layout / size of fp4_linear_forward for Y of y_dtype (returns FP4_OK
 * or an argument error; size 0 on error). */
fp4_status fp4_forward_layout(int64_t M, int64_t K, int64_t N, int32_t in_dtype, int32_t y_dtype, double q,
                              struct fp4_ws_layout *out);
size_t fp4_forward_workspace_bytes(int64_t M, int64_t K, int64_t N, int32_t in_dtype, int32_t y_dtype,
                                   double q);

/* The whole forward of one FP4 linear layer (QbitAI report, forward-quantization and
 * outlier paragraphs): quantile and clamp of A with dA, token-wise quantization of
 * A_clamped, channel-wise quantization of W, FP4 GEMM, dequantization, compensation.
 *   A  M x K, W  K x N, both of in_dtype; Y  M x N of y_dtype (out)
 *   workspace: at least fp4_forward_workspace_bytes(..., y_dtype, q) bytes (layout:
 *            fp4_forward_layout).
 * Returns FP4_OK or FP4_ERR_{NULL,SHAPE,DTYPE,QUANTILE,WORKSPACE,ALIGN,DEVICE,HIP}. */
fp4_status fp4_linear_forward(const void *A, const void *W, int32_t in_dtype, int64_t M,
                              int64_t K, int64_t N, double q, void *Y, int32_t y_dtype,
                              void *workspace, size_t ws_bytes, void *stream);

/* The forward in two stage calls, for callers that time or schedule the stages apart:
 * fp4_linear_forward(A, W, ...) enqueues exactly fp4_forward_quantize(A, W, ..., FP4_STAGE_A |
 * FP4_STAGE_W, ...) followed by fp4_forward_product(W, ...) on the same workspace.
 * fp4_forward_quantize: the quantizer stages, results in the workspace at the fp4_forward_layout
 *   offsets.  stages is a mask: FP4_STAGE_A = quantile, clamp and dA of A (T, nnz, row_ptr, the
 *   COO list) and the token-wise codes and scales of A_clamped (QbitAI report, outlier,
 *   granularity and forward-quantization paragraphs); FP4_STAGE_W = the channel-wise codes and
 *   scales of W (granularity paragraph).  A (resp. W) may be NULL when its stage is not asked
 *   for.  Asked for together (as the forward does), W's two passes share launches with the A
 *   side's select and COO build; the W stage alone takes three launches of its own.
 *   It uses the workspace up to the layout's handoff offset, which is the same for both Y
 *   types, and needs at least that many bytes.
 * fp4_forward_product: the FP4 GEMM with dequantization and the compensation dA . W (GEMM-kernel
 *   and outlier paragraphs) from the workspace's intermediates (both stages must have run on it
 *   for the same A, W, q) into Y (M x N of y_dtype); W is the original weight.
 * Returns FP4_OK or FP4_ERR_{NULL,SHAPE,DTYPE (also: unknown stage bits),QUANTILE,WORKSPACE,
 * ALIGN,DEVICE,HIP}. */
enum { FP4_STAGE_A = 1, FP4_STAGE_W = 2 };
fp4_status fp4_forward_quantize(const void *A, const void *W, int32_t in_dtype, int64_t M, int64_t K, int64_t N,
                                double q, int32_t stages, void *workspace, size_t ws_bytes, void *stream);
fp4_status fp4_forward_product(const void *W, int32_t in_dtype, int64_t M, int64_t K, int64_t N, double q, void *Y,
                               int32_t y_dtype, void *workspace, size_t ws_bytes, void *stream);

/* The same forward with W already quantized: Wq and sW as fp4_quantize(W, FP4_PER_COL)
 * produced them (N x K/2 codes, fp32[N] scales) while W is unchanged, as when the weights
 * of an inference layer are fixed.  The QbitAI report quantizes W at every forward
 * (forward-quantization paragraph); the codes depend on W alone, so reusing them gives
 * bit-identical results and skips the per-channel pass.  W itself is still read for the
 * compensation term.  Workspace and layout as for fp4_linear_forward (its Wq and sW regions
 * are left untouched).
 * Returns FP4_OK or FP4_ERR_{NULL,SHAPE,DTYPE,QUANTILE,WORKSPACE,ALIGN,DEVICE,HIP}. */
fp4_status fp4_linear_forward_wq(const void *A, const void *W, const uint8_t *Wq, const float *sW,
                                 int32_t in_dtype, int64_t M, int64_t K, int64_t N, double q,
                                 void *Y, int32_t y_dtype, void *workspace, size_t ws_bytes,
                                 void *stream);

/* Straight-through backward of the quantized product (QbitAI report, backward paragraph:
 * the hard quantizer is kept in the forward and its derivative is replaced in the
 * backward; the pages' smooth substitute is not given, so the derivative is taken as one).
 * With deq(Aq)[m][k] = value(Aq[m][k]) * sA[m] and deq(Wq)[k][n] = value(Wq[n][k]) * sW[n]
 * (the operands the forward multiplied):
 *      dA = dY . deq(Wq)^T  (M x K)        dW = deq(Aq)^T . dY  (K x N)
 * Both run on the FP4 GEMM, with the quantization axes transposed against the forward's:
 *   - G = fl32(dY[m][n] * sW[n]) is quantized per row (Gq M x N/2, sG fp32[M]) and the
 *     forward's Wq is transposed to WqT (K x N/2); dA[m][k] = fl32(acc * sG[m]) with acc the
 *     exact sum over n of value(Gq[m][n]) * value(WqT[k][n]);
 *   - H = fl32(sA[m] * dY[m][n]) is quantized per column (Hq N x M/2, sH fp32[N]) and Aq is
 *     transposed to AqT (K x M/2); dW[k][n] = fl32(acc * sH[n]) with acc the exact sum over
 *     m of value(AqT[k][m]) * value(Hq[n][m]).
 * Quantization follows the forward's rule (fl32(6/amax) multiplier, nearest E2M1 with ties
 * to even, saturation, zero vectors).  The clamp and the compensation of the forward add no
 * term.  Arguments:
 *   dY  M x N of dy_dtype (the gradient of Y)
 *   Aq, sA, Wq, sW: the forward's codes and scales (fp4_forward_layout regions of the
 *       forward workspace, or fp4_quantize's outputs); Aq/sA are needed only for dW and
 *       Wq/sW only for dA
 *   dA  NULL (not wanted) or M x K of da_dtype (out); needs N % 32 == 0, N <= 65536
 *   dW  NULL (not wanted) or K x N of dw_dtype (out); needs M % 32 == 0, M <= 65536
 *   workspace: at least fp4_backward_workspace_bytes(M, K, N) bytes; after the call it
 *       holds the intermediates at the fp4_backward_layout offsets (Gq, sG, WqT when dA
 *       was asked for; Hq, sH, AqT when dW was).
 * Kernels, in stream order: fill, [row quantization of G, transpose of Wq, GEMM],
 * [column quantization of H, transpose of Aq, GEMM]; for both products of a bf16 dY with
 * N <= 24576 the row quantization of G also collects H's column maxima (dY read once less).
 * Returns FP4_OK or FP4_ERR_{NULL,SHAPE,DTYPE,WORKSPACE,ALIGN,DEVICE,HIP}. */
struct fp4_bwd_layout {
    size_t total;        /* bytes needed */
    size_t Gq, sG;       /* M x N/2 codes, fp32[M] */
    size_t Hq, sH;       /* N x M/2 codes, fp32[N] */
    size_t WqT, AqT;     /* K x N/2 and K x M/2 codes */
    size_t ones;         /* fp32[K], internal */
    size_t part;         /* 512 x N column-maximum keys, internal */
};
fp4_status fp4_backward_layout(int64_t M, int64_t K, int64_t N, struct fp4_bwd_layout *out);
size_t fp4_backward_workspace_bytes(int64_t M, int64_t K, int64_t N);
fp4_status fp4_linear_backward(const void *dY, int32_t dy_dtype, int64_t M, int64_t K, int64_t N,
                               const uint8_t *Aq, const float *sA, const uint8_t *Wq,
                               const float *sW, void *dA, int32_t da_dtype, void *dW,
                               int32_t dw_dtype, void *workspace, size_t ws_bytes, void *stream);

/* Host-only: the kernel selection, the same rule the launches use, so a caller (a profiler
 * summary, a benchmark) can name what runs.  fp4_gemm_kernel_name: the FP4 GEMM kernel that
 * fp4_gemm and fp4_linear_forward launch for an M x N x K product on a device with num_cus
 * compute units ("k_fp4_gemm_wide": persistent 256 x 256 tiles, chosen when K % 512 == 0 and
 * there are at least two such tiles per CU; else "k_fp4_gemm": 256 x 128 tiles).
 * fp4_comp_kernel_name: the compensation kernel for M rows and a dA list of `capacity`
 * entries (fp4_outlier_capacity; the forward uses that bound) ("k_comp_block64" above 64
 * entries per row on average, else "k_comp_apply").  Both return a static string, or NULL
 * for invalid arguments (num_cus < 1, sizes out of range). */
const char *fp4_gemm_kernel_name(int64_t M, int64_t N, int64_t K, int32_t num_cus);
const char *fp4_comp_kernel_name(int64_t M, int64_t capacity);

/* Static description of a status code (never NULL). */
const char *fp4_status_string(fp4_status s);

#ifdef __cplusplus
}
#endif
#endif /* FP4LIN_H */
