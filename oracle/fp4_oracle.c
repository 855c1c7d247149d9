/*
 * Reference oracle for the FP4 quantized linear-layer forward
 *      Y = dequant(Aq . Wq) + dA . W
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark load this library.  The product path (the HIP library under
 * quantized_linear_layers_fp4_amd/) never includes, links or calls anything here,
 * and nothing here includes or calls the product.
 *
 * Plain single-threaded C99, loops only, compiled with -O2 -ffp-contract=off and
 * without fast-math, so every float operation below is one IEEE-754 operation
 * rounded to nearest-even in the precision written.
 *
 * Sources (the method is described in prose only; no formula or listing exists):
 *   [QbitAI]   QbitAI news report on "Optimizing Large Language Model Training Using
 *              FP4 Quantization" (czzqal.com repost), paragraphs on the quantization
 *              format, quantization granularity, forward quantization and the
 *              outlier clamping and compensation strategy.
 *   [Abstract] "Optimizing Large Language Model Training Using FP4 Quantization",
 *              paper-summary page (shd-paper.top), original English abstract.
 *   [topaibox] German summary "Microsoft Research bringt den ersten FP4-Genauigkeits-
 *              rahmen ...", section on FP4 simulation and training methods.
 * Readings taken where the pages are silent are listed next to the code that takes them.
 *
 * Parity pins: every function here is checked by the CPU test-suite against values the
 * pages or mathematics fix (closed forms, brute force, library routines), see
 * tests/test_oracle_pins.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_F32 = 0, ORC_BF16 = 1 };

/* Element i of an fp32 or bf16 array, widened exactly to fp32. */
static float load_elem(const void *X, int dtype, int64_t i) {
    if (dtype == ORC_BF16) {
        uint32_t b = (uint32_t)((const uint16_t *)X)[i] << 16;
        float f;
        memcpy(&f, &b, 4);
        return f;
    }
    return ((const float *)X)[i];
}

/* ---------------------------------------------------------------------------------
 * E2M1: 1 sign bit, 2 exponent bits, 1 mantissa bit ([QbitAI], format paragraph).
 * With exponent bias 1 the eight magnitudes are the table below; the table index is
 * the 3-bit exponent|mantissa field, so a 4-bit code is (sign << 3) | index.
 * ------------------------------------------------------------------------------- */
static const double E2M1_MAG[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double orc_e2m1_value(int code) {
    double v = E2M1_MAG[code & 7];
    return (code & 8) ? -v : v;
}

/* ---------------------------------------------------------------------------------
 * E4M3 (FP8 with 1 sign bit, 4 exponent bits of bias 7, 3 mantissa bits): the type the
 * pages' framework holds FP4 values in to multiply them on FP8 tensor cores ([QbitAI],
 * format paragraph; [topaibox], simulation section).  Exponent field 0 holds the
 * subnormals m/8 * 2^-6; the pattern with every exponent and mantissa bit set is NaN
 * (the format has no infinities).
 * ------------------------------------------------------------------------------- */
double orc_e4m3_value(int b) {
    const int sign = (b >> 7) & 1, e = (b >> 3) & 15, m = b & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        v = ldexp((double)m / 8.0, -6);
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -v : v;
}

/* The E4M3 byte holding the value of E2M1 code `code`, sign included (so +0 -> 0x00 and
 * -0 -> 0x80), found by searching all 256 bytes; -1 if none (every E2M1 value is
 * representable, so that is never the answer). */
int orc_e2m1_to_e4m3(int code) {
    const double v = orc_e2m1_value(code);
    const int sign = (code >> 3) & 1;
    for (int b = 0; b < 256; ++b) {
        const double w = orc_e4m3_value(b);
        if (!isnan(w) && w == v && ((b >> 7) & 1) == sign) return b;
    }
    return -1;
}

/* Expand packed E2M1 codes (two per byte, low nibble = even index) to one E4M3 byte per
 * value, in index order: nbytes in, 2 * nbytes out. */
void orc_expand_e4m3(const uint8_t *packed, int64_t nbytes, uint8_t *out) {
    for (int64_t i = 0; i < nbytes; ++i) {
        out[2 * i] = (uint8_t)orc_e2m1_to_e4m3(packed[i] & 15);
        out[2 * i + 1] = (uint8_t)orc_e2m1_to_e4m3(packed[i] >> 4);
    }
}

/* ---------------------------------------------------------------------------------
 * FP8 gradient codec: the quantize/dequantize half of the pages' FP8 gradient
 * communication ([QbitAI] and [Abstract]: gradients are exchanged in FP8; the pages give
 * no scaling rule).
 * Readings, chosen to mirror the FP4 path: per-tensor absmax scaling, multiplier
 * r = fl(448 / amax) and dequantization scale s = fl(amax / 448) in fp32 (448 = the
 * largest finite E4M3 value), amax < 2^-120 gives r = s = 0; y = fl(g * r) is rounded to
 * the nearest E4M3 value with ties to the even mantissa, |y| > 448 saturates to 448 (no
 * NaN is ever produced), and the sign is copied (-0 -> 0x80).  Dequantization is
 * fl(value(code) * s).
 * ------------------------------------------------------------------------------- */
int orc_e4m3_encode(float y) {
    double u = fabs((double)y);
    if (u > 448.0) u = 448.0;
    int best = 0;
    double best_d = u;  /* distance to code 0 */
    for (int b = 1; b < 0x7F; ++b) {  /* the finite positive codes, ascending in value */
        const double d = fabs(u - orc_e4m3_value(b));
        if (d < best_d || (d == best_d && (b & 1) == 0)) {
            best = b;
            best_d = d;
        }
    }
    return (signbit(y) ? 0x80 : 0) | best;
}

void orc_e4m3_encode_array(const float *y, int64_t n, uint8_t *out) {
    for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)orc_e4m3_encode(y[i]);
}

/* codes[i] = E4M3(fl(x[i] * r)) for n elements of X (fp32 or bf16); *scale = s. */
void orc_fp8_quantize(const void *X, int dtype, int64_t n, uint8_t *codes, float *scale) {
    float amax = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        const float v = fabsf(load_elem(X, dtype, i));
        if (v > amax) amax = v;
    }
    float r = 0.0f, s = 0.0f;
    if ((double)amax >= 7.52316384526264e-37) { /* 2^-120 */
        r = 448.0f / amax;
        s = amax / 448.0f;
    }
    for (int64_t i = 0; i < n; ++i) codes[i] = (uint8_t)orc_e4m3_encode(load_elem(X, dtype, i) * r);
    *scale = s;
}

/* out[i] = fl(value(codes[i]) * s) in fp32. */
void orc_fp8_dequantize(const uint8_t *codes, int64_t n, float s, float *out) {
    for (int64_t i = 0; i < n; ++i) out[i] = (float)orc_e4m3_value(codes[i]) * s;
}

/* Round y to the nearest E2M1 value by looking it up in the table ([QbitAI], forward
 * quantization paragraph: nearest FP4 value by table lookup).
 * Reading: at equal distance the entry with mantissa bit 0 (even index) wins, which is
 * IEEE round-to-nearest-even on the E2M1 grid; magnitudes beyond 6 saturate to 6
 * (E2M1 has no infinity).  Distances are taken in double: for |y| <= 6 the distance
 * to either of the two neighbouring table entries is exact there. */
int orc_e2m1_encode(float y) {
    double u = fabs((double)y);
    if (u > 6.0) u = 6.0; /* saturate first: far beyond the table the distances round */
    int best = 0;
    double best_d = fabs(u - E2M1_MAG[0]);
    for (int i = 1; i < 8; ++i) {
        double d = fabs(u - E2M1_MAG[i]);
        if (d < best_d || (d == best_d && (i & 1) == 0)) {
            best = i;
            best_d = d;
        }
    }
    return (signbit(y) ? 8 : 0) | best;
}

/* Encode an array of floats (used by the codec pins). */
void orc_encode_array(const float *y, int64_t n, uint8_t *out) {
    for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)orc_e2m1_encode(y[i]);
}

/* Per-vector scale ([QbitAI], scale+shift calibration paragraph).
 * Reading: symmetric absmax scaling.  The scale factor 1/amax maps the vector into
 * [-1, 1] and the second factor 6 maps [-1, 1] onto the E2M1 range [-6, 6]; both are
 * folded into one multiplier r = fl(6 / amax), computed once per vector in fp32, and
 * the dequantization scale kept for the product is s = fl(amax / 6).
 * Reading: a vector whose amax is below 2^-120 (all zero, or tiny enough that 6/amax
 * would leave the normal fp32 range) gets r = 0 and s = 0. */
#define ORC_TINY_AMAX 7.52316384526264e-37 /* 2^-120 */

static void vector_scale(float amax, float *r, float *s) {
    if (!((double)amax >= ORC_TINY_AMAX)) {
        *r = 0.0f;
        *s = 0.0f;
    } else {
        *r = 6.0f / amax;
        *s = amax / 6.0f;
    }
}

/* Token-wise (per-row) quantization of an R x C fp32 matrix X ([QbitAI], granularity
 * paragraph: the activation matrix is quantized along tokens, i.e. one range per row).
 * codes: R x C/2 bytes, element (i, j) in byte (i, j/2), low nibble for even j. */
void orc_quant_rows(const float *X, int64_t R, int64_t C, uint8_t *codes, float *scales) {
    for (int64_t i = 0; i < R; ++i) {
        const float *x = X + i * C;
        float amax = 0.0f;
        for (int64_t j = 0; j < C; ++j) {
            float v = fabsf(x[j]);
            if (v > amax) amax = v;
        }
        float r, s;
        vector_scale(amax, &r, &s);
        scales[i] = s;
        for (int64_t j = 0; j < C; j += 2) {
            float y0 = x[j] * r;
            float y1 = x[j + 1] * r;
            codes[i * (C / 2) + j / 2] =
                (uint8_t)(orc_e2m1_encode(y0) | (orc_e2m1_encode(y1) << 4));
        }
    }
}

/* Channel-wise (per output column) quantization of a K x N weight matrix W
 * ([QbitAI], granularity paragraph: the weight matrix is quantized per channel).
 * W is not clamped.  codes: N x K/2 bytes (K-contiguous per output channel),
 * element (k, n) in byte (n, k/2), low nibble for even k. */
void orc_quant_cols(const void *W, int dtype, int64_t K, int64_t N, uint8_t *codes, float *scales) {
    float *amax = (float *)calloc((size_t)N, sizeof(float));
    float *r = (float *)malloc((size_t)N * sizeof(float));
    for (int64_t k = 0; k < K; ++k)
        for (int64_t n = 0; n < N; ++n) {
            float v = fabsf(load_elem(W, dtype, k * N + n));
            if (v > amax[n]) amax[n] = v;
        }
    for (int64_t n = 0; n < N; ++n) vector_scale(amax[n], &r[n], &scales[n]);
    for (int64_t i = 0; i < N * (K / 2); ++i) codes[i] = 0;
    for (int64_t k = 0; k < K; ++k)
        for (int64_t n = 0; n < N; ++n) {
            float y = load_elem(W, dtype, k * N + n) * r[n];
            int c = orc_e2m1_encode(y);
            codes[n * (K / 2) + k / 2] |= (uint8_t)(c << (4 * (k & 1)));
        }
    free(amax);
    free(r);
}

/* ---------------------------------------------------------------------------------
 * Outlier clamping and compensation ([QbitAI], outlier paragraph; [Abstract]).
 * Reading: "quantile search" is the lower order statistic of |A| over the whole
 * tensor: T = the (k+1)-th smallest |a| with k = floor(q * (n - 1)) computed in
 * IEEE double.  T is then an element of |A|.
 * ------------------------------------------------------------------------------- */
int64_t orc_quantile_index(int64_t n, double q) {
    return (int64_t)floor(q * (double)(n - 1));
}

static void swapf(float *a, float *b) {
    float t = *a;
    *a = *b;
    *b = t;
}

/* k-th smallest (0-based) of v[0..n-1] by Hoare-partition quickselect (Hoare 1961,
 * "FIND"); v is reordered. */
static float select_kth(float *v, int64_t n, int64_t k) {
    int64_t lo = 0, hi = n - 1;
    while (lo < hi) {
        float a = v[lo], b = v[lo + (hi - lo) / 2], c = v[hi];
        float pivot = (a < b) ? ((b < c) ? b : ((a < c) ? c : a)) : ((a < c) ? a : ((b < c) ? c : b));
        int64_t i = lo, j = hi;
        while (i <= j) {
            while (v[i] < pivot) ++i;
            while (v[j] > pivot) --j;
            if (i <= j) {
                swapf(&v[i], &v[j]);
                ++i;
                --j;
            }
        }
        /* v[lo..j] <= pivot, v[i..hi] >= pivot, v[j+1..i-1] == pivot */
        if (k <= j)
            hi = j;
        else if (k >= i)
            lo = i;
        else
            return v[k];
    }
    return v[k];
}

/* T over all n entries of A (fp32 or bf16). */
float orc_abs_quantile(const void *A, int dtype, int64_t n, double q) {
    float *v = (float *)malloc((size_t)n * sizeof(float));
    for (int64_t i = 0; i < n; ++i) v[i] = fabsf(load_elem(A, dtype, i));
    float T = select_kth(v, n, orc_quantile_index(n, q));
    free(v);
    return T;
}

/* Clamp A to [-T, T] (A_clamped) and emit the sparse compensation dA = A - A_clamped in
 * COO order (row, then column).  Reading: an outlier is |a| > T strictly, so entries
 * equal to T stay and dA is non-zero exactly where clamping happened.  Each kept value
 * is delta = fl(a - copysign(T, a)).  Ac (optional) receives A_clamped (M x K fp32).
 * Returns nnz; entries beyond cap are counted but not stored. */
int64_t orc_clamp_coo(const void *A, int dtype, int64_t M, int64_t K, float T, float *Ac,
                      int32_t *coo_row, int32_t *coo_col, float *coo_val, int64_t cap,
                      int32_t *row_ptr) {
    int64_t nnz = 0;
    for (int64_t i = 0; i < M; ++i) {
        if (row_ptr) row_ptr[i] = (int32_t)nnz;
        for (int64_t j = 0; j < K; ++j) {
            float a = load_elem(A, dtype, i * K + j);
            float ac = a;
            if (fabsf(a) > T) {
                ac = copysignf(T, a);
                if (nnz < cap) {
                    coo_row[nnz] = (int32_t)i;
                    coo_col[nnz] = (int32_t)j;
                    coo_val[nnz] = a - ac;
                }
                ++nnz;
            }
            if (Ac) Ac[i * K + j] = ac;
        }
    }
    if (row_ptr) row_ptr[M] = (int32_t)nnz;
    return nnz;
}

/* ---------------------------------------------------------------------------------
 * The product of the quantized operands.  Reading: the raw accumulator is exact:
 * with a = 2 * value(codeA) and w = 2 * value(codeW) (integers in {0, +-1, .., +-12})
 * the sum S = sum_k a*w is formed in int64 and acc = S / 4 in fp32, exact because
 * |S| <= 144 K < 2^24 for K <= 65536.
 * ------------------------------------------------------------------------------- */
static const int TWICE_MAG[8] = {0, 1, 2, 3, 4, 6, 8, 12};

static int twice_value(uint8_t byte, int64_t k) {
    int c = (byte >> (4 * (k & 1))) & 15;
    int v = TWICE_MAG[c & 7];
    return (c & 8) ? -v : v;
}

static float acc_one(const uint8_t *Aq, const uint8_t *Wq, int64_t K, int64_t m, int64_t n) {
    const uint8_t *a = Aq + m * (K / 2);
    const uint8_t *w = Wq + n * (K / 2);
    int64_t S = 0;
    for (int64_t k = 0; k < K; ++k) S += (int64_t)twice_value(a[k / 2], k) * twice_value(w[k / 2], k);
    return (float)S / 4.0f;
}

void orc_accumulate(const uint8_t *Aq, const uint8_t *Wq, int64_t M, int64_t N, int64_t K, float *acc) {
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) acc[m * N + n] = acc_one(Aq, Wq, K, m, n);
}

void orc_accumulate_pairs(const uint8_t *Aq, const uint8_t *Wq, int64_t K, const int64_t *ms,
                          const int64_t *ns, int64_t count, float *acc) {
    for (int64_t i = 0; i < count; ++i) acc[i] = acc_one(Aq, Wq, K, ms[i], ns[i]);
}

/* Dequantization of the product: Y_main = fl(fl(acc * sA[m]) * sW[n]).  The per-row and
 * per-column scales factor out of the K-sum because the granularity matches the GEMM's
 * row-by-column structure ([QbitAI], granularity paragraph). */
static float dequant_one(float acc, float sa, float sw) {
    float t = acc * sa;
    return t * sw;
}

/* Compensation: Y = fl32(Y_main + sum over the row's dA entries (ascending column k) of
 * delta * W[k][n]), the sum formed in double.  W is the original (unquantized) weight.
 * denom (optional) receives |Y_main| + sum |delta * W[k][n]|, the scale of the
 * forward error of any summation order. */
static float compensate_one(float ymain, int64_t m, int64_t n, int64_t N, const int32_t *row_ptr,
                            const int32_t *coo_col, const float *coo_val, const void *W, int dtype,
                            double *denom) {
    double d = 0.0, s = fabs((double)ymain);
    if (row_ptr)
        for (int64_t e = row_ptr[m]; e < row_ptr[m + 1]; ++e) {
            double t = (double)coo_val[e] * (double)load_elem(W, dtype, (int64_t)coo_col[e] * N + n);
            d += t;
            s += fabs(t);
        }
    if (denom) *denom = s;
    return (float)((double)ymain + d);
}

void orc_output(const float *acc, const float *sA, const float *sW, int64_t M, int64_t N,
                const int32_t *row_ptr, const int32_t *coo_col, const float *coo_val, const void *W,
                int dtype, float *Y, double *denom) {
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            float ym = dequant_one(acc[m * N + n], sA[m], sW[n]);
            Y[m * N + n] = compensate_one(ym, m, n, N, row_ptr, coo_col, coo_val, W, dtype,
                                          denom ? &denom[m * N + n] : NULL);
        }
}

void orc_output_pairs(const float *acc, const float *sA, const float *sW, int64_t N,
                      const int64_t *ms, const int64_t *ns, int64_t count, const int32_t *row_ptr,
                      const int32_t *coo_col, const float *coo_val, const void *W, int dtype,
                      float *Y, double *denom) {
    for (int64_t i = 0; i < count; ++i) {
        float ym = dequant_one(acc[i], sA[ms[i]], sW[ns[i]]);
        Y[i] = compensate_one(ym, ms[i], ns[i], N, row_ptr, coo_col, coo_val, W, dtype,
                              denom ? &denom[i] : NULL);
    }
}

/* fp32 -> bf16, round to nearest even (finite inputs). */
void orc_to_bf16(const float *x, int64_t n, uint16_t *out) {
    for (int64_t i = 0; i < n; ++i) {
        uint32_t b;
        memcpy(&b, &x[i], 4);
        uint32_t lsb = (b >> 16) & 1u;
        b += 0x7FFFu + lsb;
        out[i] = (uint16_t)(b >> 16);
    }
}

/* ---------------------------------------------------------------------------------
 * The whole forward, step by step in the pages' order: quantile, clamp and dA, then
 * token-wise quantization of A_clamped, channel-wise quantization of W, the product
 * of the quantized operands, dequantization and the compensation.
 * Returns nnz, or -1 when cap is too small (outputs then incomplete).
 * ------------------------------------------------------------------------------- */
int64_t orc_forward(const void *A, const void *W, int dtype, int64_t M, int64_t K, int64_t N,
                    double q, float *T_out, int32_t *coo_row, int32_t *coo_col, float *coo_val,
                    int64_t cap, int32_t *row_ptr, uint8_t *Aq, float *sA, uint8_t *Wq, float *sW,
                    float *acc, float *Y, double *denom) {
    float T = orc_abs_quantile(A, dtype, M * K, q);
    *T_out = T;
    float *Ac = (float *)malloc((size_t)(M * K) * sizeof(float));
    int64_t nnz = orc_clamp_coo(A, dtype, M, K, T, Ac, coo_row, coo_col, coo_val, cap, row_ptr);
    if (nnz > cap) {
        free(Ac);
        return -1;
    }
    orc_quant_rows(Ac, M, K, Aq, sA);
    free(Ac);
    orc_quant_cols(W, dtype, K, N, Wq, sW);
    orc_accumulate(Aq, Wq, M, N, K, acc);
    orc_output(acc, sA, sW, M, N, row_ptr, coo_col, coo_val, W, dtype, Y, denom);
    return nnz;
}

/* ---------------------------------------------------------------------------------
 * Backward of the layer with a straight-through gradient.
 *
 * The pages: in the backward pass the derivative of the hard quantizer is zero almost
 * everywhere, and the authors replace it with the derivative of a smooth fit of the
 * quantizer (their differentiable gradient estimator) ([QbitAI], backward paragraph;
 * [Abstract]).  The pages do not give that function, so the correction is left out and
 * the quantizer's derivative is taken as one (straight-through): the gradients of
 * Y = deq(Aq) . deq(Wq) are
 *      dA = dY . deq(Wq)^T          dW = deq(Aq)^T . dY
 * with deq(Aq)[m][k] = value(Aq[m][k]) * sA[m] and deq(Wq)[k][n] = value(Wq[n][k]) * sW[n],
 * the operands the forward multiplied.
 *
 * Readings, so both products run on FP4 operands like the forward's:
 *   - the scale that lies along the contraction (sW[n] for dA, sA[m] for dW) is folded
 *     into dY in fp32: G[m][n] = fl(dY[m][n] * sW[n]), H[m][n] = fl(sA[m] * dY[m][n]);
 *   - G is quantized per row (token-wise, along n) and H per column (channel-wise, along
 *     m) with the forward's rule (scale, rounding, saturation, zero vectors): the
 *     quantization axes of the backward are the transposes of the forward's;
 *   - the forward's codes are reused unchanged, re-laid out so that the new contraction
 *     index is contiguous: WqT is K x N/2 and AqT is K x M/2;
 *   - acc is exact as in the forward (contraction length <= 65536) and each output is
 *     one rounding: dA[m][k] = fl(acc_A[m][k] * sG[m]), dW[k][n] = fl(acc_W[k][n] * sH[n]).
 * The clamp and the compensation of the forward contribute no term (the gradient is
 * taken through the quantized product only).
 * ------------------------------------------------------------------------------- */

/* R x C codes (R x C/2 bytes, element (r, c) in byte (r, c/2)) -> the same codes
 * transposed: C x R/2 bytes, element (r, c) in byte (c, r/2); low nibble = even index. */
void orc_transpose_codes(const uint8_t *in, int64_t R, int64_t C, uint8_t *out) {
    for (int64_t i = 0; i < C * (R / 2); ++i) out[i] = 0;
    for (int64_t r = 0; r < R; ++r)
        for (int64_t c = 0; c < C; ++c) {
            const int code = (in[r * (C / 2) + c / 2] >> (4 * (c & 1))) & 15;
            out[c * (R / 2) + r / 2] |= (uint8_t)(code << (4 * (r & 1)));
        }
}

/* Token-wise quantization of G = fl(X[i][j] * col_mult[j]) (R x C, X fp32 or bf16). */
void orc_scaled_quant_rows(const void *X, int dtype, int64_t R, int64_t C, const float *col_mult,
                           uint8_t *codes, float *scales) {
    float *G = (float *)malloc((size_t)(R * C) * sizeof(float));
    for (int64_t i = 0; i < R; ++i)
        for (int64_t j = 0; j < C; ++j) G[i * C + j] = load_elem(X, dtype, i * C + j) * col_mult[j];
    orc_quant_rows(G, R, C, codes, scales);
    free(G);
}

/* Channel-wise quantization of H = fl(row_mult[i] * X[i][j]) (R x C): codes C x R/2. */
void orc_scaled_quant_cols(const void *X, int dtype, int64_t R, int64_t C, const float *row_mult,
                           uint8_t *codes, float *scales) {
    float *H = (float *)malloc((size_t)(R * C) * sizeof(float));
    for (int64_t i = 0; i < R; ++i)
        for (int64_t j = 0; j < C; ++j) H[i * C + j] = row_mult[i] * load_elem(X, dtype, i * C + j);
    orc_quant_cols(H, ORC_F32, R, C, codes, scales);
    free(H);
}

/* out[i] = fl(acc[i] * s[idx[i]]): the one rounding of a backward output. */
static float scale_one(float acc, float s) { return acc * s; }

void orc_scale_pairs(const float *acc, const float *s, const int64_t *idx, int64_t count, float *out) {
    for (int64_t i = 0; i < count; ++i) out[i] = scale_one(acc[i], s[idx[i]]);
}

/* The whole backward, in the order above.  dY is M x N (fp32 or bf16); Aq, sA, Wq, sW as
 * the forward produced them.  Outputs: Gq M x N/2, sG[M], Hq N x M/2, sH[N], WqT K x N/2,
 * AqT K x M/2, dA M x K and dW K x N (fp32). */
void orc_backward(const void *dY, int dtype, int64_t M, int64_t K, int64_t N, const uint8_t *Aq,
                  const float *sA, const uint8_t *Wq, const float *sW, uint8_t *Gq, float *sG,
                  uint8_t *Hq, float *sH, uint8_t *WqT, uint8_t *AqT, float *dA, float *dW) {
    /* dA = dY . deq(Wq)^T: contraction over n */
    orc_scaled_quant_rows(dY, dtype, M, N, sW, Gq, sG);
    orc_transpose_codes(Wq, N, K, WqT);
    orc_accumulate(Gq, WqT, M, K, N, dA);
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k) dA[m * K + k] = scale_one(dA[m * K + k], sG[m]);
    /* dW = deq(Aq)^T . dY: contraction over m */
    orc_scaled_quant_cols(dY, dtype, M, N, sA, Hq, sH);
    orc_transpose_codes(Aq, M, K, AqT);
    orc_accumulate(AqT, Hq, K, N, M, dW);
    for (int64_t k = 0; k < K; ++k)
        for (int64_t n = 0; n < N; ++n) dW[k * N + n] = scale_one(dW[k * N + n], sH[n]);
}
