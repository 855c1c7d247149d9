// Host-side launchers of the gfx950 kernels (internal; the C ABI is include/fp4lin.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp4_common.h"

namespace fp4 {

// Zeroes p1[0..n1) and p2[0..n2) in one launch (n2 may be 0).
hipError_t launch_zero(uint32_t *p1, int64_t n1, uint32_t *p2, int64_t n2, hipStream_t s);
// The W side of the forward's quantizer when it shares launches with the A side: K x N W (the
// A side's dtype), its column-maximum keys (zeroed before), codes (N x K/2) and scales (N).
struct WSide {
    const void *W;
    int dt;
    int64_t K, N;
    uint32_t *keys;
    uint8_t *codes;
    float *scales;
};

// Histogram of the |A| keys and raw row maxima (ghist zero).
hipError_t launch_hist_rowmax(const void *A, int dt, int64_t M, int64_t K, uint32_t *ghist, uint32_t *rowmax_key,
                              int num_cus, hipStream_t s);
// Level 1 of the select: the bin of rank k (st zero); for bf16 inputs it fixes T.  w: NULL, or
// W's column maxima, computed in the same launch.
hipError_t launch_select_hi(const uint32_t *ghist, int dt, State *st, float *T_out, uint64_t k, const WSide *w,
                            hipStream_t s);
// Second level of the select for fp32 inputs (ghist_lo zero): fixes T.
hipError_t launch_select_lo(const void *A, int64_t n, uint32_t *ghist_lo, State *st, float *T_out, hipStream_t s);
hipError_t launch_quant_rows(const void *X, int dt, int64_t R, int64_t C, const uint32_t *rowmax_key,
                             const float *T_src, uint8_t *codes, float *scales, int32_t *row_cnt,
                             const Staging &stg, State *st, bool emit, bool write_codes, hipStream_t s);
// Exclusive scan of the row counts into row_ptr / nnz, then the staged entries (and, for rows
// that outgrew their slots, a second read of those rows of A) into the (row, col)-sorted list.
// w: NULL, or W's codes and scales from its finished column maxima, in the same launch.
hipError_t launch_coo(const int32_t *row_cnt, int64_t M, int32_t *row_ptr, int64_t *nnz_out, const Staging &stg,
                      int64_t cap, int32_t *coo_row, int32_t *coo_col, float *coo_val, const void *A, int dt,
                      int64_t K, const float *T_src, const WSide *w, hipStream_t s);
// keys_zeroed: the column-maximum keys (in scales_as_keys) were zeroed by an earlier launch.
// row_mult: NULL, or fp32[K]: quantize fl(row_mult[k] * W[k][n]) instead of W.
// scales_out: NULL (the scales replace the keys in scales_as_keys, one more launch), or a
// separate fp32[N] that the quantizing kernel fills itself.
hipError_t launch_quant_cols(const void *W, int dt, int64_t K, int64_t N, float *scales_as_keys,
                             uint8_t *codes, bool keys_zeroed, hipStream_t s, const float *row_mult = nullptr,
                             float *scales_out = nullptr);
// Backward operands: R x C codes (R x C/2 bytes) -> their transpose (C x R/2 bytes), R and C
// multiples of 32; token-wise quantization of fl(X[r][c] * mult[c]) (C <= 65536); fill.
hipError_t launch_codes_transpose(const uint8_t *in, int64_t R, int64_t C, uint8_t *out, hipStream_t s);
hipError_t launch_scaled_quant_rows(const void *X, int dt, int64_t R, int64_t C, const float *mult, uint8_t *codes,
                                    float *scales, hipStream_t s);
hipError_t launch_fill_f32(float *p, int64_t n, float v, hipStream_t s);
// One read of a bf16 X (M x C, C <= 24576): token-wise codes/scales of fl(X * mult[col]) and
// the column-maximum keys of |fl(row_mult[row] * X)| (per-workgroup partials in part, G x C
// keys, then reduced into keys[C]).  G workgroups, G <= M.
int fused_rows_cpt(int64_t C);
hipError_t launch_bwd_rows_fused(const void *X, int64_t M, int64_t C, const float *mult, const float *row_mult,
                                 uint8_t *codes, float *scales, uint32_t *part, int G, uint32_t *keys,
                                 hipStream_t s);
// The channel-wise quantization of fl(row_mult[k] * W[k][n]) with the column-maximum keys
// already in scales_as_keys (turned into scales at the end).
hipError_t launch_quant_cols_keyed(const void *W, int dt, int64_t K, int64_t N, float *scales_as_keys,
                                   uint8_t *codes, const float *row_mult, hipStream_t s);

// FP4 GEMM + dequantization: Y = fl(fl(acc * sA) * sW) in y_dt.  With y_dt == DT_Q16, Y
// receives the accumulator as int16 4*acc, and emap (esc_map_bytes(M, N) bytes) the map of
// the ESC_ROWS x ESC_COLS blocks where some |acc| > Q16_MAX_ACC left it out of range (every
// byte is written).
// acc_out: NULL or fp32[M*N].
// f8: Aq (M x K) and Wq (N x K) hold E4M3 bytes, one K value each (the emulation path).
hipError_t launch_gemm(const uint8_t *Aq, const float *sA, const uint8_t *Wq, const float *sW, int64_t M,
                       int64_t N, int64_t K, void *Y, int y_dt, float *acc_out, hipStream_t s, bool f8 = false,
                       uint8_t *emap = nullptr);
size_t esc_map_bytes(int64_t M, int64_t N);
// The escaped blocks of a DT_Q16 product (emap as launch_gemm wrote it), recomputed from the
// codes.  launch_escapes_q16: as the standalone two-byte output, fl(fl(acc*sA)*sW) into esc
// (fp32[M*N]) and Q16_ESC into their elements of Yq.  launch_escapes_comp: the final
// Y = Y_main + dA . W in y_dt for those blocks, with the compensation pass's arithmetic (the
// pass itself skips them).
hipError_t launch_escapes_q16(const uint8_t *Aq, const float *sA, const uint8_t *Wq, const float *sW, int64_t M,
                              int64_t N, int64_t K, const uint8_t *emap, int16_t *Yq, float *esc, hipStream_t s);
hipError_t launch_escapes_comp(const uint8_t *Aq, const float *sA, const uint8_t *Wq, const float *sW, int64_t M,
                               int64_t N, int64_t K, const uint8_t *emap, const int32_t *row_ptr,
                               const int32_t *coo_col, const float *coo_val, const void *W, int w_dt, void *Y,
                               int y_dt, hipStream_t s);
// The GEMM kernel launch_gemm picks for a shape on a device with `cus` compute units.
enum : int { GEMM_TILED = 0, GEMM_WIDE = 1 };
int gemm_kernel_choice(int64_t M, int64_t N, int64_t K, bool f8, int cus);
// FP8 (E4M3) gradient codec, one per-tensor scale.  key: device u32 scratch (zeroed here).
hipError_t launch_fp8_quantize(const void *X, int dt, int64_t n, uint32_t *key, uint8_t *codes, float *scale,
                               int num_cus, hipStream_t s);
hipError_t launch_fp8_dequantize(const uint8_t *codes, int64_t n, const float *scale, void *Y, int y_dt, int num_cus,
                                 hipStream_t s);
// E2M1 codes (two per byte, low nibble first) -> E4M3 bytes holding the same values, n_bytes
// input bytes -> 2 * n_bytes output bytes.
hipError_t launch_e2m1_to_e4m3(const uint8_t *codes, int64_t n_bytes, uint8_t *out, hipStream_t s);
// Y = Y_main + dA . W, accumulated in fp32 in ascending k from Y_main, rounded once to y_dt.
// Y_main comes from the GEMM's DT_Q16 output Yq and the scales sA, sW; the blocks that emap
// marks are left alone (launch_escapes_comp writes them).  Yq may be a bf16 Y itself.
// capacity: what the dA list was sized for (picks the kernel shape only; 0 if unknown).
// The compensation kernel launch_comp picks: chunk tasks up to 64 entries per row on average
// (capacity / M), 8-row blocks beyond.
enum : int { COMP_CHUNK = 0, COMP_BLOCK64 = 1 };
int comp_kernel_choice(int64_t M, int64_t capacity);
hipError_t launch_comp(const int16_t *Yq, const uint8_t *emap, const float *sA, const float *sW, void *Y, int y_dt,
                       int64_t M, int64_t N, int64_t K, const int32_t *row_ptr, const int32_t *coo_col,
                       const float *coo_val, const void *W, int w_dt, int64_t capacity, hipStream_t s);

}  // namespace fp4
