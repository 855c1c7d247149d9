// Host-side pieces of the outlier pass shared by the C ABI (abi.cpp) and the no-allocation
// entry point (noalloc.hip).  Internal header: not part of the C ABI (include/fp4lin.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "fp4lin.h"

namespace fp4 {

struct WSide;  // fp4_launch.h

// The current device must be gfx950; *cus receives its compute-unit count (cached per device).
fp4_status device_check(int *cus);

fp4_status hip_status(hipError_t e);

// Scratch of one outlier pass, byte offsets from its base.  [state, zero_end) is zero-filled at
// the start of every pass (one fill kernel, no memset); the rest is written before it is read.
struct OutlierWs {
    size_t state, hist, hist_lo, zero_end, rowmax, row_cnt, slots, total;
    int32_t S;  // staging slots per row
};
OutlierWs outlier_ws(int64_t M, int64_t K, int32_t dtype, int64_t cap);

// M*K - 1 - floor(q * (M*K - 1)), for arguments that passed the checks.
int64_t outlier_capacity_of(int64_t M, int64_t K, double q);

// The argument checks of fp4_outlier_clamp other than the workspace's (pointers, dtype, shape,
// quantile, capacity, alignment); no HIP call.
fp4_status outlier_args_check(const void *A, int32_t a_dtype, int64_t M, int64_t K, double q, const float *T,
                              const int32_t *coo_row, const int32_t *coo_col, const float *coo_val, int64_t capacity,
                              const int32_t *row_ptr, const int64_t *nnz);

// fp4_outlier_clamp on a given scratch (the caller's workspace, or a fixed device array).
fp4_status outlier_clamp_impl(const void *A, int32_t a_dtype, int64_t M, int64_t K, double q, float *T,
                              int32_t *coo_row, int32_t *coo_col, float *coo_val, int64_t capacity, int32_t *row_ptr,
                              int64_t *nnz, void *workspace, size_t ws_bytes, void *stream);

// Enqueue the outlier pass on scratch ws (layout w).  Aq/sA: NULL, or A_clamped's codes and
// scales written in the same pass.  wside: NULL, or W's quantization, done in the pass's
// launches (its keys zeroed in the zero fill, its two passes beside the select and the COO build).
fp4_status run_outliers(const void *A, int32_t dtype, int64_t M, int64_t K, double q, uint8_t *ws,
                        const OutlierWs &w, int cus, float *T, int32_t *coo_row, int32_t *coo_col,
                        float *coo_val, int64_t cap, int32_t *row_ptr, int64_t *nnz, uint8_t *Aq,
                        float *sA, const WSide *wside, hipStream_t s);

}  // namespace fp4
