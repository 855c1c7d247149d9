// fp4_outlier_clamp_noalloc (include/fp4lin.h): the outlier pass of fp4_outlier_clamp on a
// fixed scratch array that the library holds in device memory, for callers that cannot
// allocate (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc).  Same kernels, same results; nothing is allocated, freed or memset.
#include <hip/hip_runtime.h>

#include <mutex>

#include "fp4_host.h"
#include "fp4lin.h"

namespace {

// The scratch: one array per GPU the library runs on, held until the process ends.  In host
// code this name is only a host-side stand-in; its device address is looked up per device with
// hipGetSymbolAddress and only that address is handed to kernels.
constexpr size_t SCRATCH_BYTES = (size_t)FP4_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_mu;
void *g_ptr[MAX_DEVICES];  // device address of `scratch` on each device, once looked up

// The current device's scratch address (looked up on the first call on that device, with that
// device current), or NULL if the lookup failed.
void *scratch_ptr() {
    int d = 0;
    if (hipGetDevice(&d) != hipSuccess || d < 0 || d >= MAX_DEVICES) return nullptr;
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_ptr[d]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        g_ptr[d] = p;
    }
    return g_ptr[d];
}

}  // namespace

extern "C" fp4_status fp4_outlier_clamp_noalloc(const void *A, int32_t a_dtype, int64_t M, int64_t K, double q,
                                                float *T, int32_t *coo_row, int32_t *coo_col, float *coo_val,
                                                int64_t capacity, int32_t *row_ptr, int64_t *nnz, void *stream) {
    fp4_status st = fp4::outlier_args_check(A, a_dtype, M, K, q, T, coo_row, coo_col, coo_val, capacity, row_ptr, nnz);
    if (st != FP4_OK) return st;
    const fp4::OutlierWs w = fp4::outlier_ws(M, K, a_dtype, fp4::outlier_capacity_of(M, K, q));
    if (w.total > SCRATCH_BYTES) return FP4_ERR_SCRATCH;
    int cus;
    st = fp4::device_check(&cus);
    if (st != FP4_OK) return st;
    void *ws = scratch_ptr();
    if (!ws) return FP4_ERR_HIP;
    return fp4::outlier_clamp_impl(A, a_dtype, M, K, q, T, coo_row, coo_col, coo_val, capacity, row_ptr, nnz, ws,
                                   SCRATCH_BYTES, stream);
}
