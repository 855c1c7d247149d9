// C ABI of the FP4 linear forward (declared in include/fp4lin.h): host-side argument
// validation, workspace carving and stream-ordered kernel launches.  Every check runs
// before the first HIP call; the library never allocates or synchronizes.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>

#include "fp4_host.h"
#include "fp4_launch.h"
#include "fp4lin.h"

using namespace fp4;

// Element limit of the FP8 codec (its chunk indices stay far from int64 overflow).
constexpr int64_t FP8_MAX_N = (int64_t)1 << 40;

namespace {

constexpr int64_t K_MAX = 65536;
constexpr size_t ALIGN = 256;

size_t align_up(size_t x) { return (x + ALIGN - 1) & ~(ALIGN - 1); }
bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool dtype_ok(int32_t d) { return d == FP4_F32 || d == FP4_BF16; }
bool q_ok(double q) { return q >= 0.0 && q <= 1.0; }  // false for NaN
int dt_of(int32_t d) { return d == FP4_BF16 ? DT_BF16 : DT_F32; }

bool k_ok(int64_t K) { return K >= 32 && K <= K_MAX && K % 32 == 0; }
bool mk_ok(int64_t M, int64_t K) { return M >= 1 && k_ok(K) && M <= (int64_t)0xFFFFFFFF / K; }
bool n_ok(int64_t N) { return N >= 1 && N % 8 == 0 && N <= (int64_t)1 << 30; }
// Shapes of the product: Wq (N x K/2) is addressed like Aq, and the compensation gathers
// rows of the original W (K x N) with 32-bit byte offsets.
bool gemm_ok(int64_t M, int64_t N, int64_t K) { return mk_ok(M, K) && n_ok(N) && mk_ok(N, K); }
bool wcomp_ok(int64_t N, int64_t K, int32_t w_dtype) {
    return K * N * (w_dtype == FP4_BF16 ? 2 : 4) <= (int64_t)0x7FFFFFFF;
}
// Where the GEMM's two-byte accumulators and its map of escaped blocks go.  On the way to a
// compensated Y (comp): into a bf16 Y itself, or into the workspace (M*N*2 bytes) for an fp32
// Y; the escaped blocks are then written by the escape kernel, so no fp32 values are kept.
// As the standalone FP4_Q16 output: into Y, with the fp32 escape buffer (M*N*4 bytes) in the
// workspace.  The map follows in the workspace.
size_t q16_main_bytes(int64_t M, int64_t N, int32_t y_dtype, bool comp) {
    if (!comp) return align_up((size_t)M * (size_t)N * 4);
    return y_dtype == FP4_F32 ? align_up((size_t)M * (size_t)N * 2) : 0;
}
size_t q16_ws_bytes(int64_t M, int64_t N, int32_t y_dtype, bool comp) {
    return q16_main_bytes(M, N, y_dtype, comp) + align_up(esc_map_bytes(M, N));
}
struct Q16Bufs {
    int16_t *yq;
    float *esc;  // standalone FP4_Q16 output only
    uint8_t *emap;
};
Q16Bufs q16_buffers(void *Y, int32_t y_dtype, uint8_t *ws, int64_t M, int64_t N, bool comp) {
    Q16Bufs b;
    b.esc = nullptr;
    if (comp && y_dtype == FP4_F32) {
        b.yq = reinterpret_cast<int16_t *>(ws);
    } else {
        b.yq = static_cast<int16_t *>(Y);
        if (!comp) b.esc = reinterpret_cast<float *>(ws);
    }
    b.emap = ws + q16_main_bytes(M, N, y_dtype, comp);
    return b;
}
// The compensated product: the GEMM's two-byte hand-over and map, the compensation pass over
// the blocks that the hand-over holds, and the escape kernel over the others.
hipError_t launch_product_comp(const uint8_t *Aq, const float *sA, const uint8_t *Wq, const float *sW, int64_t M,
                               int64_t N, int64_t K, const int32_t *row_ptr, const int32_t *coo_col,
                               const float *coo_val, int64_t capacity, const void *W, int32_t w_dtype, void *Y,
                               int32_t y_dtype, float *acc_out, uint8_t *ws, hipStream_t s) {
    const Q16Bufs b = q16_buffers(Y, y_dtype, ws, M, N, true);
    hipError_t e = launch_gemm(Aq, sA, Wq, sW, M, N, K, b.yq, DT_Q16, acc_out, s, false, b.emap);
    if (e == hipSuccess)
        e = launch_comp(b.yq, b.emap, sA, sW, Y, dt_of(y_dtype), M, N, K, row_ptr, coo_col, coo_val, W, dt_of(w_dtype),
                        capacity, s);
    if (e == hipSuccess)
        e = launch_escapes_comp(Aq, sA, Wq, sW, M, N, K, b.emap, row_ptr, coo_col, coo_val, W, dt_of(w_dtype), Y,
                                dt_of(y_dtype), s);
    return e;
}

// The COO list of dA is indexed with int32 (row_ptr), and the kernels address it with
// 32-bit byte offsets: the capacity bound must stay below 2^29 entries.
constexpr int64_t COO_MAX = (int64_t)1 << 29;

int64_t capacity_of(int64_t M, int64_t K, double q) {
    const int64_t n = M * K;
    const int64_t k = (int64_t)std::floor(q * (double)(n - 1));
    return n - 1 - k;
}

}  // namespace

// ----------------------------------------------------------------------------- shared host helpers
// (declared in fp4_host.h; the no-alloc entry point in noalloc.hip uses them too)
namespace fp4 {

// The current device must be gfx950; its CU count sizes the histogram grid.
struct DevInfo {
    bool known = false;
    bool ok = false;
    int cus = 0;
};
static std::mutex g_dev_mu;
static DevInfo g_dev[64];

fp4_status device_check(int *cus) {
    int d = 0;
    if (hipGetDevice(&d) != hipSuccess || d < 0 || d >= 64) return FP4_ERR_HIP;
    std::lock_guard<std::mutex> lk(g_dev_mu);
    DevInfo &info = g_dev[d];
    if (!info.known) {
        hipDeviceProp_t p;
        if (hipGetDeviceProperties(&p, d) != hipSuccess) return FP4_ERR_HIP;
        info.ok = std::strncmp(p.gcnArchName, "gfx950", 6) == 0;
        info.cus = p.multiProcessorCount;
        info.known = true;
    }
    if (!info.ok) return FP4_ERR_DEVICE;
    *cus = info.cus;
    return FP4_OK;
}

// Slots per row: twice the mean outlier count per row that the capacity bound allows plus
// a margin, at least 128 (rows vary widely: with log-normal row scales a few rows hold a
// hundred times the mean), at most K.  Rows with more outliers are read again by the COO pass.
int32_t slots_per_row(int64_t M, int64_t K, int64_t cap) {
    const int64_t mean = (cap + M - 1) / M;
    int64_t S = 2 * mean + 8;
    if (S < 128) S = 128;
    return (int32_t)(S < K ? S : K);
}

OutlierWs outlier_ws(int64_t M, int64_t K, int32_t dtype, int64_t cap) {
    OutlierWs w;
    w.S = slots_per_row(M, K, cap);
    size_t off = 0;
    w.state = off;
    off += align_up(sizeof(State));
    w.hist = off;
    off += align_up((size_t)HIST_BINS * 4);
    w.hist_lo = off;
    if (dtype == FP4_F32) off += align_up((size_t)HIST_LO_BINS * 4);
    w.zero_end = off;
    w.rowmax = off;
    off += align_up((size_t)M * 4);
    w.row_cnt = off;
    off += align_up((size_t)M * 4);
    w.slots = off;
    off += align_up((size_t)M * (size_t)w.S * sizeof(SlotEntry));
    w.total = off;
    return w;
}

fp4_status hip_status(hipError_t e) { return e == hipSuccess ? FP4_OK : FP4_ERR_HIP; }

// Enqueue the outlier pass: zero, histogram + row maxima, the select of T (a second histogram
// level for fp32), then rows (clamp, optional codes, staging of dA), then the COO list.  With
// wside, W's column maxima run in the select's launch and its quantize pass in the COO build's.
fp4_status run_outliers(const void *A, int32_t dtype, int64_t M, int64_t K, double q, uint8_t *ws,
                        const OutlierWs &w, int cus, float *T, int32_t *coo_row, int32_t *coo_col,
                        float *coo_val, int64_t cap, int32_t *row_ptr, int64_t *nnz, uint8_t *Aq,
                        float *sA, const WSide *wside, hipStream_t s) {
    State *st = reinterpret_cast<State *>(ws + w.state);
    uint32_t *hist = reinterpret_cast<uint32_t *>(ws + w.hist);
    uint32_t *hist_lo = reinterpret_cast<uint32_t *>(ws + w.hist_lo);
    uint32_t *rowmax = reinterpret_cast<uint32_t *>(ws + w.rowmax);
    int32_t *row_cnt = reinterpret_cast<int32_t *>(ws + w.row_cnt);
    Staging stg;
    stg.slots = reinterpret_cast<SlotEntry *>(ws + w.slots);
    stg.S = w.S;
    const int dt = dt_of(dtype);
    const int64_t n = M * K;
    const uint64_t k = (uint64_t)std::floor(q * (double)(n - 1));
    hipError_t e = launch_zero(reinterpret_cast<uint32_t *>(ws + w.state), (int64_t)(w.zero_end - w.state) / 4,
                               wside ? wside->keys : nullptr, wside ? wside->N : 0, s);
    if (e == hipSuccess) e = launch_hist_rowmax(A, dt, M, K, hist, rowmax, cus, s);
    if (e == hipSuccess) e = launch_select_hi(hist, dt, st, T, k, wside, s);
    if (e == hipSuccess && dt == DT_F32) e = launch_select_lo(A, n, hist_lo, st, T, s);
    const bool codes = Aq != nullptr;
    if (e == hipSuccess)
        e = launch_quant_rows(A, dt, M, K, codes ? rowmax : nullptr, T, Aq, sA, row_cnt, stg, st,
                              /*emit=*/true, /*write_codes=*/codes, s);
    if (e == hipSuccess)
        e = launch_coo(row_cnt, M, row_ptr, nnz, stg, cap, coo_row, coo_col, coo_val, A, dt, K, T, wside, s);
    return hip_status(e);
}

fp4_status outlier_args_check(const void *A, int32_t a_dtype, int64_t M, int64_t K, double q, const float *T,
                              const int32_t *coo_row, const int32_t *coo_col, const float *coo_val, int64_t capacity,
                              const int32_t *row_ptr, const int64_t *nnz) {
    if (!A || !T || !coo_row || !coo_col || !coo_val || !row_ptr || !nnz) return FP4_ERR_NULL;
    if (!dtype_ok(a_dtype)) return FP4_ERR_DTYPE;
    if (!mk_ok(M, K)) return FP4_ERR_SHAPE;
    if (!q_ok(q)) return FP4_ERR_QUANTILE;
    const int64_t cap = capacity_of(M, K, q);
    if (cap > COO_MAX) return FP4_ERR_QUANTILE;
    if (capacity < cap) return FP4_ERR_CAPACITY;
    if (!aligned16(A) || !aligned16(T) || !aligned16(row_ptr)) return FP4_ERR_ALIGN;
    return FP4_OK;
}

fp4_status outlier_clamp_impl(const void *A, int32_t a_dtype, int64_t M, int64_t K, double q, float *T,
                              int32_t *coo_row, int32_t *coo_col, float *coo_val, int64_t capacity, int32_t *row_ptr,
                              int64_t *nnz, void *workspace, size_t ws_bytes, void *stream) {
    fp4_status st = outlier_args_check(A, a_dtype, M, K, q, T, coo_row, coo_col, coo_val, capacity, row_ptr, nnz);
    if (st != FP4_OK) return st;
    if (!workspace) return FP4_ERR_NULL;
    const int64_t cap = capacity_of(M, K, q);
    const OutlierWs w = outlier_ws(M, K, a_dtype, cap);
    if (ws_bytes < w.total) return FP4_ERR_WORKSPACE;
    if (!aligned16(workspace)) return FP4_ERR_ALIGN;
    int cus;
    st = device_check(&cus);
    if (st != FP4_OK) return st;
    // nnz <= cap always (T is the (k+1)-th smallest |a|), so the staging area and the COO
    // positions are bounded by the computed cap, which the workspace was sized for.
    return run_outliers(A, a_dtype, M, K, q, static_cast<uint8_t *>(workspace), w, cus, T, coo_row, coo_col, coo_val,
                        cap, row_ptr, nnz, nullptr, nullptr, nullptr, reinterpret_cast<hipStream_t>(stream));
}

int64_t outlier_capacity_of(int64_t M, int64_t K, double q) { return capacity_of(M, K, q); }

}  // namespace fp4

namespace {
// Checks shared by the forward's calls; fills the layout and the CU count.
// need_product: the product stage runs (the workspace must hold the whole layout for y_dtype);
// else only the quantizer stages, which use the part before the hand-over.
fp4_status forward_check(int64_t M, int64_t K, int64_t N, int32_t in_dtype, int32_t y_dtype, double q,
                         size_t ws_bytes, const void *workspace, bool need_product, fp4_ws_layout *l, int *cus) {
    if (!workspace) return FP4_ERR_NULL;
    if (!dtype_ok(in_dtype) || !dtype_ok(y_dtype)) return FP4_ERR_DTYPE;
    fp4_status st = fp4_forward_layout(M, K, N, in_dtype, y_dtype, q, l);
    if (st != FP4_OK) return st;
    if (ws_bytes < (need_product ? l->total : l->handoff)) return FP4_ERR_WORKSPACE;
    if (!aligned16(workspace)) return FP4_ERR_ALIGN;
    return FP4_OK;
}

// The forward's quantizer stages into the workspace: FP4_STAGE_A (quantile, clamp, dA, A's
// codes and scales) and/or FP4_STAGE_W (W's codes and scales).  W's column-maximum keys follow
// the outlier scratch.  When both stages run in one call, W's passes share the outlier pass's
// launches (its keys zeroed in the zero fill); alone, W takes a zero fill and its two passes.
fp4_status quantize_impl(const void *A, const void *W, int32_t in_dtype, int64_t M, int64_t K, int64_t N, double q,
                         int32_t stages, uint8_t *ws, const fp4_ws_layout &l, int cus, hipStream_t s) {
    const OutlierWs w = outlier_ws(M, K, in_dtype, l.capacity);
    uint32_t *wkeys = reinterpret_cast<uint32_t *>(ws + l.scratch + w.total);
    const bool sa = stages & FP4_STAGE_A, sw = stages & FP4_STAGE_W;
    if (sa) {
        WSide wside{W, dt_of(in_dtype), K, N, wkeys, ws + l.Wq, reinterpret_cast<float *>(ws + l.sW)};
        return run_outliers(A, in_dtype, M, K, q, ws + l.scratch, w, cus, reinterpret_cast<float *>(ws + l.T),
                            reinterpret_cast<int32_t *>(ws + l.coo_row), reinterpret_cast<int32_t *>(ws + l.coo_col),
                            reinterpret_cast<float *>(ws + l.coo_val), l.capacity,
                            reinterpret_cast<int32_t *>(ws + l.row_ptr), reinterpret_cast<int64_t *>(ws + l.nnz),
                            ws + l.Aq, reinterpret_cast<float *>(ws + l.sA), sw ? &wside : nullptr, s);
    }
    if (sw) {
        hipError_t e = launch_zero(wkeys, N, nullptr, 0, s);
        if (e == hipSuccess)
            e = launch_quant_cols(W, dt_of(in_dtype), K, N, reinterpret_cast<float *>(wkeys), ws + l.Wq, true, s, nullptr,
                                  reinterpret_cast<float *>(ws + l.sW));
        return hip_status(e);
    }
    return FP4_OK;
}

// The product stage: Y = Y_main + dA . W from the workspace's intermediates, through the
// two-byte hand-over in the layout's handoff region; Wq/sW: W's codes and scales (the
// workspace's, or a caller's cached ones).
fp4_status product_impl(const void *W, int32_t in_dtype, const uint8_t *Wq, const float *sW, int64_t M, int64_t K,
                        int64_t N, void *Y, int32_t y_dtype, uint8_t *ws, const fp4_ws_layout &l, hipStream_t s) {
    return hip_status(launch_product_comp(
        ws + l.Aq, reinterpret_cast<const float *>(ws + l.sA), Wq, sW, M, N, K,
        reinterpret_cast<const int32_t *>(ws + l.row_ptr), reinterpret_cast<const int32_t *>(ws + l.coo_col),
        reinterpret_cast<const float *>(ws + l.coo_val), l.capacity, W, in_dtype, Y, y_dtype, nullptr,
        ws + l.handoff, s));
}

// The forward; Wq_in/sW_in: W's codes and scales from an earlier fp4_quantize (W unchanged
// since), or NULL to quantize W here.
fp4_status forward_impl(const void *A, const void *W, const uint8_t *Wq_in, const float *sW_in, int32_t in_dtype,
                        int64_t M, int64_t K, int64_t N, double q, void *Y, int32_t y_dtype, void *workspace,
                        size_t ws_bytes, void *stream) {
    if (!A || !W || !Y || !workspace) return FP4_ERR_NULL;
    if (!dtype_ok(in_dtype) || !dtype_ok(y_dtype)) return FP4_ERR_DTYPE;
    fp4_ws_layout l;
    int cus;
    fp4_status st = forward_check(M, K, N, in_dtype, y_dtype, q, ws_bytes, workspace, true, &l, &cus);
    if (st != FP4_OK) return st;
    if (!aligned16(A) || !aligned16(W) || !aligned16(Y)) return FP4_ERR_ALIGN;
    st = device_check(&cus);
    if (st != FP4_OK) return st;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    const bool wq_given = Wq_in != nullptr;
    st = quantize_impl(A, W, in_dtype, M, K, N, q, wq_given ? FP4_STAGE_A : FP4_STAGE_A | FP4_STAGE_W, ws, l, cus, s);
    if (st != FP4_OK) return st;
    return product_impl(W, in_dtype, wq_given ? Wq_in : ws + l.Wq,
                        wq_given ? sW_in : reinterpret_cast<const float *>(ws + l.sW), M, K, N, Y, y_dtype, ws, l, s);
}

}  // namespace

extern "C" {

const char *fp4_status_string(fp4_status s) {
    switch (s) {
    case FP4_OK: return "ok";
    case FP4_ERR_NULL: return "a required pointer is NULL";
    case FP4_ERR_SHAPE: return "a size is out of range";
    case FP4_ERR_DTYPE: return "unknown dtype or axis code, or unsupported combination";
    case FP4_ERR_QUANTILE: return "q is NaN or outside [0, 1]";
    case FP4_ERR_CAPACITY: return "COO capacity below fp4_outlier_capacity()";
    case FP4_ERR_WORKSPACE: return "workspace smaller than required";
    case FP4_ERR_DEVICE: return "current HIP device is not gfx950";
    case FP4_ERR_HIP: return "a HIP runtime call or kernel launch failed";
    case FP4_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case FP4_ERR_SCRATCH: return "the problem needs more scratch than the no-alloc entry point holds";
    default: return "unknown status";
    }
}

fp4_status fp4_quantize(const void *X, int32_t x_dtype, int64_t R, int64_t C, int32_t axis,
                        const float *clamp_T, uint8_t *codes, float *scales, void *stream) {
    if (!X || !codes || !scales) return FP4_ERR_NULL;
    if (!dtype_ok(x_dtype) || (axis != FP4_PER_ROW && axis != FP4_PER_COL)) return FP4_ERR_DTYPE;
    if (axis == FP4_PER_COL && clamp_T) return FP4_ERR_DTYPE;  // W is never clamped
    if (axis == FP4_PER_ROW) {
        if (!mk_ok(R, C)) return FP4_ERR_SHAPE;
    } else {
        if (!mk_ok(C, R) || !n_ok(C)) return FP4_ERR_SHAPE;
    }
    if (!aligned16(X) || !aligned16(codes) || !aligned16(scales)) return FP4_ERR_ALIGN;
    int cus;
    fp4_status st = device_check(&cus);
    if (st != FP4_OK) return st;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (axis == FP4_PER_ROW)
        return hip_status(launch_quant_rows(X, dt_of(x_dtype), R, C, nullptr, clamp_T, codes, scales, nullptr,
                                            Staging{nullptr, 0}, nullptr, false, true, s));
    return hip_status(launch_quant_cols(X, dt_of(x_dtype), R, C, scales, codes, false, s));
}

int64_t fp4_outlier_capacity(int64_t M, int64_t K, double q) {
    if (!mk_ok(M, K) || !q_ok(q)) return -1;
    return capacity_of(M, K, q);
}

size_t fp4_outlier_workspace_bytes(int64_t M, int64_t K, int32_t a_dtype, double q) {
    if (!mk_ok(M, K) || !q_ok(q) || !dtype_ok(a_dtype)) return 0;
    return outlier_ws(M, K, a_dtype, capacity_of(M, K, q)).total;
}

fp4_status fp4_outlier_clamp(const void *A, int32_t a_dtype, int64_t M, int64_t K, double q, float *T,
                             int32_t *coo_row, int32_t *coo_col, float *coo_val, int64_t capacity,
                             int32_t *row_ptr, int64_t *nnz, void *workspace, size_t ws_bytes, void *stream) {
    return fp4::outlier_clamp_impl(A, a_dtype, M, K, q, T, coo_row, coo_col, coo_val, capacity, row_ptr, nnz,
                                   workspace, ws_bytes, stream);
}

size_t fp4_gemm_workspace_bytes(int64_t M, int64_t N, int32_t y_dtype, int32_t with_comp) {
    if (M < 1 || !n_ok(N)) return 0;
    if (y_dtype == FP4_Q16) return with_comp ? 0 : q16_ws_bytes(M, N, y_dtype, false);
    if (!dtype_ok(y_dtype) || !with_comp) return 0;
    return q16_ws_bytes(M, N, y_dtype, true);
}

fp4_status fp4_gemm(const uint8_t *Aq, const float *sA, const uint8_t *Wq, const float *sW, int64_t M, int64_t N,
                    int64_t K, const int32_t *row_ptr, const int32_t *coo_col, const float *coo_val,
                    int64_t capacity, const void *W, int32_t w_dtype, void *Y, int32_t y_dtype, float *acc_out,
                    void *workspace, size_t ws_bytes, void *stream) {
    if (!Aq || !sA || !Wq || !sW || !Y) return FP4_ERR_NULL;
    const int ncomp = (row_ptr != nullptr) + (coo_col != nullptr) + (coo_val != nullptr);
    if (ncomp != 0 && ncomp != 3) return FP4_ERR_NULL;
    const bool comp = ncomp == 3;
    if (comp && !W) return FP4_ERR_NULL;
    const bool q16 = y_dtype == FP4_Q16;
    if (!(dtype_ok(y_dtype) || q16) || (comp && (q16 || !dtype_ok(w_dtype)))) return FP4_ERR_DTYPE;
    if (!gemm_ok(M, N, K) || (comp && !wcomp_ok(N, K, w_dtype))) return FP4_ERR_SHAPE;
    const size_t need = fp4_gemm_workspace_bytes(M, N, y_dtype, comp);
    if (need && !workspace) return FP4_ERR_NULL;
    if (ws_bytes < need) return FP4_ERR_WORKSPACE;
    if (!aligned16(Aq) || !aligned16(Wq) || !aligned16(Y) || (comp && !aligned16(W)) ||
        (acc_out && !aligned16(acc_out)) || (need && !aligned16(workspace)))
        return FP4_ERR_ALIGN;
    int cus;
    fp4_status st = device_check(&cus);
    if (st != FP4_OK) return st;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (q16) {
        const Q16Bufs b = q16_buffers(Y, y_dtype, static_cast<uint8_t *>(workspace), M, N, false);
        hipError_t e = launch_gemm(Aq, sA, Wq, sW, M, N, K, b.yq, DT_Q16, acc_out, s, false, b.emap);
        if (e == hipSuccess) e = launch_escapes_q16(Aq, sA, Wq, sW, M, N, K, b.emap, b.yq, b.esc, s);
        return hip_status(e);
    }
    if (!comp) return hip_status(launch_gemm(Aq, sA, Wq, sW, M, N, K, Y, dt_of(y_dtype), acc_out, s));
    return hip_status(launch_product_comp(Aq, sA, Wq, sW, M, N, K, row_ptr, coo_col, coo_val,
                                          capacity > 0 ? capacity : 0, W, w_dtype, Y, y_dtype, acc_out,
                                          static_cast<uint8_t *>(workspace), s));
}

const char *fp4_gemm_kernel_name(int64_t M, int64_t N, int64_t K, int32_t num_cus) {
    if (num_cus < 1 || !gemm_ok(M, N, K)) return nullptr;
    return gemm_kernel_choice(M, N, K, false, num_cus) == GEMM_WIDE ? "k_fp4_gemm_wide" : "k_fp4_gemm";
}

const char *fp4_comp_kernel_name(int64_t M, int64_t capacity) {
    if (M < 1 || capacity < 0) return nullptr;
    return comp_kernel_choice(M, capacity) == COMP_BLOCK64 ? "k_comp_block64" : "k_comp_apply";
}

size_t fp4_fp8_workspace_bytes(void) { return ALIGN; }

fp4_status fp4_fp8_quantize(const void *X, int32_t x_dtype, int64_t n, uint8_t *codes, float *scale, void *workspace,
                            size_t ws_bytes, void *stream) {
    if (!X || !codes || !scale || !workspace) return FP4_ERR_NULL;
    if (!dtype_ok(x_dtype)) return FP4_ERR_DTYPE;
    if (n < 1 || n > FP8_MAX_N) return FP4_ERR_SHAPE;
    if (ws_bytes < fp4_fp8_workspace_bytes()) return FP4_ERR_WORKSPACE;
    if (!aligned16(X) || !aligned16(codes) || !aligned16(workspace)) return FP4_ERR_ALIGN;
    int cus;
    fp4_status st = device_check(&cus);
    if (st != FP4_OK) return st;
    return hip_status(launch_fp8_quantize(X, dt_of(x_dtype), n, static_cast<uint32_t *>(workspace), codes, scale, cus,
                                          reinterpret_cast<hipStream_t>(stream)));
}

fp4_status fp4_fp8_dequantize(const uint8_t *codes, int64_t n, const float *scale, void *Y, int32_t y_dtype,
                              void *stream) {
    if (!codes || !scale || !Y) return FP4_ERR_NULL;
    if (!dtype_ok(y_dtype)) return FP4_ERR_DTYPE;
    if (n < 1 || n > FP8_MAX_N) return FP4_ERR_SHAPE;
    if (!aligned16(codes) || !aligned16(Y)) return FP4_ERR_ALIGN;
    int cus;
    fp4_status st = device_check(&cus);
    if (st != FP4_OK) return st;
    return hip_status(launch_fp8_dequantize(codes, n, scale, Y, dt_of(y_dtype), cus,
                                            reinterpret_cast<hipStream_t>(stream)));
}

static bool emu_ok(int64_t M, int64_t N, int64_t K) {
    // E4M3 operands take K bytes per row; their buffer offsets stay below 2^31
    return gemm_ok(M, N, K) && M * K <= INT32_MAX && N * K <= INT32_MAX;
}

size_t fp4_gemm_fp8emu_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (!emu_ok(M, N, K)) return 0;
    return align_up((size_t)M * (size_t)K) + align_up((size_t)N * (size_t)K);
}

fp4_status fp4_gemm_fp8emu(const uint8_t *Aq, const float *sA, const uint8_t *Wq, const float *sW, int64_t M,
                           int64_t N, int64_t K, void *Y, int32_t y_dtype, float *acc_out, void *workspace,
                           size_t ws_bytes, void *stream) {
    if (!Aq || !sA || !Wq || !sW || !Y || !workspace) return FP4_ERR_NULL;
    if (!dtype_ok(y_dtype)) return FP4_ERR_DTYPE;
    if (!emu_ok(M, N, K)) return FP4_ERR_SHAPE;
    if (ws_bytes < fp4_gemm_fp8emu_workspace_bytes(M, N, K)) return FP4_ERR_WORKSPACE;
    if (!aligned16(Aq) || !aligned16(Wq) || !aligned16(Y) || !aligned16(workspace) ||
        (acc_out && !aligned16(acc_out)))
        return FP4_ERR_ALIGN;
    int cus;
    fp4_status st = device_check(&cus);
    if (st != FP4_OK) return st;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    uint8_t *A8 = static_cast<uint8_t *>(workspace);
    uint8_t *W8 = A8 + align_up((size_t)M * (size_t)K);
    hipError_t e = launch_e2m1_to_e4m3(Aq, M * (K / 2), A8, s);
    if (e == hipSuccess) e = launch_e2m1_to_e4m3(Wq, N * (K / 2), W8, s);
    if (e == hipSuccess) e = launch_gemm(A8, sA, W8, sW, M, N, K, Y, dt_of(y_dtype), acc_out, s, true);
    return hip_status(e);
}

fp4_status fp4_forward_layout(int64_t M, int64_t K, int64_t N, int32_t in_dtype, int32_t y_dtype, double q,
                              struct fp4_ws_layout *out) {
    if (!out) return FP4_ERR_NULL;
    std::memset(out, 0, sizeof(*out));
    if (!dtype_ok(in_dtype) || !dtype_ok(y_dtype)) return FP4_ERR_DTYPE;
    if (!gemm_ok(M, N, K) || !wcomp_ok(N, K, in_dtype)) return FP4_ERR_SHAPE;
    if (!q_ok(q)) return FP4_ERR_QUANTILE;
    const int64_t cap = capacity_of(M, K, q);
    if (cap > COO_MAX) return FP4_ERR_QUANTILE;
    const size_t capn = (size_t)(cap > 0 ? cap : 1);
    size_t off = 0;
    out->T = off; off += ALIGN;
    out->nnz = off; off += ALIGN;
    out->row_ptr = off; off += align_up((size_t)(M + 1) * 4);
    out->coo_row = off; off += align_up(capn * 4);
    out->coo_col = off; off += align_up(capn * 4);
    out->coo_val = off; off += align_up(capn * 4);
    out->Aq = off; off += align_up((size_t)M * (size_t)(K / 2));
    out->sA = off; off += align_up((size_t)M * 4);
    out->Wq = off; off += align_up((size_t)N * (size_t)(K / 2));
    out->sW = off; off += align_up((size_t)N * 4);
    out->scratch = off; off += outlier_ws(M, K, in_dtype, cap).total + align_up((size_t)N * 4);  // + W's keys
    out->handoff = off; off += q16_ws_bytes(M, N, y_dtype, true);  // last: the only part that depends on Y's type
    out->total = off;
    out->capacity = cap;
    return FP4_OK;
}

size_t fp4_forward_workspace_bytes(int64_t M, int64_t K, int64_t N, int32_t in_dtype, int32_t y_dtype, double q) {
    fp4_ws_layout l;
    return fp4_forward_layout(M, K, N, in_dtype, y_dtype, q, &l) == FP4_OK ? l.total : 0;
}

fp4_status fp4_linear_forward(const void *A, const void *W, int32_t in_dtype, int64_t M, int64_t K, int64_t N,
                              double q, void *Y, int32_t y_dtype, void *workspace, size_t ws_bytes, void *stream) {
    return forward_impl(A, W, nullptr, nullptr, in_dtype, M, K, N, q, Y, y_dtype, workspace, ws_bytes, stream);
}

fp4_status fp4_forward_quantize(const void *A, const void *W, int32_t in_dtype, int64_t M, int64_t K, int64_t N,
                                double q, int32_t stages, void *workspace, size_t ws_bytes, void *stream) {
    if (stages < 1 || stages > (FP4_STAGE_A | FP4_STAGE_W)) return FP4_ERR_DTYPE;
    if (((stages & FP4_STAGE_A) && !A) || ((stages & FP4_STAGE_W) && !W)) return FP4_ERR_NULL;
    fp4_ws_layout l;
    int cus;
    // the quantizer stages' part of the layout is the same for every Y type
    fp4_status st = forward_check(M, K, N, in_dtype, FP4_BF16, q, ws_bytes, workspace, false, &l, &cus);
    if (st != FP4_OK) return st;
    if (((stages & FP4_STAGE_A) && !aligned16(A)) || ((stages & FP4_STAGE_W) && !aligned16(W))) return FP4_ERR_ALIGN;
    st = device_check(&cus);
    if (st != FP4_OK) return st;
    return quantize_impl(A, W, in_dtype, M, K, N, q, stages, static_cast<uint8_t *>(workspace), l, cus,
                         reinterpret_cast<hipStream_t>(stream));
}

fp4_status fp4_forward_product(const void *W, int32_t in_dtype, int64_t M, int64_t K, int64_t N, double q, void *Y,
                               int32_t y_dtype, void *workspace, size_t ws_bytes, void *stream) {
    if (!W || !Y) return FP4_ERR_NULL;
    if (!dtype_ok(y_dtype)) return FP4_ERR_DTYPE;
    fp4_ws_layout l;
    int cus;
    fp4_status st = forward_check(M, K, N, in_dtype, y_dtype, q, ws_bytes, workspace, true, &l, &cus);
    if (st != FP4_OK) return st;
    if (!aligned16(W) || !aligned16(Y)) return FP4_ERR_ALIGN;
    st = device_check(&cus);
    if (st != FP4_OK) return st;
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    return product_impl(W, in_dtype, ws + l.Wq, reinterpret_cast<const float *>(ws + l.sW), M, K, N, Y, y_dtype, ws, l,
                        reinterpret_cast<hipStream_t>(stream));
}

fp4_status fp4_linear_forward_wq(const void *A, const void *W, const uint8_t *Wq, const float *sW, int32_t in_dtype,
                                 int64_t M, int64_t K, int64_t N, double q, void *Y, int32_t y_dtype,
                                 void *workspace, size_t ws_bytes, void *stream) {
    if (!Wq || !sW) return FP4_ERR_NULL;
    if (!aligned16(Wq)) return FP4_ERR_ALIGN;
    return forward_impl(A, W, Wq, sW, in_dtype, M, K, N, q, Y, y_dtype, workspace, ws_bytes, stream);
}

// ----------------------------------------------------------------------------- backward
// Workgroups of the fused pass over a bf16 dY (each leaves one row of column-maximum keys).
constexpr int BWD_PART_ROWS = 512;
// Shapes of the straight-through backward: the forward's (Aq, Wq), and each requested
// product's contraction (n for dA, m for dW) within the GEMM's K limits.
static fp4_status bwd_shape(int64_t M, int64_t K, int64_t N, bool want_dA, bool want_dW) {
    if (!gemm_ok(M, N, K)) return FP4_ERR_SHAPE;
    if (want_dA && !(k_ok(N) && mk_ok(M, N) && mk_ok(K, N))) return FP4_ERR_SHAPE;
    if (want_dW && !(k_ok(M) && mk_ok(N, M) && mk_ok(K, M))) return FP4_ERR_SHAPE;
    return FP4_OK;
}

fp4_status fp4_backward_layout(int64_t M, int64_t K, int64_t N, struct fp4_bwd_layout *out) {
    if (!out) return FP4_ERR_NULL;
    std::memset(out, 0, sizeof(*out));
    if (!gemm_ok(M, N, K)) return FP4_ERR_SHAPE;  // the forward's shapes; each product checks its own
    size_t off = 0;
    out->Gq = off; off += align_up((size_t)M * (size_t)(N / 2));
    out->sG = off; off += align_up((size_t)M * 4);
    out->Hq = off; off += align_up((size_t)N * (size_t)(M / 2));
    out->sH = off; off += align_up((size_t)N * 4);
    out->WqT = off; off += align_up((size_t)K * (size_t)(N / 2));
    out->AqT = off; off += align_up((size_t)K * (size_t)(M / 2));
    out->ones = off; off += align_up((size_t)K * 4);
    out->part = off; off += align_up((size_t)BWD_PART_ROWS * (size_t)N * 4);
    out->total = off;
    return FP4_OK;
}

size_t fp4_backward_workspace_bytes(int64_t M, int64_t K, int64_t N) {
    fp4_bwd_layout l;
    return fp4_backward_layout(M, K, N, &l) == FP4_OK ? l.total : 0;
}

fp4_status fp4_linear_backward(const void *dY, int32_t dy_dtype, int64_t M, int64_t K, int64_t N, const uint8_t *Aq,
                               const float *sA, const uint8_t *Wq, const float *sW, void *dA, int32_t da_dtype,
                               void *dW, int32_t dw_dtype, void *workspace, size_t ws_bytes, void *stream) {
    const bool want_dA = dA != nullptr, want_dW = dW != nullptr;
    if (!dY || !workspace || (!want_dA && !want_dW)) return FP4_ERR_NULL;
    if (want_dA && (!Wq || !sW)) return FP4_ERR_NULL;
    if (want_dW && (!Aq || !sA)) return FP4_ERR_NULL;
    if (!dtype_ok(dy_dtype) || (want_dA && !dtype_ok(da_dtype)) || (want_dW && !dtype_ok(dw_dtype)))
        return FP4_ERR_DTYPE;
    fp4_status st = bwd_shape(M, K, N, want_dA, want_dW);
    if (st != FP4_OK) return st;
    fp4_bwd_layout l;
    fp4_backward_layout(M, K, N, &l);
    if (ws_bytes < l.total) return FP4_ERR_WORKSPACE;
    if (!aligned16(dY) || !aligned16(workspace) || (want_dA && (!aligned16(Wq) || !aligned16(sW) || !aligned16(dA))) ||
        (want_dW && (!aligned16(Aq) || !aligned16(sA) || !aligned16(dW))))
        return FP4_ERR_ALIGN;
    int cus;
    st = device_check(&cus);
    if (st != FP4_OK) return st;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    float *ones = reinterpret_cast<float *>(ws + l.ones);
    const int dt = dt_of(dy_dtype);
    hipError_t e = launch_fill_f32(ones, K, 1.0f, s);
    uint8_t *Gq = ws + l.Gq, *WqT = ws + l.WqT, *Hq = ws + l.Hq, *AqT = ws + l.AqT;
    float *sG = reinterpret_cast<float *>(ws + l.sG), *sH = reinterpret_cast<float *>(ws + l.sH);
    // Both products of a bf16 dY with rows up to 24576: one pass reads dY for G's codes and for
    // H's column maxima together, so dY is read twice in all instead of three times.
    const bool fused = want_dA && want_dW && dt == DT_BF16 && fused_rows_cpt(N) <= 3;
    if (fused) {
        const int G = (int)std::min<int64_t>(M, std::min(BWD_PART_ROWS, cus));  // one 1024-thread workgroup per CU
        if (e == hipSuccess)
            e = launch_bwd_rows_fused(dY, M, N, sW, sA, Gq, sG, reinterpret_cast<uint32_t *>(ws + l.part), G,
                                      reinterpret_cast<uint32_t *>(sH), s);
    }
    if (want_dA && e == hipSuccess) {
        // dA = deq(Q_rows(dY * sW)) . value(Wq)^T: GEMM with M rows, K columns, contraction N
        if (!fused) e = launch_scaled_quant_rows(dY, dt, M, N, sW, Gq, sG, s);
        if (e == hipSuccess) e = launch_codes_transpose(Wq, N, K, WqT, s);
        if (e == hipSuccess) e = launch_gemm(Gq, sG, WqT, ones, M, K, N, dA, dt_of(da_dtype), nullptr, s);
    }
    if (want_dW && e == hipSuccess) {
        // dW = value(Aq)^T . deq(Q_cols(sA * dY)): GEMM with K rows, N columns, contraction M
        if (fused) e = launch_quant_cols_keyed(dY, dt, M, N, sH, Hq, sA, s);
        else e = launch_quant_cols(dY, dt, M, N, sH, Hq, false, s, sA);
        if (e == hipSuccess) e = launch_codes_transpose(Aq, M, K, AqT, s);
        if (e == hipSuccess) e = launch_gemm(AqT, ones, Hq, sH, K, N, M, dW, dt_of(dw_dtype), nullptr, s);
    }
    return hip_status(e);
}

}  // extern "C"
