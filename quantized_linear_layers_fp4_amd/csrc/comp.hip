// gfx950 kernels of the sparse compensation term dA . W of the FP4 linear forward (outlier
// paragraph of the QbitAI report on "Optimizing Large Language Model Training Using FP4
// Quantization": the entries clamped away from A are kept as a sparse matrix and their
// product with the weights is added back).  They run after the FP4 GEMM, which hands over
// its exact accumulator as two-byte integers 4*acc (the 128 x 64 blocks where some
// |acc| > 8191.75 does not fit are marked in a map; the pass leaves them to the escape
// kernel, escape.hip, which computes them with the same arithmetic); the pass rebuilds the dequantized product Y_main = fl(fl(acc*sA)*sW) bit for bit and writes
// Y = Y_main + dA . W in the output type, rounded once, the entries added in ascending k with
// one fp32 fma each.  The two-byte hand-over halves the bytes that an fp32 Y_main would cost
// on both sides of the pass.
//
// One wave per (row, chunk of 64*CC columns) task; lane l owns the CC columns CC*l .. of
// the chunk.  The wave first issues its accumulator and column-scale loads and the row's two
// CSR offsets together, then takes the row's dA entries 64 at a time, one (k, delta) pair per
// lane, and walks them in groups of eight W row segments loaded together.  Tasks are dealt
// out to the eight XCDs in contiguous ranges (consecutive workgroup ids go to different
// XCDs), chunk-major within a range, so each XCD streams all rows over one chunk at a time
// and the W rows that chunk gathers stay in its L2.  Up to 64 entries per row on average
// (the list's capacity over M) the tasks are (row, 512-column chunk); beyond that the gathers
// bound the pass and the tasks are (8 rows, 64-column chunk) blocks (k_comp_block64), whose
// W strip fits in L2.
// The accumulators and Y are streamed with non-temporal hints so they do not evict W.
#include "fp4_common.h"
#include "fp4_launch.h"

namespace fp4 {

constexpr int CB = 8;  // W row segments in flight per lane
typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));

// CC consecutive elements of type WDT (bf16 or fp32) at byte offset off, raw, through a
// buffer descriptor (out of range: zeros); nothing is loaded when !on.
template <int WDT, int CC>
__device__ __forceinline__ void load_seg(__amdgpu_buffer_rsrc_t rs, uint32_t off, bool on, v4i (&raw)[2]) {
    constexpr int BYTES = CC * (WDT == DT_BF16 ? 2 : 4);
    raw[0] = raw[1] = v4i{0, 0, 0, 0};
    if (!on) return;
    if constexpr (BYTES == 8) {
        const v2i q = __builtin_amdgcn_raw_buffer_load_b64(rs, (int)off, 0, 0);
        raw[0] = v4i{q.x, q.y, 0, 0};
    } else {
        raw[0] = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, 0);
        if constexpr (BYTES == 32) raw[1] = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off + 16, 0, 0);
    }
}
// element c of such a segment as fp32
template <int WDT>
__device__ __forceinline__ float seg_elem(const v4i (&raw)[2], int c) {
    if constexpr (WDT == DT_BF16) {
        const uint32_t pr = (uint32_t)raw[c >> 3][(c >> 1) & 3];
        return bf16_to_f32((c & 1) ? (pr >> 16) : (pr & 0xFFFFu));
    } else {
        return __int_as_float(raw[c >> 2][c & 3]);
    }
}

// Decodes the lane's CC int16 accumulator codes q (packed in qv) into Y_main: acc = q / 4
// exactly, Y_main = fl(fl(acc * sA) * sW) as the GEMM's own epilogue rounds it.  Yq may be Y
// itself (bf16 Y): every lane reads exactly the bytes it later writes, and no other lane
// touches them.
template <int CC>
__device__ __forceinline__ void decode_ymain(const v4i &qv, const v4i (&swv)[2], float sa, float (&y)[CC]) {
#pragma unroll
    for (int i = 0; i < CC; ++i) {
        const int q = (int)(int16_t)(((uint32_t)qv[i >> 1] >> (16 * (i & 1))) & 0xFFFFu);
        y[i] = ((float)q * 0.25f * sa) * __int_as_float(swv[i >> 2][i & 3]);
    }
}

// Y[row][col .. col+CC) in the output type (16 or 8 bytes per lane, non-temporal).
template <int YDT, int CC>
__device__ __forceinline__ void store_y(void *Y, size_t off, const float (&y)[CC]) {
    if constexpr (YDT == DT_BF16) {
        uint32_t o[CC / 2];
#pragma unroll
        for (int i = 0; i < CC / 2; ++i) o[i] = f32_to_bf16_bits(y[2 * i]) | (f32_to_bf16_bits(y[2 * i + 1]) << 16);
        uint16_t *yp = reinterpret_cast<uint16_t *>(Y) + off;
        if constexpr (CC == 8)
            __builtin_nontemporal_store(v4i{(int)o[0], (int)o[1], (int)o[2], (int)o[3]}, reinterpret_cast<v4i *>(yp));
        else
            __builtin_nontemporal_store(v2i{(int)o[0], (int)o[1]}, reinterpret_cast<v2i *>(yp));
    } else {
        f4 *yp = reinterpret_cast<f4 *>(reinterpret_cast<float *>(Y) + off);
#pragma unroll
        for (int h = 0; h < CC / 4; ++h) __builtin_nontemporal_store(f4{y[4 * h], y[4 * h + 1], y[4 * h + 2], y[4 * h + 3]}, yp + h);
    }
}

struct CompArgs {
    const int16_t *Yq;
    const uint8_t *emap;  // the GEMM's map of escaped ESC_ROWS x ESC_COLS blocks, mapN bytes per row
    int mapN;
    const float *sA, *sW;
    void *Y;
    int M, N, K;
    const int32_t *row_ptr, *coo_col;
    const float *coo_val;
    const void *W;
};

// One (row, chunk) task: lane l owns the CC columns chunk*64*CC + CC*l ...
template <int YDT, int WDT, int CC>
__device__ __forceinline__ void comp_task(const CompArgs &a, int row, int chunk, int lane) {
    const int N = a.N;
    const int col = chunk * (64 * CC) + lane * CC;
    const bool inside = col < N;  // N % 8 == 0: a lane's columns are in range together
    // The row's CSR offsets (lane l loads row_ptr[row + (l & 1)]), the lane's accumulator
    // codes and column scales, issued together; the codes and scales go through
    // descriptors, so a lane past N reads zeros.
    const int32_t rp = a.row_ptr[row + (lane & 1)];
    const __amdgpu_buffer_rsrc_t rsQ =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<int16_t *>(a.Yq) + (size_t)row * N, 0, N * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t rsS = __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(a.sW), 0, N * 4, 0x00020000);
    v4i qv = v4i{0, 0, 0, 0};
    if constexpr (CC == 8) {
        qv = __builtin_amdgcn_raw_buffer_load_b128(rsQ, col * 2, 0, 2);
    } else {
        const v2i q2 = __builtin_amdgcn_raw_buffer_load_b64(rsQ, col * 2, 0, 2);
        qv = v4i{q2.x, q2.y, 0, 0};
    }
    v4i swv[2] = {v4i{0, 0, 0, 0}, v4i{0, 0, 0, 0}};
#pragma unroll
    for (int h = 0; h < CC / 4; ++h) swv[h] = __builtin_amdgcn_raw_buffer_load_b128(rsS, col * 4 + 16 * h, 0, 0);
    const float sa = a.sA[row];
    // the map bytes under the chunk: one aligned word per wave (a uniform, scalar load); a lane's
    // CC columns lie in one block (CC divides ESC_COLS)
    constexpr int BPC = 64 * CC / ESC_COLS;  // blocks per chunk
    static_assert(BPC == 8 || BPC == 4, "map word");
    const size_t moff = (size_t)(row / ESC_ROWS) * a.mapN + (size_t)chunk * BPC;
    uint64_t mw;
    if constexpr (BPC == 8) mw = *reinterpret_cast<const uint64_t *>(a.emap + moff);
    else mw = *reinterpret_cast<const uint32_t *>(a.emap + moff);
    const bool escaped = ((mw >> (8 * (lane * CC / ESC_COLS))) & 0xFF) != 0;
    const int32_t e0 = __builtin_amdgcn_readlane(rp, 0);
    const int32_t e1 = __builtin_amdgcn_readlane(rp, 1);
    float y[CC];
    decode_ymain<CC>(qv, swv, sa, y);

    // W through a buffer descriptor.  Offsets are unsigned 32-bit: K*N*ESZ < 2^31, so the
    // largest (a lane past N on the last row of W) stays below 2^32 and reads zeros; such a
    // lane is never stored.
    constexpr int ESZ = (WDT == DT_BF16) ? 2 : 4;
    const __amdgpu_buffer_rsrc_t rsW =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(a.W), 0, (int)((int64_t)a.K * N * ESZ), 0x00020000);
    const uint32_t row_bytes = (uint32_t)N * ESZ;
    const uint32_t lane_off = (uint32_t)col * ESZ;
    for (int32_t e = e0; e < e1; e += 64) {
        int32_t kk = 0;
        float dd = 0.0f;
        if (e + lane < e1) {
            kk = a.coo_col[e + lane];
            dd = a.coo_val[e + lane];
        }
        const int nb = min(64, e1 - e);  // wave-uniform
        for (int s = 0; s < nb; s += CB) {
            v4i w[CB][2];
#pragma unroll
            for (int u = 0; u < CB; ++u) {
                const uint32_t k = (uint32_t)__builtin_amdgcn_readlane(kk, s + u);
                load_seg<WDT, CC>(rsW, k * row_bytes + lane_off, s + u < nb, w[u]);
            }
#pragma unroll
            for (int u = 0; u < CB; ++u) {
                if (s + u < nb) {  // wave-uniform
                    const float d = __builtin_bit_cast(
                        float, __builtin_amdgcn_readlane(__builtin_bit_cast(int32_t, dd), s + u));
#pragma unroll
                    for (int c = 0; c < CC; ++c) y[c] = __builtin_fmaf(d, seg_elem<WDT>(w[u], c), y[c]);
                }
            }
        }
    }
    if (inside && !escaped) store_y<YDT, CC>(a.Y, (size_t)row * N + col, y);
}

template <int YDT, int WDT, int CC>
__global__ __launch_bounds__(256) void k_comp_apply(CompArgs a, int chunks, int per_xcd) {
    const int lane = threadIdx.x & 63;
    const int logical = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    const int64_t task = (int64_t)logical * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (task >= (int64_t)chunks * a.M) return;  // whole wave
    const int chunk = (int)(task / a.M);
    const int row = (int)(task - (int64_t)chunk * a.M);
    comp_task<YDT, WDT, CC>(a, row, chunk, lane);
}

// Many entries per row: one wave per (block of 8 rows, chunk of 64 columns) task, lane
// 8r + g on row r of the block and columns 8g .. 8g+7 of the chunk.  The waves an XCD runs
// at once then gather from a W strip 64 columns wide (K x 128 bytes of bf16, 1.8 MB for
// K = 13824), which stays in its 4 MB L2, while every load instruction still moves 16 bytes
// per lane.  Each row's entries go in groups of eight: lane 8r + g loads the row's entry g
// of the group, the group's k reach the row's lanes by lane permutes, and the next group's
// entries are requested with the current group's W segments.  Every load of the entry loop
// is issued unconditionally (absent ones at an offset past their buffer: zeros, no access),
// so the compiler can count what is in flight.
template <int YDT, int WDT>
__global__ __launch_bounds__(256) void k_comp_block64(CompArgs a, int nrb, int per_xcd) {
    constexpr int CC = 8;
    const int lane = threadIdx.x & 63;
    const int logical = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    const int64_t task = (int64_t)logical * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int M = a.M, N = a.N;
    const int chunks = (N + 63) / 64;
    if (task >= (int64_t)chunks * nrb) return;  // whole wave
    const int chunk = (int)(task / nrb);
    const int r0 = (int)(task - (int64_t)chunk * nrb) * 8;
    const int r = lane >> 3, g = lane & 7;
    const int row = r0 + r;
    const int col = chunk * 64 + g * CC;
    const bool inside = row < M && col < N;  // N % 8 == 0: a lane's columns are in range together
    const int rowc = min(row, M - 1);

    const int32_t rp = a.row_ptr[min(r0 + (lane & 15), M)];
    const int32_t e0 = __shfl(rp, r), e1 = row < M ? __shfl(rp, r + 1) : e0;
    const int32_t n = e1 - e0;
    int32_t nmax = n;
#pragma unroll
    for (int o = 8; o < 64; o <<= 1) nmax = max(nmax, __shfl_xor(nmax, o));

    const __amdgpu_buffer_rsrc_t rsS = __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(a.sW), 0, N * 4, 0x00020000);
    const v4i qv = inside ? *reinterpret_cast<const v4i *>(a.Yq + (size_t)rowc * N + col) : v4i{0, 0, 0, 0};
    // the task's 8 rows and 64 columns are one block of the map: its byte from the aligned word
    // that holds it (a uniform, scalar load; the map's row stride is a multiple of 8)
    const size_t mi = (size_t)(r0 / ESC_ROWS) * a.mapN + chunk;
    const uint32_t mword = *reinterpret_cast<const uint32_t *>(a.emap + (mi & ~(size_t)3));
    const bool escaped = ((mword >> (8 * (mi & 3))) & 0xFF) != 0;
    const bool active = inside && !escaped;
    v4i swv[2];
    swv[0] = __builtin_amdgcn_raw_buffer_load_b128(rsS, col * 4, 0, 0);
    swv[1] = __builtin_amdgcn_raw_buffer_load_b128(rsS, col * 4 + 16, 0, 0);
    const float sa = a.sA[rowc];
    float y[CC];
    decode_ymain<CC>(qv, swv, sa, y);

    constexpr int ESZ = (WDT == DT_BF16) ? 2 : 4;
    const __amdgpu_buffer_rsrc_t rsW =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(a.W), 0, (int)((int64_t)a.K * N * ESZ), 0x00020000);
    // the lists through descriptors without a bound of their own (the row offsets bound every
    // real access, as in the chunk tasks); an absent entry's offset is 2^31, past the range
    const __amdgpu_buffer_rsrc_t rsK =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t *>(a.coo_col), 0, 0x7FFFFFFF, 0x00020000);
    const __amdgpu_buffer_rsrc_t rsD =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(a.coo_val), 0, 0x7FFFFFFF, 0x00020000);
    const uint32_t row_bytes = (uint32_t)N * ESZ;
    const uint32_t lane_off = (uint32_t)col * ESZ;
    // entry g of the group starting at e (past the row: an offset past the lists)
    auto load_ent = [&](int e, int32_t &kk, int32_t &dd) {
        const uint32_t off = e + g < n ? (uint32_t)(e0 + e + g) * 4u : 0x80000000u;  // nnz*4 < 2^31
        kk = __builtin_amdgcn_raw_buffer_load_b32(rsK, (int)off, 0, 0);
        dd = __builtin_amdgcn_raw_buffer_load_b32(rsD, (int)off, 0, 0);
    };
    int32_t kk, dd;
    load_ent(0, kk, dd);
    // an escaped block is written by the escape kernel: no entry to walk
    const int32_t nwalk = escaped ? 0 : nmax;
    for (int e = 0; e < nwalk; e += 8) {
        // lane 8r + g turns row r's entry e + g into the byte offset of its W row once (past the
        // row: 2^31, past the buffer, which reads zeros; K*N*ESZ < 2^31), and the row's lanes
        // take the eight offsets by lane permutes
        const uint32_t ko = e + g < n ? (uint32_t)kk * row_bytes : 0x80000000u;
        v4i w[8][2];
        float d[8];
        uint32_t off[8];
        // all sixteen permutes first, so the eight W loads go out back to back
#pragma unroll
        for (int u = 0; u < 8; ++u) off[u] = (uint32_t)__shfl((int)ko, (lane & ~7) + u);
#pragma unroll
        for (int u = 0; u < 8; ++u) d[u] = __int_as_float(__shfl(dd, (lane & ~7) + u));
#pragma unroll
        for (int u = 0; u < 8; ++u) load_seg<WDT, CC>(rsW, off[u] + lane_off, true, w[u]);
        load_ent(e + 8, kk, dd);
        // ascending k.  An entry past the row has d = 0 and reads W as zeros, and fma(0, 0, y)
        // is y exactly (y is never -0: it starts as +0 or nonzero, and an exact cancellation
        // rounds to +0), so every lane runs every step without a branch.
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
            for (int c = 0; c < CC; ++c) y[c] = __builtin_fmaf(d[u], seg_elem<WDT>(w[u], c), y[c]);
    }
    if (active) store_y<YDT, CC>(a.Y, (size_t)row * N + col, y);
}

static hipError_t launch_comp_block64(const CompArgs &a, int y_dt, int w_dt, hipStream_t s) {
    const int nrb = (a.M + 7) / 8;
    const int chunks = (a.N + 63) / 64;
    const int64_t blocks = ((int64_t)nrb * chunks + 3) / 4;
    const int per_xcd = (int)((blocks + 7) / 8);
    const dim3 grid((unsigned)per_xcd * 8u), block(256);
#define C(YD, WD) hipLaunchKernelGGL((k_comp_block64<YD, WD>), grid, block, 0, s, a, nrb, per_xcd)
    if (y_dt == DT_BF16) {
        if (w_dt == DT_BF16) C(DT_BF16, DT_BF16);
        else C(DT_BF16, DT_F32);
    } else {
        if (w_dt == DT_BF16) C(DT_F32, DT_BF16);
        else C(DT_F32, DT_F32);
    }
#undef C
    return hipGetLastError();
}

template <int CC>
static hipError_t launch_comp_tasks(const CompArgs &a, int y_dt, int w_dt, hipStream_t s) {
    const int chunks = (int)((a.N + 64 * CC - 1) / (64 * CC));
    const int64_t tasks = (int64_t)chunks * a.M;
    const int64_t blocks = (tasks + 3) / 4;
    const int per_xcd = (int)((blocks + 7) / 8);
    const dim3 grid((unsigned)per_xcd * 8u), block(256);
#define C(YD, WD) hipLaunchKernelGGL((k_comp_apply<YD, WD, CC>), grid, block, 0, s, a, chunks, per_xcd)
    if (y_dt == DT_BF16) {
        if (w_dt == DT_BF16) C(DT_BF16, DT_BF16);
        else C(DT_BF16, DT_F32);
    } else {
        if (w_dt == DT_BF16) C(DT_F32, DT_BF16);
        else C(DT_F32, DT_F32);
    }
#undef C
    return hipGetLastError();
}

int comp_kernel_choice(int64_t M, int64_t capacity) { return capacity > 64 * M ? COMP_BLOCK64 : COMP_CHUNK; }

hipError_t launch_comp(const int16_t *Yq, const uint8_t *emap, const float *sA, const float *sW, void *Y, int y_dt,
                       int64_t M, int64_t N, int64_t K, const int32_t *row_ptr, const int32_t *coo_col,
                       const float *coo_val, const void *W, int w_dt, int64_t capacity, hipStream_t s) {
    const CompArgs a{Yq, emap, esc_map_stride(N), sA, sW, Y, (int)M, (int)N, (int)K, row_ptr, coo_col, coo_val, W};
    // the list's capacity bounds the mean entries per row; past 64 the pass is bound by its
    // gathers, and the 8-row x 64-column blocks keep each XCD's W strip in its L2
    if (comp_kernel_choice(M, capacity) == COMP_BLOCK64) return launch_comp_block64(a, y_dt, w_dt, s);
    return launch_comp_tasks<8>(a, y_dt, w_dt, s);
}

}  // namespace fp4
