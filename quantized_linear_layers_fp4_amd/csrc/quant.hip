// gfx950 kernels of the bandwidth-bound half of the FP4 linear forward:
//   - |A| histogram + raw row maxima, order-statistic select of the quantile threshold T
//     (outlier paragraph of the QbitAI report on "Optimizing Large Language Model Training
//     Using FP4 Quantization": outliers are found by a quantile search over A);
//   - clamp of A to [-T, T], token-wise E2M1 quantization and staging of dA in column order
//     (granularity, forward-quantization and outlier paragraphs of the same report);
//   - exclusive scan + scatter that turns the staging into the (row, col)-sorted COO list;
//   - channel-wise column maxima and transposed E2M1 packing of W (granularity paragraph).
#include "fp4_common.h"
#include "fp4_launch.h"

namespace fp4 {

// ----------------------------------------------------------------------------- zero fill
// Zeroes p1[0..n1) and p2[0..n2) (n2 may be 0) in one launch.
__global__ void k_zero_u32(uint32_t *__restrict__ p1, int64_t n1, uint32_t *__restrict__ p2, int64_t n2) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n1 + n2; i += stride) {
        if (i < n1) p1[i] = 0u;
        else p2[i - n1] = 0u;
    }
}

// ----------------------------------------------------------------------------- select
// Level 1 (the 32768 high bins, rank k computed on the host) by one workgroup of 256 threads:
// thread t sums bins [128t, 128t + 128), a scan over the threads finds the one whose range
// holds rank k, and wave 0 then finds the bin among those 128 (two per lane).  For bf16
// inputs the bin fixes T; for fp32 inputs it leaves the rank within the bin to level 2.  Every
// count and partial sum is at most M*K < 2^32.  It needs no more than 256 threads and a few
// registers, so it can run as one workgroup of a launch that does other work.
__device__ __forceinline__ void select_hi_256(const uint32_t *__restrict__ hist, State *__restrict__ st,
                                              int final_level, float *__restrict__ T_out, uint64_t k) {
    constexpr int PER = HIST_BINS / 256;
    __shared__ uint32_t wsum[4];
    __shared__ uint32_t sel_s[2];  // the thread whose bins hold rank k, and the count before them
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint4 *src = reinterpret_cast<const uint4 *>(hist + tid * PER);
    uint32_t local = 0;
    for (int r = 0; r < PER / 4; r += 8) {
        uint4 q[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) q[u] = src[r + u];
#pragma unroll
        for (int u = 0; u < 8; ++u) local += q[u].x + q[u].y + q[u].z + q[u].w;
    }
    const uint32_t wincl = wave_incl_scan(local, lane);
    if (lane == 63) wsum[wave] = wincl;
    if (tid == 0) {  // a default in range, should the histogram not hold rank k (it always does)
        sel_s[0] = 0;
        sel_s[1] = 0;
    }
    __syncthreads();
    uint32_t before = 0;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    const uint64_t total = (uint64_t)wsum[0] + wsum[1] + wsum[2] + wsum[3];
    const uint64_t incl = (uint64_t)before + wincl, excl = incl - local;
    if (excl <= k && k < incl) {  // exactly one thread: k < total
        sel_s[0] = (uint32_t)tid;
        sel_s[1] = (uint32_t)excl;
    }
    __syncthreads();
    if (wave != 0) return;
    const int t = (int)sel_s[0];
    const uint2 p = reinterpret_cast<const uint2 *>(hist + t * PER)[lane];
    const uint32_t pc = p.x + p.y;
    const uint64_t pex = (uint64_t)sel_s[1] + wave_incl_scan(pc, lane) - pc;  // entries before bin t*PER + 2*lane
    if (pex <= k && k < pex + pc) {
        const bool first = k < pex + p.x;
        const uint32_t b = (uint32_t)(t * PER + 2 * lane + (first ? 0 : 1));
        const uint32_t cnt = first ? p.x : p.y;
        const uint64_t cum = first ? pex : pex + p.x;
        st->hi_bin = b;
        st->hi_count = cnt;
        st->k_rem = k - cum;
        st->nnz_hist = total - (cum + cnt);  // entries in later bins
        if (final_level == 1) {
            st->T_key = b << 16;
            st->T = __uint_as_float(b << 16);
            *T_out = st->T;
        }
    }
}

// Level 2 for fp32 inputs: rank st->k_rem among the 65536 low bins of the selected high bin,
// found by the 1024 threads of one workgroup; it fixes T.
__device__ __forceinline__ void select_lo_1024(const uint32_t *__restrict__ hist, State *__restrict__ st,
                                               float *__restrict__ T_out) {
    constexpr int PER = HIST_LO_BINS / 1024;
    __shared__ uint32_t wsum[16];
    __shared__ uint32_t total_s;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // the thread's PER consecutive bins stay in registers for the search below
    uint32_t cnts[PER];
#pragma unroll
    for (int i = 0; i < PER; i += 4) {
        const uint4 q = *reinterpret_cast<const uint4 *>(hist + tid * PER + i);
        cnts[i] = q.x;
        cnts[i + 1] = q.y;
        cnts[i + 2] = q.z;
        cnts[i + 3] = q.w;
    }
    uint32_t local = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) local += cnts[i];
    const uint32_t wincl = wave_incl_scan(local, lane);
    if (lane == 63) wsum[wave] = wincl;
    __syncthreads();
    if (wave == 0) {
        const uint32_t x = lane < 16 ? wsum[lane] : 0u;
        const uint32_t xi = wave_incl_scan(x, lane);
        if (lane < 16) wsum[lane] = xi - x;  // exclusive prefix of the waves
        if (lane == 15) total_s = xi;
    }
    __syncthreads();
    const uint64_t incl = (uint64_t)wsum[wave] + wincl, excl = incl - local, total = total_s;
    const uint64_t k = st->k_rem;
    if (excl <= k && k < incl) {
        // the bin of rank k among the thread's bins: branch-free over the registers
        uint64_t cum = excl;
        int bi = PER - 1;
        uint32_t cnt = cnts[PER - 1];
        uint64_t before = excl;
        bool found = false;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const bool here = !found && k < cum + cnts[i];
            if (here) {
                bi = i;
                cnt = cnts[i];
                before = cum;
            }
            found = found || here;
            cum += cnts[i];
        }
        const uint32_t b = (uint32_t)(tid * PER + bi);
        const uint64_t above = total - (before + cnt);  // entries in later bins
        const uint32_t key = (st->hi_bin << 16) | b;
        st->T_key = key;
        st->T = __uint_as_float(key);
        st->nnz_hist += above;
        *T_out = st->T;
    }
}

// ----------------------------------------------------------------------------- histogram
// One workgroup of 1024 threads per CU holds a 32768-bin histogram of key >> 16 in LDS
// (128 KiB); a wave owns one row at a time and also reduces the row's maximum key.
// Rows [r0, r1) of the block are contiguous.  Non-empty bins are merged with global atomics.
// (Selecting in the workgroup that merges last, behind a device-scope fence and a ticket, was
// measured and dropped: on this multi-XCD part the fences took 76 us, the select launch 8.)
template <int DT>
__global__ __launch_bounds__(1024) void k_hist_rowmax(const void *__restrict__ A, int64_t M, int64_t K,
                                                      uint32_t *__restrict__ ghist,
                                                      uint32_t *__restrict__ rowmax_key) {
    __shared__ uint32_t h[HIST_BINS];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int i = tid; i < HIST_BINS; i += 1024) h[i] = 0u;
    __syncthreads();
    const int64_t rows_per = (M + gridDim.x - 1) / gridDim.x;
    const int64_t r0 = blockIdx.x * rows_per;
    const int64_t r1 = min(M, r0 + rows_per);
    const int64_t nchunk = K / 8;  // 8 elements per chunk
    constexpr int U = (DT == DT_BF16) ? 8 : 4;     // chunks per lane per memory round trip
    constexpr int WPC = (DT == DT_BF16) ? 1 : 2;   // 16-byte words per chunk of 8 elements
    for (int64_t row = r0 + wave; row < r1; row += 16) {
        const int64_t base = row * K;
        uint32_t mx = 0;
        for (int64_t c0 = 0; c0 < nchunk; c0 += 64 * U) {
            uint4 raw[U][WPC];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t c = c0 + u * 64 + lane;
                if (c < nchunk) {
                    const uint4 *src = reinterpret_cast<const uint4 *>(
                        reinterpret_cast<const uint8_t *>(A) + (base + c * 8) * (DT == DT_BF16 ? 2 : 4));
#pragma unroll
                    for (int w = 0; w < WPC; ++w) raw[u][w] = src[w];
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (c0 + u * 64 + lane < nchunk) {
#pragma unroll
                    for (int w = 0; w < WPC; ++w) {
                        const uint32_t wd[4] = {raw[u][w].x, raw[u][w].y, raw[u][w].z, raw[u][w].w};
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            if constexpr (DT == DT_BF16) {
                                const uint32_t k0 = key_of_bf16(wd[i] & 0xFFFFu), k1 = key_of_bf16(wd[i] >> 16);
                                atomicAdd(&h[k0 >> 16], 1u);
                                atomicAdd(&h[k1 >> 16], 1u);
                                mx = max(mx, max(k0, k1));
                            } else {
                                const uint32_t k0 = key_of_f32(wd[i]);
                                atomicAdd(&h[k0 >> 16], 1u);
                                mx = max(mx, k0);
                            }
                        }
                    }
                }
            }
        }
        mx = wave_max_u32(mx);
        if (lane == 0) rowmax_key[row] = mx;
    }
    __syncthreads();
    for (int i = tid; i < HIST_BINS; i += 1024) {
        uint32_t c = h[i];
        if (c) atomicAdd(&ghist[i], c);
    }
}

// The level-1 select alone (one workgroup of 256 threads).
__global__ __launch_bounds__(256) void k_select_hi(const uint32_t *__restrict__ hist, State *__restrict__ st,
                                                   int final_level, float *__restrict__ T_out, uint64_t k_level1) {
    select_hi_256(hist, st, final_level, T_out, k_level1);
}

// Second level for fp32 inputs: among the entries whose key >> 16 is the selected bin,
// histogram the low 16 bits (few entries: global atomics).
__global__ __launch_bounds__(256) void k_hist_lo(const uint32_t *__restrict__ A, int64_t n,
                                                 const State *__restrict__ st,
                                                 uint32_t *__restrict__ ghist_lo) {
    const uint32_t hi = st->hi_bin;
    int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += stride) {
        uint32_t k = key_of_f32(A[i]);
        if ((k >> 16) == hi) atomicAdd(&ghist_lo[k & 0xFFFFu], 1u);
    }
}

// The level-2 select of fp32 inputs (one workgroup).
__global__ __launch_bounds__(1024) void k_select_lo(const uint32_t *__restrict__ hist_lo, State *__restrict__ st,
                                                    float *__restrict__ T_out) {
    select_lo_1024(hist_lo, st, T_out);
}

// ----------------------------------------------------------------------------- rows (A)
// One wave per row.  Optionally clamps to [-T, T] (T from *T_src), writes the row's E2M1
// codes and scale, and stages the clamped-away residuals dA in ascending column order.
//   HAVE_ROWMAX: the raw row maximum key comes from rowmax_key (histogram pass); otherwise
//                a first sweep over the row computes it.
template <int DT, bool CLAMP, bool HAVE_ROWMAX, bool CODES, bool EMIT>
__global__ __launch_bounds__(256) void k_quant_rows(const void *__restrict__ X, int64_t R, int64_t C,
                                                    const uint32_t *__restrict__ rowmax_key,
                                                    const float *__restrict__ T_src,
                                                    uint8_t *__restrict__ codes, float *__restrict__ scales,
                                                    int32_t *__restrict__ row_cnt, Staging stg,
                                                    State *__restrict__ st) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= R) return;  // whole wave exits together
    const int64_t base = row * C;
    const int64_t nchunk = C / 8;
    const uint32_t tkey = CLAMP ? key_of_f32(__float_as_uint(*T_src)) : 0xFFFFFFFFu;

    uint32_t mx = 0;
    if constexpr (HAVE_ROWMAX) {
        mx = rowmax_key[row];
    } else if constexpr (CODES) {
        for (int64_t c = lane; c < nchunk; c += 64) {
            float v[8];
            uint32_t key[8], sg[8];
            load8<DT>(X, base + c * 8, v, key, sg);
#pragma unroll
            for (int e = 0; e < 8; ++e) mx = max(mx, key[e]);
        }
        mx = wave_max_u32(mx);
    }
    mx = min(mx, tkey);  // max |clamp(a)| = min(max |a|, T)
    float r = 0.0f, s = 0.0f;
    if constexpr (CODES) {
        vector_scale(__uint_as_float(mx), r, s);
        if (lane == 0) scales[row] = s;
    }
    uint32_t running = 0;  // outliers of this row emitted so far
    // U chunks of 8 elements per lane are loaded before any is processed, so a row of
    // 64*8*U elements costs one memory round trip.  Chunks are processed in ascending
    // column order (the staging order of dA).
    constexpr int U = (DT == DT_BF16) ? 8 : 4;
    constexpr int WPC = (DT == DT_BF16) ? 1 : 2;  // 16-byte words per chunk
    for (int64_t c0 = 0; c0 < nchunk; c0 += 64 * U) {
        uint4 raw[U][WPC];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t c = c0 + u * 64 + lane;
            if (c < nchunk) {
                const uint4 *src = reinterpret_cast<const uint4 *>(
                    reinterpret_cast<const uint8_t *>(X) + (base + c * 8) * (DT == DT_BF16 ? 2 : 4));
#pragma unroll
                for (int w = 0; w < WPC; ++w) raw[u][w] = src[w];
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t c = c0 + u * 64 + lane;
            if (c0 + u * 64 >= nchunk) break;  // wave-uniform: no lane has chunk u
            const bool valid = c < nchunk;
            float v[8];
            uint32_t key[8], sg[8];
            if constexpr (DT == DT_BF16) {
                const uint32_t wd[4] = {raw[u][0].x, raw[u][0].y, raw[u][0].z, raw[u][0].w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t lo = wd[i] & 0xFFFFu, hi = wd[i] >> 16;
                    v[2 * i] = bf16_to_f32(lo);
                    v[2 * i + 1] = bf16_to_f32(hi);
                    key[2 * i] = key_of_bf16(lo);
                    key[2 * i + 1] = key_of_bf16(hi);
                    sg[2 * i] = (lo << 16) & 0x80000000u;
                    sg[2 * i + 1] = (hi << 16) & 0x80000000u;
                }
            } else {
                const uint32_t wd[8] = {raw[u][0].x, raw[u][0].y, raw[u][0].z, raw[u][0].w,
                                        raw[u][1].x, raw[u][1].y, raw[u][1].z, raw[u][1].w};
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    v[i] = __uint_as_float(wd[i]);
                    key[i] = key_of_f32(wd[i]);
                    sg[i] = wd[i] & 0x80000000u;
                }
            }
            uint32_t omask = 0;
            float y[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const bool out = valid && key[e] > tkey;
                omask |= (uint32_t)out << e;
                const float ac = out ? __uint_as_float(sg[e] | tkey) : v[e];
                y[e] = ac * r;
            }
            if constexpr (CODES) {
                if (valid) *reinterpret_cast<uint32_t *>(codes + row * (C / 2) + c * 4) = e2m1_pack8(y);
            }
            if constexpr (EMIT) {
                if (__ballot(omask != 0)) {
                    // rank of this lane's first outlier = outliers in the lower lanes: one
                    // ballot per element position, counted below the lane with mbcnt (no
                    // cross-lane shuffles, whose LDS round trips made this path slow)
                    uint32_t before = 0, total = 0;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const uint64_t b = __ballot((omask >> e) & 1u);
                        before += __builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32),
                                                            __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0u));
                        total += (uint32_t)__popcll(b);
                    }
                    uint32_t rank = running + before;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        if (omask & (1u << e)) {
                            const int32_t col = (int32_t)(c * 8 + e);
                            const float val = v[e] - __uint_as_float(sg[e] | tkey);
                            if (rank < (uint32_t)stg.S) {  // ranks past S: see k_coo_build
                                SlotEntry se;
                                se.col = col;
                                se.val = val;
                                stg.slots[row * stg.S + rank] = se;
                            }
                            ++rank;
                        }
                    }
                    running += total;
                }
            }
        }
    }
    if constexpr (EMIT) {
        if (lane == 0) row_cnt[row] = (int32_t)running;
    }
}

// ----------------------------------------------------------------------------- COO
// Exclusive scan of the per-row outlier counts (one workgroup of 1024 threads, 16 rows
// per thread per pass, wave scans + one cross-wave step).  Used ahead of k_coo_build when
// M is too large for every workgroup of that kernel to sum the counts before its rows.
__global__ __launch_bounds__(1024) void k_coo_scan(const int32_t *__restrict__ row_cnt, int64_t M,
                                                   int32_t *__restrict__ row_ptr,
                                                   int64_t *__restrict__ nnz_out) {
    constexpr int ITEMS = 16;
    __shared__ uint32_t wsum[16];
    __shared__ uint32_t carry_s;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint32_t carry = 0;
    for (int64_t b0 = 0; b0 < M; b0 += 1024 * ITEMS) {
        uint32_t c[ITEMS], local = 0;
        const int64_t r0 = b0 + (int64_t)tid * ITEMS;
        if (r0 + ITEMS <= M) {
            // row_cnt is 16-byte aligned and r0 a multiple of 16: four 16-byte loads
#pragma unroll
            for (int i = 0; i < ITEMS; i += 4) {
                const int4 q = *reinterpret_cast<const int4 *>(row_cnt + r0 + i);
                c[i] = (uint32_t)q.x;
                c[i + 1] = (uint32_t)q.y;
                c[i + 2] = (uint32_t)q.z;
                c[i + 3] = (uint32_t)q.w;
            }
        } else {
#pragma unroll
            for (int i = 0; i < ITEMS; ++i) c[i] = (r0 + i < M) ? (uint32_t)row_cnt[r0 + i] : 0u;
        }
#pragma unroll
        for (int i = 0; i < ITEMS; ++i) local += c[i];
        const uint32_t incl = wave_incl_scan(local, lane);
        if (lane == 63) wsum[wave] = incl;
        __syncthreads();
        if (wave == 0) {
            uint32_t x = lane < 16 ? wsum[lane] : 0u;
            const uint32_t xi = wave_incl_scan(x, lane);
            if (lane < 16) wsum[lane] = xi - x;  // exclusive
            if (lane == 15) carry_s = xi;          // total of this pass
        }
        __syncthreads();
        uint32_t run = carry + wsum[wave] + incl - local;
        int32_t out[ITEMS];
#pragma unroll
        for (int i = 0; i < ITEMS; ++i) {
            out[i] = (int32_t)run;
            run += c[i];
        }
        if (r0 + ITEMS <= M) {
#pragma unroll
            for (int i = 0; i < ITEMS; i += 4)
                *reinterpret_cast<int4 *>(row_ptr + r0 + i) = make_int4(out[i], out[i + 1], out[i + 2], out[i + 3]);
        } else {
#pragma unroll
            for (int i = 0; i < ITEMS; ++i)
                if (r0 + i < M) row_ptr[r0 + i] = out[i];
        }
        carry += carry_s;
        __syncthreads();
    }
    if (tid == 0) {
        row_ptr[M] = (int32_t)carry;
        *nnz_out = (int64_t)carry;
    }
}

// The outliers of rank >= S of one row that outgrew its staging slots: the row of A is read
// again, its outliers ranked as the quantize pass ranked them (ascending column), and those of
// rank >= S written straight to row_ptr[row] + rank.
template <int DT>
__device__ __forceinline__ void coo_overflow_row(int64_t row, int64_t base, int32_t S, int64_t cap,
                                                 const void *__restrict__ A, int64_t K, uint32_t tkey, int lane,
                                                 int32_t *__restrict__ coo_row, int32_t *__restrict__ coo_col,
                                                 float *__restrict__ coo_val) {
    const int64_t nchunk = K / 8;
    uint32_t run = 0;
    // U chunks of 8 per lane are loaded together: one memory round trip per 512*U elements
    // (rows this long are rare; a small U keeps the registers of the COO build low)
    constexpr int U = 2;
    for (int64_t cg = 0; cg < nchunk; cg += 64 * U) {
        float vv[U][8];
        uint32_t kk[U][8], ss[U][8];
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (cg + u * 64 + lane < nchunk) load8<DT>(A, row * K + (cg + u * 64 + lane) * 8, vv[u], kk[u], ss[u]);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t c = cg + u * 64 + lane;
            const float *v = vv[u];
            const uint32_t *sg = ss[u];
            uint32_t omask = 0;
            if (c < nchunk) {
#pragma unroll
                for (int e = 0; e < 8; ++e) omask |= (uint32_t)(kk[u][e] > tkey) << e;
            }
            uint32_t before = 0, total = 0;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint64_t b = __ballot((omask >> e) & 1u);
                before += __builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0u));
                total += (uint32_t)__popcll(b);
            }
            uint32_t rank = run + before;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                if (omask & (1u << e)) {
                    const int64_t pos = base + rank;
                    if (rank >= (uint32_t)S && pos < cap) {
                        if (coo_row) coo_row[pos] = (int32_t)row;
                        coo_col[pos] = (int32_t)(c * 8 + e);
                        coo_val[pos] = v[e] - __uint_as_float(sg[e] | tkey);
                    }
                    ++rank;
                }
            }
            run += total;
        }
    }
}

// The (row, col)-sorted COO list from the staging, one workgroup per 64 rows:
//   1. PREFIX: the row offset of the workgroup's first row is the sum of the counts before it,
//      which the workgroup reads itself (at most COO_PREFIX_ROWS counts, from L2), so no
//      separate scan launch precedes it; otherwise row_ptr was written by k_coo_scan;
//   2. a wave scan of the 64 counts gives the rows' offsets (row_ptr, and nnz from the last);
//   3. the 256 threads copy the staged entries (ranks below S) of the 64 rows as one list;
//   4. rows that outgrew their slots are read again for their ranks >= S.
constexpr int64_t COO_PREFIX_ROWS = 16384;
template <int DT, bool PREFIX>
__device__ __forceinline__ void coo_block(Staging stg, const int32_t *__restrict__ row_cnt,
                                          int32_t *__restrict__ row_ptr, int64_t *__restrict__ nnz_out, int64_t M,
                                          int64_t cap, int32_t *__restrict__ coo_row, int32_t *__restrict__ coo_col,
                                          float *__restrict__ coo_val, const void *__restrict__ A, int64_t K,
                                          const float *__restrict__ T_src, int bx) {
    __shared__ uint32_t wsum[4];
    __shared__ int32_t off_s[64], cnt_s[64], sc_s[65];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t r0 = (int64_t)bx * 64;
    // wave 0's lanes hold the counts of the workgroup's 64 rows; their load is issued together
    // with the prefix loads (one memory round trip for both)
    const int64_t rl = r0 + lane;
    const uint32_t c = (wave == 0 && rl < M) ? (uint32_t)row_cnt[rl] : 0u;
    uint32_t base = 0;
    if constexpr (PREFIX) {
        // row_cnt is 16-byte aligned and r0 a multiple of 64: whole 16-byte groups, at most
        // COO_PREFIX_ROWS / 1024 of them per thread, in two rounds of loads issued together
        constexpr int PI = (int)(COO_PREFIX_ROWS / 1024), PH = PI / 2;
        uint32_t part = 0;
#pragma unroll 1
        for (int h = 0; h < PI / PH; ++h) {
            int4 q[PH];
#pragma unroll
            for (int u = 0; u < PH; ++u) {
                const int64_t i = (int64_t)tid * 4 + (int64_t)(h * PH + u) * 1024;
                q[u] = i < r0 ? *reinterpret_cast<const int4 *>(row_cnt + i) : make_int4(0, 0, 0, 0);
            }
#pragma unroll
            for (int u = 0; u < PH; ++u) part += (uint32_t)q[u].x + (uint32_t)q[u].y + (uint32_t)q[u].z + (uint32_t)q[u].w;
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) part += (uint32_t)__shfl_xor((int)part, o, 64);
        if (lane == 0) wsum[wave] = part;
        __syncthreads();
        base = wsum[0] + wsum[1] + wsum[2] + wsum[3];
    }
    if (wave == 0) {
        const uint32_t incl = wave_incl_scan(c, lane);
        int32_t off;
        if constexpr (PREFIX) {
            off = (int32_t)(base + incl - c);
            if (rl < M) row_ptr[rl] = off;
            if (rl == M - 1) {
                row_ptr[M] = (int32_t)(base + incl);
                *nnz_out = (int64_t)(base + incl);
            }
        } else {
            off = rl < M ? row_ptr[rl] : 0;
        }
        off_s[lane] = off;
        cnt_s[lane] = (int32_t)c;
        // the rows' staged entries (ranks below S) as one flat list: its prefix
        const uint32_t st = min(c, (uint32_t)stg.S);
        const uint32_t sincl = wave_incl_scan(st, lane);
        sc_s[lane] = (int32_t)(sincl - st);
        if (lane == 63) sc_s[64] = (int32_t)sincl;
    }
    __syncthreads();
    // the row of entry e is found by a binary search in the rows' staged-count prefix
    for (int32_t e = tid; e < sc_s[64]; e += 256) {
        int lo = 0, hi = 64;  // the last j with sc_s[j] <= e (rows with no staged entry are skipped)
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (sc_s[mid] <= e) lo = mid;
            else hi = mid;
        }
        const int32_t t = e - sc_s[lo];
        const int64_t row = r0 + lo;
        const SlotEntry se = stg.slots[row * stg.S + t];
        const int64_t pos = (int64_t)off_s[lo] + t;
        if (pos < cap) {
            if (coo_row) coo_row[pos] = (int32_t)row;
            coo_col[pos] = se.col;
            coo_val[pos] = se.val;
        }
    }
    // rows past S are rare (S is at least 128 and twice the mean count plus a margin)
    const uint64_t todo = __ballot(r0 + lane < M && cnt_s[lane] > stg.S);  // the same in every wave
    if (!todo) return;
    const uint32_t tkey = key_of_f32(__float_as_uint(*T_src));
    uint64_t t = todo;
    for (int i = 0; t; ++i) {
        const int bit = __builtin_ctzll(t);
        t &= t - 1;
        if ((i & 3) != wave) continue;  // dealt to the four waves in turn
        coo_overflow_row<DT>(r0 + bit, off_s[bit], stg.S, cap, A, K, tkey, lane, coo_row, coo_col, coo_val);
    }
}

template <int DT, bool PREFIX>
__global__ __launch_bounds__(256) void k_coo_build(Staging stg, const int32_t *__restrict__ row_cnt,
                                                   int32_t *__restrict__ row_ptr, int64_t *__restrict__ nnz_out,
                                                   int64_t M, int64_t cap, int32_t *__restrict__ coo_row,
                                                   int32_t *__restrict__ coo_col, float *__restrict__ coo_val,
                                                   const void *__restrict__ A, int64_t K,
                                                   const float *__restrict__ T_src) {
    coo_block<DT, PREFIX>(stg, row_cnt, row_ptr, nnz_out, M, cap, coo_row, coo_col, coo_val, A, K, T_src, blockIdx.x);
}

// ----------------------------------------------------------------------------- columns (W)
// Row k of the matrix as quantized: the input itself, or (RM) fl(row_mult[k] * x), the
// form the backward quantizes per column.
template <int DT, bool RM>
__device__ __forceinline__ void load8_rm(const void *__restrict__ W, const float *__restrict__ row_mult, int64_t k,
                                         int64_t N, int64_t col, float v[8], uint32_t key[8]) {
    uint32_t sg[8];
    load8<DT>(W, k * N + col, v, key, sg);
    if constexpr (RM) {
        const float m = row_mult[k];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            v[e] = m * v[e];
            key[e] = __float_as_uint(v[e]) & 0x7FFFFFFFu;
        }
    }
}

// Column maxima of K x N W (keys), merged with atomicMax into colmax_key (zeroed before).
// Tile (bx, by): 256 threads = 4 waves over the same 512 columns (8 per lane), rows split by wave.
template <int DT, bool RM>
__device__ __forceinline__ void colmax_tile(const void *__restrict__ W, int64_t K, int64_t N, int rows_per_block,
                                            const float *__restrict__ row_mult, uint32_t *__restrict__ colmax_key,
                                            int bx, int by) {
    __shared__ uint32_t red[4][512];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t col = (int64_t)bx * 512 + lane * 8;
    const int64_t r0 = (int64_t)by * rows_per_block;
    const int64_t r1 = min(K, r0 + rows_per_block);
    uint32_t mx[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (col < N) {
        int64_t r = r0 + wave;
        for (; r + 12 < r1; r += 16) {
            float v[4][8];
            uint32_t key[4][8];
#pragma unroll
            for (int u = 0; u < 4; ++u) load8_rm<DT, RM>(W, row_mult, r + 4 * u, N, col, v[u], key[u]);
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int e = 0; e < 8; ++e) mx[e] = max(mx[e], key[u][e]);
        }
        for (; r < r1; r += 4) {
            float v[8];
            uint32_t key[8];
            load8_rm<DT, RM>(W, row_mult, r, N, col, v, key);
#pragma unroll
            for (int e = 0; e < 8; ++e) mx[e] = max(mx[e], key[e]);
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) red[wave][lane * 8 + e] = mx[e];
    __syncthreads();
    for (int i = threadIdx.x; i < 512; i += 256) {
        uint32_t m = max(max(red[0][i], red[1][i]), max(red[2][i], red[3][i]));
        int64_t c = (int64_t)bx * 512 + i;
        if (c < N && m) atomicMax(&colmax_key[c], m);
    }
}

template <int DT, bool RM>
__global__ __launch_bounds__(256) void k_colmax(const void *__restrict__ W, int64_t K, int64_t N,
                                                int rows_per_block, const float *__restrict__ row_mult,
                                                uint32_t *__restrict__ colmax_key) {
    colmax_tile<DT, RM>(W, K, N, rows_per_block, row_mult, colmax_key, blockIdx.x, blockIdx.y);
}

// Quantize a 256 (k) x TN (n) tile of W with the finished column maxima and write it
// transposed: Wq[n][k/2].  Loads: TN/8 threads per row (16 bytes = 8 columns each); each thread
// takes 8 consecutive rows (4 pairs of k) of its 8 columns, so it forms 4 output bytes of each
// column in a register and writes them to LDS as one dword.  The transpose tile holds a column's
// 128 bytes (256 values of k) as 32 dwords; dword j of column c sits at j ^ 4*((c/8) % 8), which
// spreads a wave's writes over all banks (two lanes per bank) and keeps each 16-byte group whole
// for the read-out, which writes 128-byte rows of Wq.
// scales_out: NULL, or fp32[N] (a buffer other than the keys) that the workgroups of the first
// tile row fill with the dequantization scales of their columns.
template <int DT, bool RM, int TN>
__device__ __forceinline__ void qcols_tile(const void *__restrict__ W, int64_t K, int64_t N,
                                           const float *__restrict__ row_mult,
                                           const uint32_t *__restrict__ colmax_key, uint8_t *__restrict__ codes,
                                           float *__restrict__ scales_out, int bx, int by) {
    constexpr int TPR = TN / 8;         // threads per row
    constexpr int GPP = 256 / TPR;      // groups of 8 rows per pass
    constexpr int PASSES = 32 / GPP;    // 32 groups of 8 rows = 256 rows per tile
    constexpr int TPN = 256 / TN;       // threads per output row
    constexpr int DPT = 32 / TPN;       // output dwords per thread
    __shared__ float rs[TN];
    __shared__ __attribute__((aligned(16))) uint32_t tile[TN][32];
    const int tid = threadIdx.x;
    const int64_t n0 = (int64_t)bx * TN, k0 = (int64_t)by * 256;
    if (tid < TN) {
        float r = 0.0f, s;
        if (n0 + tid < N) {
            vector_scale(__uint_as_float(colmax_key[n0 + tid]), r, s);
            if (scales_out && by == 0) scales_out[n0 + tid] = s;
        }
        rs[tid] = r;
    }
    __syncthreads();
    const int c8 = tid % TPR;         // columns n0 + 8*c8 .. +7
    const int64_t col = n0 + c8 * 8;
    const int swz = 4 * (c8 & 7);     // the dword swizzle of the thread's columns
    float r8[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) r8[e] = rs[c8 * 8 + e];
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        const int jj = tid / TPR + GPP * p;  // rows 8*jj .. 8*jj+7 of the tile: output dword jj
        const int64_t k = k0 + 8 * jj;
        uint32_t w[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        if (col < N && k < K) {  // K % 32 == 0: the 8 rows are in range together
            float v[8][8];
            uint32_t key[8][8];
#pragma unroll
            for (int q = 0; q < 8; ++q) load8_rm<DT, RM>(W, row_mult, k + q, N, col, v[q], key[q]);
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    w[e] |= (e2m1_pack2<0>(0u, v[2 * q][e] * r8[e], v[2 * q + 1][e] * r8[e]) & 0xFFu) << (8 * q);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) tile[c8 * 8 + e][jj ^ swz] = w[e];
    }
    __syncthreads();
    // write out: n = tid / TPN, DPT dwords (8*DPT values of k) per thread
    const int nl = tid / TPN, part = tid % TPN;
    const int64_t n = n0 + nl;
    const int rswz = 4 * ((nl >> 3) & 7);
    const int64_t kb = k0 / 2 + part * DPT * 4;  // byte offset within the row of Wq
    if (n < N) {
#pragma unroll
        for (int h = 0; h < DPT / 4; ++h) {
            if (kb + h * 16 < K / 2) {
                const uint4 q = *reinterpret_cast<const uint4 *>(&tile[nl][(part * DPT + 4 * h) ^ rswz]);
                *reinterpret_cast<uint4 *>(codes + n * (K / 2) + kb + h * 16) = q;
            }
        }
    }
}

template <int DT, bool RM, int TN>
__global__ __launch_bounds__(256) void k_quant_cols(const void *__restrict__ W, int64_t K, int64_t N,
                                                    const float *__restrict__ row_mult,
                                                    const uint32_t *__restrict__ colmax_key,
                                                    uint8_t *__restrict__ codes, float *__restrict__ scales_out) {
    qcols_tile<DT, RM, TN>(W, K, N, row_mult, colmax_key, codes, scales_out, blockIdx.x, blockIdx.y);
}

// Column width of the transposing tile: 128 (256-byte row segments of the input; 3 % faster
// than 64 on the 16384 x 22016 gradient, equal on the 4096 x 22016 weight).  A compile-time
// tuning aid: 64 or 128.
#ifndef FP4_QCOLS_TN
#define FP4_QCOLS_TN 128
#endif
static_assert(FP4_QCOLS_TN == 64 || FP4_QCOLS_TN == 128, "FP4_QCOLS_TN is 64 or 128");

template <int DT, bool RM>
static void launch_qcols_tile(const void *W, int64_t K, int64_t N, const float *row_mult, const uint32_t *keys,
                              uint8_t *codes, float *scales_out, hipStream_t s) {
    if constexpr (FP4_QCOLS_TN == 128) {
        dim3 g((unsigned)((N + 127) / 128), (unsigned)((K + 255) / 256));
        hipLaunchKernelGGL((k_quant_cols<DT, RM, 128>), g, dim3(256), 0, s, W, K, N, row_mult, keys, codes, scales_out);
    } else {
        dim3 g((unsigned)((N + 63) / 64), (unsigned)((K + 255) / 256));
        hipLaunchKernelGGL((k_quant_cols<DT, RM, 64>), g, dim3(256), 0, s, W, K, N, row_mult, keys, codes, scales_out);
    }
}

// Column maxima keys -> dequantization scales, in place.
__global__ void k_col_scales(uint32_t *__restrict__ colmax_key_then_scale, int64_t N) {
    int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (i < N) {
        float r, s;
        vector_scale(__uint_as_float(colmax_key_then_scale[i]), r, s);
        colmax_key_then_scale[i] = __float_as_uint(s);
    }
}

// ----------------------------------------------------------------------------- shared launches
// When the forward quantizes A and W in one call, the W side's two passes share launches with
// the A side's latency-bound steps, which are independent of them: the level-1 select (one
// workgroup) runs beside W's column maxima, and the COO build beside W's quantize pass.  Each
// workgroup takes one part by its index (a uniform branch), so both parts keep their own
// tiling; the short A-side workgroups come first in the dispatch order.
constexpr int COLMAX_ROWS = 256;  // rows of W per column-maximum workgroup

template <int DT>
__global__ __launch_bounds__(256) void k_select_colmax(const uint32_t *__restrict__ hist, State *__restrict__ st,
                                                       int final_level, float *__restrict__ T_out, uint64_t k_level1,
                                                       WSide w, int gx) {
    if (blockIdx.x == 0) {
        select_hi_256(hist, st, final_level, T_out, k_level1);
        return;
    }
    const int b = (int)blockIdx.x - 1;
    colmax_tile<DT, false>(w.W, w.K, w.N, COLMAX_ROWS, nullptr, w.keys, b % gx, b / gx);
}

template <int DT, bool PREFIX>
__global__ __launch_bounds__(256) void k_coo_qcols(Staging stg, const int32_t *__restrict__ row_cnt,
                                                   int32_t *__restrict__ row_ptr, int64_t *__restrict__ nnz_out,
                                                   int64_t M, int64_t cap, int32_t *__restrict__ coo_row,
                                                   int32_t *__restrict__ coo_col, float *__restrict__ coo_val,
                                                   const void *__restrict__ A, int64_t K,
                                                   const float *__restrict__ T_src, int ncoo, WSide w, int gx) {
    if ((int)blockIdx.x < ncoo) {
        coo_block<DT, PREFIX>(stg, row_cnt, row_ptr, nnz_out, M, cap, coo_row, coo_col, coo_val, A, K, T_src,
                              blockIdx.x);
        return;
    }
    const int b = (int)blockIdx.x - ncoo;
    qcols_tile<DT, false, FP4_QCOLS_TN>(w.W, w.K, w.N, nullptr, w.keys, w.codes, w.scales, b % gx, b / gx);
}

// ----------------------------------------------------------------------------- launchers
static inline int blocks_for(int64_t n, int threads, int cap) {
    int64_t b = (n + threads - 1) / threads;
    if (b > cap) b = cap;
    return (int)(b < 1 ? 1 : b);
}

hipError_t launch_zero(uint32_t *p1, int64_t n1, uint32_t *p2, int64_t n2, hipStream_t s) {
    if (n1 + n2 <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_zero_u32, dim3(blocks_for(n1 + n2, 256, 1024)), dim3(256), 0, s, p1, n1, p2, n2);
    return hipGetLastError();
}

hipError_t launch_hist_rowmax(const void *A, int dt, int64_t M, int64_t K, uint32_t *ghist, uint32_t *rowmax_key,
                              int num_cus, hipStream_t s) {
    int blocks = (int)(M < (int64_t)num_cus ? M : (int64_t)num_cus);
    if (dt == DT_BF16)
        hipLaunchKernelGGL(k_hist_rowmax<DT_BF16>, dim3(blocks), dim3(1024), 0, s, A, M, K, ghist, rowmax_key);
    else
        hipLaunchKernelGGL(k_hist_rowmax<DT_F32>, dim3(blocks), dim3(1024), 0, s, A, M, K, ghist, rowmax_key);
    return hipGetLastError();
}

hipError_t launch_select_hi(const uint32_t *ghist, int dt, State *st, float *T_out, uint64_t k, const WSide *w,
                            hipStream_t s) {
    const int final_level = dt == DT_BF16 ? 1 : 2;
    if (!w) {
        hipLaunchKernelGGL(k_select_hi, dim3(1), dim3(256), 0, s, ghist, st, final_level, T_out, k);
        return hipGetLastError();
    }
    const int gx = (int)((w->N + 511) / 512), gy = (int)((w->K + COLMAX_ROWS - 1) / COLMAX_ROWS);
    const dim3 grid((unsigned)(1 + gx * gy));
    if (w->dt == DT_BF16)
        hipLaunchKernelGGL(k_select_colmax<DT_BF16>, grid, dim3(256), 0, s, ghist, st, final_level, T_out, k, *w, gx);
    else
        hipLaunchKernelGGL(k_select_colmax<DT_F32>, grid, dim3(256), 0, s, ghist, st, final_level, T_out, k, *w, gx);
    return hipGetLastError();
}

hipError_t launch_select_lo(const void *A, int64_t n, uint32_t *ghist_lo, State *st, float *T_out, hipStream_t s) {
    hipLaunchKernelGGL(k_hist_lo, dim3(blocks_for(n, 256, 2048)), dim3(256), 0, s, (const uint32_t *)A, n, st,
                       ghist_lo);
    hipLaunchKernelGGL(k_select_lo, dim3(1), dim3(1024), 0, s, ghist_lo, st, T_out);
    return hipGetLastError();
}

hipError_t launch_quant_rows(const void *X, int dt, int64_t R, int64_t C, const uint32_t *rowmax_key,
                             const float *T_src, uint8_t *codes, float *scales, int32_t *row_cnt,
                             const Staging &stg, State *st, bool emit, bool write_codes, hipStream_t s) {
    dim3 grid((unsigned)((R + 3) / 4)), block(256);
    const bool clamp = T_src != nullptr;
    const bool have_rm = rowmax_key != nullptr;
#define QR(DT, CL, HR, CO, EM)                                                                      \
    hipLaunchKernelGGL((k_quant_rows<DT, CL, HR, CO, EM>), grid, block, 0, s, X, R, C, rowmax_key, T_src, \
                       codes, scales, row_cnt, stg, st)
    if (dt == DT_BF16) {
        if (emit && write_codes && have_rm) QR(DT_BF16, true, true, true, true);
        else if (emit && !write_codes) QR(DT_BF16, true, false, false, true);
        else if (clamp) QR(DT_BF16, true, false, true, false);
        else QR(DT_BF16, false, false, true, false);
    } else {
        if (emit && write_codes && have_rm) QR(DT_F32, true, true, true, true);
        else if (emit && !write_codes) QR(DT_F32, true, false, false, true);
        else if (clamp) QR(DT_F32, true, false, true, false);
        else QR(DT_F32, false, false, true, false);
    }
#undef QR
    return hipGetLastError();
}

hipError_t launch_coo(const int32_t *row_cnt, int64_t M, int32_t *row_ptr, int64_t *nnz_out, const Staging &stg,
                      int64_t cap, int32_t *coo_row, int32_t *coo_col, float *coo_val, const void *A, int dt,
                      int64_t K, const float *T_src, const WSide *w, hipStream_t s) {
    const int ncoo = (int)((M + 63) / 64);  // 64 rows per workgroup
    const bool prefix = M <= COO_PREFIX_ROWS;
    if (!prefix) hipLaunchKernelGGL(k_coo_scan, dim3(1), dim3(1024), 0, s, row_cnt, M, row_ptr, nnz_out);
    if (w) {
        const int gx = (int)((w->N + FP4_QCOLS_TN - 1) / FP4_QCOLS_TN), gy = (int)((w->K + 255) / 256);
        const dim3 grid((unsigned)(ncoo + gx * gy));
#define CQ(DT, PF)                                                                                              \
    hipLaunchKernelGGL((k_coo_qcols<DT, PF>), grid, dim3(256), 0, s, stg, row_cnt, row_ptr, nnz_out, M, cap, coo_row, \
                       coo_col, coo_val, A, K, T_src, ncoo, *w, gx)
        if (dt == DT_BF16) {
            if (prefix) CQ(DT_BF16, true);
            else CQ(DT_BF16, false);
        } else {
            if (prefix) CQ(DT_F32, true);
            else CQ(DT_F32, false);
        }
#undef CQ
        return hipGetLastError();
    }
    const dim3 grid((unsigned)ncoo), block(256);
#define CB(DT, PF)                                                                                              \
    hipLaunchKernelGGL((k_coo_build<DT, PF>), grid, block, 0, s, stg, row_cnt, row_ptr, nnz_out, M, cap, coo_row, \
                       coo_col, coo_val, A, K, T_src)
    if (dt == DT_BF16) {
        if (prefix) CB(DT_BF16, true);
        else CB(DT_BF16, false);
    } else {
        if (prefix) CB(DT_F32, true);
        else CB(DT_F32, false);
    }
#undef CB
    return hipGetLastError();
}

hipError_t launch_quant_cols(const void *W, int dt, int64_t K, int64_t N, float *scales_as_keys,
                             uint8_t *codes, bool keys_zeroed, hipStream_t s, const float *row_mult,
                             float *scales_out) {
    uint32_t *keys = reinterpret_cast<uint32_t *>(scales_as_keys);
    if (!keys_zeroed) {
        hipError_t e = launch_zero(keys, N, nullptr, 0, s);
        if (e != hipSuccess) return e;
    }
    const int rows_per_block = COLMAX_ROWS;
    dim3 g1((unsigned)((N + 511) / 512), (unsigned)((K + rows_per_block - 1) / rows_per_block));
#define QC(DT, RM)                                                                                         \
    do {                                                                                                   \
        hipLaunchKernelGGL((k_colmax<DT, RM>), g1, dim3(256), 0, s, W, K, N, rows_per_block, row_mult, keys); \
        launch_qcols_tile<DT, RM>(W, K, N, row_mult, keys, codes, scales_out, s);                           \
    } while (0)
    if (dt == DT_BF16) {
        if (row_mult) QC(DT_BF16, true);
        else QC(DT_BF16, false);
    } else {
        if (row_mult) QC(DT_F32, true);
        else QC(DT_F32, false);
    }
#undef QC
    if (!scales_out) hipLaunchKernelGGL(k_col_scales, dim3(blocks_for(N, 256, 1 << 20)), dim3(256), 0, s, keys, N);
    return hipGetLastError();
}

hipError_t launch_quant_cols_keyed(const void *W, int dt, int64_t K, int64_t N, float *scales_as_keys,
                                   uint8_t *codes, const float *row_mult, hipStream_t s) {
    uint32_t *keys = reinterpret_cast<uint32_t *>(scales_as_keys);
    if (dt == DT_BF16) {
        if (row_mult) launch_qcols_tile<DT_BF16, true>(W, K, N, row_mult, keys, codes, nullptr, s);
        else launch_qcols_tile<DT_BF16, false>(W, K, N, row_mult, keys, codes, nullptr, s);
    } else {
        if (row_mult) launch_qcols_tile<DT_F32, true>(W, K, N, row_mult, keys, codes, nullptr, s);
        else launch_qcols_tile<DT_F32, false>(W, K, N, row_mult, keys, codes, nullptr, s);
    }
    hipLaunchKernelGGL(k_col_scales, dim3(blocks_for(N, 256, 1 << 20)), dim3(256), 0, s, keys, N);
    return hipGetLastError();
}

}  // namespace fp4
