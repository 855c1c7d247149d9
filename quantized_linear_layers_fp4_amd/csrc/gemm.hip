// gfx950 FP4 GEMM of the quantized operands with the dequantization and the sparse
// compensation fused into its output (QbitAI report on "Optimizing Large Language Model
// Training Using FP4 Quantization": GEMM-kernel paragraph for the FP4 tiled product,
// granularity paragraph for the row/column scales that factor out of the K-sum, outlier
// paragraph for dA).  The pages' kernel emulates FP4 on FP8 tensor cores and reduces in
// FP16; here the CDNA4 matrix cores multiply E2M1 operands natively (unit E8M0 block
// scales) and accumulate in fp32, which is exact for these operands.
//
// Workgroup: 8 waves (two per SIMD) own a 256 x 256 output tile; wave (wm, wn) owns rows
// 128*wm.. and columns 64*wn.. as 4 x 2 tiles of V_MFMA_SCALE_F32_32X32X64_F8F6F4.
// K advances 128 codes (64 bytes per row) per stage.  Operand tiles travel from global
// memory straight into one of four LDS stage buffers (buffer loads with the LDS flag,
// issued three stages ahead); rows or K chunks outside the matrices read as zero.  One
// barrier per stage; the fragments of the next stage's first K-step are read before it, so
// the matrix cores restart right after each barrier.  The row/column scales and the row pointers of dA for the tile are
// fetched into LDS under the first stage loads.
//
// Epilogue: 32 rows at a time through an fp32 slab in LDS.  The tile's dA entries (sorted
// by row, then column) stream through in rounds of 32 KiB of gathered W row segments:
// the (column, delta) pairs of a round are copied into a small LDS ring one round before
// its gather, and each gather is issued two rounds before it is applied, so the gathers'
// latency runs under the application of the rounds before.
#include "fp4_common.h"
#include "fp4_launch.h"

#include <cstdlib>

namespace fp4 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
#define LDS_PTR(p) ((__attribute__((address_space(3))) void *)(p))

constexpr int BM = 256, BN = 256, NW = 8, NT = 64 * NW;
constexpr int BKB = 64;                    // bytes of K per row per stage (128 codes)
constexpr int OPB = 256 * BKB;             // one operand tile per stage: 16 KiB
constexpr int STB = 2 * OPB;               // A then B: 32 KiB per stage buffer
constexpr int UNIT_SCALE = 0x7F7F7F7F;     // E8M0 127 = 2^0 in every byte
constexpr int BUF_FLAGS = 0x00020000;      // raw buffer descriptor word 3 (gfx9 family)
constexpr int OOB = 0x7FFFFFF0;            // an offset past every buffer: the load returns 0
constexpr int SLAB = 32;                   // epilogue rows per pass (one 32-row MFMA tile)
constexpr int GBYTES = 3 * STB;            // gather space of one round: the three free stage buffers
constexpr int RING = 192;                  // dA entries per ring slot
constexpr int LPR = GBYTES / 1024 / NW;    // gather loads per wave per round (12)

// 16-byte slot of (row, chunk) in a 256-row x 4-chunk operand tile.  A 16-lane group
// reading 16 consecutive rows of one chunk hits 16 distinct slots modulo 16.
__device__ __forceinline__ int slot16(int row, int chunk) { return row * 4 + (chunk ^ ((row >> 2) & 3)); }

// fp32 epilogue slab (32 rows x 256 columns): columns of rows with bit 2 set are XORed
// with 32 so the two half-waves of an MFMA register write different banks.
__device__ __forceinline__ int eidx(int row, int col) { return row * BN + (col ^ ((row & 4) << 3)); }

struct TileArgs {
    const uint8_t *Aq, *Wq;
    const float *sA, *sW;
    int M, N, K;
    const int32_t *row_ptr, *coo_row, *coo_col;
    const float *coo_val;
    const void *Wc;
    void *Y;
    float *acc_out;
    int tilesM, tilesN, raster_group;
};

// LDS bookkeeping of one tile (written with ordinary stores).
struct Book {
    float sA[BM];
    float sW[BN];
    int32_t rp[BM + 4];        // row_ptr[m0 .. m0+256] (clamped to M)
    float X[NW][BN];           // first-row partial sums of each wave's share of a pass
    int32_t Xrow[NW];          // (slab row of X[w], or -1)
};

// The dA entries of the rounds in flight, one slot per round (filled by buffer loads with
// the LDS flag).
struct Ring {
    int32_t kc[2][RING];       // columns
    float dv[2][RING];         // values
    int32_t kr[2][RING];       // rows
};

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)LDS_PTR(const_cast<void *>(p));
}

// Reads of LDS that buffer loads with the LDS flag fill.  The loads' completion is waited
// for explicitly (vmcnt, then a barrier); these reads carry their own lgkmcnt wait, so the
// compiler does not add a wait for every buffer load still in flight.
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void lds_read2_u32(uint32_t a, uint32_t b, uint32_t &x, uint32_t &y) {
    asm volatile("ds_read_b32 %0, %2\n\tds_read_b32 %1, %3\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(x), "=&v"(y)
                 : "v"(a), "v"(b));
}
__device__ __forceinline__ void lds_read4_u32(const uint32_t (&a)[4], uint32_t (&x)[4]) {
    asm volatile(
        "ds_read_b32 %0, %4\n\tds_read_b32 %1, %5\n\tds_read_b32 %2, %6\n\tds_read_b32 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]));
}
__device__ __forceinline__ void lds_read4_b64(const uint32_t (&a)[4], u32x2 (&x)[4]) {
    asm volatile(
        "ds_read_b64 %0, %4\n\tds_read_b64 %1, %5\n\tds_read_b64 %2, %6\n\tds_read_b64 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]));
}
__device__ __forceinline__ void lds_read4_b128(const uint32_t (&a)[4], u32x4 (&x)[4]) {
    asm volatile(
        "ds_read_b128 %0, %4\n\tds_read_b128 %1, %5\n\tds_read_b128 %2, %6\n\tds_read_b128 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]));
}

// Workgroup barrier for LDS traffic only: this wave's LDS reads and writes are done, then
// s_barrier.  Buffer loads and global stores stay in flight (their waits are explicit).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt and expcnt unconstrained
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
}

// One stage of DMA for this wave: 2 loads of A (rows 32w..32w+31) and 2 of B.  Lane i of
// load j fills slot 64*(2w+j) + i: row 16*(2w+j) + i/4, at the swizzled position i%4.
__device__ __forceinline__ void stage_dma(__amdgpu_buffer_rsrc_t rsA, __amdgpu_buffer_rsrc_t rsB, uint8_t *buf,
                                          int wave, const int (&offA)[2], const int (&offB)[2], int kt, int KB,
                                          int lane_chunk16) {
    const bool kin = kt * BKB + lane_chunk16 < KB;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int oa = (kin && offA[j] != OOB) ? offA[j] + kt * BKB : OOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsA, LDS_PTR(buf + (wave * 2 + j) * 1024), 16, oa, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int ob = (kin && offB[j] != OOB) ? offB[j] + kt * BKB : OOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsB, LDS_PTR(buf + OPB + (wave * 2 + j) * 1024), 16, ob, 0, 0, 0);
    }
}

// Fragments of K-step s (0 or 1) of a stage: lane l reads row l%32 of each 32-row tile and
// the 16-byte chunk 2s + l/32 (32 codes).
__device__ __forceinline__ void frag_load(const uint8_t *buf, int wm, int wn, int lane, int s, u32x4 (&a)[4],
                                          u32x4 (&b)[2]) {
    const int chunk = 2 * s + (lane >> 5);
#pragma unroll
    for (int i = 0; i < 4; ++i)
        a[i] = *reinterpret_cast<const u32x4 *>(buf + slot16(wm * 128 + i * 32 + (lane & 31), chunk) * 16);
#pragma unroll
    for (int j = 0; j < 2; ++j)
        b[j] = *reinterpret_cast<const u32x4 *>(buf + OPB + slot16(wn * 64 + j * 32 + (lane & 31), chunk) * 16);
}

__device__ __forceinline__ void mfma_block(v16f (&acc)[4][2], const u32x4 (&a)[4], const u32x4 (&b)[2]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const v8i av = v8i{(int)a[i].x, (int)a[i].y, (int)a[i].z, (int)a[i].w, 0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const v8i bv = v8i{(int)b[j].x, (int)b[j].y, (int)b[j].z, (int)b[j].w, 0, 0, 0, 0};
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc[i][j], 4, 4, 0, UNIT_SCALE, 0,
                                                                        UNIT_SCALE);
        }
    }
}

// s_waitcnt vmcnt(n), other counters untouched (gfx9 encoding)
#define WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | 0x0F70)

// Byte `off` of the gather space, which spans the three free stage buffers in order.  A
// select between the LDS arrays themselves keeps the accesses in the LDS address space.
__device__ __forceinline__ uint8_t *gather_at(int off, uint8_t *g0, uint8_t *g1, uint8_t *g2) {
    const int b = off / STB;
    return (b == 0 ? g0 : (b == 1 ? g1 : g2)) + (off - b * STB);
}

// The dA stream of one tile: entries [E0, E0 + n) of the COO list, in rounds of RE entries
// whose W row segments (BN columns each) fill one 32 KiB gather buffer.
template <int WDT>
struct Stream {
    static constexpr int ESZ = (WDT == DT_BF16) ? 2 : 4;
    static constexpr int ROW_BYTES = BN * ESZ;
    static constexpr int RE = GBYTES / ROW_BYTES;   // 192 (bf16 W) or 96 (fp32 W) entries per round
    static_assert(RE <= RING, "ring slot holds a round");
    __amdgpu_buffer_rsrc_t rsK, rsV, rsR, rsW;   // the tile's columns, values and rows, and W
    int n;                                       // entries of the tile
    int N, n0, wave, lane;

    // (column, delta, row) of the entries of round u into ring slot u%4: wave 0 copies the
    // columns, wave 1 the values, wave 2 the rows (one 4-byte load per lane; past the
    // tile's entries they read 0).
    __device__ __forceinline__ void issue_pairs(Ring &rg, int u) const {
#pragma unroll
        for (int c = 0; c < (RE + 63) / 64; ++c) {
            const int o = (u * RE + c * 64 + lane) * 4;
            if (wave == 0)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rsK, LDS_PTR(&rg.kc[u & 1][c * 64]), 4, o, 0, 0, 0);
            else if (wave == 1)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rsV, LDS_PTR(&rg.dv[u & 1][c * 64]), 4, o, 0, 0, 0);
            else if (wave == 2)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rsR, LDS_PTR(&rg.kr[u & 1][c * 64]), 4, o, 0, 0, 0);
        }
    }
    // W[k][n0 .. n0+BN-1] of every entry of round u, back to back into buffer u%3.  A load
    // moves 1 KiB: lane i carries bytes 16i.. of it.  Every wave issues LPR loads.
    __device__ __forceinline__ void issue_gather(const Ring &rg, int u, uint8_t *g0, uint8_t *g1, uint8_t *g2) const {
        uint32_t ka[LPR], kv[LPR];
        int el[LPR], col[LPR];
#pragma unroll
        for (int j = 0; j < LPR; ++j) {
            const int byte = (wave * LPR + j) * 1024 + lane * 16;
            el[j] = byte / ROW_BYTES;
            col[j] = n0 + (byte % ROW_BYTES) / ESZ;
            ka[j] = lds_addr(&rg.kc[u & 1][el[j]]);
        }
#pragma unroll
        for (int j = 0; j < LPR; j += 4) {
            const uint32_t a4[4] = {ka[j], ka[j + 1], ka[j + 2], ka[j + 3]};
            uint32_t v4[4];
            lds_read4_u32(a4, v4);
            kv[j] = v4[0];
            kv[j + 1] = v4[1];
            kv[j + 2] = v4[2];
            kv[j + 3] = v4[3];
        }
#pragma unroll
        for (int j = 0; j < LPR; ++j) {
            const int L = wave * LPR + j;
            int o = OOB;
            if (u * RE + el[j] < n && col[j] < N) o = ((int)kv[j] * N + col[j]) * ESZ;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsW, LDS_PTR(gather_at(L * 1024, g0, g1, g2)), 16, o, 0, 0, 0);
        }
    }
};

template <int YDT, int WDT, bool COMP, bool ACCOUT>
__global__ __launch_bounds__(NT, 2) void k_fp4_gemm(TileArgs p) {
    __shared__ __attribute__((aligned(16))) uint8_t sb0[STB];
    __shared__ __attribute__((aligned(16))) uint8_t sb1[STB];
    __shared__ __attribute__((aligned(16))) uint8_t sb2[STB];
    __shared__ __attribute__((aligned(16))) uint8_t sb3[STB];
    __shared__ __attribute__((aligned(16))) Book bk;
    __shared__ __attribute__((aligned(16))) Ring rg;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 2, wn = wave & 3;
    const int M = p.M, N = p.N, K = p.K;

    // XCD-aware order: consecutive workgroup ids go to different XCDs, so give each XCD a
    // contiguous range of logical tiles; within it raster_group tile-rows sweep the
    // tile-columns together, so the tiles an XCD runs at once share operand strips (and
    // the compensation's W rows) in its L2.
    const int per_xcd = gridDim.x / 8;
    const int logical = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    if (logical >= p.tilesM * p.tilesN) return;
    const int group = logical / (p.raster_group * p.tilesN);
    const int first_m = group * p.raster_group;
    const int gm = min(p.raster_group, p.tilesM - first_m);
    const int in_group = logical - group * p.raster_group * p.tilesN;
    const int m0 = (first_m + in_group % gm) * BM;
    const int n0 = (in_group / gm) * BN;

    const int KB = K / 2;
    const int kstages = (KB + BKB - 1) / BKB;
    const __amdgpu_buffer_rsrc_t rsA =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(p.Aq), 0, M * KB, BUF_FLAGS);
    const __amdgpu_buffer_rsrc_t rsB =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(p.Wq), 0, N * KB, BUF_FLAGS);
    const int lane_chunk16 = ((lane & 3) ^ ((lane >> 4) & 3)) * 16;
    int offA[2], offB[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int r = (wave * 2 + j) * 16 + (lane >> 2);
        offA[j] = (m0 + r < M) ? (m0 + r) * KB + lane_chunk16 : OOB;
        offB[j] = (n0 + r < N) ? (n0 + r) * KB + lane_chunk16 : OOB;
    }

    v16f acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // prologue: stage 0, the tile's scales and row pointers, then stages 1 and 2.  The
    // bookkeeping loads are older than the later stages' loads, so the wait for stages 0
    // and 1 covers them too.
    stage_dma(rsA, rsB, sb0, wave, offA, offB, 0, KB, lane_chunk16);
    __builtin_amdgcn_sched_barrier(0);
    float bA = 0.0f, bW = 0.0f;
    int bR0 = 0, bR1 = 0;
    if (tid < 256) {
        if (m0 + tid < M) bA = p.sA[m0 + tid];
        if (n0 + tid < N) bW = p.sW[n0 + tid];
        if constexpr (COMP) bR0 = p.row_ptr[min(m0 + tid, M)];
    } else if (COMP && tid < 260) {
        bR1 = p.row_ptr[min(m0 + tid, M)];
    }
    __builtin_amdgcn_sched_barrier(0);
    stage_dma(rsA, rsB, sb1, wave, offA, offB, 1, KB, lane_chunk16);
    stage_dma(rsA, rsB, sb2, wave, offA, offB, 2, KB, lane_chunk16);
    __builtin_amdgcn_sched_barrier(0);
    WAIT_VMCNT(4);
    if (tid < 256) {
        bk.sA[tid] = bA;
        bk.sW[tid] = bW;
        if constexpr (COMP) bk.rp[tid] = bR0;
    } else if (COMP && tid < 260) {
        bk.rp[tid] = bR1;
    }
    __builtin_amdgcn_s_barrier();

    // Stage kt lives in buffer kt%4; its loads are issued at step kt-3.  At the start of
    // step kt the K-step-0 fragments of stage kt are already in registers and stage kt+1 is
    // complete; the step reads stage kt's K-step-1 fragments under the first eight MFMAs
    // and stage kt+1's K-step-0 fragments under the second eight.  Each wave then waits for
    // its own loads of stage kt+2 before the barrier that ends the step, so after it stage
    // kt+2 is complete and stage kt-1's buffer (read last in step kt-1) takes stage kt+3.
    u32x4 a0[4], b0[2];
    __builtin_amdgcn_sched_barrier(0);
    frag_load(sb0, wm, wn, lane, 0, a0, b0);
    auto step = [&](int kt, const uint8_t *cur, const uint8_t *nxt, uint8_t *ahead) {
        __builtin_amdgcn_sched_barrier(0);
        stage_dma(rsA, rsB, ahead, wave, offA, offB, kt + 3, KB, lane_chunk16);
        u32x4 a1[4], b1[2];
        frag_load(cur, wm, wn, lane, 1, a1, b1);
        __builtin_amdgcn_sched_barrier(0);
        mfma_block(acc, a0, b0);
        __builtin_amdgcn_sched_barrier(0);
        frag_load(nxt, wm, wn, lane, 0, a0, b0);
        __builtin_amdgcn_sched_barrier(0);
        mfma_block(acc, a1, b1);
        __builtin_amdgcn_sched_barrier(0);
        WAIT_VMCNT(4);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };
    // whole groups of four stages (a group may run past the last stage on zeros: one exit
    // keeps the accumulators in one set of registers)
    for (int kt = 0; kt < kstages; kt += 4) {
        step(kt, sb0, sb1, sb3);
        step(kt + 1, sb1, sb2, sb0);
        step(kt + 2, sb2, sb3, sb1);
        step(kt + 3, sb3, sb0, sb2);
    }
    WAIT_VMCNT(0);  // look-ahead loads past the end (zeros) land before the buffers are reused
    __syncthreads();

    // ---- epilogue: Y = fl(fl(acc * sA) * sW), then + sum of delta * W[k][n] over the row's
    // dA entries in ascending k, 32 rows at a time through an fp32 slab in LDS.
    // MFMA 32x32 output layout: lane l, register r -> row 8*(r/4) + 4*(l/32) + r%4, col l%32.
    using S = Stream<WDT>;
    constexpr int RE = S::RE, ROW_BYTES = S::ROW_BYTES, ESZ = S::ESZ;
    float *E = reinterpret_cast<float *>(sb0);
    float sw[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) sw[j] = bk.sW[wn * 64 + j * 32 + (lane & 31)];
    const int g = tid >> 5;    // 16 row groups: slab rows g and g + 16
    const int c8 = tid & 31;   // columns n0 + 8*c8 .. +7
    const int gn = n0 + c8 * 8;

    S st;
    int visited = 0;           // rounds whose first application has started
    int E0 = 0;
    if constexpr (COMP) {
        E0 = bk.rp[0];
        st.n = bk.rp[BM] - E0;
        st.N = N;
        st.n0 = n0;
        st.wave = wave;
        st.lane = lane;
        st.rsK = __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t *>(p.coo_col + E0), 0, st.n * 4, BUF_FLAGS);
        st.rsV = __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(p.coo_val + E0), 0, st.n * 4, BUF_FLAGS);
        st.rsR = __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t *>(p.coo_row + E0), 0, st.n * 4, BUF_FLAGS);
        st.rsW = __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p.Wc), 0, K * N * ESZ, BUF_FLAGS);
        if (st.n > 0) {
            // prime: the entries of round 0 in the ring
            st.issue_pairs(rg, 0);
            WAIT_VMCNT(0);
            lds_barrier();
        }
    }

    // slab q holds tile rows 32q..32q+31: MFMA tile q%4 of the waves with wm == q/4.  The
    // slabs go in ascending row order (the dA stream is sorted by row); the tile index must
    // be a compile-time constant, so the four tiles of a half are unrolled.
#pragma unroll 1
    for (int qh = 0; qh < 2; ++qh) {
#pragma unroll
        for (int qi = 0; qi < 4; ++qi) {
            const int q = qh * 4 + qi;
            if (wm == qh) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int lr = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                    const float sa = bk.sA[q * SLAB + lr];
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const int lc = wn * 64 + j * 32 + (lane & 31);
                        const float a = acc[qi][j][r];
                        if constexpr (ACCOUT) {
                            const int grow = m0 + q * SLAB + lr;
                            if (grow < M && n0 + lc < N) p.acc_out[(size_t)grow * N + n0 + lc] = a;
                        }
                        const float t = a * sa;
                        E[eidx(lr, lc)] = t * sw[j];
                    }
                }
            }
            lds_barrier();
            if constexpr (COMP) {
                const int e_lo = bk.rp[q * SLAB] - E0, e_hi = bk.rp[q * SLAB + SLAB] - E0;
                if (e_hi > e_lo) {
#pragma unroll 1
                    for (int t = e_lo / RE; t <= (e_hi - 1) / RE; ++t) {
                        if (t >= visited) {
                            // first use of round t: every wave is past round t-1, whose gather
                            // space and ring slot are free; gather round t and copy the entries
                            // of round t+1, then wait for both
                            lds_barrier();
                            st.issue_gather(rg, t, sb1, sb2, sb3);
                            st.issue_pairs(rg, t + 1);
                            WAIT_VMCNT(0);
                            lds_barrier();
                            visited = t + 1;
                        }

                        // one pass: the round's entries of slab q split into NW contiguous
                        // shares, wave w adding share w over all BN columns (4 per lane).
                        // Entries are sorted by row, so a share owns its rows except the first,
                        // which may continue the previous share's last row: that partial sum
                        // goes to X[w] and is added after the barrier, shares in order.
                        const int a = max(e_lo, t * RE) - t * RE;
                        const int b = min(e_hi, t * RE + RE) - t * RE;
                        const int pa = a + ((b - a) * wave) / NW, pb = a + ((b - a) * (wave + 1)) / NW;
                        const int rbase = m0 + q * SLAB;
                        // the share's rows and deltas: one LDS read per lane, then broadcast
                        const int ns = pb - pa;   // at most RE / NW <= 24 entries
                        int krl = 0;
                        float dvl = 0.0f;
                        {
                            const int ei = pa + min(lane, max(ns - 1, 0));
                            uint32_t kx, dx;
                            lds_read2_u32(lds_addr(&rg.kr[t & 1][ei]), lds_addr(&rg.dv[t & 1][ei]), kx, dx);
                            krl = ((int)kx - rbase) & (SLAB - 1);
                            dvl = __uint_as_float(dx);
                        }
                        const int first_row = ns > 0 ? __builtin_amdgcn_readfirstlane(krl) : -1;
                        if (lane == 0) bk.Xrow[wave] = first_row;
                        float4 part = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
                        int cur = first_row;
                        auto add_to_E = [&](int row, const float4 &v) {
                            float4 *ep = reinterpret_cast<float4 *>(&E[eidx(row, lane * 4)]);
                            float4 y = *ep;
                            y.x += v.x;
                            y.y += v.y;
                            y.z += v.z;
                            y.w += v.w;
                            *ep = y;
                        };
                        // four entries' W segments are read together, then added in order
#pragma unroll
                        for (int i0 = 0; i0 < RE / NW; i0 += 4) {
                            if (i0 >= ns) break;
                            float wf[4][4];
                            uint32_t wa[4];
#pragma unroll
                            for (int u = 0; u < 4; ++u)
                                wa[u] = lds_addr(gather_at((pa + min(i0 + u, ns - 1)) * ROW_BYTES + lane * 4 * ESZ,
                                                           sb1, sb2, sb3));
                            if constexpr (WDT == DT_BF16) {
                                u32x2 w2[4];
                                lds_read4_b64(wa, w2);
#pragma unroll
                                for (int u = 0; u < 4; ++u) {
                                    wf[u][0] = bf16_to_f32(w2[u].x & 0xFFFFu);
                                    wf[u][1] = bf16_to_f32(w2[u].x >> 16);
                                    wf[u][2] = bf16_to_f32(w2[u].y & 0xFFFFu);
                                    wf[u][3] = bf16_to_f32(w2[u].y >> 16);
                                }
                            } else {
                                u32x4 w4[4];
                                lds_read4_b128(wa, w4);
#pragma unroll
                                for (int u = 0; u < 4; ++u) {
                                    wf[u][0] = __uint_as_float(w4[u].x);
                                    wf[u][1] = __uint_as_float(w4[u].y);
                                    wf[u][2] = __uint_as_float(w4[u].z);
                                    wf[u][3] = __uint_as_float(w4[u].w);
                                }
                            }
#pragma unroll
                            for (int u = 0; u < 4; ++u) {
                                if (i0 + u >= ns) break;
                                const int row = __builtin_amdgcn_readlane(krl, i0 + u);
                                const float d = __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                    __builtin_bit_cast(int, dvl), i0 + u));
                                if (row != cur) {
                                    // rows are sorted: cur is complete (only the first row of a
                                    // share can continue the previous share's last row)
                                    if (wave > 0 && cur == first_row)
                                        *reinterpret_cast<float4 *>(&bk.X[wave][lane * 4]) = part;
                                    else
                                        add_to_E(cur, part);
                                    cur = row;
                                    part = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
                                }
                                part.x = __builtin_fmaf(d, wf[u][0], part.x);
                                part.y = __builtin_fmaf(d, wf[u][1], part.y);
                                part.z = __builtin_fmaf(d, wf[u][2], part.z);
                                part.w = __builtin_fmaf(d, wf[u][3], part.w);
                            }
                        }
                        if (ns > 0) {
                            if (wave > 0 && cur == first_row)
                                *reinterpret_cast<float4 *>(&bk.X[wave][lane * 4]) = part;
                            else
                                add_to_E(cur, part);
                        }
                        lds_barrier();
                        if (wave == 0) {
                            // the shares' first-row partial sums in share order; a run of one
                            // row is summed first and added to E once
                            const int xr = lane < NW ? bk.Xrow[lane] : -1;
                            float4 x[NW];
#pragma unroll
                            for (int w = 1; w < NW; ++w) x[w] = *reinterpret_cast<const float4 *>(&bk.X[w][lane * 4]);
                            int rr = -1;
                            float4 run = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
                            for (int w = 1; w < NW; ++w) {
                                const int r = __builtin_amdgcn_readlane(xr, w);
                                if (r < 0) continue;
                                if (r == rr) {
                                    run.x += x[w].x;
                                    run.y += x[w].y;
                                    run.z += x[w].z;
                                    run.w += x[w].w;
                                } else {
                                    if (rr >= 0) add_to_E(rr, run);
                                    rr = r;
                                    run = x[w];
                                }
                            }
                            if (rr >= 0) add_to_E(rr, run);
                        }
                        lds_barrier();
                    }
                }
            }
            // store the slab: 32 rows x 32 chunks of 8 columns, 32 threads per row
            if (gn < N) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int lr = g + 16 * h;
                    const int grow = m0 + q * SLAB + lr;
                    if (grow < M) {
                        const float4 e0 = *reinterpret_cast<const float4 *>(&E[eidx(lr, c8 * 8)]);
                        const float4 e1 = *reinterpret_cast<const float4 *>(&E[eidx(lr, c8 * 8 + 4)]);
                        if constexpr (YDT == DT_BF16) {
                            uint4 o;
                            o.x = f32_to_bf16_bits(e0.x) | (f32_to_bf16_bits(e0.y) << 16);
                            o.y = f32_to_bf16_bits(e0.z) | (f32_to_bf16_bits(e0.w) << 16);
                            o.z = f32_to_bf16_bits(e1.x) | (f32_to_bf16_bits(e1.y) << 16);
                            o.w = f32_to_bf16_bits(e1.z) | (f32_to_bf16_bits(e1.w) << 16);
                            *reinterpret_cast<uint4 *>(reinterpret_cast<uint16_t *>(p.Y) + (size_t)grow * N + gn) = o;
                        } else {
                            float4 *yp =
                                reinterpret_cast<float4 *>(reinterpret_cast<float *>(p.Y) + (size_t)grow * N + gn);
                            yp[0] = e0;
                            yp[1] = e1;
                        }
                    }
                }
            }
            lds_barrier();
        }
    }
    if constexpr (COMP) WAIT_VMCNT(0);  // the look-ahead gathers land before the workgroup ends
}

// Tile-rows per column sweep within an XCD.  FP4_GEMM_RASTER overrides (tuning aid).
static int raster_group_for(int tilesM, bool comp) {
    static int env = -2;
    if (env == -2) {
        const char *e = getenv("FP4_GEMM_RASTER");
        env = e ? atoi(e) : -1;
    }
    const int g = env > 0 ? env : (comp ? 32 : 8);
    return g < tilesM ? g : tilesM;
}

hipError_t launch_gemm(const uint8_t *Aq, const float *sA, const uint8_t *Wq, const float *sW, int64_t M,
                       int64_t N, int64_t K, const int32_t *row_ptr, const int32_t *coo_row, const int32_t *coo_col,
                       const float *coo_val, const void *W, int w_dt, void *Y, int y_dt, float *acc_out,
                       hipStream_t s) {
    TileArgs p;
    p.Aq = Aq;
    p.Wq = Wq;
    p.sA = sA;
    p.sW = sW;
    p.M = (int)M;
    p.N = (int)N;
    p.K = (int)K;
    p.row_ptr = row_ptr;
    p.coo_row = coo_row;
    p.coo_col = coo_col;
    p.coo_val = coo_val;
    p.Wc = W;
    p.Y = Y;
    p.acc_out = acc_out;
    p.tilesM = (int)((M + BM - 1) / BM);
    p.tilesN = (int)((N + BN - 1) / BN);
    const bool comp = row_ptr != nullptr;
    p.raster_group = raster_group_for(p.tilesM, comp);
    const int64_t tiles = (int64_t)p.tilesM * p.tilesN;
    const int blocks = (int)((tiles + 7) / 8 * 8);
#define G(YD, WD, CO, AO) hipLaunchKernelGGL((k_fp4_gemm<YD, WD, CO, AO>), dim3(blocks), dim3(NT), 0, s, p)
#define G2(YD, WD)                                    \
    do {                                              \
        if (comp && acc_out) G(YD, WD, true, true);   \
        else if (comp) G(YD, WD, true, false);        \
        else if (acc_out) G(YD, WD, false, true);     \
        else G(YD, WD, false, false);                 \
    } while (0)
    if (y_dt == DT_BF16) {
        if (w_dt == DT_BF16) G2(DT_BF16, DT_BF16);
        else G2(DT_BF16, DT_F32);
    } else {
        if (w_dt == DT_BF16) G2(DT_F32, DT_BF16);
        else G2(DT_F32, DT_F32);
    }
#undef G2
#undef G
    return hipGetLastError();
}

}  // namespace fp4
