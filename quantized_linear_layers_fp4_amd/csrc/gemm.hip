// gfx950 FP4 GEMM of the quantized operands with the dequantization fused into its output
// (QbitAI report on "Optimizing Large Language Model Training Using FP4 Quantization":
// GEMM-kernel paragraph for the FP4 tiled product, granularity paragraph for the row/column
// scales that factor out of the K-sum).  The pages' kernel emulates FP4 on FP8 tensor cores and reduces in
// FP16; here the CDNA4 matrix cores multiply E2M1 operands natively (unit E8M0 block
// scales) and accumulate in fp32, which is exact for these operands.
//
// Workgroup: 8 waves (two per SIMD) own a 256 x 256 output tile; wave (wm, wn) owns rows
// 128*wm.. and columns 64*wn.. as 4 x 2 tiles of V_MFMA_SCALE_F32_32X32X64_F8F6F4.
// K advances 128 codes (64 bytes per row) per stage.  Operand tiles travel from global
// memory straight into one of four LDS stage buffers (buffer loads with the LDS flag,
// issued three stages ahead); rows or K chunks outside the matrices read as zero.  One
// barrier per stage; the fragments of the next stage's first K-step are read before it, so
// the matrix cores restart right after each barrier.  The row/column scales of the tile are
// fetched into LDS under the first stage loads.
//
// Epilogue: Y = fl(fl(acc * sA) * sW), 32 rows at a time through an fp32 slab in LDS so
// every store is a 16-byte row segment.  The sparse compensation dA . W is a separate
// kernel (comp.hip) that runs on the fp32 result.
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
    void *Y;
    float *acc_out;
    int tilesM, tilesN, raster_group;
};

// The tile's row and column scales, fetched into LDS under the first stage loads.
struct Book {
    float sA[BM];
    float sW[BN];
};

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

// Workgroup barrier for LDS traffic only: this wave's LDS reads and writes are done, then
// s_barrier.  Global stores stay in flight.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt and expcnt unconstrained
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
}

template <int YDT, bool ACCOUT>
__global__ __launch_bounds__(NT, 2) void k_fp4_gemm(TileArgs p) {
    __shared__ __attribute__((aligned(16))) uint8_t sb0[STB];
    __shared__ __attribute__((aligned(16))) uint8_t sb1[STB];
    __shared__ __attribute__((aligned(16))) uint8_t sb2[STB];
    __shared__ __attribute__((aligned(16))) uint8_t sb3[STB];
    __shared__ __attribute__((aligned(16))) Book bk;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 2, wn = wave & 3;
    const int M = p.M, N = p.N, K = p.K;

    // XCD-aware order: consecutive workgroup ids go to different XCDs, so give each XCD a
    // contiguous range of logical tiles; within it raster_group tile-rows sweep the
    // tile-columns together, so the tiles an XCD runs at once share operand strips in its L2.
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

    // prologue: stage 0, the tile's scales, then stages 1 and 2.  The scale loads are older
    // than the later stages' loads, so the wait for stages 0 and 1 covers them too.
    stage_dma(rsA, rsB, sb0, wave, offA, offB, 0, KB, lane_chunk16);
    __builtin_amdgcn_sched_barrier(0);
    float bA = 0.0f, bW = 0.0f;
    if (tid < 256) {
        if (m0 + tid < M) bA = p.sA[m0 + tid];
        if (n0 + tid < N) bW = p.sW[n0 + tid];
    }
    __builtin_amdgcn_sched_barrier(0);
    stage_dma(rsA, rsB, sb1, wave, offA, offB, 1, KB, lane_chunk16);
    stage_dma(rsA, rsB, sb2, wave, offA, offB, 2, KB, lane_chunk16);
    __builtin_amdgcn_sched_barrier(0);
    WAIT_VMCNT(4);
    if (tid < 256) {
        bk.sA[tid] = bA;
        bk.sW[tid] = bW;
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

    // ---- epilogue: Y = fl(fl(acc * sA) * sW), 32 rows at a time through an fp32 slab in LDS.
    // MFMA 32x32 output layout: lane l, register r -> row 8*(r/4) + 4*(l/32) + r%4, col l%32.
    float *E = reinterpret_cast<float *>(sb0);
    float sw[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) sw[j] = bk.sW[wn * 64 + j * 32 + (lane & 31)];
    const int g = tid >> 5;    // 16 row groups: slab rows g and g + 16
    const int c8 = tid & 31;   // columns n0 + 8*c8 .. +7
    const int gn = n0 + c8 * 8;

    // slab q holds tile rows 32q..32q+31: MFMA tile q%4 of the waves with wm == q/4 (the
    // tile index must be a compile-time constant, so the four tiles of a half are unrolled)
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
}

// Tile-rows per column sweep within an XCD.  FP4_GEMM_RASTER overrides (tuning aid).
static int raster_group_for(int tilesM) {
    static int env = -2;
    if (env == -2) {
        const char *e = getenv("FP4_GEMM_RASTER");
        env = e ? atoi(e) : -1;
    }
    const int g = env > 0 ? env : 8;
    return g < tilesM ? g : tilesM;
}

hipError_t launch_gemm(const uint8_t *Aq, const float *sA, const uint8_t *Wq, const float *sW, int64_t M,
                       int64_t N, int64_t K, void *Y, int y_dt, float *acc_out, hipStream_t s) {
    TileArgs p;
    p.Aq = Aq;
    p.Wq = Wq;
    p.sA = sA;
    p.sW = sW;
    p.M = (int)M;
    p.N = (int)N;
    p.K = (int)K;
    p.Y = Y;
    p.acc_out = acc_out;
    p.tilesM = (int)((M + BM - 1) / BM);
    p.tilesN = (int)((N + BN - 1) / BN);
    p.raster_group = raster_group_for(p.tilesM);
    const int64_t tiles = (int64_t)p.tilesM * p.tilesN;
    const int blocks = (int)((tiles + 7) / 8 * 8);
#define G(YD, AO) hipLaunchKernelGGL((k_fp4_gemm<YD, AO>), dim3(blocks), dim3(NT), 0, s, p)
    if (y_dt == DT_BF16) {
        if (acc_out) G(DT_BF16, true);
        else G(DT_BF16, false);
    } else {
        if (acc_out) G(DT_F32, true);
        else G(DT_F32, false);
    }
#undef G
    return hipGetLastError();
}

}  // namespace fp4
