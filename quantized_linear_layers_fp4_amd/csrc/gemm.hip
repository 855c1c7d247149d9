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
// barrier per stage.
#include "fp4_common.h"
#include "fp4_launch.h"

#include <cstdlib>

namespace fp4 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
#define LDS_PTR(p) ((__attribute__((address_space(3))) void *)(p))

constexpr int BM = 256, BN = 256, NT = 512;
constexpr int BKB = 64;                    // bytes of K per row per stage (128 codes)
constexpr int OPB = 256 * BKB;             // one operand tile per stage: 16 KiB
constexpr int STB = 2 * OPB;               // A then B: 32 KiB per stage buffer
constexpr int UNIT_SCALE = 0x7F7F7F7F;     // E8M0 127 = 2^0 in every byte
constexpr int BUF_FLAGS = 0x00020000;      // raw buffer descriptor word 3 (gfx9 family)
constexpr int OOB = 0x7FFFFFF0;            // an offset past every buffer: the load returns 0
constexpr int SLAB = 32;                   // epilogue rows per pass (one 32-row MFMA tile)
constexpr int RP_OFF = 0, KC_OFF = 264, DV_OFF = 264 + 192;  // bookkeeping layout (ints)

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
    const int32_t *row_ptr, *coo_col;
    const float *coo_val;
    const void *Wc;
    void *Y;
    float *acc_out;
    int tilesM, tilesN, raster_group;
    int pf_dist;   // stages ahead that the L2 warm-up touches (0: off)
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

// The rest of one epilogue slab, after its scaled products are in E: add the dA * W
// compensation (W rows gathered into the freed stage buffers) and store 32 rows of Y.
template <int YDT, int WDT, bool COMP>
__device__ __forceinline__ void slab_finish(const TileArgs &p, int q, int m0, int n0, int tid, int wave, int lane,
                                            float *E, const int32_t *rp_s, int32_t *kc_s, float *dv_s, uint8_t *sb1,
                                            uint8_t *sb2, uint8_t *sb3, __amdgpu_buffer_rsrc_t rsW) {
    constexpr int ESZ = (WDT == DT_BF16) ? 2 : 4;
    constexpr int ROW_BYTES = BN * ESZ;          // one gathered W row segment
    constexpr int ROUND = 3 * STB / ROW_BYTES;   // entries gathered per round (3 buffers)
    const int M = p.M, N = p.N;
    const int g = tid >> 5;   // 16 row groups: rows g and g + 16 of the slab
    const int c8 = tid & 31;  // columns n0 + 8*c8 .. +7
    const int gn = n0 + c8 * 8;
        __syncthreads();
        if constexpr (COMP) {
            const int e_lo = rp_s[q * SLAB], e_hi = rp_s[q * SLAB + SLAB];
#pragma unroll 1
            for (int cb = e_lo; cb < e_hi; cb += ROUND) {
                const int n_e = min(ROUND, e_hi - cb);
                for (int t = tid; t < n_e; t += NT) {
                    kc_s[t] = p.coo_col[cb + t];
                    dv_s[t] = p.coo_val[cb + t];
                }
                __syncthreads();
                // gather W[k][n0 .. n0+255] of every entry into sb1..sb3 back to back; a load
                // moves 1 KiB: lane i carries bytes 16i.. of it
                const int loads = (n_e * ROW_BYTES + 1023) / 1024;
                for (int L = wave; L < loads; L += NT / 64) {
                    const int byte = L * 1024 + lane * 16;
                    const int e = byte / ROW_BYTES;
                    const int col = n0 + (byte % ROW_BYTES) / ESZ;
                    int o = OOB;
                    if (e < n_e && col < N) o = (kc_s[e] * N + col) * ESZ;
                    const int bsel = (L * 1024) / STB, within = L * 1024 - bsel * STB;
                    uint8_t *dst = bsel == 0 ? sb1 : (bsel == 1 ? sb2 : sb3);
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsW, LDS_PTR(dst + within), 16, o, 0, 0, 0);
                }
                WAIT_VMCNT(0);
                __syncthreads();
                if (gn < N) {
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int lr = g + 16 * h;
                        const int rel = q * SLAB + lr;
                        const int a0 = max(rp_s[rel], cb) - cb;
                        const int a1 = min(rp_s[rel + 1], cb + n_e) - cb;
                        if (a0 >= a1) continue;
                        float4 *ep0 = reinterpret_cast<float4 *>(&E[eidx(lr, c8 * 8)]);
                        float4 *ep1 = reinterpret_cast<float4 *>(&E[eidx(lr, c8 * 8 + 4)]);
                        float4 y0 = *ep0, y1 = *ep1;
                        for (int e = a0; e < a1; ++e) {
                            const int byte = e * ROW_BYTES + c8 * 8 * ESZ;
                            const int bsel = byte / STB;
                            const uint8_t *src = (bsel == 0 ? sb1 : (bsel == 1 ? sb2 : sb3)) + (byte - bsel * STB);
                            float wf[8];
                            if constexpr (WDT == DT_BF16) {
                                const u32x4 q4 = *reinterpret_cast<const u32x4 *>(src);
                                const uint32_t ws[4] = {q4.x, q4.y, q4.z, q4.w};
#pragma unroll
                                for (int t = 0; t < 4; ++t) {
                                    wf[2 * t] = bf16_to_f32(ws[t] & 0xFFFFu);
                                    wf[2 * t + 1] = bf16_to_f32(ws[t] >> 16);
                                }
                            } else {
                                const u32x4 q0 = *reinterpret_cast<const u32x4 *>(src);
                                const u32x4 q1 = *reinterpret_cast<const u32x4 *>(src + 16);
                                const uint32_t ws[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
                                for (int t = 0; t < 8; ++t) wf[t] = __uint_as_float(ws[t]);
                            }
                            const float d = dv_s[e];
                            y0.x = __builtin_fmaf(d, wf[0], y0.x);
                            y0.y = __builtin_fmaf(d, wf[1], y0.y);
                            y0.z = __builtin_fmaf(d, wf[2], y0.z);
                            y0.w = __builtin_fmaf(d, wf[3], y0.w);
                            y1.x = __builtin_fmaf(d, wf[4], y1.x);
                            y1.y = __builtin_fmaf(d, wf[5], y1.y);
                            y1.z = __builtin_fmaf(d, wf[6], y1.z);
                            y1.w = __builtin_fmaf(d, wf[7], y1.w);
                        }
                        *ep0 = y0;
                        *ep1 = y1;
                    }
                }
                __syncthreads();
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
                        float4 *yp = reinterpret_cast<float4 *>(reinterpret_cast<float *>(p.Y) + (size_t)grow * N + gn);
                        yp[0] = e0;
                        yp[1] = e1;
                    }
                }
            }
        }
        __syncthreads();
}

template <int YDT, int WDT, bool COMP, bool ACCOUT>
__global__ __launch_bounds__(NT) void k_fp4_gemm(TileArgs p) {
    __shared__ __attribute__((aligned(16))) uint8_t sb0[STB];
    __shared__ __attribute__((aligned(16))) uint8_t sb1[STB];
    __shared__ __attribute__((aligned(16))) uint8_t sb2[STB];
    __shared__ __attribute__((aligned(16))) uint8_t sb3[STB];
    __shared__ __attribute__((aligned(16))) int32_t sx[1024];  // epilogue bookkeeping
    __shared__ __attribute__((aligned(16))) uint32_t sink[8 * 64];  // target of the L2 warm-up loads
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 2, wn = wave & 3;
    const int M = p.M, N = p.N, K = p.K;

    // XCD-aware order: consecutive workgroup ids go to different XCDs, so give each XCD a
    // contiguous range of logical tiles; within it raster_group tile-rows sweep the
    // tile-columns together, so the tiles an XCD runs at once share their W column strip
    // (operand codes and the compensation's W rows) in its L2.
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

    stage_dma(rsA, rsB, sb0, wave, offA, offB, 0, KB, lane_chunk16);
    stage_dma(rsA, rsB, sb1, wave, offA, offB, 1, KB, lane_chunk16);
    stage_dma(rsA, rsB, sb2, wave, offA, offB, 2, KB, lane_chunk16);
    WAIT_VMCNT(8);
    __builtin_amdgcn_s_barrier();

    // L2 warm-up: one 4-byte load per 64-byte line of stage kt + pf_dist (waves 0-3 cover
    // the 256 A rows, waves 4-7 the 256 B rows), landing in a scratch LDS word.  It pulls
    // the lines into the XCD's L2 ahead of the stage loads, which then hit.
    const int pf_row = (wave & 3) * 64 + lane;
    const int pf_base = (wave < 4) ? ((m0 + pf_row < M) ? (m0 + pf_row) * KB : OOB)
                                   : ((n0 + pf_row < N) ? (n0 + pf_row) * KB : OOB);
    const __amdgpu_buffer_rsrc_t rsPF = (wave < 4) ? rsA : rsB;
    auto warm = [&](int kt) {
        const int s = kt + p.pf_dist;
        const int o = (p.pf_dist > 0 && pf_base != OOB && s * BKB < KB) ? pf_base + s * BKB : OOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsPF, LDS_PTR(sink + wave * 64), 4, o, 0, 0, 0);
    };

    // Stage kt lives in buffer kt%4.  Its loads were issued at stage kt-3; each wave waits
    // for its own loads of stage kt+1 before the barrier that ends stage kt, so after that
    // barrier stage kt+1 is complete and stage kt's buffer is free for stage kt+4.  Per
    // stage a wave issues 4 stage loads then 1 warm-up load: 11 loads follow those of
    // stage kt+1.
    auto step = [&](int kt, const uint8_t *cur, uint8_t *ahead) {
        __builtin_amdgcn_sched_barrier(0);
        stage_dma(rsA, rsB, ahead, wave, offA, offB, kt + 3, KB, lane_chunk16);
        warm(kt);
        u32x4 a0[4], b0[2], a1[4], b1[2];
        frag_load(cur, wm, wn, lane, 0, a0, b0);
        frag_load(cur, wm, wn, lane, 1, a1, b1);
        __builtin_amdgcn_sched_barrier(0);
        mfma_block(acc, a0, b0);
        __builtin_amdgcn_sched_barrier(0);
        mfma_block(acc, a1, b1);
        __builtin_amdgcn_sched_barrier(0);
        WAIT_VMCNT(11);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };
    // whole groups of four stages (a group may run past the last stage on zeros: one exit
    // keeps the accumulators in one set of registers)
    for (int kt = 0; kt < kstages; kt += 4) {
        step(kt, sb0, sb3);
        step(kt + 1, sb1, sb0);
        step(kt + 2, sb2, sb1);
        step(kt + 3, sb3, sb2);
    }
    WAIT_VMCNT(0);  // look-ahead loads past the end (zeros) land before the buffers are reused
    __syncthreads();

    // ---- epilogue: Y = fl(fl(acc * sA) * sW), then + sum of delta * W[k][n] over the row's
    // dA entries in ascending k, 32 rows at a time through an fp32 slab in LDS.
    // MFMA 32x32 output layout: lane l, register r -> row 8*(r/4) + 4*(l/32) + r%4, col l%32.
    constexpr int ESZ = (WDT == DT_BF16) ? 2 : 4;
    constexpr int ROW_BYTES = BN * ESZ;                 // one gathered W row segment
    constexpr int ROUND = 3 * STB / ROW_BYTES;          // entries gathered per round (3 buffers)
    static_assert(ROUND <= 192, "bookkeeping holds 192 entries");
    float *E = reinterpret_cast<float *>(sb0);
    int32_t *rp_s = sx + RP_OFF;
    int32_t *kc_s = sx + KC_OFF;
    float *dv_s = reinterpret_cast<float *>(sx + DV_OFF);
    if constexpr (COMP) {
        for (int t = tid; t <= BM; t += NT) rp_s[t] = p.row_ptr[min(m0 + t, M)];
    }
    float sw[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int gcol = n0 + wn * 64 + j * 32 + (lane & 31);
        sw[j] = gcol < N ? p.sW[gcol] : 0.0f;
    }
    const __amdgpu_buffer_rsrc_t rsW =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p.Wc), 0, COMP ? K * N * ESZ : 0, BUF_FLAGS);

    // slab q holds tile rows 32q..32q+31: MFMA tile q%4 of the waves with wm == q/4 (the
    // tile index must be a compile-time constant, so the four tiles are unrolled)
#pragma unroll
    for (int qi = 0; qi < 4; ++qi) {
#pragma unroll 1
        for (int qh = 0; qh < 2; ++qh) {
            const int q = qh * 4 + qi;
            if (wm == qh) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int lr = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                    const int grow = m0 + q * SLAB + lr;
                    const float sa = grow < M ? p.sA[grow] : 0.0f;
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const int lc = wn * 64 + j * 32 + (lane & 31);
                        const float a = acc[qi][j][r];
                        if constexpr (ACCOUT) {
                            if (grow < M && n0 + lc < N) p.acc_out[(size_t)grow * N + n0 + lc] = a;
                        }
                        const float t = a * sa;
                        E[eidx(lr, lc)] = t * sw[j];
                    }
                }
            }
            slab_finish<YDT, WDT, COMP>(p, q, m0, n0, tid, wave, lane, E, rp_s, kc_s, dv_s, sb1, sb2, sb3, rsW);
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
    const int g = env > 0 ? env : 32;
    return g < tilesM ? g : tilesM;
}

// Stages ahead of the one being multiplied that the L2 warm-up touches.  FP4_GEMM_PF
// overrides (tuning aid; 0 disables).
static int pf_dist_default() {
    static int env = -2;
    if (env == -2) {
        const char *e = getenv("FP4_GEMM_PF");
        env = e ? atoi(e) : -1;
    }
    return env >= 0 ? env : 8;
}

hipError_t launch_gemm(const uint8_t *Aq, const float *sA, const uint8_t *Wq, const float *sW, int64_t M,
                       int64_t N, int64_t K, const int32_t *row_ptr, const int32_t *coo_col,
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
    p.coo_col = coo_col;
    p.coo_val = coo_val;
    p.Wc = W;
    p.Y = Y;
    p.acc_out = acc_out;
    p.tilesM = (int)((M + BM - 1) / BM);
    p.tilesN = (int)((N + BN - 1) / BN);
    p.raster_group = raster_group_for(p.tilesM);
    p.pf_dist = pf_dist_default();
    const int64_t tiles = (int64_t)p.tilesM * p.tilesN;
    const int blocks = (int)((tiles + 7) / 8 * 8);
    const bool comp = row_ptr != nullptr;
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
