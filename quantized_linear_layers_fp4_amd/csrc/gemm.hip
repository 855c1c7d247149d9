// gfx950 FP4 GEMM of the quantized operands with the dequantization and the sparse
// compensation fused into its output (QbitAI report on "Optimizing Large Language Model
// Training Using FP4 Quantization": GEMM-kernel paragraph for the FP4 tiled product,
// granularity paragraph for the row/column scales that factor out of the K-sum, outlier
// paragraph for dA).  The pages' kernel emulates FP4 on FP8 tensor cores and reduces in
// FP16; here the CDNA4 matrix cores multiply E2M1 operands natively (unit E8M0 block
// scales) and accumulate in fp32, which is exact for these operands.
//
// Tile: 256 x 256 outputs per workgroup of 4 waves, each wave 128 x 128 as 4 x 4 tiles of
// V_MFMA_SCALE_F32_32X32X64_F8F6F4.  K advances 256 codes (128 bytes per row) per stage;
// two LDS stages of A and B (2 x 64 KiB) with an XOR swizzle of the 16-byte chunks.
#include "fp4_common.h"
#include "fp4_launch.h"

namespace fp4 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int BM = 256, BN = 256;
constexpr int BKB = 128;                   // bytes of K per stage per row (256 codes)
constexpr int STAGE_BYTES = (BM + BN) * BKB;
constexpr int EPI_ROWS = 128;              // epilogue processes half a tile at a time
constexpr int EPI_LD = BN + 4;             // fp32 per LDS row in the epilogue
constexpr int EPI_BYTES = EPI_ROWS * EPI_LD * 4;
constexpr int LDS_BYTES = (2 * STAGE_BYTES > EPI_BYTES) ? 2 * STAGE_BYTES : EPI_BYTES;
constexpr int RASTER_GROUP = 8;            // tile-rows that sweep the tile-columns together
constexpr int UNIT_SCALE = 0x7F7F7F7F;     // E8M0 127 = 2^0 in every byte

// 16-byte slot of (row, chunk) in a 256-row x 8-chunk operand tile.  Reads (32 rows, one
// chunk) and writes (2 rows, all chunks) of 16 lanes each touch 16 distinct slots mod 16.
__device__ __forceinline__ int slot16(int row, int chunk) { return row * 8 + (chunk ^ ((row >> 1) & 7)); }

template <int YDT, int WDT, bool COMP, bool ACCOUT>
__global__ __launch_bounds__(256) void k_fp4_gemm(const uint8_t *__restrict__ Aq, const float *__restrict__ sA,
                                                  const uint8_t *__restrict__ Wq, const float *__restrict__ sW,
                                                  int M, int N, int K, const int32_t *__restrict__ row_ptr,
                                                  const int32_t *__restrict__ coo_col,
                                                  const float *__restrict__ coo_val, const void *__restrict__ Wc,
                                                  void *__restrict__ Y, float *__restrict__ acc_out, int tilesM,
                                                  int tilesN) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[LDS_BYTES];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    // XCD-aware order: consecutive workgroup ids go to different XCDs, so give each XCD a
    // contiguous range of logical tiles, then raster RASTER_GROUP tile-rows per column
    // sweep so the tiles an XCD runs together share operand strips in its L2.
    const int per_xcd = gridDim.x / 8;
    const int logical = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    if (logical >= tilesM * tilesN) return;
    const int group = logical / (RASTER_GROUP * tilesN);
    const int first_m = group * RASTER_GROUP;
    const int gm = min(RASTER_GROUP, tilesM - first_m);
    const int in_group = logical - group * RASTER_GROUP * tilesN;
    const int tm = first_m + in_group % gm;
    const int tn = in_group / gm;
    const int m0 = tm * BM, n0 = tn * BN;

    const int KB = K / 2;
    const int kstages = (KB + BKB - 1) / BKB;

    // global -> LDS assignment: pass p moves rows p*32 + tid/8, 16-byte chunk tid%8
    const int lrow = tid >> 3, lchunk = tid & 7;
    uint4 ra[8], rb[8];
    auto gload = [&](int kt) {
        const int kb = kt * BKB + lchunk * 16;
        const bool kin = kb < KB;
#pragma unroll
        for (int p = 0; p < 8; ++p) {
            const int r = p * 32 + lrow;
            const int am = m0 + r, bn = n0 + r;
            ra[p] = (kin && am < M) ? *reinterpret_cast<const uint4 *>(Aq + (size_t)am * KB + kb) : make_uint4(0, 0, 0, 0);
            rb[p] = (kin && bn < N) ? *reinterpret_cast<const uint4 *>(Wq + (size_t)bn * KB + kb) : make_uint4(0, 0, 0, 0);
        }
    };
    auto lstore = [&](int buf) {
        uint8_t *As = lds + buf * STAGE_BYTES;
        uint8_t *Bs = As + BM * BKB;
#pragma unroll
        for (int p = 0; p < 8; ++p) {
            const int r = p * 32 + lrow;
            *reinterpret_cast<uint4 *>(As + slot16(r, lchunk) * 16) = ra[p];
            *reinterpret_cast<uint4 *>(Bs + slot16(r, lchunk) * 16) = rb[p];
        }
    };

    v16f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    gload(0);
    lstore(0);
    __syncthreads();
    for (int kt = 0; kt < kstages; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < kstages) gload(kt + 1);
        const uint8_t *As = lds + buf * STAGE_BYTES;
        const uint8_t *Bs = As + BM * BKB;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            // lane l holds row l%32 of each 32-row tile and the 32 codes of K-half l/32
            const int chunk = 2 * s + (lane >> 5);
            v8i a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint4 q = *reinterpret_cast<const uint4 *>(As + slot16(wm * 128 + i * 32 + (lane & 31), chunk) * 16);
                a[i] = v8i{(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint4 q = *reinterpret_cast<const uint4 *>(Bs + slot16(wn * 128 + j * 32 + (lane & 31), chunk) * 16);
                b[j] = v8i{(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[j], acc[i][j], 4, 4, 0, UNIT_SCALE,
                                                                                0, UNIT_SCALE);
        }
        if (kt + 1 < kstages) lstore(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: Y = fl(fl(acc * sA) * sW) (+ compensation), half a tile at a time
    // MFMA 32x32 output layout: lane l, register r -> row 8*(r/4) + 4*(l/32) + r%4, col l%32.
    float *E = reinterpret_cast<float *>(lds);
    for (int half = 0; half < 2; ++half) {
        if (wm == half) {
            float sw[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int gn = n0 + wn * 128 + j * 32 + (lane & 31);
                sw[j] = gn < N ? sW[gn] : 0.0f;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int lr = i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                    const int grow = m0 + half * 128 + lr;
                    const float sa = grow < M ? sA[grow] : 0.0f;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int lc = wn * 128 + j * 32 + (lane & 31);
                        const float a = acc[i][j][r];
                        if constexpr (ACCOUT) {
                            if (grow < M && n0 + lc < N) acc_out[(size_t)grow * N + n0 + lc] = a;
                        }
                        const float t = a * sa;
                        E[lr * EPI_LD + lc] = t * sw[j];
                    }
                }
        }
        __syncthreads();
        // row-wise pass: 128 rows x 32 chunks of 8 columns; 32 threads per row
        const int c8 = tid & 31;
        const int gn = n0 + c8 * 8;
        for (int it = 0; it < 16; ++it) {
            const int lr = it * 8 + (tid >> 5);
            const int grow = m0 + half * 128 + lr;
            if (grow < M && gn < N) {
                float y[8];
                const float4 e0 = *reinterpret_cast<const float4 *>(&E[lr * EPI_LD + c8 * 8]);
                const float4 e1 = *reinterpret_cast<const float4 *>(&E[lr * EPI_LD + c8 * 8 + 4]);
                y[0] = e0.x; y[1] = e0.y; y[2] = e0.z; y[3] = e0.w;
                y[4] = e1.x; y[5] = e1.y; y[6] = e1.z; y[7] = e1.w;
                if constexpr (COMP) {
                    float d[8] = {0, 0, 0, 0, 0, 0, 0, 0};
                    const int e_end = row_ptr[grow + 1];
                    for (int e = row_ptr[grow]; e < e_end; ++e) {
                        const int k = coo_col[e];
                        const float dv = coo_val[e];
                        float w[8];
                        if constexpr (WDT == DT_BF16) {
                            const uint4 q = *reinterpret_cast<const uint4 *>(
                                reinterpret_cast<const uint16_t *>(Wc) + (size_t)k * N + gn);
                            const uint32_t ws[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
                            for (int t = 0; t < 4; ++t) {
                                w[2 * t] = bf16_to_f32(ws[t] & 0xFFFFu);
                                w[2 * t + 1] = bf16_to_f32(ws[t] >> 16);
                            }
                        } else {
                            const float4 *p = reinterpret_cast<const float4 *>(
                                reinterpret_cast<const float *>(Wc) + (size_t)k * N + gn);
                            const float4 q0 = p[0], q1 = p[1];
                            w[0] = q0.x; w[1] = q0.y; w[2] = q0.z; w[3] = q0.w;
                            w[4] = q1.x; w[5] = q1.y; w[6] = q1.z; w[7] = q1.w;
                        }
#pragma unroll
                        for (int t = 0; t < 8; ++t) d[t] = __builtin_fmaf(dv, w[t], d[t]);
                    }
#pragma unroll
                    for (int t = 0; t < 8; ++t) y[t] = y[t] + d[t];
                }
                if constexpr (YDT == DT_BF16) {
                    uint4 o;
                    o.x = f32_to_bf16_bits(y[0]) | (f32_to_bf16_bits(y[1]) << 16);
                    o.y = f32_to_bf16_bits(y[2]) | (f32_to_bf16_bits(y[3]) << 16);
                    o.z = f32_to_bf16_bits(y[4]) | (f32_to_bf16_bits(y[5]) << 16);
                    o.w = f32_to_bf16_bits(y[6]) | (f32_to_bf16_bits(y[7]) << 16);
                    *reinterpret_cast<uint4 *>(reinterpret_cast<uint16_t *>(Y) + (size_t)grow * N + gn) = o;
                } else {
                    float4 *p = reinterpret_cast<float4 *>(reinterpret_cast<float *>(Y) + (size_t)grow * N + gn);
                    p[0] = make_float4(y[0], y[1], y[2], y[3]);
                    p[1] = make_float4(y[4], y[5], y[6], y[7]);
                }
            }
        }
        __syncthreads();
    }
}

hipError_t launch_gemm(const uint8_t *Aq, const float *sA, const uint8_t *Wq, const float *sW, int64_t M,
                       int64_t N, int64_t K, const int32_t *row_ptr, const int32_t *coo_col,
                       const float *coo_val, const void *W, int w_dt, void *Y, int y_dt, float *acc_out,
                       hipStream_t s) {
    const int tilesM = (int)((M + BM - 1) / BM), tilesN = (int)((N + BN - 1) / BN);
    const int64_t tiles = (int64_t)tilesM * tilesN;
    const int blocks = (int)((tiles + 7) / 8 * 8);
    const bool comp = row_ptr != nullptr;
    const int m = (int)M, n = (int)N, k = (int)K;
#define G(YD, WD, CO, AO)                                                                                   \
    hipLaunchKernelGGL((k_fp4_gemm<YD, WD, CO, AO>), dim3(blocks), dim3(256), 0, s, Aq, sA, Wq, sW, m, n, k, \
                       row_ptr, coo_col, coo_val, W, Y, acc_out, tilesM, tilesN)
#define G2(YD, WD)                                  \
    do {                                            \
        if (comp && acc_out) G(YD, WD, true, true);   \
        else if (comp) G(YD, WD, true, false);        \
        else if (acc_out) G(YD, WD, false, true);     \
        else G(YD, WD, false, false);                 \
    } while (0)
    if (y_dt == DT_BF16) {
        if (w_dt == DT_BF16) G2(DT_BF16, DT_BF16); else G2(DT_BF16, DT_F32);
    } else {
        if (w_dt == DT_BF16) G2(DT_F32, DT_BF16); else G2(DT_F32, DT_F32);
    }
#undef G2
#undef G
    return hipGetLastError();
}

}  // namespace fp4
