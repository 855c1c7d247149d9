// gfx950 FP4 GEMM of the quantized operands with the dequantization fused into its output
// (QbitAI report on "Optimizing Large Language Model Training Using FP4 Quantization":
// GEMM-kernel paragraph for the FP4 tiled product, granularity paragraph for the row/column
// scales that factor out of the K-sum).  The pages' kernel emulates FP4 on FP8 tensor cores and reduces in
// FP16; here the CDNA4 matrix cores multiply E2M1 operands natively (the F8F6F4 MFMA in its
// unscaled form, i.e. unit block scales) and accumulate in fp32, which is exact for these operands.
//
// Workgroup: 4 waves (one per SIMD) own a 256 x 128 output tile; wave (wm, wn) owns rows
// 128*wm.. and columns 64*wn.. as 4 x 2 tiles of V_MFMA_F32_32X32X64_F8F6F4.  Two
// workgroups share a CU (73.5 KiB of LDS each), so one's epilogue and barriers run under
// the other's matrix work.  K advances 128 codes (64 bytes per row) per stage.  Operand
// tiles travel from global memory straight into one of three LDS stage buffers (buffer
// loads with the LDS flag, issued two stages ahead); rows or K chunks outside the matrices
// read as zero.  One barrier per stage; the second K-step's fragments are read under the
// first K-step's MFMAs.  The row/column scales of the tile are fetched into LDS with the
// first stage.
//
// Epilogue: Y = fl(fl(acc * sA) * sW); each wave reorders its result tiles through a
// private patch of LDS so that the stores are 16 bytes per lane along rows.  In front of the
// sparse compensation dA . W (a separate kernel, comp.hip) the output is instead the exact
// accumulator as the int16 4*acc (DT_Q16), with a map of the 128 x 64 output blocks where it
// does not fit (escape.hip recomputes those); the compensation pass rebuilds Y_main from it.
//
// Large products (K a multiple of 512 and at least two 256 x 256 tiles per CU) run on a
// second, persistent kernel with 256 x 256 tiles (see "wide tiles" below); both compute the
// same exact accumulator and epilogue, so their outputs are identical.
#include "fp4_common.h"
#include "fp4_launch.h"

namespace fp4 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));
#define LDS_PTR(p) ((__attribute__((address_space(3))) void *)(p))

constexpr int BM = 256, BN = 128, NW = 4, NT = 64 * NW;
constexpr int BKB = 64;                    // bytes of K per row per stage (128 codes)
constexpr int OPA = BM * BKB;              // A tile per stage: 16 KiB
constexpr int STB = (BM + BN) * BKB;       // A then B: 24 KiB per stage buffer
// Block scales of the MFMA: 0 in both scale operands selects the unscaled form of the
// instruction (V_MFMA_F32_32X32X64_F8F6F4, unit scales).  Its results equal those with explicit
// E8M0 unit scales (127 in every byte), and it issues faster: 32.7 against 34.4 cycles per
// MFMA in a chain of independent FP4 MFMAs on one box, at a 4 % higher clock.
constexpr int UNIT_SCALE = 0;
constexpr int BUF_FLAGS = 0x00020000;      // raw buffer descriptor word 3 (gfx9 family)
constexpr int OOB = 0x7FFFFFF0;            // an offset past every buffer: the load returns 0

// 16-byte slot of (row, chunk) in an operand tile of 4 chunks per row.  A 16-lane group
// reading 16 consecutive rows of one chunk hits 16 distinct slots modulo 16.
__device__ __forceinline__ int slot16(int row, int chunk) { return row * 4 + (chunk ^ ((row >> 2) & 3)); }

struct TileArgs {
    const uint8_t *Aq, *Wq;
    const float *sA, *sW;
    int M, N, K;
    void *Y;
    float *acc_out;
    uint8_t *emap;   // DT_Q16: one byte per 128 x 64 output block (row-major, stride mapN),
                     // 1 when the wave block it lies in holds some |acc| > Q16_MAX_ACC
    int cellsM, cellsN, mapN;
    int tilesM, tilesN, raster_group;
};

// The tile's row and column scales, fetched into LDS with the first stage.
struct Book {
    float sA[BM];
    float sW[BN];
};

// One stage of DMA for this wave: 4 loads of A (rows 64w..64w+63) and NB of B (rows
// 16*NB*w ..).  Lane i of a load fills slot 64*blk + i: row 16*blk + i/4, at the swizzled
// position i%4.  KFULL (K a multiple of 128: every stage is whole): the stage's K offset
// goes in the scalar offset and rows past the matrix read zeros through their offset
// alone; the look-ahead stages past the end reload the last stage (never consumed), so
// every address stays inside its row.  Otherwise each lane also checks its chunk against
// K, so a partial last stage and the stages past the end read zeros.  opa: bytes of the
// A tile in the stage buffer.
template <bool KFULL, int NB>
__device__ __forceinline__ void stage_dma(__amdgpu_buffer_rsrc_t rsA, __amdgpu_buffer_rsrc_t rsB, uint8_t *buf,
                                          int wave, const int (&offA)[4], const int (&offB)[NB], int kt, int KB,
                                          int lane_chunk16, int opa = OPA) {
    const bool kin = KFULL || kt * BKB + lane_chunk16 < KB;
    const int soff = KFULL ? min(kt, KB / BKB - 1) * BKB : 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int oa = KFULL ? offA[j] : ((kin && offA[j] != OOB) ? offA[j] + kt * BKB : OOB);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsA, LDS_PTR(buf + (wave * 4 + j) * 1024), 16, oa, soff, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        const int ob = KFULL ? offB[j] : ((kin && offB[j] != OOB) ? offB[j] + kt * BKB : OOB);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsB, LDS_PTR(buf + opa + (wave * NB + j) * 1024), 16, ob, soff, 0,
                                                 0);
    }
}

// Fragments of K-step s (0 or 1) of a stage: lane l reads row l%32 of each 32-row tile and
// the 16-byte chunk 2s + l/32 (32 codes).  The wave's tiles: 4 of A from row 128*wm and NJ
// of B from row 32*NJ*wn.
template <int NJ>
__device__ __forceinline__ void frag_load(const uint8_t *buf, int wm, int wn, int lane, int s, u32x4 (&a)[4],
                                          u32x4 (&b)[NJ], int opa = OPA) {
    const int chunk = 2 * s + (lane >> 5);
#pragma unroll
    for (int i = 0; i < 4; ++i)
        a[i] = *reinterpret_cast<const u32x4 *>(buf + slot16(wm * 128 + i * 32 + (lane & 31), chunk) * 16);
#pragma unroll
    for (int j = 0; j < NJ; ++j)
        b[j] = *reinterpret_cast<const u32x4 *>(buf + opa + slot16(wn * 32 * NJ + j * 32 + (lane & 31), chunk) * 16);
}

// FP8 operands (the emulation path): lane l reads row l%32 and the two 16-byte chunks
// 2*(l/32), 2*(l/32)+1 (32 consecutive K values, one per byte) of the stage's one K-step.
__device__ __forceinline__ void frag_load8(const uint8_t *buf, int wm, int wn, int lane, u32x4 (&a)[4][2],
                                           u32x4 (&b)[2][2]) {
    const int chunk = 2 * (lane >> 5);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            a[i][h] = *reinterpret_cast<const u32x4 *>(buf + slot16(wm * 128 + i * 32 + (lane & 31), chunk + h) * 16);
#pragma unroll
        for (int j = 0; j < 2; ++j)
            b[j][h] =
                *reinterpret_cast<const u32x4 *>(buf + OPA + slot16(wn * 64 + j * 32 + (lane & 31), chunk + h) * 16);
    }
}

// The same tile product on E4M3 operands (format code 0): 32 bytes per lane and MFMA.
__device__ __forceinline__ void mfma_block8(v16f (&acc)[4][2], const u32x4 (&a)[4][2], const u32x4 (&b)[2][2]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const v8i av = v8i{(int)a[i][0].x, (int)a[i][0].y, (int)a[i][0].z, (int)a[i][0].w,
                           (int)a[i][1].x, (int)a[i][1].y, (int)a[i][1].z, (int)a[i][1].w};
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const v8i bv = v8i{(int)b[j][0].x, (int)b[j][0].y, (int)b[j][0].z, (int)b[j][0].w,
                               (int)b[j][1].x, (int)b[j][1].y, (int)b[j][1].z, (int)b[j][1].w};
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc[i][j], 0, 0, 0, UNIT_SCALE, 0,
                                                                        UNIT_SCALE);
        }
    }
}

// SW: the operands swapped, so tile (i, j) holds the transpose (lane l: row l%32 of the
// product, columns 8(r/4) + 4(l/32) + r%4 in register r: four consecutive columns per quad).
template <int NJ, bool SW = false>
__device__ __forceinline__ void mfma_block(v16f (&acc)[4][NJ], const u32x4 (&a)[4], const u32x4 (&b)[NJ]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const v8i av = v8i{(int)a[i].x, (int)a[i].y, (int)a[i].z, (int)a[i].w, 0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const v8i bv = v8i{(int)b[j].x, (int)b[j].y, (int)b[j].z, (int)b[j].w, 0, 0, 0, 0};
            if constexpr (SW)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bv, av, acc[i][j], 4, 4, 0, UNIT_SCALE, 0,
                                                                            UNIT_SCALE);
            else
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc[i][j], 4, 4, 0, UNIT_SCALE, 0,
                                                                            UNIT_SCALE);
        }
    }
}

// s_waitcnt vmcnt(n), other counters untouched (gfx9 encoding)
#define WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | 0x0F70)

// Workgroup barrier for LDS traffic only: this wave's LDS reads and writes are done, then
// s_barrier.  Buffer loads stay in flight (their waits are explicit).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt and expcnt unconstrained
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
}

// The epilogue of two side-by-side 32 x 32 tiles (rows row0.., columns col0.. and col0+32..)
// computed with swapped MFMA operands (mfma_block<.., true>): lane l holds row l%32 and, per
// quad a, the four consecutive columns 8a + 4(l/32) ...
// DT_Q16: the low 16 bits of fl(4*acc + 1.5*2^23), which are 4*acc as int16 whenever
// |acc| <= Q16_MAX_ACC; esc is set when some lane of the wave holds a larger |acc| (one ballot
// per pair: a running maximum over the whole tile pushed the wide kernel into spills).
// DT_BF16: the bf16 (nearest-even) of fl(fl(acc * sA) * sW); sa: the lane's row scale, sWp:
// the pair's 64 column scales (LDS).
// Read-back chunk c = 64k + lane holds row c/8 = 8k + lane/8, columns 8(c%8)..; loff0: its
// row-major offset (elements) for k = 0.  Each quad goes to the patch as one 8-byte write (two 16-bit values
// per dword), rows 68 values apart so the 32 rows' writes fall on distinct banks; the
// read-back takes each 16-byte row chunk as two 8-byte reads and stores it, so each row
// segment is 128 bytes.  The patch is private to the wave and a wave's LDS accesses execute
// in order, so the read-back sees the writes and the next call's writes cannot overtake it.
template <int YDT>
__device__ __forceinline__ void epi_pair_t(const v16f &x0, const v16f &x1, bool &esc, float sa, const float *sWp,
                                           uint16_t *P, int lane, int row0, int col0, int M, int N, bool full,
                                           uint16_t *Yo, uint32_t loff0) {
    constexpr int PS = 68;  // patch row stride, 16-bit values
    const int lr = lane & 31, h = lane >> 5;
    float m = 0.0f;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const v16f &x = t ? x1 : x0;
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            uint32_t q[4];
            if constexpr (YDT == DT_Q16) {
#pragma unroll
                for (int e = 0; e < 4; ++e) q[e] = __float_as_uint(__builtin_fmaf(x[4 * a + e], 4.0f, Q16_MAGIC));
                asm("v_max3_f32 %0, |%1|, |%2|, %3" : "=v"(m) : "v"(x[4 * a]), "v"(x[4 * a + 1]), "v"(m));
                asm("v_max3_f32 %0, |%1|, |%2|, %3" : "=v"(m) : "v"(x[4 * a + 2]), "v"(x[4 * a + 3]), "v"(m));
            } else {
                const float4 sw = *reinterpret_cast<const float4 *>(&sWp[32 * t + 8 * a + 4 * h]);
                q[0] = f32_to_bf16_bits((x[4 * a] * sa) * sw.x);
                q[1] = f32_to_bf16_bits((x[4 * a + 1] * sa) * sw.y);
                q[2] = f32_to_bf16_bits((x[4 * a + 2] * sa) * sw.z);
                q[3] = f32_to_bf16_bits((x[4 * a + 3] * sa) * sw.w);
            }
            const uint32_t w0 = (q[0] & 0xFFFFu) | (q[1] << 16), w1 = (q[2] & 0xFFFFu) | (q[3] << 16);
            *reinterpret_cast<uint2 *>(&P[lr * PS + 32 * t + 8 * a + 4 * h]) = make_uint2(w0, w1);
        }
    }
    if constexpr (YDT == DT_Q16) esc |= __builtin_amdgcn_ballot_w64(m > Q16_MAX_ACC) != 0;  // wave-uniform
    v4i e[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int c = k * 64 + lane;
        const uint2 u0 = *reinterpret_cast<const uint2 *>(&P[(c >> 3) * PS + (c & 7) * 8]);
        const uint2 u1 = *reinterpret_cast<const uint2 *>(&P[(c >> 3) * PS + (c & 7) * 8 + 4]);
        e[k] = v4i{(int)u0.x, (int)u0.y, (int)u1.x, (int)u1.y};
    }
    if (full) {
        uint16_t *base = Yo + (size_t)row0 * N + col0;
#pragma unroll
        for (int k = 0; k < 4; ++k)
            __builtin_nontemporal_store(e[k], reinterpret_cast<v4i *>(base + loff0 + (uint32_t)(8 * k) * (uint32_t)N));
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int c = k * 64 + lane, grow = row0 + (c >> 3), gcol = col0 + (c & 7) * 8;
            if (grow < M && gcol < N)
                __builtin_nontemporal_store(e[k], reinterpret_cast<v4i *>(Yo + (size_t)grow * N + gcol));
        }
    }
}

// The two halves of epi_pair_t, for an epilogue whose stores are deferred into the next
// tile's main loop: pair_pack turns the pair into 16 packed words per lane (quad (t, a) in
// words 2(4t + a), 2(4t + a) + 1), pair_store writes them through the patch.
template <int YDT>
__device__ __forceinline__ void pair_pack(const v16f &x0, const v16f &x1, float &m, float sa, const float *sWp,
                                          int lane, uint32_t (&pk)[16]) {
    const int h = lane >> 5;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const v16f &x = t ? x1 : x0;
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            uint32_t q[4];
            if constexpr (YDT == DT_Q16) {
#pragma unroll
                for (int e = 0; e < 4; ++e) q[e] = __float_as_uint(__builtin_fmaf(x[4 * a + e], 4.0f, Q16_MAGIC));
                asm("v_max3_f32 %0, |%1|, |%2|, %3" : "=v"(m) : "v"(x[4 * a]), "v"(x[4 * a + 1]), "v"(m));
                asm("v_max3_f32 %0, |%1|, |%2|, %3" : "=v"(m) : "v"(x[4 * a + 2]), "v"(x[4 * a + 3]), "v"(m));
            } else {
                const float4 sw = *reinterpret_cast<const float4 *>(&sWp[32 * t + 8 * a + 4 * h]);
                q[0] = f32_to_bf16_bits((x[4 * a] * sa) * sw.x);
                q[1] = f32_to_bf16_bits((x[4 * a + 1] * sa) * sw.y);
                q[2] = f32_to_bf16_bits((x[4 * a + 2] * sa) * sw.z);
                q[3] = f32_to_bf16_bits((x[4 * a + 3] * sa) * sw.w);
            }
            // low halves of two words into one (byte select 0x05040100): one v_perm_b32
            pk[2 * (4 * t + a)] = __builtin_amdgcn_perm(q[1], q[0], 0x05040100u);
            pk[2 * (4 * t + a) + 1] = __builtin_amdgcn_perm(q[3], q[2], 0x05040100u);
        }
    }
}

__device__ __forceinline__ void pair_store(const uint32_t (&pk)[16], uint16_t *P, int lane, int row0, int col0,
                                           int M, int N, bool full, uint16_t *Yo, uint32_t loff0) {
    constexpr int PS = 68;
    const int lr = lane & 31, h = lane >> 5;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int a = 0; a < 4; ++a)
            *reinterpret_cast<uint2 *>(&P[lr * PS + 32 * t + 8 * a + 4 * h]) =
                make_uint2(pk[2 * (4 * t + a)], pk[2 * (4 * t + a) + 1]);
    v4i e[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int c = k * 64 + lane;
        const uint2 u0 = *reinterpret_cast<const uint2 *>(&P[(c >> 3) * PS + (c & 7) * 8]);
        const uint2 u1 = *reinterpret_cast<const uint2 *>(&P[(c >> 3) * PS + (c & 7) * 8 + 4]);
        e[k] = v4i{(int)u0.x, (int)u0.y, (int)u1.x, (int)u1.y};
    }
    if (full) {
        uint16_t *base = Yo + (size_t)row0 * N + col0;
#pragma unroll
        for (int k = 0; k < 4; ++k)
            __builtin_nontemporal_store(e[k], reinterpret_cast<v4i *>(base + loff0 + (uint32_t)(8 * k) * (uint32_t)N));
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int c = k * 64 + lane, grow = row0 + (c >> 3), gcol = col0 + (c & 7) * 8;
            if (grow < M && gcol < N)
                __builtin_nontemporal_store(e[k], reinterpret_cast<v4i *>(Yo + (size_t)grow * N + gcol));
        }
    }
}
// F8: the operands are E4M3 bytes (one K value per byte) instead of packed E2M1 codes.
template <int YDT, bool ACCOUT, bool KFULL, bool F8>
__global__ __launch_bounds__(NT, 2) void k_fp4_gemm(TileArgs p) {
    // two-byte outputs run on the transposed product (swapped MFMA operands, see epi_pair_t)
    constexpr bool TR = YDT != DT_F32 && !F8;
    __shared__ __attribute__((aligned(16))) uint8_t sb0[STB];
    __shared__ __attribute__((aligned(16))) uint8_t sb1[STB];
    __shared__ __attribute__((aligned(16))) uint8_t sb2[STB];
    __shared__ __attribute__((aligned(16))) Book bk;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
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

    const int KB = F8 ? K : K / 2;  // operand bytes per row
    const int kstages = (KB + BKB - 1) / BKB;
    const __amdgpu_buffer_rsrc_t rsA =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(p.Aq), 0, M * KB, BUF_FLAGS);
    const __amdgpu_buffer_rsrc_t rsB =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(p.Wq), 0, N * KB, BUF_FLAGS);
    const int lane_chunk16 = ((lane & 3) ^ ((lane >> 4) & 3)) * 16;
    int offA[4], offB[2];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = (wave * 4 + j) * 16 + (lane >> 2);
        offA[j] = (m0 + r < M) ? (m0 + r) * KB + lane_chunk16 : OOB;
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int r = (wave * 2 + j) * 16 + (lane >> 2);
        offB[j] = (n0 + r < N) ? (n0 + r) * KB + lane_chunk16 : OOB;
    }

    v16f acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // prologue: stage 0, the tile's scales, then stage 1.  The scale loads are older than
    // stage 1's loads, so the wait for stage 0 covers them too.
    stage_dma<KFULL>(rsA, rsB, sb0, wave, offA, offB, 0, KB, lane_chunk16);
    __builtin_amdgcn_sched_barrier(0);
    const float bA = (m0 + tid < M) ? p.sA[m0 + tid] : 0.0f;
    const float bW = (tid < BN && n0 + tid < N) ? p.sW[n0 + tid] : 0.0f;
    __builtin_amdgcn_sched_barrier(0);
    stage_dma<KFULL>(rsA, rsB, sb1, wave, offA, offB, 1, KB, lane_chunk16);
    __builtin_amdgcn_sched_barrier(0);
    WAIT_VMCNT(6);
    bk.sA[tid] = bA;
    if (tid < BN) bk.sW[tid] = bW;
    __builtin_amdgcn_s_barrier();

    // Stage kt lives in buffer kt%3; its loads are issued at the start of step kt-2, into
    // the buffer step kt-3 read.  Step kt reads stage kt's K-step-0 fragments, issues stage
    // kt+2, reads the K-step-1 fragments under the first eight MFMAs, runs the second
    // eight, and waits for its own loads of stage kt+1 before the barrier that ends it.
    auto step = [&](int kt, const uint8_t *cur, uint8_t *ahead) {
        if constexpr (F8) {  // one K-step of 64 values per stage
            u32x4 a8[4][2], b8[2][2];
            __builtin_amdgcn_sched_barrier(0);
            frag_load8(cur, wm, wn, lane, a8, b8);
            __builtin_amdgcn_sched_barrier(0);
            stage_dma<KFULL>(rsA, rsB, ahead, wave, offA, offB, kt + 2, KB, lane_chunk16);
            __builtin_amdgcn_sched_barrier(0);
            mfma_block8(acc, a8, b8);
            __builtin_amdgcn_sched_barrier(0);
            WAIT_VMCNT(6);
            lds_barrier();
            return;
        }
        u32x4 a0[4], b0[2], a1[4], b1[2];
        __builtin_amdgcn_sched_barrier(0);
        frag_load(cur, wm, wn, lane, 0, a0, b0);
        __builtin_amdgcn_sched_barrier(0);
        stage_dma<KFULL>(rsA, rsB, ahead, wave, offA, offB, kt + 2, KB, lane_chunk16);
        __builtin_amdgcn_sched_barrier(0);
        frag_load(cur, wm, wn, lane, 1, a1, b1);
        mfma_block<2, TR>(acc, a0, b0);
#pragma unroll
        for (int q = 0; q < 6; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_barrier(0);
        mfma_block<2, TR>(acc, a1, b1);
        __builtin_amdgcn_sched_barrier(0);
        WAIT_VMCNT(6);
        lds_barrier();
    };
    // whole groups of three stages, then the last one or two (a loop exit between the
    // steps of a group costs a full drain of the loads in flight at every iteration)
    int kt = 0;
    for (; kt + 3 <= kstages; kt += 3) {
        step(kt, sb0, sb2);
        step(kt + 1, sb1, sb0);
        step(kt + 2, sb2, sb1);
    }
    if (kt < kstages) {
        step(kt, sb0, sb2);
        if (kt + 1 < kstages) step(kt + 1, sb1, sb0);
    }
    WAIT_VMCNT(0);  // look-ahead loads past the end (zeros) land before the workgroup ends

    // ---- epilogue: Y = fl(fl(acc * sA) * sW).  Each wave turns its 32 x 32 result tiles
    // into row-major order through a private 4 KiB patch of LDS, so every store writes 16
    // contiguous bytes per lane.  The patch lies in the buffer of the last real stage: all
    // waves finished reading it before the last barrier, and no look-ahead load targets it.
    // MFMA 32x32 output layout: lane l, register r -> row 8*(r/4) + 4*(l/32) + r%4, col l%32.
    const int last = (kstages + 2) % 3;
    uint8_t *stg = last == 0 ? sb0 : (last == 1 ? sb1 : sb2);
    float *E = reinterpret_cast<float *>(stg + wave * 4352);  // 4 x 4352 bytes fit the 24 KiB stage buffer
    float sw[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) sw[j] = bk.sW[wn * 64 + j * 32 + (lane & 31)];
    const bool full = (m0 + BM <= M) && (n0 + BN <= N);
    const uint32_t qoff = (uint32_t)(lane >> 3) * (uint32_t)N + (uint32_t)((lane & 7) * 8);  // epi_pair_t read-back
    bool qesc = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float sa[16];
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const float4 v = *reinterpret_cast<const float4 *>(&bk.sA[wm * 128 + i * 32 + 8 * r4 + 4 * (lane >> 5)]);
            sa[4 * r4] = v.x;
            sa[4 * r4 + 1] = v.y;
            sa[4 * r4 + 2] = v.z;
            sa[4 * r4 + 3] = v.w;
        }
        const int row0 = m0 + wm * 128 + i * 32;  // first row of this 32-row tile
        if constexpr (TR) {  // the transposed product: both tiles of the row band as one pair
            if constexpr (ACCOUT) {  // row lane%32, columns 8(r/4) + 4(lane/32) + r%4
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int grow = row0 + (lane & 31);
                        const int gcol = n0 + wn * 64 + j * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                        if (full || (grow < M && gcol < N)) p.acc_out[(size_t)grow * N + gcol] = acc[i][j][r];
                    }
            }
            epi_pair_t<YDT>(acc[i][0], acc[i][1], qesc, bk.sA[wm * 128 + i * 32 + (lane & 31)], &bk.sW[wn * 64],
                            reinterpret_cast<uint16_t *>(E), lane, row0, n0 + wn * 64, M, N, full,
                            static_cast<uint16_t *>(p.Y), qoff);
            continue;
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int col0 = n0 + wn * 64 + j * 32;
            if constexpr (ACCOUT) {  // raw accumulator, a check aid: plain stores
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int grow = row0 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                    if (full || (grow < M && col0 + (lane & 31) < N))
                        p.acc_out[(size_t)grow * N + col0 + (lane & 31)] = acc[i][j][r];
                }
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int lr = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                E[lr * 32 + (lane & 31)] = (acc[i][j][r] * sa[r]) * sw[j];
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            // streaming stores: Y is not read back soon enough to be worth caching, and
            // leaving it out of the caches keeps the operand strips there
            // all of the patch is read back before the first store is issued
            f4 e[4];
            if constexpr (YDT == DT_BF16) {
                // chunk c = 64k + lane: row c/4, columns 8(c%4) .. +7 (floats 8c .. 8c+7)
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                    e[2 * k] = *reinterpret_cast<const f4 *>(&E[8 * (k * 64 + lane)]);
                    e[2 * k + 1] = *reinterpret_cast<const f4 *>(&E[8 * (k * 64 + lane) + 4]);
                }
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                    const int c = k * 64 + lane, lr = c >> 2, cc = (c & 3) * 8;
                    const f4 e0 = e[2 * k], e1 = e[2 * k + 1];
                    const int grow = row0 + lr, gcol = col0 + cc;
                    if (full || (grow < M && gcol < N)) {
                        v4i o;
                        o[0] = (int)(f32_to_bf16_bits(e0[0]) | (f32_to_bf16_bits(e0[1]) << 16));
                        o[1] = (int)(f32_to_bf16_bits(e0[2]) | (f32_to_bf16_bits(e0[3]) << 16));
                        o[2] = (int)(f32_to_bf16_bits(e1[0]) | (f32_to_bf16_bits(e1[1]) << 16));
                        o[3] = (int)(f32_to_bf16_bits(e1[2]) | (f32_to_bf16_bits(e1[3]) << 16));
                        __builtin_nontemporal_store(
                            o, reinterpret_cast<v4i *>(reinterpret_cast<uint16_t *>(p.Y) + (size_t)grow * N + gcol));
                    }
                }
            } else {
                // chunk c = 64k + lane: row c/8, columns 4(c%8) .. +3 (floats 4c .. 4c+3)
#pragma unroll
                for (int k = 0; k < 4; ++k) e[k] = *reinterpret_cast<const f4 *>(&E[4 * (k * 64 + lane)]);
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int c = k * 64 + lane, lr = c >> 3, cc = (c & 7) * 4;
                    const int grow = row0 + lr, gcol = col0 + cc;
                    if (full || (grow < M && gcol < N))
                        __builtin_nontemporal_store(
                            e[k], reinterpret_cast<f4 *>(reinterpret_cast<float *>(p.Y) + (size_t)grow * N + gcol));
                }
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
    }
    if constexpr (YDT == DT_Q16) {  // the wave's 128 x 64 block is one cell of the map
        const int cm = m0 / 128 + wm, cn = n0 / 64 + wn;
        if (lane == 0 && cm < p.cellsM && cn < p.cellsN) p.emap[(size_t)cm * p.mapN + cn] = qesc ? 1 : 0;
    }
}

// ----------------------------------------------------------------------------- wide tiles
// For large products: a 256 x 256 tile per workgroup, 4 waves of 128 x 128 (4 x 4 MFMA tiles:
// 8 fragment reads per 16 MFMAs instead of 6 per 8, and a third less operand traffic per
// output than 256 x 128), one workgroup per CU (the accumulators fill the 256 AGPRs), four
// LDS stage buffers (three stages of look-ahead) and a barrier between the two K-steps of a
// stage.  A stage's direct-to-LDS loads are split: A's half after the barrier of the step that
// frees the buffer, W's half in the first K-step of the step after it, so each K-step issues four
// (about 1 % faster than all eight in the second K-step).  Persistent: the workgroup walks its
// XCD's tiles, and the DMA of the next tile's first four stages is issued during the current
// tile's last four steps (the last W half at the next tile's first step), so they land while the
// epilogue runs.  Needs K % 512 == 0 (whole groups of four 128-code stages).
constexpr int WBN = 256;
constexpr int WSTB = (BM + WBN) * BKB;  // 32 KiB per stage buffer

struct WBook {
    float sA[BM];
    float sW[WBN];
};

// 16 MFMAs with 8 fragment reads spread among them
#define INTERLEAVE16()                                         \
    do {                                                       \
        _Pragma("unroll") for (int q = 0; q < 8; ++q) {        \
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0); \
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0); \
        }                                                      \
        __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);     \
    } while (0)

// The A half and the B half of stage_dma<true, 4>, issued apart.
__device__ __forceinline__ void stage_dma_ha(__amdgpu_buffer_rsrc_t rsA, uint8_t *buf, int wave, const int (&offA)[4],
                                             int kt, int KB) {
    const int soff = min(kt, KB / BKB - 1) * BKB;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsA, LDS_PTR(buf + (wave * 4 + j) * 1024), 16, offA[j], soff, 0, 0);
}
__device__ __forceinline__ void stage_dma_hb(__amdgpu_buffer_rsrc_t rsB, uint8_t *buf, int wave, const int (&offB)[4],
                                             int kt, int KB) {
    const int soff = min(kt, KB / BKB - 1) * BKB;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsB, LDS_PTR(buf + OPA + (wave * 4 + j) * 1024), 16, offB[j], soff, 0,
                                                 0);
}

template <int YDT, bool ACCOUT>
__global__ __launch_bounds__(NT, 1) void k_fp4_gemm_wide(TileArgs p) {
    __shared__ __attribute__((aligned(16))) uint8_t sb0[WSTB];
    __shared__ __attribute__((aligned(16))) uint8_t sb1[WSTB];
    __shared__ __attribute__((aligned(16))) uint8_t sb2[WSTB];
    __shared__ __attribute__((aligned(16))) uint8_t sb3[WSTB];
    __shared__ __attribute__((aligned(16))) float patch[NW][1088];  // 32 x 68 int16 for the transposed pair
    __shared__ __attribute__((aligned(16))) WBook bk[2];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int M = p.M, N = p.N, K = p.K;

    const int tiles = p.tilesM * p.tilesN;
    const int per_xcd_wg = gridDim.x / 8;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int tpx = (tiles + 7) / 8;
    const int hi = min((xcd + 1) * tpx, tiles);
    int logical = xcd * tpx + slot;
    if (logical >= hi) return;

    auto origin = [&](int lg, int &m0, int &n0) {
        const int group = lg / (p.raster_group * p.tilesN);
        const int first_m = group * p.raster_group;
        const int gm = min(p.raster_group, p.tilesM - first_m);
        const int in_group = lg - group * p.raster_group * p.tilesN;
        m0 = (first_m + in_group % gm) * BM;
        n0 = (in_group / gm) * WBN;
    };
    const int KB = K / 2;
    const int kstages = KB / BKB;  // a multiple of 4
    const __amdgpu_buffer_rsrc_t rsA =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(p.Aq), 0, M * KB, BUF_FLAGS);
    const __amdgpu_buffer_rsrc_t rsB =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(p.Wq), 0, N * KB, BUF_FLAGS);
    const int lane_chunk16 = ((lane & 3) ^ ((lane >> 4) & 3)) * 16;
    auto offsets = [&](int m0, int n0, int (&oa)[4], int (&ob)[4]) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = (wave * 4 + j) * 16 + (lane >> 2);
            oa[j] = (m0 + r < M) ? (m0 + r) * KB + lane_chunk16 : OOB;
            ob[j] = (n0 + r < N) ? (n0 + r) * KB + lane_chunk16 : OOB;
        }
    };
    int m0, n0, offA[4], offB[4];
    origin(logical, m0, n0);
    offsets(m0, n0, offA, offB);

    v16f acc[4][4];
    u32x4 a0[4], b0[4], a1[4], b1[4];

    // prologue of the first tile
    stage_dma<true, 4>(rsA, rsB, sb0, wave, offA, offB, 0, KB, lane_chunk16);
    __builtin_amdgcn_sched_barrier(0);
    {
        const float bA = (m0 + tid < M) ? p.sA[m0 + tid] : 0.0f;
        const float bW = (n0 + tid < N) ? p.sW[n0 + tid] : 0.0f;
        __builtin_amdgcn_sched_barrier(0);
        stage_dma<true, 4>(rsA, rsB, sb1, wave, offA, offB, 1, KB, lane_chunk16);
        stage_dma<true, 4>(rsA, rsB, sb2, wave, offA, offB, 2, KB, lane_chunk16);
        stage_dma_ha(rsA, sb3, wave, offA, 3, KB);
        __builtin_amdgcn_sched_barrier(0);
        WAIT_VMCNT(20);
        bk[0].sA[tid] = bA;
        bk[0].sW[tid] = bW;
    }
    lds_barrier();
    frag_load(sb0, wm, wn, lane, 0, a0, b0);
    // W's half of each stage's direct-to-LDS loads is issued in the next step's first K-step, so
    // the loads are spread over both K-steps (pending: buffer, offsets and stage of that half)
    uint8_t *pbuf = sb3;
    int pob[4], pst = 3;
#pragma unroll
    for (int j = 0; j < 4; ++j) pob[j] = offB[j];

    auto step = [&](uint8_t *cur, const uint8_t *nxt, const int (&oa)[4], const int (&ob)[4], int dma_stage,
                    bool load_next) {
        __builtin_amdgcn_sched_barrier(0);
        frag_load(cur, wm, wn, lane, 1, a1, b1);
        stage_dma_hb(rsB, pbuf, wave, pob, pst, KB);
        mfma_block<4, YDT != DT_F32>(acc, a0, b0);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // buffer load to LDS
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        __builtin_amdgcn_sched_barrier(0);
        WAIT_VMCNT(16);
        lds_barrier();
        // A's half of the refill and the next fragments' eight reads go between the K-step-1
        // MFMAs; W's half is left for the next step
        stage_dma_ha(rsA, cur, wave, oa, dma_stage, KB);
        pbuf = cur;
        pst = dma_stage;
#pragma unroll
        for (int j = 0; j < 4; ++j) pob[j] = ob[j];
        if (load_next) {
            frag_load(nxt, wm, wn, lane, 0, a0, b0);
            mfma_block<4, YDT != DT_F32>(acc, a1, b1);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // buffer load to LDS
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        } else {
            mfma_block<4, YDT != DT_F32>(acc, a1, b1);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    // DT_Q16 outputs: the last ND pairs of a tile are packed in registers and stored during the
    // next tile's first steps, under its MFMAs (the bf16 epilogue stores at once: deferring it spills)
    constexpr bool DEFER = YDT == DT_Q16;
    // pairs deferred (the tile's last ND; the others are stored at once).  The next tile's first
    // two steps flush exactly four (two each), so ND is 4 here; with the flushes spread to match,
    // 2, 4 and 6 measured within noise of each other on four layer shapes, and 8 spills.
    constexpr int ND = 4;
    static_assert(ND == 4, "the first two steps of a tile flush four deferred pairs");
    uint32_t pk[ND][16];
    bool pend = false;
    int pr0 = 0, pc0 = 0;
    bool pfull = false;
    uint32_t dloff = (uint32_t)(lane >> 3) * (uint32_t)N + (uint32_t)((lane & 7) * 8);
    auto flush_pair = [&](const uint32_t (&q)[16], int pp) {
        pair_store(q, reinterpret_cast<uint16_t *>(patch[wave]), lane, pr0 + ((pp + 8 - ND) >> 1) * 32, pc0 + (pp & 1) * 64, M, N,
                   pfull, static_cast<uint16_t *>(p.Y), dloff);
    };
    auto step_d = [&](uint8_t *cur, const uint8_t *nxt, const int (&oa)[4], const int (&ob)[4], int dma_stage,
                      const uint32_t (&qa)[16], int pa, const uint32_t (&qb)[16], int pb) {
        __builtin_amdgcn_sched_barrier(0);
        frag_load(cur, wm, wn, lane, 1, a1, b1);
        stage_dma_hb(rsB, pbuf, wave, pob, pst, KB);
        mfma_block<4, YDT != DT_F32>(acc, a0, b0);
        flush_pair(qa, pa);
        INTERLEAVE16();
        __builtin_amdgcn_sched_barrier(0);
        WAIT_VMCNT(16);
        lds_barrier();
        stage_dma_ha(rsA, cur, wave, oa, dma_stage, KB);
        pbuf = cur;
        pst = dma_stage;
#pragma unroll
        for (int j = 0; j < 4; ++j) pob[j] = ob[j];
        frag_load(nxt, wm, wn, lane, 0, a0, b0);
        mfma_block<4, YDT != DT_F32>(acc, a1, b1);
        flush_pair(qb, pb);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    for (int tt = 0;; ++tt) {
        const int nlog = logical + per_xcd_wg;
        const bool has_next = nlog < hi;
        int nm0 = m0, nn0 = n0, noffA[4], noffB[4];
        if (has_next) origin(nlog, nm0, nn0);
        offsets(nm0, nn0, noffA, noffB);
        // without a next tile the last four loads re-read this tile's last stage (in bounds,
        // never consumed)
        const int nbase = has_next ? 0 : kstages - 1;
        const int nstep = has_next ? 1 : 0;

#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
        int kt = 0;
        if constexpr (DEFER) {
            if (pend) {
                if (kstages >= 8) {  // the previous tile's stores under this tile's first four steps
                    step_d(sb0, sb1, offA, offB, 4, pk[0], 0, pk[1], 1);
                    step_d(sb1, sb2, offA, offB, 5, pk[2], 2, pk[3], 3);
                    step(sb2, sb3, offA, offB, 6, true);
                    step(sb3, sb0, offA, offB, 7, true);
                    kt = 4;
                } else {
#pragma unroll
                    for (int pp = 0; pp < ND; ++pp) flush_pair(pk[pp], pp);
                }
                pend = false;
            }
        }
        for (; kt + 4 < kstages; kt += 4) {
            step(sb0, sb1, offA, offB, kt + 4, true);
            step(sb1, sb2, offA, offB, kt + 5, true);
            step(sb2, sb3, offA, offB, kt + 6, true);
            step(sb3, sb0, offA, offB, kt + 7, true);
        }
        step(sb0, sb1, noffA, noffB, nbase, true);
        step(sb1, sb2, noffA, noffB, nbase + nstep, true);
        step(sb2, sb3, noffA, noffB, nbase + 2 * nstep, true);
        step(sb3, sb0, noffA, noffB, nbase + 3 * nstep, false);

        // pin the accumulators here: keeps the last step's MFMAs (and their fragments) out of
        // the epilogue's blocks
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) asm volatile("" : "+a"(acc[i][j]));
        // next tile's scales, fetched under this epilogue
        const float nbA = (has_next && nm0 + tid < M) ? p.sA[nm0 + tid] : 0.0f;
        const float nbW = (has_next && nn0 + tid < N) ? p.sW[nn0 + tid] : 0.0f;

        const WBook &b = bk[tt & 1];
        float *E = patch[wave];
        float sw[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) sw[j] = b.sW[wn * 128 + j * 32 + (lane & 31)];
        const bool full = (m0 + BM <= M) && (n0 + WBN <= N);
        // Row-major read-back of a 32 x 32 patch, the same lanes for every tile: chunk
        // c = 64k + lane holds row c/8, columns 4(c%8).. (fp32) or row c/4, columns 8(c%4).. (bf16).
        constexpr int NK = YDT == DT_F32 ? 4 : 1;
        int lrow[NK], lcol[NK];
        uint32_t loff[NK];
#pragma unroll
        for (int k = 0; k < NK; ++k) {
            const int c = k * 64 + lane;
            lrow[k] = c >> 3;
            lcol[k] = (c & 7) * (YDT == DT_F32 ? 4 : 8);
            loff[k] = (uint32_t)lrow[k] * (uint32_t)N + (uint32_t)lcol[k];
        }
        bool qesc = false;  // DT_Q16: some |acc| of the wave's block is past the int16 range
        float qmx = 0.0f;   // DT_Q16: the lane's largest |acc|
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float sa[16];
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const float4 v = *reinterpret_cast<const float4 *>(&b.sA[wm * 128 + i * 32 + 8 * r4 + 4 * (lane >> 5)]);
                sa[4 * r4] = v.x;
                sa[4 * r4 + 1] = v.y;
                sa[4 * r4 + 2] = v.z;
                sa[4 * r4 + 3] = v.w;
            }
            const int row0 = m0 + wm * 128 + i * 32;
            if constexpr (YDT != DT_F32) {  // the transposed product: pairs of tiles
                const float sar = b.sA[wm * 128 + i * 32 + (lane & 31)];
#pragma unroll
                for (int jp = 0; jp < 2; ++jp) {
                    if constexpr (!DEFER) __builtin_amdgcn_sched_barrier(0);
                    if constexpr (ACCOUT) {  // the swapped layout: row lane%32, columns 8(r/4) + 4(lane/32) + r%4
#pragma unroll
                        for (int j = 2 * jp; j < 2 * jp + 2; ++j)
#pragma unroll
                            for (int r = 0; r < 16; ++r) {
                                const int grow = row0 + (lane & 31);
                                const int gcol = n0 + wn * 128 + j * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                                if (full || (grow < M && gcol < N)) p.acc_out[(size_t)grow * N + gcol] = acc[i][j][r];
                            }
                    }
                    if constexpr (DEFER) {  // packed now; the tile's last ND pairs are stored later
                        if (2 * i + jp >= 8 - ND) {
                            pair_pack<YDT>(acc[i][2 * jp], acc[i][2 * jp + 1], qmx, sar, &b.sW[wn * 128 + 64 * jp], lane,
                                           pk[2 * i + jp - (8 - ND)]);
                        } else {
                            uint32_t q[16];
                            pair_pack<YDT>(acc[i][2 * jp], acc[i][2 * jp + 1], qmx, sar, &b.sW[wn * 128 + 64 * jp], lane, q);
                            pair_store(q, reinterpret_cast<uint16_t *>(E), lane, row0, n0 + wn * 128 + 64 * jp, M, N, full,
                                       static_cast<uint16_t *>(p.Y), loff[0]);
                        }
                    } else {
                        epi_pair_t<YDT>(acc[i][2 * jp], acc[i][2 * jp + 1], qesc, sar, &b.sW[wn * 128 + 64 * jp],
                                        reinterpret_cast<uint16_t *>(E), lane, row0, n0 + wn * 128 + 64 * jp, M, N, full,
                                        static_cast<uint16_t *>(p.Y), loff[0]);
                    }
                }
                continue;
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                __builtin_amdgcn_sched_barrier(0);
                const int col0 = n0 + wn * 128 + j * 32;
                if constexpr (ACCOUT) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int grow = row0 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                        if (full || (grow < M && col0 + (lane & 31) < N))
                            p.acc_out[(size_t)grow * N + col0 + (lane & 31)] = acc[i][j][r];
                    }
                }
                // The patch is private to the wave and a wave's LDS accesses execute in
                // order, so the read-back sees these writes and the next tile's writes
                // cannot overtake it: no barrier.
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int lr = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                    E[lr * 32 + (lane & 31)] = (acc[i][j][r] * sa[r]) * sw[j];
                }
                f4 e[4];
                if constexpr (YDT == DT_BF16) {
#pragma unroll
                    for (int k = 0; k < 2; ++k) {
                        e[2 * k] = *reinterpret_cast<const f4 *>(&E[8 * (k * 64 + lane)]);
                        e[2 * k + 1] = *reinterpret_cast<const f4 *>(&E[8 * (k * 64 + lane) + 4]);
                    }
                    v4i o[2];
#pragma unroll
                    for (int k = 0; k < 2; ++k) {
                        const f4 e0 = e[2 * k], e1 = e[2 * k + 1];
                        o[k][0] = (int)(f32_to_bf16_bits(e0[0]) | (f32_to_bf16_bits(e0[1]) << 16));
                        o[k][1] = (int)(f32_to_bf16_bits(e0[2]) | (f32_to_bf16_bits(e0[3]) << 16));
                        o[k][2] = (int)(f32_to_bf16_bits(e1[0]) | (f32_to_bf16_bits(e1[1]) << 16));
                        o[k][3] = (int)(f32_to_bf16_bits(e1[2]) | (f32_to_bf16_bits(e1[3]) << 16));
                    }
                    uint16_t *Yb = reinterpret_cast<uint16_t *>(p.Y);
                    if (full) {
                        uint16_t *base = Yb + (size_t)row0 * N + col0;
#pragma unroll
                        for (int k = 0; k < 2; ++k) __builtin_nontemporal_store(o[k], reinterpret_cast<v4i *>(base + loff[k]));
                    } else {
#pragma unroll
                        for (int k = 0; k < 2; ++k) {
                            const int grow = row0 + lrow[k], gcol = col0 + lcol[k];
                            if (grow < M && gcol < N)
                                __builtin_nontemporal_store(o[k], reinterpret_cast<v4i *>(Yb + (size_t)grow * N + gcol));
                        }
                    }
                } else {
#pragma unroll
                    for (int k = 0; k < 4; ++k) e[k] = *reinterpret_cast<const f4 *>(&E[4 * (k * 64 + lane)]);
                    float *Yf = reinterpret_cast<float *>(p.Y);
                    if (full) {
                        float *base = Yf + (size_t)row0 * N + col0;
#pragma unroll
                        for (int k = 0; k < 4; ++k) __builtin_nontemporal_store(e[k], reinterpret_cast<f4 *>(base + loff[k]));
                    } else {
#pragma unroll
                        for (int k = 0; k < 4; ++k) {
                            const int grow = row0 + lrow[k], gcol = col0 + lcol[k];
                            if (grow < M && gcol < N)
                                __builtin_nontemporal_store(e[k], reinterpret_cast<f4 *>(Yf + (size_t)grow * N + gcol));
                        }
                    }
                }
            }
        }
        if constexpr (YDT == DT_Q16) {
            qesc = __builtin_amdgcn_ballot_w64(qmx > Q16_MAX_ACC) != 0;
            // the wave's 128 x 128 block is two cells of the map
            const int cm = m0 / 128 + wm, cn = n0 / 64 + 2 * wn;
            if (lane < 2 && cm < p.cellsM && cn + lane < p.cellsN)
                p.emap[(size_t)cm * p.mapN + cn + lane] = qesc ? 1 : 0;
        }
        if constexpr (DEFER) {
            pr0 = m0 + wm * 128;
            pc0 = n0 + wn * 128;
            pfull = full;
            if (has_next) {
                pend = true;
            } else {
#pragma unroll
                for (int pp = 0; pp < ND; ++pp) flush_pair(pk[pp], pp);
            }
        }
        bk[(tt + 1) & 1].sA[tid] = nbA;
        bk[(tt + 1) & 1].sW[tid] = nbW;
        if (!has_next) break;
        // the next tile's stage 0 landed before the last step's barrier
        frag_load(sb0, wm, wn, lane, 0, a0, b0);
        logical = nlog;
        m0 = nm0;
        n0 = nn0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            offA[j] = noffA[j];
            offB[j] = noffB[j];
        }
    }
    WAIT_VMCNT(0);
}

// Tile-rows per column sweep within an XCD (measured on five layer shapes: 2, 4 and 8 within
// 3 % of each other, 4 best on most; 16 and more lose L2 reuse).  A compile-time tuning aid.
#ifndef FP4_GEMM_RASTER_GROUP
#define FP4_GEMM_RASTER_GROUP 4
#endif
static int raster_group_for(int tilesM) {
    const int g = FP4_GEMM_RASTER_GROUP;
    return g < tilesM ? g : tilesM;
}

// CUs of the current device (the persistent grid's size), looked up once per device.
static int num_cus() {
    static int cache[64];
    int d = 0;
    if (hipGetDevice(&d) != hipSuccess || d < 0 || d >= 64) return 0;
    int n = __atomic_load_n(&cache[d], __ATOMIC_RELAXED);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, d) != hipSuccess) return 0;
        __atomic_store_n(&cache[d], n, __ATOMIC_RELAXED);
    }
    return n;
}

int gemm_kernel_choice(int64_t M, int64_t N, int64_t K, bool f8, int cus) {
    // wide persistent tiles when K is whole groups of four stages and there are at least two
    // such tiles per CU (with fewer, the per-tile prologue and epilogue of the large tiles are
    // left exposed)
    const int64_t wtiles = ((M + BM - 1) / BM) * ((N + WBN - 1) / WBN);
    if (!f8 && K % 512 == 0 && cus >= 8 && wtiles >= 2 * (int64_t)cus) return GEMM_WIDE;
    return GEMM_TILED;
}

// One launch of the product.
static hipError_t launch_gemm_one(const TileArgs &p0, int y_dt, bool acc, bool f8, hipStream_t s) {
    TileArgs p = p0;
    const int64_t M = p.M, N = p.N, K = p.K;
    const int cus = num_cus();
    if (gemm_kernel_choice(M, N, K, f8, cus) == GEMM_WIDE) {
        p.tilesN = (int)((N + WBN - 1) / WBN);
        const int blocks = cus / 8 * 8;
#define W2(YD, AO) hipLaunchKernelGGL((k_fp4_gemm_wide<YD, AO>), dim3(blocks), dim3(NT), 0, s, p)
        if (y_dt == DT_Q16) {
            if (acc) W2(DT_Q16, true);
            else W2(DT_Q16, false);
        } else if (y_dt == DT_BF16) {
            if (acc) W2(DT_BF16, true);
            else W2(DT_BF16, false);
        } else {
            if (acc) W2(DT_F32, true);
            else W2(DT_F32, false);
        }
#undef W2
        return hipGetLastError();
    }
    const int64_t tiles = (int64_t)p.tilesM * p.tilesN;
    const int blocks = (int)((tiles + 7) / 8 * 8);
    const bool kfull = f8 ? (K % 64 == 0) : (K % 128 == 0);  // every stage whole
#define G3(YD, AO, KF, F) hipLaunchKernelGGL((k_fp4_gemm<YD, AO, KF, F>), dim3(blocks), dim3(NT), 0, s, p)
#define G2(YD, AO, F)                        \
    do {                                     \
        if (kfull) G3(YD, AO, true, F);      \
        else G3(YD, AO, false, F);           \
    } while (0)
#define G1(YD, AO)                  \
    do {                            \
        if (f8) G2(YD, AO, true);   \
        else G2(YD, AO, false);     \
    } while (0)
    if (y_dt == DT_Q16) {  // never F8
        if (acc) G2(DT_Q16, true, false);
        else G2(DT_Q16, false, false);
    } else if (y_dt == DT_BF16) {
        if (acc) G1(DT_BF16, true);
        else G1(DT_BF16, false);
    } else {
        if (acc) G1(DT_F32, true);
        else G1(DT_F32, false);
    }
#undef G1
#undef G2
#undef G3
    return hipGetLastError();
}

hipError_t launch_gemm(const uint8_t *Aq, const float *sA, const uint8_t *Wq, const float *sW, int64_t M,
                       int64_t N, int64_t K, void *Y, int y_dt, float *acc_out, hipStream_t s, bool f8,
                       uint8_t *emap) {
    if (y_dt == DT_Q16 && (f8 || !emap)) return hipErrorInvalidValue;
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
    p.emap = emap;
    p.cellsM = (int)((M + ESC_ROWS - 1) / ESC_ROWS);
    p.cellsN = (int)((N + ESC_COLS - 1) / ESC_COLS);
    p.mapN = esc_map_stride(N);
    p.tilesM = (int)((M + BM - 1) / BM);
    p.tilesN = (int)((N + BN - 1) / BN);
    p.raster_group = raster_group_for(p.tilesM);
    return launch_gemm_one(p, y_dt, acc_out != nullptr, f8, s);
}

}  // namespace fp4
