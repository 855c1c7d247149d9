// gfx950 kernel for the output blocks that the GEMM's two-byte hand-over cannot hold.  The
// hand-over (gemm.hip, DT_Q16) stores the exact FP4 accumulator as the int16 4*acc, which
// covers |acc| <= 8191.75; the GEMM marks in a map every aligned 128 x 64 block of a wave block
// where some |acc| is larger.  Such blocks are rare: |acc| reaches 36*K only when a row of A and
// a column of W are both near their scale maximum with aligned signs.  This kernel finds the
// marked blocks and recomputes their exact accumulator on the FP4 matrix cores straight from
// the codes, then writes either
//   * the standalone two-byte output's escapes: fl(fl(acc*sA)*sW) in fp32 into an escape
//     buffer and -32768 into the int16 elements, or
//   * the final Y = Y_main + dA . W of the forward (QbitAI report on "Optimizing Large
//     Language Model Training Using FP4 Quantization", outlier paragraph: the clamped-away
//     entries of A times the weights are added back), with the arithmetic of the compensation
//     pass: Y_main = fl(fl(acc*sA)*sW), then one fp32 fma per entry in ascending k, rounded
//     once to the output type.  The compensation pass skips the marked blocks, so every element
//     of Y is written by exactly one of the two kernels.
// Each workgroup checks 256 blocks of the map at a time and collects the marked ones in LDS;
// its four waves then take 32 rows of each such block, as two 32 x 32 MFMA tiles.
#include "fp4_common.h"
#include "fp4_launch.h"

namespace fp4 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

enum : int { ESC_Q16 = 0, ESC_COMP = 1 };

struct EscArgs {
    const uint8_t *Aq, *Wq;  // M x K/2 and N x K/2 E2M1 codes, two per byte, low nibble first
    const float *sA, *sW;
    int M, N, K;
    const uint8_t *emap;  // cellsM rows of mapN bytes, one per ESC_ROWS x ESC_COLS block (cellsN used)
    int cellsM, cellsN, mapN;
    int16_t *Yq;  // ESC_Q16: the two-byte output, and its fp32 escape buffer
    float *esc;
    const int32_t *row_ptr, *coo_col;  // ESC_COMP: dA (CSR offsets, columns, values), W, Y
    const float *coo_val;
    const void *W;
    void *Y;
};

// The exact accumulator of the 32 x 64 block at rows r0.., columns c0.. (two 32 x 32 tiles).
// Each MFMA consumes 64 codes of K: lane l supplies row l%32 of A (or of Wq) and the 32 codes
// 32(l/32) .. of the step, 16 bytes read straight from global memory.  Rows past M or N, and
// the second half of a last step that K (a multiple of 32) leaves half full, read as zeros.
// Result layout of tile j: lane l holds column c0 + 32j + l%32 and, in register r, row
// r0 + 8(r/4) + 4(l/32) + r%4.
__device__ __forceinline__ void block_acc(const EscArgs &a, int r0, int c0, int lane, v16f (&acc)[2]) {
    const int KB = a.K / 2;
    const int lr = lane & 31, h = lane >> 5;
    const bool aok = r0 + lr < a.M;
    const uint8_t *ap = a.Aq + (size_t)(aok ? r0 + lr : 0) * KB;
    bool bok[2];
    const uint8_t *bp[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int brow = c0 + 32 * j + lr;
        bok[j] = brow < a.N;
        bp[j] = a.Wq + (size_t)(bok[j] ? brow : 0) * KB;
    }
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;
    for (int kb = 0; kb < KB; kb += 32) {
        const int off = kb + 16 * h;  // KB is a multiple of 16: a chunk is wholly in or out
        const bool kin = off < KB;
        u32x4 av = u32x4{0, 0, 0, 0};
        if (aok && kin) av = *reinterpret_cast<const u32x4 *>(ap + off);
        const v8i A = v8i{(int)av.x, (int)av.y, (int)av.z, (int)av.w, 0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            u32x4 bv = u32x4{0, 0, 0, 0};
            if (bok[j] && kin) bv = *reinterpret_cast<const u32x4 *>(bp[j] + off);
            const v8i B = v8i{(int)bv.x, (int)bv.y, (int)bv.z, (int)bv.w, 0, 0, 0, 0};
            // FP4 (format code 4) on both sides, unit block scales (scale operands 0)
            acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B, acc[j], 4, 4, 0, 0, 0, 0);
        }
    }
}

template <int WDT>
__device__ __forceinline__ float w_elem(const void *W, size_t i) {
    if constexpr (WDT == DT_BF16) return bf16_to_f32(reinterpret_cast<const uint16_t *>(W)[i]);
    else return reinterpret_cast<const float *>(W)[i];
}

// The block's outputs from its accumulator (layout of block_acc).
template <int MODE, int YDT, int WDT>
__device__ __forceinline__ void block_write(const EscArgs &a, int r0, int c0, int lane, const v16f (&acc)[2]) {
    const int lr = lane & 31, h = lane >> 5;
    const int M = a.M, N = a.N;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int n = c0 + 32 * j + lr;
        if (n >= N) continue;
        const float sw = a.sW[n];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int m = r0 + 8 * (r >> 2) + 4 * h + (r & 3);
            if (m >= M) continue;
            const size_t o = (size_t)m * N + n;
            const float ymain = (acc[j][r] * a.sA[m]) * sw;
            if constexpr (MODE == ESC_Q16) {
                a.esc[o] = ymain;
                a.Yq[o] = (int16_t)Q16_ESC;
            } else {
                float y = ymain;
                const int32_t e1 = a.row_ptr[m + 1];
                for (int32_t e = a.row_ptr[m]; e < e1; ++e)
                    y = __builtin_fmaf(a.coo_val[e], w_elem<WDT>(a.W, (size_t)a.coo_col[e] * N + n), y);
                if constexpr (YDT == DT_BF16) reinterpret_cast<uint16_t *>(a.Y)[o] = (uint16_t)f32_to_bf16_bits(y);
                else reinterpret_cast<float *>(a.Y)[o] = y;
            }
        }
    }
}

template <int MODE, int YDT, int WDT>
__global__ __launch_bounds__(256) void k_q16_escapes(EscArgs a) {
    __shared__ int list[256];
    __shared__ int count;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int cells = a.cellsM * a.mapN;
    for (int base = blockIdx.x * 256; base < cells; base += gridDim.x * 256) {
        if (tid == 0) count = 0;
        __syncthreads();
        const int c = base + tid;
        // the row padding past cellsN is never written: not a block
        if (c < cells && c % a.mapN < a.cellsN && a.emap[c]) list[atomicAdd(&count, 1)] = c;  // LDS: <= 256
        __syncthreads();
        const int n = count;
        for (int i = 0; i < n; ++i) {
            const int cell = list[i];
            const int r0 = (cell / a.mapN) * ESC_ROWS + 32 * wave, c0 = (cell % a.mapN) * ESC_COLS;
            if (r0 < a.M) {  // wave-uniform
                v16f acc[2];
                block_acc(a, r0, c0, lane, acc);
                block_write<MODE, YDT, WDT>(a, r0, c0, lane, acc);
            }
        }
        __syncthreads();  // the list is refilled next round
    }
}

size_t esc_map_bytes(int64_t M, int64_t N) { return (size_t)((M + ESC_ROWS - 1) / ESC_ROWS) * esc_map_stride(N); }

static EscArgs esc_args(const uint8_t *Aq, const float *sA, const uint8_t *Wq, const float *sW, int64_t M, int64_t N,
                        int64_t K, const uint8_t *emap) {
    EscArgs a{};
    a.Aq = Aq;
    a.Wq = Wq;
    a.sA = sA;
    a.sW = sW;
    a.M = (int)M;
    a.N = (int)N;
    a.K = (int)K;
    a.emap = emap;
    a.cellsM = (int)((M + ESC_ROWS - 1) / ESC_ROWS);
    a.cellsN = (int)((N + ESC_COLS - 1) / ESC_COLS);
    a.mapN = esc_map_stride(N);
    return a;
}

// one round of 256 map bytes per workgroup covers the map with up to 4096 workgroups; larger
// maps take further rounds
static dim3 esc_grid(const EscArgs &a) {
    const int64_t rounds = ((int64_t)a.cellsM * a.mapN + 255) / 256;
    return dim3((unsigned)(rounds < 4096 ? rounds : 4096));
}

hipError_t launch_escapes_q16(const uint8_t *Aq, const float *sA, const uint8_t *Wq, const float *sW, int64_t M,
                              int64_t N, int64_t K, const uint8_t *emap, int16_t *Yq, float *esc, hipStream_t s) {
    EscArgs a = esc_args(Aq, sA, Wq, sW, M, N, K, emap);
    a.Yq = Yq;
    a.esc = esc;
    hipLaunchKernelGGL((k_q16_escapes<ESC_Q16, DT_F32, DT_F32>), esc_grid(a), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_escapes_comp(const uint8_t *Aq, const float *sA, const uint8_t *Wq, const float *sW, int64_t M,
                               int64_t N, int64_t K, const uint8_t *emap, const int32_t *row_ptr,
                               const int32_t *coo_col, const float *coo_val, const void *W, int w_dt, void *Y,
                               int y_dt, hipStream_t s) {
    EscArgs a = esc_args(Aq, sA, Wq, sW, M, N, K, emap);
    a.row_ptr = row_ptr;
    a.coo_col = coo_col;
    a.coo_val = coo_val;
    a.W = W;
    a.Y = Y;
    const dim3 g = esc_grid(a);
#define E(YD, WD) hipLaunchKernelGGL((k_q16_escapes<ESC_COMP, YD, WD>), g, dim3(256), 0, s, a)
    if (y_dt == DT_BF16) {
        if (w_dt == DT_BF16) E(DT_BF16, DT_BF16);
        else E(DT_BF16, DT_F32);
    } else {
        if (w_dt == DT_BF16) E(DT_F32, DT_BF16);
        else E(DT_F32, DT_F32);
    }
#undef E
    return hipGetLastError();
}

}  // namespace fp4
