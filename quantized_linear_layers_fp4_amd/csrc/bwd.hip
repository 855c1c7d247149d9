// gfx950 kernels of the straight-through backward of the FP4 product (backward paragraph of
// the QbitAI report on "Optimizing Large Language Model Training Using FP4 Quantization":
// the hard quantizer stays in the forward, and the backward takes its derivative from a
// substitute; here the identity).  The two products
//      dA = dY . deq(Wq)^T      (contraction over the output channels n)
//      dW = deq(Aq)^T . dY      (contraction over the tokens m)
// run on the same FP4 GEMM as the forward, so each operand needs its codes contiguous
// along the new contraction index and its scale on the other index:
//   - dY is multiplied by the scale that lies along the contraction (sW[n], resp. sA[m])
//     and quantized per row (for dA) or per column (for dW, in quant.hip);
//   - the forward's codes are transposed: Wq (N x K/2) -> WqT (K x N/2) and
//     Aq (M x K/2) -> AqT (K x M/2).
#include "fp4_common.h"
#include "fp4_launch.h"

namespace fp4 {

// ----------------------------------------------------------------------------- transpose
// R x C codes (R x C/2 bytes) -> C x R/2 bytes.  One workgroup per 64 (r) x 128 (c) tile:
// each thread loads 16 bytes (32 codes) of one input row, the tile goes through LDS, and
// each thread writes 16 bytes (32 values of r) of one output row.  R % 32 == 0 and
// C % 32 == 0, so every 16-byte piece is wholly inside or outside the matrix.
__global__ __launch_bounds__(256) void k_codes_transpose(const uint8_t *__restrict__ in, int64_t R, int64_t C,
                                                         uint8_t *__restrict__ out) {
    __shared__ uint32_t tile[64][17];  // 64 rows x 64 bytes, one word of padding per row
    const int tid = threadIdx.x;
    const int64_t c0 = (int64_t)blockIdx.x * 128, r0 = (int64_t)blockIdx.y * 64;
    {
        const int rr = tid >> 2, part = tid & 3;
        const int64_t r = r0 + rr, cb = c0 / 2 + part * 16;  // byte column of the input row
        uint4 q = make_uint4(0u, 0u, 0u, 0u);
        if (r < R && cb < C / 2) q = *reinterpret_cast<const uint4 *>(in + r * (C / 2) + cb);
        tile[rr][part * 4 + 0] = q.x;
        tile[rr][part * 4 + 1] = q.y;
        tile[rr][part * 4 + 2] = q.z;
        tile[rr][part * 4 + 3] = q.w;
    }
    __syncthreads();
    const int cl = tid >> 1, half = tid & 1;  // output row c0 + cl, input rows half*32 ..
    const int64_t c = c0 + cl, ob = r0 / 2 + half * 16;
    if (c >= C || ob >= R / 2) return;
    const int word = cl >> 3, shift = (cl & 7) * 4;  // code cl of a tile row: word cl/8, nibble cl%8
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t w = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int ra = half * 32 + (4 * i + j) * 2;
            const uint32_t lo = (tile[ra][word] >> shift) & 15u, hi = (tile[ra + 1][word] >> shift) & 15u;
            w |= (lo | (hi << 4)) << (8 * j);
        }
        o[i] = w;
    }
    *reinterpret_cast<uint4 *>(out + c * (R / 2) + ob) = make_uint4(o[0], o[1], o[2], o[3]);
}

// ----------------------------------------------------------------------------- rows of G
// Token-wise quantization of G = fl(X[row][j] * mult[j]): one workgroup of 256 threads per
// row holds G's row in registers (CPT chunks of 8 elements per thread, chunk i*256 + tid),
// reduces max |G| over the workgroup, then scales, rounds and packs from registers.
template <int DT>
__device__ __forceinline__ void load_raw8(const void *X, int64_t elem, uint4 (&raw)[2]) {
    if constexpr (DT == DT_BF16) {
        raw[0] = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(X) + elem);
    } else {
        const uint4 *p = reinterpret_cast<const uint4 *>(reinterpret_cast<const float *>(X) + elem);
        raw[0] = p[0];
        raw[1] = p[1];
    }
}

template <int DT>
__device__ __forceinline__ void scaled8(const uint4 (&raw)[2], const float *__restrict__ mult, int64_t j0,
                                        float g[8]) {
    const float4 m0 = *reinterpret_cast<const float4 *>(mult + j0);
    const float4 m1 = *reinterpret_cast<const float4 *>(mult + j0 + 4);
    const float m[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
    float v[8];
    if constexpr (DT == DT_BF16) {
        const uint32_t w[4] = {raw[0].x, raw[0].y, raw[0].z, raw[0].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
            v[2 * i + 1] = bf16_to_f32(w[i] >> 16);
        }
    } else {
        const uint32_t w[8] = {raw[0].x, raw[0].y, raw[0].z, raw[0].w, raw[1].x, raw[1].y, raw[1].z, raw[1].w};
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = __uint_as_float(w[i]);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) g[e] = v[e] * m[e];
}

template <int DT, int CPT>
__global__ __launch_bounds__(256) void k_scaled_rows(const void *__restrict__ X, int64_t C,
                                                     const float *__restrict__ mult, uint8_t *__restrict__ codes,
                                                     float *__restrict__ scales) {
    __shared__ uint32_t red[4];
    const int tid = threadIdx.x;
    const int64_t row = blockIdx.x;
    const int64_t nchunk = C / 8, base = row * C;
    uint4 raw[CPT][2];
#pragma unroll
    for (int i = 0; i < CPT; ++i)
        if (i * 256 + tid < nchunk) load_raw8<DT>(X, base + (int64_t)(i * 256 + tid) * 8, raw[i]);
    // G is kept in registers between the two phases (8 values per chunk)
    float g[CPT][8];
    uint32_t mx = 0;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        const int64_t c = i * 256 + tid;
        if (c < nchunk) {
            scaled8<DT>(raw[i], mult, c * 8, g[i]);
#pragma unroll
            for (int e = 0; e < 8; ++e) mx = max(mx, __float_as_uint(g[i][e]) & 0x7FFFFFFFu);
        }
    }
    mx = wave_max_u32(mx);
    if ((tid & 63) == 0) red[tid >> 6] = mx;
    __syncthreads();
    mx = max(max(red[0], red[1]), max(red[2], red[3]));
    float r, s;
    vector_scale(__uint_as_float(mx), r, s);
    if (tid == 0) scales[row] = s;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        const int64_t c = i * 256 + tid;
        if (c < nchunk) {
            float y[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] = g[i][e] * r;
            *reinterpret_cast<uint32_t *>(codes + row * (C / 2) + c * 4) = e2m1_pack8(y);
        }
    }
}

// Both per-row reads of a bf16 dY in one pass: the token-wise quantization of
// G = fl(dY[m][n] * sW[n]) as above, and for the channel-wise quantization of
// H = fl(sA[m] * dY[m][n]) the maximum over the workgroup's rows of |H| for each column,
// kept by the thread that owns the column (chunk i*1024 + tid) and written once per workgroup
// as a row of keys into part[blockIdx.x][N].  Workgroup g takes rows g, g + G, g + 2G, ...
// 1024 threads per row keep the per-thread state (the row's CPT chunks and their 8*CPT
// column maxima) small enough for two workgroups per CU.
template <int CPT>
__global__ __launch_bounds__(1024) void k_bwd_rows_fused(const void *__restrict__ X, int64_t M, int64_t C,
                                                         const float *__restrict__ mult,
                                                         const float *__restrict__ row_mult,
                                                         uint8_t *__restrict__ codes, float *__restrict__ scales,
                                                         uint32_t *__restrict__ part) {
    __shared__ uint32_t red[2][16];
    const int tid = threadIdx.x;
    const int64_t nchunk = C / 8;
    // the thread's columns are the same in every row: their multipliers stay in registers
    float m[CPT][8];
    uint32_t cmax[CPT][8];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        const int64_t c = i * 1024 + tid;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            m[i][e] = c < nchunk ? mult[c * 8 + e] : 0.0f;
            cmax[i][e] = 0u;
        }
    }
    int par = 0;
    // the next row's loads are issued before this row is processed
    uint4 raw[CPT][2], nxt[CPT][2];
    float rm_nxt = 0.0f;
    auto load_row = [&](int64_t row, uint4 (&dst)[CPT][2]) {
#pragma unroll
        for (int i = 0; i < CPT; ++i)
            if (i * 1024 + tid < nchunk) load_raw8<DT_BF16>(X, row * C + (int64_t)(i * 1024 + tid) * 8, dst[i]);
    };
    if (blockIdx.x < M) {
        load_row(blockIdx.x, nxt);
        rm_nxt = row_mult[blockIdx.x];
    }
    for (int64_t row = blockIdx.x; row < M; row += gridDim.x, par ^= 1) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            raw[i][0] = nxt[i][0];
            raw[i][1] = nxt[i][1];
        }
        const float rm = rm_nxt;
        if (row + gridDim.x < M) {
            load_row(row + gridDim.x, nxt);
            rm_nxt = row_mult[row + gridDim.x];
        }
        float g[CPT][8];
        uint32_t mx = 0;
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int64_t c = i * 1024 + tid;
            if (c < nchunk) {
                const uint32_t w[4] = {raw[i][0].x, raw[i][0].y, raw[i][0].z, raw[i][0].w};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float v = bf16_to_f32((e & 1) ? (w[e >> 1] >> 16) : (w[e >> 1] & 0xFFFFu));
                    g[i][e] = v * m[i][e];
                    mx = max(mx, __float_as_uint(g[i][e]) & 0x7FFFFFFFu);
                    cmax[i][e] = max(cmax[i][e], __float_as_uint(rm * v) & 0x7FFFFFFFu);
                }
            }
        }
        // one slot set per row parity: a wave may start the next row's reduction while a
        // slower wave still reads this one's
        mx = wave_max_u32(mx);
        if ((tid & 63) == 0) red[par][tid >> 6] = mx;
        __syncthreads();
#pragma unroll
        for (int w = 0; w < 16; ++w) mx = max(mx, red[par][w]);
        float r, s;
        vector_scale(__uint_as_float(mx), r, s);
        if (tid == 0) scales[row] = s;
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int64_t c = i * 1024 + tid;
            if (c < nchunk) {
                float y[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) y[e] = g[i][e] * r;
                *reinterpret_cast<uint32_t *>(codes + row * (C / 2) + c * 4) = e2m1_pack8(y);
            }
        }
    }
    uint32_t *out = part + (int64_t)blockIdx.x * C;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        const int64_t c = i * 1024 + tid;
        if (c < nchunk) {
            uint4 *o = reinterpret_cast<uint4 *>(out + c * 8);
            o[0] = make_uint4(cmax[i][0], cmax[i][1], cmax[i][2], cmax[i][3]);
            o[1] = make_uint4(cmax[i][4], cmax[i][5], cmax[i][6], cmax[i][7]);
        }
    }
}

// keys[n] = max over the G partial rows of part[g][n]; eight rows' loads in flight per thread.
__global__ __launch_bounds__(256) void k_colmax_reduce(const uint32_t *__restrict__ part, int G, int64_t C,
                                                       uint32_t *__restrict__ keys) {
    const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (n >= C) return;
    uint32_t m[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    int g = 0;
    for (; g + 8 <= G; g += 8) {
#pragma unroll
        for (int u = 0; u < 8; ++u) m[u] = max(m[u], part[(int64_t)(g + u) * C + n]);
    }
    for (; g < G; ++g) m[0] = max(m[0], part[(int64_t)g * C + n]);
#pragma unroll
    for (int u = 1; u < 8; ++u) m[0] = max(m[0], m[u]);
    keys[n] = m[0];
}

__global__ void k_fill_f32(float *__restrict__ p, int64_t n, float v) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

// ----------------------------------------------------------------------------- launchers
hipError_t launch_codes_transpose(const uint8_t *in, int64_t R, int64_t C, uint8_t *out, hipStream_t s) {
    const dim3 grid((unsigned)((C + 127) / 128), (unsigned)((R + 63) / 64));
    hipLaunchKernelGGL(k_codes_transpose, grid, dim3(256), 0, s, in, R, C, out);
    return hipGetLastError();
}

hipError_t launch_scaled_quant_rows(const void *X, int dt, int64_t R, int64_t C, const float *mult, uint8_t *codes,
                                    float *scales, hipStream_t s) {
    const int64_t per = (C / 8 + 255) / 256;  // chunks per thread; C <= 65536 -> <= 32
    const dim3 grid((unsigned)R), block(256);
#define SR(CPT)                                                                                         \
    do {                                                                                                \
        if (dt == DT_BF16) hipLaunchKernelGGL((k_scaled_rows<DT_BF16, CPT>), grid, block, 0, s, X, C, mult, codes, scales); \
        else hipLaunchKernelGGL((k_scaled_rows<DT_F32, CPT>), grid, block, 0, s, X, C, mult, codes, scales);            \
    } while (0)
    if (per <= 4) SR(4);
    else if (per <= 8) SR(8);
    else if (per <= 12) SR(12);
    else if (per <= 16) SR(16);
    else if (per <= 24) SR(24);
    else SR(32);
#undef SR
    return hipGetLastError();
}

int fused_rows_cpt(int64_t C) { return (int)((C / 8 + 1023) / 1024); }

hipError_t launch_bwd_rows_fused(const void *X, int64_t M, int64_t C, const float *mult, const float *row_mult,
                                 uint8_t *codes, float *scales, uint32_t *part, int G, uint32_t *keys,
                                 hipStream_t s) {
    const int per = fused_rows_cpt(C);
#define FR(CPT) hipLaunchKernelGGL((k_bwd_rows_fused<CPT>), dim3((unsigned)G), dim3(1024), 0, s, X, M, C, mult, \
                                   row_mult, codes, scales, part)
    if (per <= 1) FR(1);
    else if (per <= 2) FR(2);
    else FR(3);
#undef FR
    hipLaunchKernelGGL(k_colmax_reduce, dim3((unsigned)((C + 255) / 256)), dim3(256), 0, s, part, G, C, keys);
    return hipGetLastError();
}

hipError_t launch_fill_f32(float *p, int64_t n, float v, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_fill_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n, v);
    return hipGetLastError();
}

}  // namespace fp4
