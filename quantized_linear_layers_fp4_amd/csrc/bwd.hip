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

hipError_t launch_fill_f32(float *p, int64_t n, float v, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_fill_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n, v);
    return hipGetLastError();
}

}  // namespace fp4
