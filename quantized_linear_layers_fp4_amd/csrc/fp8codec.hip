// gfx950 kernels of the FP8 (E4M3) gradient codec: the single-GPU quantize/dequantize half
// of the FP8 gradient communication that the QbitAI report and the paper abstract pair with
// FP4 training (gradients travel in FP8; the pages give no scaling rule).
//
// One per-tensor scale: amax over the tensor (keys merged with atomicMax), multiplier
// r = fl(448 / amax) and dequantization scale s = fl(amax / 448), both zero when
// amax < 2^-120; each value becomes E4M3(fl(x * r)), rounded to nearest with ties to the
// even mantissa, saturating at 448 and keeping the sign.  Dequantization is
// fl(value(code) * s).  Elements go eight at a time (one or two 16-byte loads, one 8-byte
// store); a tail of n % 8 elements is handled element by element.
#include "fp4_common.h"
#include "fp4_launch.h"

namespace fp4 {

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Element i of X as fp32 (bf16 widened exactly).
template <int DT>
__device__ __forceinline__ float elem(const void *X, int64_t i) {
    if constexpr (DT == DT_BF16) return bf16_to_f32(reinterpret_cast<const uint16_t *>(X)[i]);
    else return reinterpret_cast<const float *>(X)[i];
}

// Eight consecutive elements starting at 8*c as fp32.
template <int DT>
__device__ __forceinline__ void load8f(const void *X, int64_t c, float v[8]) {
    if constexpr (DT == DT_BF16) {
        const u32x4 q = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(X) + c);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = bf16_to_f32(q[i] & 0xFFFFu);
            v[2 * i + 1] = bf16_to_f32(q[i] >> 16);
        }
    } else {
        const u32x4 *p = reinterpret_cast<const u32x4 *>(X) + 2 * c;
        const u32x4 q0 = __builtin_nontemporal_load(p), q1 = __builtin_nontemporal_load(p + 1);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[i] = __uint_as_float(q0[i]);
            v[4 + i] = __uint_as_float(q1[i]);
        }
    }
}

// fp32 -> E4M3 byte: nearest, ties to the even mantissa, |y| > 448 saturates to 448.
// Branch-free: for |y| >= 2^-6 the code is the fp32 pattern rounded to 3 mantissa bits
// (adding 0x7FFFF plus the kept LSB rounds to nearest-even; a mantissa carry moves into the
// exponent field, which is the right code) with the exponent rebased from 127 to 7; below
// 2^-6 it is the multiple of 2^-9, rounded to nearest-even by rint.
__device__ __forceinline__ uint32_t e4m3_encode(float y) {
    const uint32_t b = __float_as_uint(y);
    const uint32_t a = b & 0x7FFFFFFFu;
    const uint32_t normal = ((a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20) - (120u << 3);
    const uint32_t sub = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
    const uint32_t code = a > 0x43E00000u ? 0x7Eu : (a >= 0x3C800000u ? normal : sub);
    return ((b >> 24) & 0x80u) | code;
}

// E4M3 byte -> its value in fp32 (exact).
__device__ __forceinline__ float e4m3_value(uint32_t c) {
    const uint32_t e = (c >> 3) & 15u, m = c & 7u;
    float v;
    if (e == 0u) v = (float)m * 0x1p-9f;
    else if (e == 15u && m == 7u) v = __uint_as_float(0x7FC00000u);
    else v = __uint_as_float(((e + 120u) << 23) | (m << 20));
    return (c & 0x80u) ? -v : v;
}

__device__ __forceinline__ void fp8_scales(uint32_t amax_key, float &r, float &s) {
    const float amax = __uint_as_float(amax_key);
    if (!(amax >= 0x1p-120f)) {
        r = 0.0f;
        s = 0.0f;
    } else {
        r = __fdiv_rn(448.0f, amax);
        s = __fdiv_rn(amax, 448.0f);
    }
}

constexpr int CU = 4;  // chunks of 8 elements per thread and round trip

template <int DT>
__global__ __launch_bounds__(256) void k_fp8_amax(const void *__restrict__ X, int64_t n, uint32_t *__restrict__ key) {
    const int64_t nc = n / 8, stride = (int64_t)gridDim.x * blockDim.x;
    uint32_t mx = 0;
    for (int64_t c0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c0 < nc; c0 += CU * stride) {
        float v[CU][8];
#pragma unroll
        for (int u = 0; u < CU; ++u)
            if (c0 + u * stride < nc) load8f<DT>(X, c0 + u * stride, v[u]);
#pragma unroll
        for (int u = 0; u < CU; ++u)
            if (c0 + u * stride < nc)
#pragma unroll
                for (int i = 0; i < 8; ++i) mx = max(mx, __float_as_uint(v[u][i]) & 0x7FFFFFFFu);
    }
    if (blockIdx.x == 0)
        for (int64_t i = nc * 8 + threadIdx.x; i < n; i += blockDim.x)
            mx = max(mx, __float_as_uint(elem<DT>(X, i)) & 0x7FFFFFFFu);
    // one atomic per workgroup: thousands of same-address atomics serialize in L2
    __shared__ uint32_t red[4];
    mx = wave_max_u32(mx);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
    __syncthreads();
    if (threadIdx.x == 0) {
        mx = max(max(red[0], red[1]), max(red[2], red[3]));
        if (mx) atomicMax(key, mx);
    }
}

template <int DT>
__global__ __launch_bounds__(256) void k_fp8_quant(const void *__restrict__ X, int64_t n,
                                                   const uint32_t *__restrict__ key, uint8_t *__restrict__ codes,
                                                   float *__restrict__ scale) {
    float r, s;
    fp8_scales(*key, r, s);
    if (blockIdx.x == 0 && threadIdx.x == 0) *scale = s;
    const int64_t nc = n / 8, stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t c0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c0 < nc; c0 += CU * stride) {
        float v[CU][8];
#pragma unroll
        for (int u = 0; u < CU; ++u)
            if (c0 + u * stride < nc) load8f<DT>(X, c0 + u * stride, v[u]);
#pragma unroll
        for (int u = 0; u < CU; ++u) {
            if (c0 + u * stride < nc) {
                u32x2 o = {0u, 0u};
#pragma unroll
                for (int i = 0; i < 8; ++i) o[i >> 2] |= e4m3_encode(v[u][i] * r) << (8 * (i & 3));
                __builtin_nontemporal_store(o, reinterpret_cast<u32x2 *>(codes) + c0 + u * stride);
            }
        }
    }
    if (blockIdx.x == 0)
        for (int64_t i = nc * 8 + threadIdx.x; i < n; i += blockDim.x) codes[i] = (uint8_t)e4m3_encode(elem<DT>(X, i) * r);
}

template <int YDT>
__global__ __launch_bounds__(256) void k_fp8_dequant(const uint8_t *__restrict__ codes, int64_t n,
                                                     const float *__restrict__ scale, void *__restrict__ Y) {
    const float s = *scale;
    const int64_t nc = n / 8, stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < nc; c += stride) {
        const u32x2 q = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(codes) + c);
        float v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = e4m3_value((q[i >> 2] >> (8 * (i & 3))) & 0xFFu) * s;
        if constexpr (YDT == DT_BF16) {
            u32x4 o;
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = f32_to_bf16_bits(v[2 * i]) | (f32_to_bf16_bits(v[2 * i + 1]) << 16);
            __builtin_nontemporal_store(o, reinterpret_cast<u32x4 *>(Y) + c);
        } else {
            u32x4 *p = reinterpret_cast<u32x4 *>(Y) + 2 * c;
            __builtin_nontemporal_store(u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                                              __float_as_uint(v[3])}, p);
            __builtin_nontemporal_store(u32x4{__float_as_uint(v[4]), __float_as_uint(v[5]), __float_as_uint(v[6]),
                                              __float_as_uint(v[7])}, p + 1);
        }
    }
    if (blockIdx.x == 0)
        for (int64_t i = nc * 8 + threadIdx.x; i < n; i += blockDim.x) {
            const float v = e4m3_value(codes[i]) * s;
            if constexpr (YDT == DT_BF16) reinterpret_cast<uint16_t *>(Y)[i] = (uint16_t)f32_to_bf16_bits(v);
            else reinterpret_cast<float *>(Y)[i] = v;
        }
}

static unsigned grid_for(int64_t n, int num_cus) {
    int64_t b = (n / 8 + 255) / 256;
    const int64_t cap = (int64_t)num_cus * 8;
    if (b > cap) b = cap;
    return (unsigned)(b < 1 ? 1 : b);
}

hipError_t launch_fp8_quantize(const void *X, int dt, int64_t n, uint32_t *key, uint8_t *codes, float *scale,
                               int num_cus, hipStream_t s) {
    hipError_t e = launch_zero(key, 1, nullptr, 0, s);
    if (e != hipSuccess) return e;
    const unsigned g = grid_for(n, num_cus);
    const unsigned ga = g < (unsigned)(2 * num_cus) ? g : (unsigned)(2 * num_cus);  // few same-address atomics
    if (dt == DT_BF16) {
        hipLaunchKernelGGL(k_fp8_amax<DT_BF16>, dim3(ga), dim3(256), 0, s, X, n, key);
        hipLaunchKernelGGL(k_fp8_quant<DT_BF16>, dim3(g), dim3(256), 0, s, X, n, key, codes, scale);
    } else {
        hipLaunchKernelGGL(k_fp8_amax<DT_F32>, dim3(ga), dim3(256), 0, s, X, n, key);
        hipLaunchKernelGGL(k_fp8_quant<DT_F32>, dim3(g), dim3(256), 0, s, X, n, key, codes, scale);
    }
    return hipGetLastError();
}

hipError_t launch_fp8_dequantize(const uint8_t *codes, int64_t n, const float *scale, void *Y, int y_dt, int num_cus,
                                 hipStream_t s) {
    const unsigned g = grid_for(n, num_cus);
    if (y_dt == DT_BF16) hipLaunchKernelGGL(k_fp8_dequant<DT_BF16>, dim3(g), dim3(256), 0, s, codes, n, scale, Y);
    else hipLaunchKernelGGL(k_fp8_dequant<DT_F32>, dim3(g), dim3(256), 0, s, codes, n, scale, Y);
    return hipGetLastError();
}

}  // namespace fp4
