// Matrix-core issue-rate probe (include/fp4probe.h): the FP4 MFMA rate and shader clock the
// present device sustains with nothing else running, the denominator the FP4 GEMM of the
// linear forward is measured against (QbitAI report on "Optimizing Large Language Model
// Training Using FP4 Quantization", GEMM-kernel paragraph).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp4probe.h"

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int CHAINS = 8;  // independent accumulators: enough to keep the matrix pipe full
// Scale operands 0: the unscaled form of the instruction (unit block scales), the form the FP4
// GEMM issues.

__global__ __launch_bounds__(256, 1) void k_probe_mfma_fp4(int iters, uint64_t *__restrict__ clocks,
                                                           float *__restrict__ sink) {
    const int lane = threadIdx.x & 63;
    const int wave = (int)(blockIdx.x * 4 + (threadIdx.x >> 6));
    // operands: FP4 codes derived from the lane id (values are irrelevant to the timing)
    const int seed = 0x11111111 * ((lane & 7) + 1);
    v8i a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = i < 4 ? (seed ^ (i * 0x01010101)) : 0;
        b[i] = i < 4 ? (seed + i * 0x02020202) : 0;
    }
    v16f acc[CHAINS];
#pragma unroll
    for (int c = 0; c < CHAINS; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;
    const uint64_t c0 = __builtin_amdgcn_s_memtime();
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < CHAINS; ++c)
            acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[c], 4, 4, 0, 0, 0, 0);
    }
    // the end stamps wait for the last results
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < CHAINS; ++c) s += acc[c][0] + acc[c][15];
    asm volatile("" : "+v"(s));
    const uint64_t c1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    sink[blockIdx.x * 256 + threadIdx.x] = s;
    if (lane == 0) {
        uint64_t *o = clocks + (size_t)wave * 4;
        o[0] = c0;
        o[1] = c1;
        o[2] = r0;
        o[3] = r1;
    }
}

}  // namespace

extern "C" int32_t fp4_probe_mfma_fp4(int32_t blocks, int32_t iters, uint64_t *clocks, float *sink, void *stream) {
    if (blocks < 1 || iters < 1 || !clocks || !sink) return 1;
    hipLaunchKernelGGL(k_probe_mfma_fp4, dim3((unsigned)blocks), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                       iters, clocks, sink);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}
