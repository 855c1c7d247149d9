// FP4-on-FP8 emulation (the execution mode of the pages' own framework: the QbitAI report's
// format paragraph and the topaibox summary's simulation section describe FP4 values held in
// FP8 and multiplied on FP8 matrix cores).  Every E2M1 value {0, 0.5, 1, 1.5, 2, 3, 4, 6} and
// its negation is exactly representable in E4M3, so the expansion is a 16-entry table and the
// FP8 product equals the FP4 one.
//
// E4M3 bytes (bias 7): 0 -> 0x00, 0.5 -> 0x30, 1 -> 0x38, 1.5 -> 0x3C, 2 -> 0x40, 3 -> 0x44,
// 4 -> 0x48, 6 -> 0x4C; the E2M1 sign bit (bit 3) becomes bit 7.
#include "fp4_common.h"
#include "fp4_launch.h"

namespace fp4 {

// Four codes (nibbles 0..3 of x) -> four E4M3 bytes: byte_perm picks byte (code & 7) of the
// 8-byte magnitude table, then the sign bit moves from bit 3 to bit 7 of its byte.
__device__ __forceinline__ uint32_t expand4(uint32_t x) {
    const uint32_t spread = (x & 0x000Fu) | ((x & 0x00F0u) << 4) | ((x & 0x0F00u) << 8) | ((x & 0xF000u) << 12);
    const uint32_t mag = __builtin_amdgcn_perm(0x4C484440u, 0x3C383000u, spread & 0x07070707u);
    return mag | ((spread & 0x08080808u) << 4);
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void k_e2m1_to_e4m3(const u32x4 *__restrict__ in, int64_t n16,
                                                      u32x4 *__restrict__ out) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) {
        const u32x4 v = __builtin_nontemporal_load(in + i);
        u32x4 o0, o1;
        o0[0] = expand4(v[0] & 0xFFFFu);
        o0[1] = expand4(v[0] >> 16);
        o0[2] = expand4(v[1] & 0xFFFFu);
        o0[3] = expand4(v[1] >> 16);
        o1[0] = expand4(v[2] & 0xFFFFu);
        o1[1] = expand4(v[2] >> 16);
        o1[2] = expand4(v[3] & 0xFFFFu);
        o1[3] = expand4(v[3] >> 16);
        out[2 * i] = o0;
        out[2 * i + 1] = o1;
    }
}

hipError_t launch_e2m1_to_e4m3(const uint8_t *codes, int64_t n_bytes, uint8_t *out, hipStream_t s) {
    const int64_t n16 = n_bytes / 16;  // callers pass multiples of 16 bytes (K % 32 == 0)
    int64_t blocks = (n16 + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(k_e2m1_to_e4m3, dim3((unsigned)blocks), dim3(256), 0, s,
                       reinterpret_cast<const u32x4 *>(codes), n16, reinterpret_cast<u32x4 *>(out));
    return hipGetLastError();
}

}  // namespace fp4
