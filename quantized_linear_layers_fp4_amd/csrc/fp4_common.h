// Device-side helpers shared by the gfx950 kernels of the FP4 linear forward.
// Internal header: not part of the C ABI (include/fp4lin.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4 {

enum : int { DT_F32 = 0, DT_BF16 = 1, DT_Q16 = 2 };

// DT_Q16: the GEMM's accumulator handed to the compensation pass in two bytes.  The FP4
// products are multiples of 1/4 and their fp32 sum is exact, so 4*acc is an integer, stored
// as int16 when |acc| <= Q16_MAX_ACC.  The GEMM also writes a map with one byte per aligned
// ESC_ROWS x ESC_COLS output block, set for the blocks of a wave block that holds a larger
// |acc|; the escape kernel (escape.hip) recomputes those blocks and the compensation pass
// skips them.  As the standalone two-byte output, escaped elements hold Q16_ESC and an fp32
// buffer their fl(fl(acc*sA)*sW).
constexpr int ESC_ROWS = 128, ESC_COLS = 64;
// Row stride of the map in bytes: a multiple of 8, so the eight blocks under a 512-column chunk
// are one aligned 8-byte word (the padding bytes are never written or read as blocks).
__host__ __device__ inline int esc_map_stride(int64_t N) { return (int)((N + 8 * ESC_COLS - 1) / (8 * ESC_COLS)) * 8; }
constexpr int Q16_ESC = -32768;
constexpr float Q16_MAX_ACC = 8191.75f;  // largest |acc| stored inline
// fl(acc * 4 + 1.5 * 2^23) is exact for |4*acc| < 2^22 and its low 16 bits are 4*acc as int16
constexpr float Q16_MAGIC = 12582912.0f;

// |x| as an unsigned key: the fp32 bit pattern of |x|.  For non-negative finite floats
// the unsigned order of the bit patterns is the numeric order, so every comparison of
// magnitudes below is an integer comparison, independent of the denormal mode.  For
// bf16 inputs the key is the widened pattern (low 16 bits zero).
__device__ __forceinline__ uint32_t key_of_bf16(uint32_t b16) { return (b16 & 0x7FFFu) << 16; }
__device__ __forceinline__ uint32_t key_of_f32(uint32_t b32) { return b32 & 0x7FFFFFFFu; }

constexpr int HIST_BINS = 32768;     // level-1 histogram: key >> 16 (15 bits)
constexpr int HIST_LO_BINS = 65536;  // level-2 histogram for fp32 keys: key & 0xFFFF

// Device-resident scalars of one outlier pass (lives in the caller's workspace).
struct State {
    uint64_t k_rem;        // rank left inside the level-1 bin (fp32 inputs)
    uint64_t nnz_hist;     // #{|a| > T} counted from the histograms
    uint32_t T_key;        // key of T
    float T;               // T itself
    uint32_t hi_bin;       // selected level-1 bin
    uint32_t hi_count;     // population of that bin
};
static_assert(sizeof(State) == 32, "State layout");

// Outlier staging.  Row m owns S slots; the outlier of rank j (ascending column) in row m
// goes to slot m*S + j when j < S.  A row with more outliers (rare: S is at least 128 and twice
// the mean count per row plus a margin) is read again when the COO list is assembled, and its
// outliers of rank >= S are written straight to their final positions there.  No atomic is
// involved.
struct SlotEntry {
    int32_t col;
    float val;   // delta = a - copysign(T, a)
};
struct Staging {
    SlotEntry *slots;
    int32_t S;
};

// Per-vector scales: r = fl(6 / amax) multiplies, s = fl(amax / 6) dequantizes; a vector
// whose amax is below 2^-120 gets r = s = 0.  Both divisions are IEEE round-to-nearest.
__device__ __forceinline__ void vector_scale(float amax, float &r, float &s) {
    if (!(amax >= 0x1p-120f)) {
        r = 0.0f;
        s = 0.0f;
    } else {
        r = __fdiv_rn(6.0f, amax);
        s = __fdiv_rn(amax, 6.0f);
    }
}

// E2M1 round-to-nearest-even with saturation of two floats into byte SEL of `word`
// (first value in the low nibble).  The gfx950 converter with unit scale performs
// exactly that rounding on every finite fp32 input.
template <int SEL>
__device__ __forceinline__ uint32_t e2m1_pack2(uint32_t word, float lo, float hi) {
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, lo, hi, 1.0f, SEL);
}

__device__ __forceinline__ uint32_t e2m1_pack8(const float y[8]) {
    uint32_t w = 0;
    w = e2m1_pack2<0>(w, y[0], y[1]);
    w = e2m1_pack2<1>(w, y[2], y[3]);
    w = e2m1_pack2<2>(w, y[4], y[5]);
    w = e2m1_pack2<3>(w, y[6], y[7]);
    return w;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t b = __float_as_uint(f);
    return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// Load 8 consecutive elements of an fp32 or bf16 row as fp32 values plus their keys and
// raw sign bits.  p must be 16-byte aligned.
template <int DT>
__device__ __forceinline__ void load8(const void *__restrict__ base, int64_t elem, float v[8],
                                      uint32_t key[8], uint32_t sgn[8]) {
    if constexpr (DT == DT_BF16) {
        uint4 q = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(base) + elem);
        uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint32_t lo = w[i] & 0xFFFFu, hi = w[i] >> 16;
            v[2 * i] = bf16_to_f32(lo);
            v[2 * i + 1] = bf16_to_f32(hi);
            key[2 * i] = key_of_bf16(lo);
            key[2 * i + 1] = key_of_bf16(hi);
            sgn[2 * i] = (lo << 16) & 0x80000000u;
            sgn[2 * i + 1] = (hi << 16) & 0x80000000u;
        }
    } else {
        const uint4 *p = reinterpret_cast<const uint4 *>(reinterpret_cast<const float *>(base) + elem);
        uint4 q0 = p[0], q1 = p[1];
        uint32_t w[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            v[i] = __uint_as_float(w[i]);
            key[i] = key_of_f32(w[i]);
            sgn[i] = w[i] & 0x80000000u;
        }
    }
}

// Wave-wide (64 lanes) reductions and scans.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x = max(x, (uint32_t)__shfl_xor((int)x, off, 64));
    return x;
}

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x, int lane) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        uint32_t y = (uint32_t)__shfl_up((int)x, off, 64);
        if (lane >= off) x += y;
    }
    return x;
}

}  // namespace fp4
