// Device helpers shared by the gfx950 kernels of the quantized MoE decode layer.
//
// Weight format (mlxcel PR #276, "Scope / flags" and "Next": affine 4/8-bit
// and 6-bit weights): codes are packed LSB-first into little-endian uint32
// words per row; w = scale * q + bias with one scale and bias per group of 64
// codes along the contraction dimension.
//
// A lane always loads whole "chunks" of a row:
//   4-bit: 16 bytes = 32 codes (half a group)
//   8-bit: 16 bytes = 16 codes (a quarter group)
//   6-bit: 12 bytes = 16 codes (a quarter group; 16 codes fill exactly 3 words)
// so every chunk starts on a code boundary and lies inside one group.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_decode.h"

namespace moe {

constexpr int kWave = 64;
constexpr int kGroup = 64;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int BITS> struct Fmt;
template <> struct Fmt<4> { static constexpr int kCodes = 32, kWords = 4, kChunksPerGroup = 2; };
template <> struct Fmt<8> { static constexpr int kCodes = 16, kWords = 4, kChunksPerGroup = 4; };
template <> struct Fmt<6> { static constexpr int kCodes = 16, kWords = 3, kChunksPerGroup = 4; };

// A chunk of packed codes held in registers.
template <int BITS> struct Chunk { uint32_t w[Fmt<BITS>::kWords]; };

// Streaming (non-temporal) load of one chunk: the weights are read once per step.
template <int BITS>
__device__ __forceinline__ Chunk<BITS> load_chunk(const uint32_t *p) {
    Chunk<BITS> c;
    if constexpr (Fmt<BITS>::kWords == 4) {
        u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
        c.w[0] = v.x; c.w[1] = v.y; c.w[2] = v.z; c.w[3] = v.w;
    } else {
        c.w[0] = __builtin_nontemporal_load(p + 0);
        c.w[1] = __builtin_nontemporal_load(p + 1);
        c.w[2] = __builtin_nontemporal_load(p + 2);
    }
    return c;
}

// Unpack a chunk into its codes as floats, in code order.
template <int BITS>
__device__ __forceinline__ void unpack(const Chunk<BITS> &c, float *q) {
    if constexpr (BITS == 4) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t lo = c.w[k] & 0x0F0F0F0Fu;          // codes 8k, 8k+2, 8k+4, 8k+6
            const uint32_t hi = (c.w[k] >> 4) & 0x0F0F0F0Fu;   // codes 8k+1, 8k+3, 8k+5, 8k+7
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                q[8 * k + 2 * b] = (float)((lo >> (8 * b)) & 0xFFu);
                q[8 * k + 2 * b + 1] = (float)((hi >> (8 * b)) & 0xFFu);
            }
        }
    } else if constexpr (BITS == 8) {
#pragma unroll
        for (int k = 0; k < 4; ++k)
#pragma unroll
            for (int b = 0; b < 4; ++b)
                q[4 * k + b] = (float)((c.w[k] >> (8 * b)) & 0xFFu);
    } else {
        // 96 bits hold 16 six-bit codes; code i is bits [6i, 6i+6).
        const uint64_t lo = (uint64_t)c.w[0] | ((uint64_t)c.w[1] << 32);
#pragma unroll
        for (int i = 0; i < 10; ++i)
            q[i] = (float)((uint32_t)(lo >> (6 * i)) & 63u);
        q[10] = (float)(((uint32_t)(lo >> 60) | (c.w[2] << 4)) & 63u);
#pragma unroll
        for (int i = 11; i < 16; ++i)
            q[i] = (float)((c.w[2] >> (6 * i - 64)) & 63u);
    }
}

// A 16-bit scale or bias bit pattern as float.
template <int SB>
__device__ __forceinline__ float sb_to_float(uint16_t h) {
    if constexpr (SB == MOE_BF16) {
        return __uint_as_float((uint32_t)h << 16);
    } else {
        _Float16 f;
        __builtin_memcpy(&f, &h, 2);
        return (float)f;
    }
}

template <int SB>
__device__ __forceinline__ float load_sb(const uint16_t *p, int64_t i) {
    return sb_to_float<SB>(p[i]);
}

// Activation element of a given dtype as float.
__device__ __forceinline__ float load_act(const void *p, int dt, int64_t i) {
    if (dt == MOE_F32) return reinterpret_cast<const float *>(p)[i];
    const uint16_t h = reinterpret_cast<const uint16_t *>(p)[i];
    if (dt == MOE_BF16) return __uint_as_float((uint32_t)h << 16);
    _Float16 f;
    __builtin_memcpy(&f, &h, 2);
    return (float)f;
}

// Sum over aligned groups of `width` lanes (a power of two <= 64); every lane
// of the group ends with the same bits.
__device__ __forceinline__ float group_sum(float v, int width) {
    for (int m = width >> 1; m > 0; m >>= 1)
        v += __shfl_xor(v, m, kWave);
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m > 0; m >>= 1)
        v += __shfl_xor(v, m, kWave);
    return v;
}

__device__ __forceinline__ float sigmoidf_(float z) { return 1.0f / (1.0f + __expf(-z)); }

}  // namespace moe
