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

// Rounding to the output dtypes: the nearest value of dtype dt, ties to even.
// bf16 keeps the top 16 bits of the fp32 pattern after adding half of the
// dropped part's range (plus the kept part's lowest bit, for ties to even);
// NaN stays a quiet NaN.  fp16 uses the hardware conversion, which rounds to
// nearest even in the default mode.  Both are computed and one is selected,
// so the callers' code has no branches on dt but the store width.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float v) {
    const uint32_t u = __float_as_uint(v);
    const uint32_t r = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
    return (u & 0x7fffffffu) > 0x7f800000u ? ((u >> 16) | 0x40u) : r;
}

__device__ __forceinline__ uint32_t f32_to_f16_bits(float v) {
    const _Float16 h = (_Float16)v;
    uint16_t b;
    __builtin_memcpy(&b, &h, 2);
    return b;
}

// v rounded to dtype dt, as a float (F32: v itself).
__device__ __forceinline__ float round_to_dtype(int dt, float v) {
    const float b = __uint_as_float(f32_to_bf16_rne(v) << 16);
    const float h = (float)(_Float16)v;
    return dt == MOE_BF16 ? b : (dt == MOE_F16 ? h : v);
}

// Element i of p, of dtype dt, set to v, which already holds a value of dt
// (round_to_dtype): the conversion back to 16 bits is exact.
__device__ __forceinline__ void store_rounded(void *p, int dt, int64_t i, float v) {
    if (dt == MOE_F32) {
        reinterpret_cast<float *>(p)[i] = v;
    } else {
        const uint32_t bits = dt == MOE_BF16 ? (__float_as_uint(v) >> 16) : f32_to_f16_bits(v);
        reinterpret_cast<uint16_t *>(p)[i] = (uint16_t)bits;
    }
}

// Element i of p, of dtype dt, set to v rounded to dt.
__device__ __forceinline__ void store_act(void *p, int dt, int64_t i, float v) {
    store_rounded(p, dt, i, round_to_dtype(dt, v));
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}

// v + (value of DPP control CTRL) in the rows of ROW_MASK; other rows add 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_add_rows(float v) {
    return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xf, false));
}

// Sum over aligned groups of W lanes (a power of two <= 64) with DPP only:
// within a row of 16 every lane gets the sum (quad permutations, half-mirror,
// mirror); across rows the row broadcasts carry it forward, so for W >= 32
// only the group's last lane holds the total.  Read the result there.
template <int W>
__device__ __forceinline__ float group_sum_last(float v) {
    if constexpr (W >= 2) v += dpp_f<0xB1>(v);     // quad_perm [1,0,3,2]
    if constexpr (W >= 4) v += dpp_f<0x4E>(v);     // quad_perm [2,3,0,1]
    if constexpr (W >= 8) v += dpp_f<0x141>(v);    // row_half_mirror
    if constexpr (W >= 16) v += dpp_f<0x140>(v);   // row_mirror
    if constexpr (W >= 32) v = dpp_add_rows<0x142, 0xA>(v);   // row_bcast:15 into rows 1 and 3
    if constexpr (W >= 64) v = dpp_add_rows<0x143, 0xC>(v);   // row_bcast:31 into rows 2 and 3
    return v;
}

// DPP control that pairs every lane with the lane across bit B (B <= 3) of
// its index within a row: row_ror:8 for bit 3, row_half_mirror (lanes r and
// 7 - r, which differ in bit 2) for bit 2, quad permutations for bits 1, 0.
template <int B>
constexpr int dpp_across_bit() {
    return B == 3 ? 0x128 : B == 2 ? 0x141 : B == 1 ? 0x4E : 0xB1;
}

// The gfx950 permlane swap across lane bit B (5: lanes l and l ^ 32; 4: l
// and l ^ 16) of two registers a, b.  In the lower lane of each pair, r0 is
// its own a and r1 its partner's a; in the upper lane, r0 is its partner's b
// and r1 its own b.  So r0 + r1 is a's pair sum in lower lanes and b's in
// upper lanes, and with a = b = x the partner's x is r1 (lower) or r0 (upper).
template <int B>
__device__ __forceinline__ void swap_across(float a, float b, float &r0, float &r1) {
    static_assert(B == 4 || B == 5, "permlane swaps cover lane bits 4 and 5");
    if constexpr (B == 5) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
        r0 = __uint_as_float(r[0]);
        r1 = __uint_as_float(r[1]);
    } else {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
        r0 = __uint_as_float(r[0]);
        r1 = __uint_as_float(r[1]);
    }
}

template <int K, int LW, int LV, int V>
__device__ __forceinline__ void multi_sum_step(float (&v)[V], int lane) {
    if constexpr (K < LW) {
        constexpr int B = LW - 1 - K;
        if constexpr (K < LV) {               // halve: keep one half, add the partner's
            constexpr int H = (V >> K) / 2;
#pragma unroll
            for (int j = 0; j < H; ++j) {
                if constexpr (B >= 4) {
                    float r0, r1;
                    swap_across<B>(v[j], v[j + H], r0, r1);
                    v[j] = r0 + r1;
                } else {
                    const bool hi = (lane >> B) & 1;
                    const float keep = hi ? v[j + H] : v[j], send = hi ? v[j] : v[j + H];
                    v[j] = keep + dpp_f<dpp_across_bit<B>()>(send);
                }
            }
        } else {                              // add across the bit
            if constexpr (B >= 4) {
                float r0, r1;
                swap_across<B>(v[0], v[0], r0, r1);
                v[0] = r0 + r1;
            } else {
                v[0] += dpp_f<dpp_across_bit<B>()>(v[0]);
            }
        }
        multi_sum_step<K + 1, LW, LV, V>(v, lane);
    }
}

constexpr int ilog2(int n) { return n <= 1 ? 0 : 1 + ilog2(n / 2); }

// Sums of V values over aligned groups of W lanes at once (W and V powers of
// two, V <= W, W <= 64): lane l ends with, in v[0], the group sum of value
// (l mod W) >> (log2 W - log2 V), so each value's sum sits in W / V
// consecutive lanes.  Each of the first log2 V steps halves the values a
// lane holds (a lane and its partner across one lane bit each keep one half
// and add the other's half), the remaining steps add across the remaining
// bits: V - 1 + log2 W additions in all, against V log2 W for V separate
// reductions.  The partners are the gfx950 permlane swaps for bits 5 and 4
// and DPP for bits 3..0.
template <int W, int V>
__device__ __forceinline__ void group_multi_sum(float (&v)[V]) {
    static_assert(ilog2(V) <= ilog2(W) && W <= 64, "at most one value per lane of the group");
    multi_sum_step<0, ilog2(W), ilog2(V), V>(v, threadIdx.x & (kWave - 1));
}

// x of the lane across the top bit of its W-lane group (W >= 16).
template <int W>
__device__ __forceinline__ float group_partner(float x) {
    static_assert(W >= 16 && W <= 64, "partner across lane bit 3, 4 or 5");
    constexpr int B = ilog2(W) - 1;
    if constexpr (B == 3) {
        return dpp_f<dpp_across_bit<3>()>(x);
    } else {
        float r0, r1;
        swap_across<B>(x, x, r0, r1);
        return ((threadIdx.x >> B) & 1) ? r0 : r1;
    }
}

// Sum over the whole wave, the same value in every lane (DPP reduction into
// lane 63, then a broadcast of that lane).
__device__ __forceinline__ float wave_sum(float v) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(group_sum_last<kWave>(v)), kWave - 1));
}

// fn(IntC-like tag with ::value = 1 << shift) for a wave-uniform shift in 0..6.
template <int N>
struct WidthC {
    static constexpr int value = N;
};
template <typename Fn>
__device__ __forceinline__ void with_width(int shift, Fn fn) {
    switch (shift) {
    case 0: fn(WidthC<1>{}); break;
    case 1: fn(WidthC<2>{}); break;
    case 2: fn(WidthC<4>{}); break;
    case 3: fn(WidthC<8>{}); break;
    case 4: fn(WidthC<16>{}); break;
    case 5: fn(WidthC<32>{}); break;
    default: fn(WidthC<64>{}); break;
    }
}

// Maximum over the wave with DPP row shifts and row broadcasts; every lane
// gets the result.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float fmax_dpp(float v) {
    const int o = __builtin_amdgcn_update_dpp(__float_as_int(-INFINITY), __float_as_int(v), CTRL, ROW_MASK,
                                              0xf, false);
    return fmaxf(v, __int_as_float(o));
}

__device__ __forceinline__ float wave_max(float v) {
    v = fmax_dpp<0x111, 0xf>(v);   // row_shr:1
    v = fmax_dpp<0x112, 0xf>(v);   // row_shr:2
    v = fmax_dpp<0x114, 0xf>(v);   // row_shr:4
    v = fmax_dpp<0x118, 0xf>(v);   // row_shr:8  (lane 15 of each row: the row maximum)
    v = fmax_dpp<0x142, 0xa>(v);   // row_bcast:15
    v = fmax_dpp<0x143, 0xc>(v);   // row_bcast:31 (lane 63: the wave maximum)
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ float sigmoidf_(float z) { return 1.0f / (1.0f + __expf(-z)); }

}  // namespace moe
