// Building blocks of the quantized GEMV rows used by kernels A and B.
//
// A row of a quantized matrix is handled by LR lanes of a wave64 (LR a power
// of two); lane j of the row owns the chunks j, j+LR, j+2LR, ... (a chunk is
// 32 codes for 4-bit, 16 codes for 6/8-bit; see common.hpp).  A lane handles
// NR rows at once (r0, r0+rstep, ...): `load_block` issues every load of
// those rows for one chunk position before anything waits on them, and
// `dot_block` consumes them against one input chunk.  The chunk's
// contribution is factored per quantization group:
//     sum_i (s q_i + b) x_i = s * sum_i q_i x_i + b * sum_i x_i,
// so the per-weight work is one code conversion and one FMA.
#pragma once

#include "common.hpp"

namespace moe {

// One quantized projection stack as the kernels see it.
struct QM {
    const uint32_t *q;
    const uint16_t *s;
    const uint16_t *b;
    int rows, cols, wpr, gpr;   // words and groups per row
    int bits_, sb_;             // host-side kernel selection only
};

template <int BITS, int NM, int NR>
struct BlockRegs {
    Chunk<BITS> w[NM][NR];
    uint16_t sr[NM][NR], br[NM][NR];
    bool live[NR];
    int cc;      // the chunk position actually loaded (in bounds)
};

// Loads of NR rows x NM matrices at chunk position c.  Rows past row_end and
// chunks past the row read an in-bounds neighbour (the same cache lines) and
// are masked out in dot_block, so the loads need no branches.
template <int BITS, int NM, int NR>
__device__ __forceinline__ void load_block(BlockRegs<BITS, NM, NR> &R, const QM *mats, int64_t erow0,
                                           int r0, int rstep, int row_end, int c, int cpr) {
    using F = Fmt<BITS>;
    const bool okc = c < cpr;
    R.cc = okc ? c : 0;
#pragma unroll
    for (int n = 0; n < NR; ++n) R.live[n] = okc && (r0 + n * rstep < row_end);
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int n = 0; n < NR; ++n) {
            const int r = min(r0 + n * rstep, row_end - 1);
            const int64_t row = erow0 + r;
            R.w[m][n] = load_chunk<BITS>(mats[m].q + row * mats[m].wpr + R.cc * F::kWords);
            const int64_t gi = row * mats[m].gpr + R.cc / F::kChunksPerGroup;
            R.sr[m][n] = mats[m].s[gi];
            R.br[m][n] = mats[m].b[gi];
        }
}

// acc[m][n] += s * (q . xv) + b * xsum for the loaded chunk of every row.
template <int BITS, int SB, int NM, int NR>
__device__ __forceinline__ void dot_block(const BlockRegs<BITS, NM, NR> &R, const float *xv, float xsum,
                                          float (&acc)[NM][NR]) {
    constexpr int CODES = Fmt<BITS>::kCodes;
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int n = 0; n < NR; ++n) {
            float q[CODES];
            unpack<BITS>(R.w[m][n], q);
            float d = 0.f;
#pragma unroll
            for (int i = 0; i < CODES; ++i) d += q[i] * xv[i];
            const float s = R.live[n] ? sb_to_float<SB>(R.sr[m][n]) : 0.f;
            const float b = R.live[n] ? sb_to_float<SB>(R.br[m][n]) : 0.f;
            acc[m][n] += s * d + b * xsum;
        }
}

// Input chunk of CODES consecutive values, read straight from global memory.
template <int XT, int CODES>
__device__ __forceinline__ void load_x_chunk(const void *x, int64_t off, float *xv) {
    if constexpr (XT == MOE_F32) {
        const f32x4 *p = reinterpret_cast<const f32x4 *>(reinterpret_cast<const float *>(x) + off);
#pragma unroll
        for (int i = 0; i < CODES / 4; ++i) {
            const f32x4 v = p[i];
            xv[4 * i] = v.x; xv[4 * i + 1] = v.y; xv[4 * i + 2] = v.z; xv[4 * i + 3] = v.w;
        }
    } else {
        const u32x4 *p = reinterpret_cast<const u32x4 *>(reinterpret_cast<const uint16_t *>(x) + off);
#pragma unroll
        for (int i = 0; i < CODES / 8; ++i) {
            const u32x4 v = p[i];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                if constexpr (XT == MOE_BF16) {
                    xv[8 * i + 2 * k] = __uint_as_float(v[k] << 16);
                    xv[8 * i + 2 * k + 1] = __uint_as_float(v[k] & 0xFFFF0000u);
                } else {
                    _Float16 lo, hi;
                    const uint16_t l16 = (uint16_t)(v[k] & 0xFFFFu), h16 = (uint16_t)(v[k] >> 16);
                    __builtin_memcpy(&lo, &l16, 2);
                    __builtin_memcpy(&hi, &h16, 2);
                    xv[8 * i + 2 * k] = (float)lo;
                    xv[8 * i + 2 * k + 1] = (float)hi;
                }
            }
        }
    }
}

template <int N>
__device__ __forceinline__ float sum_n(const float *v) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < N; ++i) s += v[i];
    return s;
}

// LDS layout of staged input vectors: vector t, chunk c occupies floats
// [(t*cpr + c)*(CODES+4), +CODES) and its sum sits at +CODES.  The 4-float pad
// puts the 16-byte reads of consecutive chunks by consecutive lanes in
// distinct LDS banks.
template <int CODES>
__device__ __forceinline__ const float *staged_chunk(const float *xs, int t, int cpr, int c) {
    return xs + (t * cpr + c) * (CODES + 4);
}

// Fill the staged layout for nt vectors; src(t, i) gives element i of vector t.
// WITH_SUMS also stores each chunk's sum after it.  Ends with a workgroup
// barrier.
template <int CODES, bool WITH_SUMS = true, typename Src>
__device__ __forceinline__ void stage_inputs(float *xs, int nt, int cpr, Src src) {
    constexpr int SLOT = CODES + 4;
    const int tid = threadIdx.x;
    const int per_vec = cpr * CODES;
    for (int i = tid; i < nt * per_vec; i += blockDim.x) {
        const int t = i / per_vec, rem = i - t * per_vec;
        const int c = rem / CODES, q = rem - c * CODES;
        xs[(t * cpr + c) * SLOT + q] = src(t, rem);
    }
    __syncthreads();
    if (!WITH_SUMS) return;
    for (int i = tid; i < nt * cpr; i += blockDim.x) {
        float *p = xs + i * SLOT;
        float sum = 0.f;
#pragma unroll
        for (int q = 0; q < CODES; ++q) sum += p[q];
        p[CODES] = sum;
    }
    __syncthreads();
}

// Read a staged chunk (CODES values) into registers.
template <int CODES>
__device__ __forceinline__ void read_staged(const float *p, float *xv) {
    const f32x4 *v = reinterpret_cast<const f32x4 *>(p);
#pragma unroll
    for (int i = 0; i < CODES / 4; ++i) {
        const f32x4 a = v[i];
        xv[4 * i] = a.x; xv[4 * i + 1] = a.y; xv[4 * i + 2] = a.z; xv[4 * i + 3] = a.w;
    }
}

}  // namespace moe
