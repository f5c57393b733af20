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
// are masked out in dot_block, so the loads need no branches.  With SBASE,
// erow0 (the expert's first row, the same for the whole wave) gives the
// expert's base addresses once in scalar registers and each lane adds a
// 32-bit offset (24-bit multiplies: rows and row lengths are at most 8192),
// so a load costs a couple of vector instructions instead of a 64-bit
// address computation; without it every address is formed per lane in 64
// bits, which schedules better in some kernels.
template <int BITS, int NM, int NR, bool SBASE = true>
__device__ __forceinline__ void load_block(BlockRegs<BITS, NM, NR> &R, const QM *mats, int64_t erow0,
                                           int r0, int rstep, int row_end, int c, int cpr) {
    using F = Fmt<BITS>;
    const bool okc = c < cpr;
    R.cc = okc ? c : 0;
    if constexpr (!SBASE) {
#pragma unroll
        for (int n = 0; n < NR; ++n) R.live[n] = okc && (r0 + n * rstep < row_end);
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int n = 0; n < NR; ++n) {
                const int64_t row = erow0 + min(r0 + n * rstep, row_end - 1);
                R.w[m][n] = load_chunk<BITS>(mats[m].q + row * mats[m].wpr + R.cc * F::kWords);
                const int64_t gi = row * mats[m].gpr + R.cc / F::kChunksPerGroup;
                R.sr[m][n] = mats[m].s[gi];
                R.br[m][n] = mats[m].b[gi];
            }
        __builtin_amdgcn_sched_barrier(0);
        return;
    }
    const uint32_t e_lo = __builtin_amdgcn_readfirstlane((uint32_t)erow0);
    const uint32_t e_hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)erow0 >> 32));
    const int64_t er = (int64_t)(((uint64_t)e_hi << 32) | e_lo);
    uint32_t rr[NR];
#pragma unroll
    for (int n = 0; n < NR; ++n) {
        R.live[n] = okc && (r0 + n * rstep < row_end);
        rr[n] = (uint32_t)min(r0 + n * rstep, row_end - 1);
    }
#pragma unroll
    for (int m = 0; m < NM; ++m) {
        const uint32_t *qb = mats[m].q + er * mats[m].wpr;
        const uint16_t *sb = mats[m].s + er * mats[m].gpr;
        const uint16_t *bb = mats[m].b + er * mats[m].gpr;
#pragma unroll
        for (int n = 0; n < NR; ++n) {
            R.w[m][n] = load_chunk<BITS>(qb + (__umul24(rr[n], (uint32_t)mats[m].wpr) + (uint32_t)R.cc * F::kWords));
            const uint32_t gi = __umul24(rr[n], (uint32_t)mats[m].gpr) + (uint32_t)R.cc / F::kChunksPerGroup;
            R.sr[m][n] = sb[gi];
            R.br[m][n] = bb[gi];
        }
    }
    // Keep every load of the block here: left alone, the compiler sinks the
    // scale/bias loads down to their first use, after the codes have arrived,
    // which costs a second memory round trip per block.
    __builtin_amdgcn_sched_barrier(0);
}

// The codes of word k of a 4- or 8-bit chunk as floats.
template <int BITS>
__device__ __forceinline__ void unpack_word(uint32_t w, float *q) {
    if constexpr (BITS == 4) {
        const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            q[2 * b] = (float)((lo >> (8 * b)) & 0xFFu);
            q[2 * b + 1] = (float)((hi >> (8 * b)) & 0xFFu);
        }
    } else {
#pragma unroll
        for (int b = 0; b < 4; ++b) q[b] = (float)((w >> (8 * b)) & 0xFFu);
    }
}

// acc[m][n] += s * (q . xv) + b * xsum for the loaded chunk of every row.
// For 4- and 8-bit codes the loop walks the chunk word by word across all
// rows, so the NM*NR dot products form independent FMA chains that hide each
// other's latency; 6-bit chunks (codes straddle words) are unpacked whole.
template <int BITS, int SB, int NM, int NR>
__device__ __forceinline__ void dot_block(const BlockRegs<BITS, NM, NR> &R, const float *xv, float xsum,
                                          float (&acc)[NM][NR]) {
    constexpr int CODES = Fmt<BITS>::kCodes;
    float d[NM][NR];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int n = 0; n < NR; ++n) d[m][n] = 0.f;
    if constexpr (BITS == 6) {
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int n = 0; n < NR; ++n) {
                float q[CODES];
                unpack<BITS>(R.w[m][n], q);
#pragma unroll
                for (int i = 0; i < CODES; ++i) d[m][n] += q[i] * xv[i];
            }
    } else {
        constexpr int PER_WORD = 32 / BITS;
#pragma unroll
        for (int k = 0; k < Fmt<BITS>::kWords; ++k)
#pragma unroll
            for (int m = 0; m < NM; ++m)
#pragma unroll
                for (int n = 0; n < NR; ++n) {
                    float q[PER_WORD];
                    unpack_word<BITS>(R.w[m][n].w[k], q);
#pragma unroll
                    for (int i = 0; i < PER_WORD; ++i) d[m][n] += q[i] * xv[k * PER_WORD + i];
                }
    }
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int n = 0; n < NR; ++n) {
            const float s = R.live[n] ? sb_to_float<SB>(R.sr[m][n]) : 0.f;
            const float b = R.live[n] ? sb_to_float<SB>(R.br[m][n]) : 0.f;
            acc[m][n] += s * d[m][n] + b * xsum;
        }
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// The four code pairs of a 4-bit word for the packed dot instructions: pair p
// holds codes p and p + 4 (the nibbles at bits 4p and 16 + 4p) as the low and
// high 16-bit halves, each MAGIC << 8 | q.  With MAGIC = 0x43 that is the bf16
// 128 + q, with MAGIC = 0x64 the fp16 1024 + q (both exact).  Masking the even
// and the odd nibbles once and placing bytes with v_perm costs seven
// instructions per word, where shift-mask-or per pair costs eleven (this
// target has no literal operand for a three-input and-or).
template <uint32_t MAGIC>
__device__ __forceinline__ void nibble_pairs(uint32_t w, uint32_t (&q)[4]) {
    constexpr uint32_t kMagic4 = MAGIC * 0x01010101u;
    const uint32_t lo = w & 0x0F0F0F0Fu;            // byte b: nibble 2b
    const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;     // byte b: nibble 2b + 1
    q[0] = __builtin_amdgcn_perm(kMagic4, lo, 0x04020400u);     // nibbles 0, 4
    q[1] = __builtin_amdgcn_perm(kMagic4, hi, 0x04020400u);     // nibbles 1, 5
    q[2] = __builtin_amdgcn_perm(kMagic4, lo, 0x04030401u);     // nibbles 2, 6
    q[3] = __builtin_amdgcn_perm(kMagic4, hi, 0x04030401u);     // nibbles 3, 7
}

// 4-bit codes against bf16 inputs with the packed dot instruction.  Each
// code q is turned into the bf16 number 128 + q (exact: 0x4300 | q, by
// nibble_pairs), and v_dot2 multiplies two such numbers by two
// bf16 inputs and adds both products (exact in fp32) to the accumulator:
//     sum_i (s q_i + b) x_i = s * sum_i (128 + q_i) x_i + (b - 128 s) * sum_i x_i.
// Pair p of word k holds codes (8k+p, 8k+p+4) (nibbles p and p+4), so the
// inputs are paired the same way, once per chunk, with byte permutes.
// xw: the chunk's 32 bf16 inputs as 16 words (element 2i in the low half of
// word i).
template <int SB, int NM, int NR>
__device__ __forceinline__ void dot_block_q4_bf16(const BlockRegs<4, NM, NR> &R, const uint32_t *xw,
                                                  float xsum, float (&acc)[NM][NR]) {
    uint32_t xp[4][4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t x0 = xw[4 * k], x1 = xw[4 * k + 1], x2 = xw[4 * k + 2], x3 = xw[4 * k + 3];
        xp[k][0] = __builtin_amdgcn_perm(x2, x0, 0x05040100u);   // (x[8k],   x[8k+4])
        xp[k][1] = __builtin_amdgcn_perm(x2, x0, 0x07060302u);   // (x[8k+1], x[8k+5])
        xp[k][2] = __builtin_amdgcn_perm(x3, x1, 0x05040100u);   // (x[8k+2], x[8k+6])
        xp[k][3] = __builtin_amdgcn_perm(x3, x1, 0x07060302u);   // (x[8k+3], x[8k+7])
    }
    float d[NM][NR];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int n = 0; n < NR; ++n) d[m][n] = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int n = 0; n < NR; ++n) {
                uint32_t qw[4];
                nibble_pairs<0x43u>(R.w[m][n].w[k], qw);
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const uint32_t qp = qw[p];
                    d[m][n] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qp),
                                                              __builtin_bit_cast(bf16x2_t, xp[k][p]),
                                                              d[m][n], false);
                }
            }
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int n = 0; n < NR; ++n) {
            const float s = R.live[n] ? sb_to_float<SB>(R.sr[m][n]) : 0.f;
            const float b = R.live[n] ? sb_to_float<SB>(R.br[m][n]) : 0.f;
            acc[m][n] += s * d[m][n] + (b - 128.0f * s) * xsum;
        }
}

// Input chunk of CODES consecutive values, read straight from global memory.
// Raw words of one input chunk: CODES elements of dtype XT (4 or 2 bytes).
template <int XT, int CODES>
struct XRaw {
    static constexpr int kVecs = CODES * (XT == MOE_F32 ? 4 : 2) / 16;
    u32x4 v[kVecs];
};

// Issue the loads of an input chunk (elements off .. off+CODES of x); the
// values are converted later by convert_x, so the loads can be issued ahead
// of the weight loads without waiting on them.
template <int XT, int CODES>
__device__ __forceinline__ void load_x_raw(const void *x, int64_t off, XRaw<XT, CODES> &r) {
    constexpr int kElem = XT == MOE_F32 ? 4 : 2;
    const u32x4 *p = reinterpret_cast<const u32x4 *>(reinterpret_cast<const char *>(x) + off * kElem);
#pragma unroll
    for (int i = 0; i < XRaw<XT, CODES>::kVecs; ++i) r.v[i] = p[i];
}

template <int XT, int CODES>
__device__ __forceinline__ void convert_x(const XRaw<XT, CODES> &r, float *xv) {
    if constexpr (XT == MOE_F32) {
#pragma unroll
        for (int i = 0; i < CODES / 4; ++i)
#pragma unroll
            for (int k = 0; k < 4; ++k) xv[4 * i + k] = __uint_as_float(r.v[i][k]);
    } else {
#pragma unroll
        for (int i = 0; i < CODES / 8; ++i) {
            const u32x4 v = r.v[i];
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

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// fp16 inputs of one 4-bit chunk staged for dot_block_q4_f16: 16 pairs, pair
// 4k + p = (input 8k+p, input 8k+p+4) (the codes a nibble pair of word k
// holds), then 16 bytes of padding.
constexpr int kF16ChunkBytes = 16 * 4 + 16;

// Staging of fp32 act as fp16 for the packed fp16 dot of a 4-bit down
// projection.  Every value is multiplied by kActF16Prescale = 2^8 before it is
// rounded (exact), and the dot products by 2^-8 afterwards (exact, folded into
// the score).  fp16's normal range then holds |act| from 2^-22 to 255.9 with
// 11-bit precision; a smaller value is an fp16 subnormal with an absolute
// error of at most 2^-25 after scaling, 2^-33 before, so over a row of n <=
// 8192 terms such errors stay below n 2^-33 |w|max.  A value of
// kActF16Overflow = 65520 / 2^8 or more would round to fp16 infinity: the
// stagers check for it and then stage the vector again with a factor fitted
// to its largest magnitude m (f16_stage_scale).
constexpr float kActF16Prescale = 256.0f;
constexpr float kActF16Postscale = 1.0f / 256.0f;
constexpr float kActF16Overflow = 255.9375f;

// The power-of-two staging factor for a vector whose largest magnitude has
// the bit pattern m: values are multiplied by inv = 2^-k before rounding and
// the dot products by the returned 2^k afterwards (both exact), k chosen so
// that m 2^-k lies in [2^14, 2^15): nothing overflows, and every value within
// 2^-28 of m keeps fp16's 11-bit precision.  m's biased exponent e gives m in
// [2^(e-127), 2^(e-126)), so inv = 2^(141-e); exponents below 15 (m < 2^-112,
// zero included) take e = 15, keeping both factors normal floats.
__device__ __forceinline__ float f16_stage_scale(uint32_t max_abs_bits, float &inv) {
    const int e = max((int)(max_abs_bits >> 23), 15);
    inv = __uint_as_float((uint32_t)(268 - e) << 23);
    return __uint_as_float((uint32_t)(e - 14) << 23);
}

// LDS byte offset (within a chunk) of input i of the chunk, in that order.
__device__ __forceinline__ int f16_pair_offset(int i) {
    const int k = i >> 3, r = i & 7;
    return (4 * k + (r & 3)) * 4 + (r >> 2) * 2;
}

// 4-bit codes against fp16 inputs with the packed fp16 dot instruction.  A
// pair of codes becomes the fp16 pair (1024 + q, 1024 + q') (nibble_pairs:
// 0x6400 | q is 1024 + q exactly) and then (q, q') with one packed fp16
// subtraction (exact), so no large offset has to cancel later; v_dot2
// multiplies it by two fp16 inputs (products exact in fp32) and adds both to
// the fp32 accumulator.  ap: the chunk's 16 staged pairs; asum: their sum.
template <int SB, int NM, int NR>
__device__ __forceinline__ void dot_block_q4_f16(const BlockRegs<4, NM, NR> &R, const uint32_t *ap, float asum,
                                                 float (&acc)[NM][NR]) {
    const f16x2_t off = {(_Float16)1024.0f, (_Float16)1024.0f};
    float d[NM][NR];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int n = 0; n < NR; ++n) d[m][n] = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int n = 0; n < NR; ++n) {
                uint32_t qw[4];
                nibble_pairs<0x64u>(R.w[m][n].w[k], qw);
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const f16x2_t q = __builtin_bit_cast(f16x2_t, qw[p]) - off;
                    d[m][n] = __builtin_amdgcn_fdot2(q, __builtin_bit_cast(f16x2_t, ap[4 * k + p]), d[m][n], false);
                }
            }
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int n = 0; n < NR; ++n) {
            const float s = R.live[n] ? sb_to_float<SB>(R.sr[m][n]) : 0.f;
            const float b = R.live[n] ? sb_to_float<SB>(R.br[m][n]) : 0.f;
            acc[m][n] += s * d[m][n] + b * asum;
        }
}

// The codes of a 4-bit block as the exact fp16 pairs dot_block_q4_f16 forms,
// unpacked ahead of their inputs (while those are still on their way):
// pre[m][n][4k + p] is pair p of word k.
template <int NM, int NR>
__device__ __forceinline__ void unpack_q4_f16(const BlockRegs<4, NM, NR> &R, uint32_t (&pre)[NM][NR][16]) {
    const f16x2_t off = {(_Float16)1024.0f, (_Float16)1024.0f};
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int n = 0; n < NR; ++n)
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                uint32_t qw[4];
                nibble_pairs<0x64u>(R.w[m][n].w[k], qw);
#pragma unroll
                for (int p = 0; p < 4; ++p)
                    pre[m][n][4 * k + p] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, qw[p]) - off);
            }
}

// dot_block_q4_f16 on codes already unpacked by unpack_q4_f16 (R supplies the
// scales, biases and row validity).
template <int SB, int NM, int NR>
__device__ __forceinline__ void dot_pre_q4_f16(const BlockRegs<4, NM, NR> &R, const uint32_t (&pre)[NM][NR][16],
                                               const uint32_t *ap, float asum, float (&acc)[NM][NR]) {
    float d[NM][NR];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int n = 0; n < NR; ++n) d[m][n] = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i)
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int n = 0; n < NR; ++n)
                d[m][n] = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, pre[m][n][i]),
                                                 __builtin_bit_cast(f16x2_t, ap[i]), d[m][n], false);
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int n = 0; n < NR; ++n) {
            const float s = R.live[n] ? sb_to_float<SB>(R.sr[m][n]) : 0.f;
            const float b = R.live[n] ? sb_to_float<SB>(R.br[m][n]) : 0.f;
            acc[m][n] += s * d[m][n] + b * asum;
        }
}

// Sum of a chunk's NP staged fp16 pairs, in fp32.
template <int NP = 16>
__device__ __forceinline__ float f16_pairs_sum(const uint32_t *ap) {
    const f16x2_t one = {(_Float16)1.0f, (_Float16)1.0f};
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NP; ++i) s = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, ap[i]), one, s, false);
    return s;
}

// fp16 inputs of one 6- or 8-bit chunk (16 values) staged for
// dot_block_f16x16: in order, pair p = (input 2p, input 2p + 1), then 16 bytes
// of padding.
constexpr int kF16Chunk16Bytes = 16 * 2 + 16;

// Bytes of one staged fp16 input chunk of a BITS-bit down projection, and the
// LDS byte offset of input i of the whole vector in that staging.
template <int BITS>
constexpr int f16_chunk_bytes() { return BITS == 4 ? kF16ChunkBytes : kF16Chunk16Bytes; }

template <int BITS>
__device__ __forceinline__ int f16_stage_offset(int i) {
    if constexpr (BITS == 4) return (i >> 5) * kF16ChunkBytes + f16_pair_offset(i & 31);
    else return (i >> 4) * kF16Chunk16Bytes + (i & 15) * 2;
}

typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

// The eight code pairs (2p, 2p + 1) of a 6- or 8-bit chunk as fp16 pairs
// whose bit patterns are the codes themselves: an fp16 pattern q < 1024 is the
// subnormal q 2^-24, exact, so a packed fp16 dot of such a pair with two
// inputs is 2^-24 (q x + q' x') with exact products, and the 2^24 joins the
// scale.  8-bit: one byte permute per pair.  6-bit: the four codes of each
// 3-byte group lie in two 16-bit windows (bytes B0 B1 and B1 B2); a permute
// puts a window in both halves of a word, a packed 16-bit shift moves each
// half's code to bit 0 (shifts 0 and 6 in B0 B1, 4 and 10 in B1 B2) and a
// mask keeps 6 bits.
template <int BITS>
__device__ __forceinline__ void code_pairs16(const Chunk<BITS> &c, uint32_t (&q)[8]) {
    if constexpr (BITS == 8) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            q[2 * k] = __builtin_amdgcn_perm(0u, c.w[k], 0x04010400u);         // bytes 0, 1
            q[2 * k + 1] = __builtin_amdgcn_perm(0u, c.w[k], 0x04030402u);     // bytes 2, 3
        }
    } else {
        static_assert(BITS == 6, "code_pairs16 takes 6- or 8-bit chunks");
        // group g: bytes 3g .. 3g + 2 of the 12; perm(hi, lo, sel) picks bytes
        // 0-3 from lo and 4-7 from hi
        const uint32_t lo[4] = {c.w[0], c.w[0], c.w[1], c.w[2]};
        const uint32_t hi[4] = {c.w[0], c.w[1], c.w[2], c.w[2]};
        constexpr uint32_t b0[4] = {0, 3, 2, 1};           // selector of the group's first byte
        const u16x2_t sh01 = {0, 6}, sh23 = {4, 10};
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const uint32_t B0 = b0[g], B1 = b0[g] + 1, B2 = b0[g] + 2;
            const uint32_t t01 = __builtin_amdgcn_perm(hi[g], lo[g], B0 | B1 << 8 | B0 << 16 | B1 << 24);
            const uint32_t t23 = __builtin_amdgcn_perm(hi[g], lo[g], B1 | B2 << 8 | B1 << 16 | B2 << 24);
            q[2 * g] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2_t, t01) >> sh01) & 0x003F003Fu;
            q[2 * g + 1] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2_t, t23) >> sh23) & 0x003F003Fu;
        }
    }
}

// 6- or 8-bit codes against fp16 inputs staged in order (kF16Chunk16Bytes per
// chunk) with the packed fp16 dot instruction: the code pairs of
// code_pairs16, eight dots per row, the scale times 2^24 (exact).  ap: the
// chunk's 8 staged pairs; asum: their sum.
template <int BITS, int SB, int NM, int NR>
__device__ __forceinline__ void dot_block_f16x16(const BlockRegs<BITS, NM, NR> &R, const uint32_t *ap, float asum,
                                                 float (&acc)[NM][NR]) {
    float d[NM][NR];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int n = 0; n < NR; ++n) {
            uint32_t qp[8];
            code_pairs16<BITS>(R.w[m][n], qp);
            d[m][n] = 0.f;
#pragma unroll
            for (int p = 0; p < 8; ++p)
                d[m][n] = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, qp[p]), __builtin_bit_cast(f16x2_t, ap[p]),
                                                 d[m][n], false);
        }
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int n = 0; n < NR; ++n) {
            const float s = R.live[n] ? sb_to_float<SB>(R.sr[m][n]) * 16777216.0f : 0.f;
            const float b = R.live[n] ? sb_to_float<SB>(R.br[m][n]) : 0.f;
            acc[m][n] += s * d[m][n] + b * asum;
        }
}

// Input chunks staged raw in LDS: chunk c at byte c * xraw_stride (16 bytes of
// padding per chunk keep 16-byte reads of consecutive chunks by consecutive
// lanes free of bank conflicts).
template <int XT, int CODES>
constexpr int xraw_stride() {
    return XRaw<XT, CODES>::kVecs * 16 + 16;
}

// Copy the cpr chunks of x (16-byte aligned) into that layout, all threads of
// the block; the caller's next barrier makes them visible.
template <int XT, int CODES>
__device__ __forceinline__ void stage_x_raw(const void *x, int cpr, void *lds) {
    constexpr int V = XRaw<XT, CODES>::kVecs;
    const u32x4 *src = reinterpret_cast<const u32x4 *>(x);
    char *dst = reinterpret_cast<char *>(lds);
    for (int i = threadIdx.x; i < cpr * V; i += blockDim.x) {
        const int c = i / V, v = i - c * V;
        *reinterpret_cast<u32x4 *>(dst + c * xraw_stride<XT, CODES>() + v * 16) = src[i];
    }
}

template <int XT, int CODES>
__device__ __forceinline__ void read_x_raw(const void *lds, int c, XRaw<XT, CODES> &r) {
    const u32x4 *p =
        reinterpret_cast<const u32x4 *>(reinterpret_cast<const char *>(lds) + c * xraw_stride<XT, CODES>());
#pragma unroll
    for (int i = 0; i < XRaw<XT, CODES>::kVecs; ++i) r.v[i] = p[i];
}

template <int XT, int CODES>
__device__ __forceinline__ void load_x_chunk(const void *x, int64_t off, float *xv) {
    XRaw<XT, CODES> r;
    load_x_raw<XT, CODES>(x, off, r);
    convert_x<XT, CODES>(r, xv);
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
