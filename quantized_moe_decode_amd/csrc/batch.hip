// Small-batch decode (several tokens per step) with 4-bit weights: each work
// item is one expert and at most kBatchTok of its tokens (mlxcel PR #276, "What
// changed" step 2, applied to every token routed to the expert), so each
// touched expert's rows are streamed once per work item and applied to all
// of its tokens.
//
// A workgroup first stages its tokens' inputs in LDS, paired the way the
// packed dot instructions consume them (see dot_block_q4_bf16 and
// dot_block_q4_f16): record (t, c) holds chunk c of token t as 16 pairs,
// pair 4k + p = (v[8k+p], v[8k+p+4]), then the fp32 sum of the chunk.  The
// codes of a word are turned into a 16-bit pair once and multiplied into
// every token's accumulator:
//   kernel A: bf16 x, codes as bf16 128 + q, bias folded as b - 128 s;
//   kernel B: act rounded to fp16 after a power-of-two factor (2^8, or one
//             fitted to the token's vector if that would overflow fp16),
//             codes as fp16 1024 + q, bias folded as b - 1024 s, the token's
//             sums scaled back when stored.
#include <hip/hip_runtime.h>

#include "api.hpp"
#include "common.hpp"
#include "ffn.hpp"
#include "qgemv.hpp"

namespace moe {

constexpr int kRec = 80;         // bytes per staged chunk: 64 of pairs, the chunk sum, padding
constexpr int kRecSum = 64;
constexpr int kBatchThreads = kFfnThreads;

size_t batch_lds_bytes(int cols) { return (size_t)kBatchTok * (cols / 32) * kRec; }

// Pairs (v[8k+p], v[8k+p+4]) of 8 consecutive 16-bit inputs held as 4 words.
__device__ __forceinline__ u32x4 pair_words(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3) {
    u32x4 v;
    v[0] = __builtin_amdgcn_perm(w2, w0, 0x05040100u);
    v[1] = __builtin_amdgcn_perm(w2, w0, 0x07060302u);
    v[2] = __builtin_amdgcn_perm(w3, w1, 0x05040100u);
    v[3] = __builtin_amdgcn_perm(w3, w1, 0x07060302u);
    return v;
}

// Quad sum (lanes 4i..4i+3 end with the same value).
__device__ __forceinline__ float quad_sum(float v) {
    v += dpp_f<0xB1>(v);
    return v + dpp_f<0x4E>(v);
}

// Quad maximum of unsigned values (lanes 4i..4i+3 end with the same value).
__device__ __forceinline__ uint32_t quad_max_u(uint32_t x) {
    x = max(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xf, 0xf, false));
    return max(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xf, 0xf, false));
}

// Stage nt tokens' inputs.  Thread i handles token t, chunk c, word k (8
// inputs); the four k of a chunk are consecutive lanes.  Src(t, c, k, v)
// fills v with 4 pair words and returns the inputs' sum.
template <typename Src>
__device__ __forceinline__ void stage_pairs(char *lds, int nt, int cpr, Src src) {
    const int n = nt * cpr * 4;
    for (int i0 = 0; i0 < n; i0 += blockDim.x) {       // uniform trip count: the quad sum needs whole quads
        const int i = i0 + threadIdx.x;
        const bool ok = i < n;
        const int k = i & 3, tc = i >> 2;
        const int t = ok ? tc / cpr : 0, c = ok ? tc - t * cpr : 0;
        u32x4 v = {0u, 0u, 0u, 0u};
        float sum = 0.f;
        if (ok) sum = src(t, c, k, v);
        sum = quad_sum(sum);
        if (ok) {
            char *rec = lds + (t * cpr + c) * kRec;
            *reinterpret_cast<u32x4 *>(rec + k * 16) = v;
            if (k == 0) *reinterpret_cast<float *>(rec + kRecSum) = sum;
        }
    }
}

// Stage nt act vectors (fp32 [.., cpr*32]) as fp16 pairs; s_cs[t] gets the
// factor by which token t's dot products are to be multiplied.  Thread i
// handles act row t, chunk c, word k (8 values); the four k of a chunk are a
// quad.  The values are staged times kActF16Prescale (s_cs = its inverse)
// unless some value would overflow fp16 that way (one compare per value; the
// waves' ballots meet in LDS over a barrier): then each token's largest
// magnitude is found (LDS atomic maxima) and every token is staged again with
// the factor fitted to it (f16_stage_scale).  Ends with a workgroup barrier.
__device__ __forceinline__ void stage_act_f16(char *lds, int nt, int cpr, const Work &wk, const float *act,
                                              int d_ff, float *s_cs) {
    constexpr int kWaves = kBatchThreads / kWave;
    static_assert(kWaves == 4, "one flag word per wave, read as one 16-byte word");
    __shared__ __align__(16) uint32_t s_wave[kWaves];
    __shared__ uint32_t s_max[kBatchTok];
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
    const int n = nt * cpr * 4;
    auto load = [&](int i, float (&f)[8], int &t) {
        const int k = i & 3, tc = i >> 2;
        t = tc / cpr;
        const int c = tc - t * cpr;
        const f32x4 *src = reinterpret_cast<const f32x4 *>(act + (int64_t)pair_at(wk, t) * d_ff + c * 32 + k * 8);
        const f32x4 lo = src[0], hi = src[1];
        f[0] = lo.x; f[1] = lo.y; f[2] = lo.z; f[3] = lo.w;
        f[4] = hi.x; f[5] = hi.y; f[6] = hi.z; f[7] = hi.w;
    };
    // one pass: every value times its token's factor, rounded and placed;
    // returns whether any value of this thread reaches kActF16Overflow
    auto stage = [&](auto inv_of) {
        bool over = false;
        for (int i0 = 0; i0 < n; i0 += kBatchThreads) {       // uniform trip count: whole quads
            const int i = i0 + threadIdx.x;
            float f[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            int t = 0;
            if (i < n) load(i, f, t);
            const float inv = inv_of(t);
            uint32_t h[8];
            float sum = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                over |= !(__builtin_fabsf(f[e]) < kActF16Overflow);      // NaN counts as over
                const _Float16 q = (_Float16)(f[e] * inv);
                sum += (float)q;
                h[e] = __builtin_bit_cast(uint16_t, q);
            }
            sum = quad_sum(sum);
            if (i < n) {
                char *rec = lds + (i >> 2) * kRec;
                *reinterpret_cast<u32x4 *>(rec + (i & 3) * 16) =
                    pair_words(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
                if ((i & 3) == 0) *reinterpret_cast<float *>(rec + kRecSum) = sum;
            }
        }
        return over;
    };
    const bool over = stage([](int) { return kActF16Prescale; });
    const uint64_t b_over = __builtin_amdgcn_ballot_w64(over);
    if (lane == 0) s_wave[wave] = b_over ? 1u : 0u;
    if (threadIdx.x < kBatchTok) {
        s_cs[threadIdx.x] = kActF16Postscale;
        s_max[threadIdx.x] = 0;
    }
    __syncthreads();
    const u32x4 fl = *reinterpret_cast<const u32x4 *>(s_wave);
    if (!(fl.x | fl.y | fl.z | fl.w)) return;
    // a value past fp16's range at 2^8: per-token maxima, then all again, fitted
    for (int i = threadIdx.x; i < n; i += kBatchThreads) {
        float f[8];
        int t;
        load(i, f, t);
        uint32_t m = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) m = max(m, __float_as_uint(f[e]) & 0x7FFFFFFFu);
        atomicMax(&s_max[t], m);
    }
    __syncthreads();
    (void)stage([&](int t) {
        float inv;
        (void)f16_stage_scale(s_max[t], inv);
        return inv;
    });
    if (threadIdx.x < kBatchTok) {
        float inv;
        s_cs[threadIdx.x] = f16_stage_scale(s_max[threadIdx.x], inv);
    }
    __syncthreads();
}

// fn(tag) for a workgroup-uniform nt in 1..kBatchTok, with ::value = nt for
// nt <= 2 and 4 otherwise: the compute loops see a compile-time token count
// NT >= nt and run all NT tokens (tokens past nt compute on stale LDS and are
// never stored).  Three instantiations rather than four: with a three-token
// one as well, kernel A needs 139 VGPRs (three waves per SIMD) instead of
// 123 (four), and the 32-token step measured 3.6% slower; the one-token
// instantiation (a single pair per work item is the commonest case at 32
// tokens with top-8 of 128 experts) took that step 4.84 -> 4.73 ms together
// with kernel B's folded code offset.
template <int N>
struct TokC {
    static constexpr int value = N;
};
template <typename Fn>
__device__ __forceinline__ void with_tokens(int nt, Fn fn) {
    static_assert(kBatchTok == 4, "token dispatch covers 1..4");
    if (nt == 1) fn(TokC<1>{});
    else if (nt == 2) fn(TokC<2>{});
    else fn(TokC<4>{});
}

// Kernel A: gate and up projections of one work item over a tile of rows, then SwiGLU.
template <int SB>
__global__ __launch_bounds__(kBatchThreads) void gate_up_batch_q4(FfnArgs a) {
    constexpr int NR = kBatchNRA;
    extern __shared__ __align__(16) char lds[];
    Work wk;
    if (!get_work(a, blockIdx.y, wk)) return;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
    const int row0 = blockIdx.x * a.rows_per_wg;
    const int row_end = min(row0 + a.rows_per_wg, a.d_ff);
    const int nt = wk.npairs;
    if (wk.e < 0 || wk.e >= a.E) {
        for (int i = 0; i < nt; ++i) {
            const int64_t p = pair_at(wk, i);
            for (int r = row0 + tid; r < row_end; r += blockDim.x) a.act[p * a.d_ff + r] = 0.f;
        }
        return;
    }
    const int cpr = a.d_in / 32;
    const uint16_t *x = reinterpret_cast<const uint16_t *>(a.x);
    stage_pairs(lds, nt, cpr, [&](int t, int c, int k, u32x4 &v) {
        const int64_t tok = pair_at(wk, t) / a.K;
        const u32x4 w = *reinterpret_cast<const u32x4 *>(x + tok * a.d_in + c * 32 + k * 8);
        v = pair_words(w[0], w[1], w[2], w[3]);
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) s += __uint_as_float(w[i] << 16) + __uint_as_float(w[i] & 0xFFFF0000u);
        return s;
    });
    __syncthreads();

    const int lr = 1 << a.lr_shift, j = lane & (lr - 1), rsub = lane >> a.lr_shift, rpw = kWave >> a.lr_shift;
    const QM mats[2] = {a.gate, a.up};
    const int64_t erow0 = (int64_t)wk.e * a.d_ff;
    with_tokens(nt, [&](auto ntc) {
        constexpr int NT = decltype(ntc)::value;
        for (int rb = row0 + wave * rpw * NR; rb < row_end; rb += 4 * rpw * NR) {
            const int r0 = rb + rsub;
            float acc[2][NR][NT];
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int n = 0; n < NR; ++n)
#pragma unroll
                    for (int t = 0; t < NT; ++t) acc[m][n][t] = 0.f;
            for (int c0 = 0; c0 < cpr; c0 += lr) {
                BlockRegs<4, 2, NR> R;
                load_block<4, 2, NR>(R, mats, erow0, r0, rpw, row_end, c0 + j, cpr);
                float d[2][NR][NT];
#pragma unroll
                for (int m = 0; m < 2; ++m)
#pragma unroll
                    for (int n = 0; n < NR; ++n)
#pragma unroll
                        for (int t = 0; t < NT; ++t) d[m][n][t] = 0.f;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    uint32_t xk[NT][4];     // plain words: bit casts of vector elements are not used
#pragma unroll
                    for (int t = 0; t < NT; ++t) {
                        const u32x4 v = *reinterpret_cast<const u32x4 *>(lds + (t * cpr + R.cc) * kRec + k * 16);
#pragma unroll
                        for (int p = 0; p < 4; ++p) xk[t][p] = v[p];
                    }
#pragma unroll
                    for (int m = 0; m < 2; ++m)
#pragma unroll
                        for (int n = 0; n < NR; ++n) {
                            uint32_t qw[4];
                            nibble_pairs<0x43u>(R.w[m][n].w[k], qw);
#pragma unroll
                            for (int p = 0; p < 4; ++p) {
                                const bf16x2_t q = __builtin_bit_cast(bf16x2_t, qw[p]);
#pragma unroll
                                for (int t = 0; t < NT; ++t)
                                    d[m][n][t] = __builtin_amdgcn_fdot2_f32_bf16(
                                        q, __builtin_bit_cast(bf16x2_t, xk[t][p]), d[m][n][t], false);
                            }
                        }
                }
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    const float xsum = *reinterpret_cast<const float *>(lds + (t * cpr + R.cc) * kRec + kRecSum);
#pragma unroll
                    for (int m = 0; m < 2; ++m)
#pragma unroll
                        for (int n = 0; n < NR; ++n) {
                            const float s = R.live[n] ? sb_to_float<SB>(R.sr[m][n]) : 0.f;
                            const float b = R.live[n] ? sb_to_float<SB>(R.br[m][n]) : 0.f;
                            acc[m][n][t] += s * d[m][n][t] + (b - 128.0f * s) * xsum;
                        }
                }
            }
            with_width(a.lr_shift, [&](auto wd) {
                constexpr int W = decltype(wd)::value;
                if constexpr (W >= 16) {
                    // every (projection, row, token) sum of the lane group at once:
                    // value m * V/2 + n * NTP + t ends in the lanes of index
                    // (that value) << SH, where the gate sum (m = 0) meets the up
                    // sum from across the group's top lane bit
                    constexpr int NTP = NT == 3 ? 4 : NT;
                    constexpr int V = 2 * NR * NTP, SH = ilog2(W) - ilog2(V);
                    float sv[V];
#pragma unroll
                    for (int m = 0; m < 2; ++m)
#pragma unroll
                        for (int n = 0; n < NR; ++n)
#pragma unroll
                            for (int t = 0; t < NTP; ++t)
                                sv[m * (V / 2) + n * NTP + t] = t < NT ? acc[m][n][t] : 0.f;
                    group_multi_sum<W, V>(sv);
                    const float u = group_partner<W>(sv[0]);
                    const int li = lane & (W - 1), idx = li >> SH;
                    if ((li & ((1 << SH) - 1)) == 0 && idx < V / 2) {
                        const int n = idx / NTP, t = idx - n * NTP;
                        const int r = r0 + n * rpw;
                        const float g = sv[0];
                        if (t < nt && r < row_end) a.act[(int64_t)pair_at(wk, t) * a.d_ff + r] = g * sigmoidf_(g) * u;
                    }
                } else {
#pragma unroll
                    for (int m = 0; m < 2; ++m)
#pragma unroll
                        for (int n = 0; n < NR; ++n)
#pragma unroll
                            for (int t = 0; t < NT; ++t) acc[m][n][t] = group_sum_last<W>(acc[m][n][t]);
                    if (j == lr - 1) {
#pragma unroll
                        for (int n = 0; n < NR; ++n) {
                            const int r = r0 + n * rpw;
                            if (r < row_end) {
#pragma unroll
                                for (int t = 0; t < NT; ++t) {
                                    if (t >= nt) break;
                                    const float g = acc[0][n][t], u = acc[1][n][t];
                                    a.act[(int64_t)pair_at(wk, t) * a.d_ff + r] = g * sigmoidf_(g) * u;
                                }
                            }
                        }
                    }
                }
            });
        }
    });
}

// Kernel B: down projection of one work item over a tile of output rows, times each pair's score.
// Six workgroups per CU (at most 80 VGPRs; the compiler spills one
// loop-invariant value, reloaded once per row pass) measured faster than five
// without the spill.
template <int SB>
__global__ __launch_bounds__(kBatchThreads, 6) void down_batch_q4(FfnArgs a) {
    constexpr int NR = kBatchNRB;
    extern __shared__ __align__(16) char lds[];
    Work wk;
    if (!get_work(a, blockIdx.y, wk)) return;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
    const int row0 = blockIdx.x * a.rows_per_wg;
    const int row_end = min(row0 + a.rows_per_wg, a.d_in);
    const int nt = wk.npairs;
    if (wk.e < 0 || wk.e >= a.E) {
        for (int i = 0; i < nt; ++i) {
            const int64_t p = pair_at(wk, i);
            for (int r = row0 + tid; r < row_end; r += blockDim.x) a.partial[p * a.d_in + r] = 0.f;
        }
        return;
    }
    const int cpr = a.d_ff / 32;
    __shared__ float s_cs[kBatchTok];
    stage_act_f16(lds, nt, cpr, wk, a.act, a.d_ff, s_cs);

    const int lr = 1 << a.lr_shift, j = lane & (lr - 1), rsub = lane >> a.lr_shift, rpw = kWave >> a.lr_shift;
    const QM mats[1] = {a.down};
    const int64_t erow0 = (int64_t)wk.e * a.d_in;
    with_tokens(nt, [&](auto ntc) {
        constexpr int NT = decltype(ntc)::value;
        for (int rb = row0 + wave * rpw * NR; rb < row_end; rb += 4 * rpw * NR) {
            const int r0 = rb + rsub;
            float acc[NR][NT];
#pragma unroll
            for (int n = 0; n < NR; ++n)
#pragma unroll
                for (int t = 0; t < NT; ++t) acc[n][t] = 0.f;
            for (int c0 = 0; c0 < cpr; c0 += lr) {
                BlockRegs<4, 1, NR> R;
                load_block<4, 1, NR>(R, mats, erow0, r0, rpw, row_end, c0 + j, cpr);
                float d[NR][NT];
#pragma unroll
                for (int n = 0; n < NR; ++n)
#pragma unroll
                    for (int t = 0; t < NT; ++t) d[n][t] = 0.f;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    uint32_t xk[NT][4];     // plain words: bit casts of vector elements are not used
#pragma unroll
                    for (int t = 0; t < NT; ++t) {
                        const u32x4 v = *reinterpret_cast<const u32x4 *>(lds + (t * cpr + R.cc) * kRec + k * 16);
#pragma unroll
                        for (int p = 0; p < 4; ++p) xk[t][p] = v[p];
                    }
#pragma unroll
                    for (int n = 0; n < NR; ++n) {
                        uint32_t qw[4];
                        nibble_pairs<0x64u>(R.w[0][n].w[k], qw);
#pragma unroll
                        for (int p = 0; p < 4; ++p) {
                            const f16x2_t q = __builtin_bit_cast(f16x2_t, qw[p]);      // 1024 + q
#pragma unroll
                            for (int t = 0; t < NT; ++t)
                                d[n][t] = __builtin_amdgcn_fdot2(q, __builtin_bit_cast(f16x2_t, xk[t][p]), d[n][t],
                                                                 false);
                        }
                    }
                }
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    const float asum = *reinterpret_cast<const float *>(lds + (t * cpr + R.cc) * kRec + kRecSum);
#pragma unroll
                    for (int n = 0; n < NR; ++n) {
                        const float s = R.live[n] ? sb_to_float<SB>(R.sr[0][n]) : 0.f;
                        const float b = R.live[n] ? sb_to_float<SB>(R.br[0][n]) : 0.f;
                        acc[n][t] += s * d[n][t] + (b - 1024.0f * s) * asum;
                    }
                }
            }
            with_width(a.lr_shift, [&](auto wd) {
                constexpr int W = decltype(wd)::value;
                if constexpr (W >= 16) {
                    // every (row, token) sum of the lane group at once: value
                    // n * NTP + t ends in the lanes of index (that value) << SH
                    constexpr int NTP = NT == 3 ? 4 : NT;
                    constexpr int V = NR * NTP, SH = ilog2(W) - ilog2(V);
                    float sv[V];
#pragma unroll
                    for (int n = 0; n < NR; ++n)
#pragma unroll
                        for (int t = 0; t < NTP; ++t) sv[n * NTP + t] = t < NT ? acc[n][t] : 0.f;
                    group_multi_sum<W, V>(sv);
                    const int li = lane & (W - 1), idx = li >> SH;
                    if ((li & ((1 << SH) - 1)) == 0) {
                        const int n = idx / NTP, t = idx - n * NTP;
                        const int r = r0 + n * rpw;
                        if (t < nt && r < row_end) {
                            const int64_t p = pair_at(wk, t);
                            const float sc = (a.scores ? a.scores[p] : 1.0f) * s_cs[t];   // exact: a power of two
                            a.partial[p * a.d_in + r] = sc * sv[0];
                        }
                    }
                } else {
#pragma unroll
                    for (int n = 0; n < NR; ++n)
#pragma unroll
                        for (int t = 0; t < NT; ++t) acc[n][t] = group_sum_last<W>(acc[n][t]);
                    if (j == lr - 1) {
#pragma unroll
                        for (int n = 0; n < NR; ++n) {
                            const int r = r0 + n * rpw;
                            if (r < row_end) {
#pragma unroll
                                for (int t = 0; t < NT; ++t) {
                                    if (t >= nt) break;
                                    const int64_t p = pair_at(wk, t);
                                    const float sc = (a.scores ? a.scores[p] : 1.0f) * s_cs[t];
                                    a.partial[p * a.d_in + r] = sc * acc[n][t];
                                }
                            }
                        }
                    }
                }
            });
        }
    });
}

KernelFn batch_gate_up_q4(int sb) {
    return sb == MOE_BF16 ? gate_up_batch_q4<MOE_BF16> : sb == MOE_F16 ? gate_up_batch_q4<MOE_F16> : nullptr;
}

KernelFn batch_down_q4(int sb) {
    return sb == MOE_BF16 ? down_batch_q4<MOE_BF16> : sb == MOE_F16 ? down_batch_q4<MOE_F16> : nullptr;
}

}  // namespace moe
