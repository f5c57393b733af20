// Expert FFN of the MoE decode layer on gfx950.
//
// The two-kernel split of mlxcel PR #276 ("What changed", step 2):
//   kernel A (gate_up_kernel): act[t][k][r] = silu(W_gate[e] x_t)_r * (W_up[e] x_t)_r
//   kernel B (down_kernel):    partial[t][k][i] = score[t][k] * (W_down[e] act[t][k])_i
// Every output row is independent work, so the grid spans (row tiles x
// selected experts) and fills the whole GPU; each weight byte is read once
// per step.
//
// Mapping on a 64-wide wavefront: a row is handled by LR lanes (a power of
// two chosen on the host from the row length); a wave processes 64/LR rows
// at once.  Lane j of a row reads chunks j, j+LR, j+2LR, ... of that row
// (16-byte loads for 4/8-bit, 12-byte loads for 6-bit) so that the LR lanes
// of a row read contiguous memory.  The codes of a chunk are unpacked in
// registers; the chunk's contribution is factored per quantization group:
//   sum_i (s q_i + b) x_i = s * sum_i q_i x_i + b * sum_i x_i
// with the per-chunk input sums precomputed once per workgroup in LDS.  The
// LR partial sums of a row are combined with a butterfly over lanes.
//
// Input vectors (x for kernel A, act for kernel B) are staged in LDS as fp32.
// With several tokens per expert (small-batch decode), an expert's weight
// chunk is unpacked once and applied to all of its tokens (up to MAXT per
// LDS pass), so each touched expert's weights are read once per step.
#include <hip/hip_runtime.h>

#include <mutex>

#include "api.hpp"
#include "common.hpp"
#include "qgemv.hpp"
#include "ffn.hpp"

namespace moe {

// Dot products of kNR rows (r0, r0+rstep, ...) of NM matrices of the expert
// whose first row is erow0, accumulated per lane (the caller combines the
// row's LR lanes).  MAXT == 1 reads the single token's input chunk from
// global memory (x_src, dtype XT); MAXT > 1 reads the staged LDS copy.
template <int BITS, int SB, int XT, int NM, int MAXT>
__device__ __forceinline__ void row_block(const QM *mats, int64_t erow0, int r0, int rstep, int row_end,
                                          int j, int lr, int cpr, const void *x_src, int64_t x_off,
                                          const float *xs, int nt, float (&acc)[NM][kNR][MAXT]) {
    constexpr int CODES = Fmt<BITS>::kCodes;
    float a1[NM][kNR];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int n = 0; n < kNR; ++n) {
            a1[m][n] = 0.f;
#pragma unroll
            for (int t = 0; t < MAXT; ++t) acc[m][n][t] = 0.f;
        }
    for (int c0 = 0; c0 < cpr; c0 += lr) {          // same trip count on every lane
        BlockRegs<BITS, NM, kNR> R;
        load_block<BITS, NM, kNR>(R, mats, erow0, r0, rstep, row_end, c0 + j, cpr);
        if constexpr (MAXT == 1 && BITS == 4 && XT == MOE_BF16) {
            // raw bf16 inputs for the packed bf16 dot (exact products)
            XRaw<XT, CODES> xr;
            load_x_raw<XT, CODES>(x_src, x_off + (int64_t)R.cc * CODES, xr);
            uint32_t xw[16];
            float xsum = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const uint32_t v = xr.v[i][k];
                    xw[4 * i + k] = v;
                    xsum += __uint_as_float(v << 16) + __uint_as_float(v & 0xFFFF0000u);
                }
            dot_block_q4_bf16<SB, NM, kNR>(R, xw, xsum, a1);
        } else if constexpr (MAXT == 1) {
            float xv[CODES];
            load_x_chunk<XT, CODES>(x_src, x_off + (int64_t)R.cc * CODES, xv);
            dot_block<BITS, SB, NM, kNR>(R, xv, sum_n<CODES>(xv), a1);
        } else {
#pragma unroll
            for (int t = 0; t < MAXT; ++t) {
                if (t < nt) {
                    const float *p = staged_chunk<CODES>(xs, t, cpr, R.cc);
                    float xv[CODES];
                    read_staged<CODES>(p, xv);
                    float part[NM][kNR];
#pragma unroll
                    for (int m = 0; m < NM; ++m)
#pragma unroll
                        for (int n = 0; n < kNR; ++n) part[m][n] = 0.f;
                    dot_block<BITS, SB, NM, kNR>(R, xv, p[CODES], part);
#pragma unroll
                    for (int m = 0; m < NM; ++m)
#pragma unroll
                        for (int n = 0; n < kNR; ++n) acc[m][n][t] += part[m][n];
                }
            }
        }
    }
    if constexpr (MAXT == 1) {
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int n = 0; n < kNR; ++n) acc[m][n][0] = a1[m][n];
    }
}

// Kernel A: gate and up projections of one expert over a tile of rows, then SwiGLU.
template <int BITS, int SB, int XT, int MAXT>
__global__ __launch_bounds__(256) void gate_up_kernel(FfnArgs a) {
    using F = Fmt<BITS>;
    extern __shared__ float lds[];
    Work wk;
    if (!get_work(a, blockIdx.y, wk)) return;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
    const int row0 = blockIdx.x * a.rows_per_wg;
    const int row_end = min(row0 + a.rows_per_wg, a.d_ff);
    if (wk.e < 0 || wk.e >= a.E) {
        for (int i = 0; i < wk.npairs; ++i) {
            const int64_t p = pair_at(wk, i);
            for (int r = row0 + tid; r < row_end; r += blockDim.x) a.act[p * a.d_ff + r] = 0.f;
        }
        return;
    }
    const int cpr = a.d_in / F::kCodes;
    const int lr = 1 << a.lr_shift, j = lane & (lr - 1), rsub = lane >> a.lr_shift, rpw = kWave >> a.lr_shift;
    const QM mats[2] = {a.gate, a.up};
    const int64_t erow0 = (int64_t)wk.e * a.d_ff;

    for (int pb = 0; pb < wk.npairs; pb += a.tpp) {
        const int nt = min(a.tpp, wk.npairs - pb);
        int64_t x_off = 0;
        if constexpr (MAXT == 1) {
            x_off = (int64_t)(pair_at(wk, pb) / a.K) * a.d_in;
        } else {
            __syncthreads();
            stage_inputs<F::kCodes>(lds, nt, cpr, [&](int tt, int c) {
                const int64_t tok = pair_at(wk, pb + tt) / a.K;
                return load_act(a.x, a.x_dt, tok * a.d_in + c);
            });
        }
        for (int rb = row0 + wave * rpw * kNR; rb < row_end; rb += 4 * rpw * kNR) {
            const int r0 = rb + rsub;
            float acc[2][kNR][MAXT];
            row_block<BITS, SB, XT, 2, MAXT>(mats, erow0, r0, rpw, row_end, j, lr, cpr, a.x, x_off, lds, nt, acc);
            with_width(__builtin_ctz(lr), [&](auto w) {
#pragma unroll
                for (int n = 0; n < kNR; ++n)
#pragma unroll
                    for (int t = 0; t < MAXT; ++t) {
                        acc[0][n][t] = group_sum_last<decltype(w)::value>(acc[0][n][t]);
                        acc[1][n][t] = group_sum_last<decltype(w)::value>(acc[1][n][t]);
                    }
            });
            if (j == lr - 1) {
#pragma unroll
                for (int n = 0; n < kNR; ++n) {
                    const int r = r0 + n * rpw;
                    if (r < row_end) {
#pragma unroll
                        for (int t = 0; t < MAXT; ++t)
                            if (t < nt) {
                                const float g = acc[0][n][t], u = acc[1][n][t];
                                a.act[(int64_t)pair_at(wk, pb + t) * a.d_ff + r] = g * sigmoidf_(g) * u;
                            }
                    }
                }
            }
        }
    }
}

// Kernel B: down projection of one expert over a tile of output rows, times the score.
template <int BITS, int SB, int MAXT>
__global__ __launch_bounds__(256) void down_kernel(FfnArgs a) {
    using F = Fmt<BITS>;
    extern __shared__ float lds[];
    Work wk;
    if (!get_work(a, blockIdx.y, wk)) return;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
    const int row0 = blockIdx.x * a.rows_per_wg;
    const int row_end = min(row0 + a.rows_per_wg, a.d_in);
    if (wk.e < 0 || wk.e >= a.E) {
        for (int i = 0; i < wk.npairs; ++i) {
            const int64_t p = pair_at(wk, i);
            for (int r = row0 + tid; r < row_end; r += blockDim.x) a.partial[p * a.d_in + r] = 0.f;
        }
        return;
    }
    const int cpr = a.d_ff / F::kCodes;
    const int lr = 1 << a.lr_shift, j = lane & (lr - 1), rsub = lane >> a.lr_shift, rpw = kWave >> a.lr_shift;
    const QM mats[1] = {a.down};
    const int64_t erow0 = (int64_t)wk.e * a.d_in;

    for (int pb = 0; pb < wk.npairs; pb += a.tpp) {
        const int nt = min(a.tpp, wk.npairs - pb);
        int64_t x_off = 0;
        if constexpr (MAXT == 1) {
            x_off = (int64_t)pair_at(wk, pb) * a.d_ff;
        } else {
            __syncthreads();
            stage_inputs<F::kCodes>(lds, nt, cpr, [&](int tt, int c) {
                return a.act[(int64_t)pair_at(wk, pb + tt) * a.d_ff + c];
            });
        }
        for (int rb = row0 + wave * rpw * kNR; rb < row_end; rb += 4 * rpw * kNR) {
            const int r0 = rb + rsub;
            float acc[1][kNR][MAXT];
            row_block<BITS, SB, MOE_F32, 1, MAXT>(mats, erow0, r0, rpw, row_end, j, lr, cpr, a.act, x_off, lds, nt, acc);
            with_width(__builtin_ctz(lr), [&](auto w) {
#pragma unroll
                for (int n = 0; n < kNR; ++n)
#pragma unroll
                    for (int t = 0; t < MAXT; ++t) acc[0][n][t] = group_sum_last<decltype(w)::value>(acc[0][n][t]);
            });
            if (j == lr - 1) {
#pragma unroll
                for (int n = 0; n < kNR; ++n) {
                    const int r = r0 + n * rpw;
                    if (r < row_end) {
#pragma unroll
                        for (int t = 0; t < MAXT; ++t)
                            if (t < nt) {
                                const int64_t p = pair_at(wk, pb + t);
                                const float sc = a.scores ? a.scores[p] : 1.0f;
                                a.partial[p * a.d_in + r] = sc * acc[0][n][t];
                            }
                    }
                }
            }
        }
    }
}

// Kernel B for one token with the packed fp16 dots (the arithmetic of the
// fused layer's kernel-B units): the workgroup issues the loads of its first
// block of weights, stages its slot's act row in LDS as fp16 in the layout
// the dots read (f16_stage_offset), each value times 2^8 (exact; the inverse
// joins the score), and if some value would overflow fp16 that way (one
// compare per value, flags exchanged over the staging's barrier) stages it
// again with the power of two fitted to the row's largest magnitude
// (f16_stage_scale).  Then it streams its rows: 4-bit codes through
// dot_block_q4_f16, 6- and 8-bit codes through dot_block_f16x16.
template <int BITS, int SB>
__global__ __launch_bounds__(kFfnThreads) void down_kernel_t1(FfnArgs a) {
    using F = Fmt<BITS>;
    constexpr int CODES = F::kCodes, NP = CODES / 2;
    constexpr int kWaves = kFfnThreads / kWave;
    static_assert(kWaves == 4, "one flag word per wave, read as one 16-byte word");
    extern __shared__ __align__(16) char lds_h[];
    __shared__ __align__(16) uint32_t s_wave[2][kWaves];      // per wave: overflow flag, largest magnitude
    const int k = blockIdx.y;
    const int e = a.ids[k];
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
    const int row0 = blockIdx.x * a.rows_per_wg;
    const int row_end = min(row0 + a.rows_per_wg, a.d_in);
    float *part = a.partial + (int64_t)k * a.d_in;
    if (e < 0 || e >= a.E) {
        for (int r = row0 + tid; r < row_end; r += kFfnThreads) part[r] = 0.f;
        return;
    }
    const float *act = a.act + (int64_t)k * a.d_ff;
    const int n = a.d_ff;
    const int cpr = n / CODES;
    const int lr = 1 << a.lr_shift, j = lane & (lr - 1), rsub = lane >> a.lr_shift, rpw = kWave >> a.lr_shift;
    const QM mats[1] = {a.down};
    const int64_t erow0 = (int64_t)e * a.d_in;
    const int rb_first = row0 + wave * rpw * kNR, rb_step = 4 * rpw * kNR;
    // the first block's weights are on their way while act is staged
    BlockRegs<BITS, 1, kNR> R;
    if (rb_first < row_end) load_block<BITS, 1, kNR>(R, mats, erow0, rb_first + rsub, rpw, row_end, j, cpr);
    auto place = [&](int i, float v) { *reinterpret_cast<_Float16 *>(lds_h + f16_stage_offset<BITS>(i)) = (_Float16)v; };
    // fn(i, act[i]) for every i: 16-byte loads of four values (n is a multiple
    // of 64), eight per thread in flight at a time
    auto each_act = [&](auto fn) __attribute__((always_inline)) {
        constexpr int kPer = 8;
        const f32x4 *act4 = reinterpret_cast<const f32x4 *>(act);
        const int n4 = n / 4;
        for (int base = 0; base < n4; base += kPer * kFfnThreads) {
            f32x4 v[kPer];
#pragma unroll
            for (int u = 0; u < kPer; ++u) {
                const int i = base + u * kFfnThreads + tid;
                v[u] = i < n4 ? act4[i] : f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int u = 0; u < kPer; ++u) {
                const int i = base + u * kFfnThreads + tid;
                if (i < n4) {
                    fn(4 * i, v[u].x);
                    fn(4 * i + 1, v[u].y);
                    fn(4 * i + 2, v[u].z);
                    fn(4 * i + 3, v[u].w);
                }
            }
        }
    };
    bool over = false;
    each_act([&](int i, float v) {
        over |= !(__builtin_fabsf(v) < kActF16Overflow);      // NaN counts as over
        place(i, v * kActF16Prescale);
    });
    if (lane == 0) s_wave[0][wave] = __ballot(over) ? 1u : 0u;
    __syncthreads();
    float cs = kActF16Postscale;
    const u32x4 f = *reinterpret_cast<const u32x4 *>(s_wave[0]);
    if (f.x | f.y | f.z | f.w) {
        uint32_t mx = 0;                 // magnitudes order like their bit patterns
        each_act([&](int, float v) { mx = max(mx, __float_as_uint(v) & 0x7FFFFFFFu); });
        const float wm = wave_max(__uint_as_float(mx));
        if (lane == 0) s_wave[1][wave] = __float_as_uint(wm);
        __syncthreads();
        uint32_t m = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) m = max(m, s_wave[1][w]);
        float inv;
        cs = f16_stage_scale(m, inv);
        each_act([&](int i, float v) { place(i, v * inv); });
        __syncthreads();
    }
    const float sc = (a.scores ? a.scores[k] : 1.0f) * cs;      // exact: cs is a power of two
    for (int rb = rb_first; rb < row_end; rb += rb_step) {
        const int r0 = rb + rsub;
        float acc[1][kNR];
#pragma unroll
        for (int r = 0; r < kNR; ++r) acc[0][r] = 0.f;
        for (int c0 = 0; c0 < cpr; c0 += lr) {          // same trip count on every lane
            if (rb != rb_first || c0 != 0) load_block<BITS, 1, kNR>(R, mats, erow0, r0, rpw, row_end, c0 + j, cpr);
            const u32x4 *src = reinterpret_cast<const u32x4 *>(lds_h + R.cc * f16_chunk_bytes<BITS>());
            uint32_t ap[NP];
#pragma unroll
            for (int i = 0; i < NP / 4; ++i) {
                const u32x4 v = src[i];
#pragma unroll
                for (int q = 0; q < 4; ++q) ap[4 * i + q] = v[q];
            }
            if constexpr (BITS == 4) dot_block_q4_f16<SB, 1, kNR>(R, ap, f16_pairs_sum<NP>(ap), acc);
            else dot_block_f16x16<BITS, SB, 1, kNR>(R, ap, f16_pairs_sum<NP>(ap), acc);
        }
        with_width(__builtin_ctz(lr), [&](auto w) {
#pragma unroll
            for (int r = 0; r < kNR; ++r) acc[0][r] = group_sum_last<decltype(w)::value>(acc[0][r]);
        });
        if (j == lr - 1) {
#pragma unroll
            for (int r = 0; r < kNR; ++r) {
                const int row = r0 + r * rpw;
                if (row < row_end) part[row] = sc * acc[0][r];
            }
        }
    }
}

// Small-batch bucketing: groups the (token, slot) pairs by expert with a
// stable counting sort (pairs stay in ascending t*K + k order inside an
// expert) and cuts each expert's list into work items of at most max_tok
// pairs.  Work items list the touched experts in ascending id order, then
// the items (expert -1) collecting every out-of-range id.  One workgroup:
// histogram by LDS atomics, a block scan, and each pair's rank among the
// earlier pairs of its bucket.  A token selects an expert at most once, so
// for in-range buckets that rank is the number of earlier tokens in the
// bucket's token mask; ids that repeat within a token, and the out-of-range
// bucket, take the direct count instead.
constexpr int kBucketThreads = 256;
constexpr int kScanMax = MOE_MAX_EXPERTS + 2;   // bucket entries (E + 1 buckets and the total)

// Exclusive prefix sums of a[0..n) and b[0..n) together, in place; a[n] and
// b[n] receive the totals.  Thread t owns a run of consecutive entries: the
// runs' sums are scanned across each wave with lane shuffles and across the
// waves through LDS, then every thread rewrites its own run, so the whole
// scan takes two barriers.  All threads of the block call it.
__device__ void block_exclusive_scan2(int *a, int *b, int n) {
    __shared__ int wsum_a[kBucketThreads / kWave], wsum_b[kBucketThreads / kWave];
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave, nw = blockDim.x / kWave;
    const int per = (n + blockDim.x - 1) / blockDim.x;
    const int i0 = min(tid * per, n), i1 = min(i0 + per, n);
    int ra = 0, rb = 0;
    for (int i = i0; i < i1; ++i) {
        ra += a[i];
        rb += b[i];
    }
    int xa = ra, xb = rb;     // inclusive scan of the run sums over the wave
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int ya = __shfl_up(xa, d), yb = __shfl_up(xb, d);
        if (lane >= d) {
            xa += ya;
            xb += yb;
        }
    }
    if (lane == kWave - 1) {
        wsum_a[wave] = xa;
        wsum_b[wave] = xb;
    }
    __syncthreads();
    int pa = xa - ra, pb = xb - rb, ta = 0, tb = 0;
    for (int w = 0; w < nw; ++w) {
        if (w < wave) {
            pa += wsum_a[w];
            pb += wsum_b[w];
        }
        ta += wsum_a[w];
        tb += wsum_b[w];
    }
    for (int i = i0; i < i1; ++i) {
        const int va = a[i], vb = b[i];
        a[i] = pa;
        b[i] = pb;
        pa += va;
        pb += vb;
    }
    if (tid == 0) {
        a[n] = ta;
        b[n] = tb;
    }
    __syncthreads();
}

__global__ __launch_bounds__(kBucketThreads) void bucket_kernel(const int32_t *ids, int n_pairs, int top_k, int E,
                                                                int max_tok, int32_t *work_expert,
                                                                int32_t *work_begin, int32_t *pair_list,
                                                                int32_t *n_work) {
    __shared__ int off[kScanMax];       // pairs, then first pair, per bucket (bucket E: out-of-range ids)
    __shared__ int ioff[kScanMax];      // work items, then first work item, per bucket
    __shared__ int cnt[MOE_MAX_EXPERTS + 1];
    __shared__ uint32_t tmask[MOE_MAX_EXPERTS + 1];     // tokens with a pair in the bucket
    __shared__ __align__(16) int bucket[MOE_MAX_TOKENS * MOE_MAX_TOP_K];
    __shared__ int s_repeat;
    static_assert(MOE_MAX_TOKENS <= 32, "one mask bit per token");
    const int tid = threadIdx.x, nb = E + 1;
    for (int i = tid; i < nb; i += blockDim.x) {
        cnt[i] = 0;
        tmask[i] = 0;
    }
    if (tid == 0) s_repeat = 0;
    __syncthreads();
    for (int p = tid; p < n_pairs; p += blockDim.x) {
        const int e = ids[p];
        const int b = (e >= 0 && e < E) ? e : E;
        bucket[p] = b;
        atomicAdd(&cnt[b], 1);
        if (b < E) {
            const uint32_t bit = 1u << (p / top_k);
            if (atomicOr(&tmask[b], bit) & bit) s_repeat = 1;
        }
    }
    __syncthreads();
    for (int i = tid; i < nb; i += blockDim.x) {
        off[i] = cnt[i];
        ioff[i] = (cnt[i] + max_tok - 1) / max_tok;
    }
    __syncthreads();
    block_exclusive_scan2(off, ioff, nb);    // off[nb] = n_pairs, ioff[nb] = work items
    // a pair's rank among the earlier pairs of its bucket
    const int4 *b4 = reinterpret_cast<const int4 *>(bucket);
    const bool repeat = s_repeat != 0;
    for (int p = tid; p < n_pairs; p += blockDim.x) {
        const int b = bucket[p];
        int r = 0;
        if (b < E && !repeat) {
            r = __popc(tmask[b] & ((1u << (p / top_k)) - 1u));
        } else {    // direct count, 16-byte LDS reads
            int q = 0;
            for (; q + 4 <= p; q += 4) {
                const int4 v = b4[q >> 2];
                r += (v.x == b ? 1 : 0) + (v.y == b ? 1 : 0) + (v.z == b ? 1 : 0) + (v.w == b ? 1 : 0);
            }
            for (; q < p; ++q) r += bucket[q] == b ? 1 : 0;
        }
        pair_list[off[b] + r] = p;
    }
    for (int b = tid; b < nb; b += blockDim.x) {
        const int items = ioff[b + 1] - ioff[b];
        for (int i = 0; i < items; ++i) {
            work_expert[ioff[b] + i] = b < E ? b : -1;
            work_begin[ioff[b] + i] = off[b] + i * max_tok;
        }
    }
    if (tid == 0) {
        work_begin[ioff[nb]] = n_pairs;
        *n_work = ioff[nb];
    }
}

// ------------------------------------------------------------------ host side

// Kernel A instantiations: bits x scale dtype x (single-token input dtype, or
// staged multi-token inputs).
template <int BITS, int SB>
static KernelFn pick_gate_up(int x_dt, bool multi) {
    if (multi) return gate_up_kernel<BITS, SB, -1, 8>;
    switch (x_dt) {
    case MOE_F32: return gate_up_kernel<BITS, SB, MOE_F32, 1>;
    case MOE_F16: return gate_up_kernel<BITS, SB, MOE_F16, 1>;
    default: return gate_up_kernel<BITS, SB, MOE_BF16, 1>;
    }
}

template <int BITS, int SB>
static KernelFn pick_down(bool multi) {
    return multi ? down_kernel<BITS, SB, 8> : down_kernel_t1<BITS, SB>;
}

static KernelFn select_gate_up(int bits, int sb, int x_dt, bool multi) {
#define MOE_PICK(B, S) if (bits == B && sb == S) return pick_gate_up<B, S>(x_dt, multi);
    MOE_PICK(4, MOE_BF16) MOE_PICK(4, MOE_F16)
    MOE_PICK(6, MOE_BF16) MOE_PICK(6, MOE_F16)
    MOE_PICK(8, MOE_BF16) MOE_PICK(8, MOE_F16)
#undef MOE_PICK
    return nullptr;
}

static KernelFn select_down(int bits, int sb, bool multi) {
#define MOE_PICK(B, S) if (bits == B && sb == S) return pick_down<B, S>(multi);
    MOE_PICK(4, MOE_BF16) MOE_PICK(4, MOE_F16)
    MOE_PICK(6, MOE_BF16) MOE_PICK(6, MOE_F16)
    MOE_PICK(8, MOE_BF16) MOE_PICK(8, MOE_F16)
#undef MOE_PICK
    return nullptr;
}

static int codes_per_chunk(int bits) { return bits == 4 ? 32 : 16; }

// Lanes per row: the chunk count rounded up to a power of two, at most 64
// (lanes past the row's last chunk stay idle; longer rows loop).
static int pick_lr_shift(int cpr) {
    int s = 0;
    while (s < 6 && (1 << s) < cpr) ++s;
    return s;
}

static QM to_qm(const moe_qmat *m) {
    QM q;
    q.q = m->q;
    q.s = reinterpret_cast<const uint16_t *>(m->scales);
    q.b = reinterpret_cast<const uint16_t *>(m->biases);
    q.rows = m->rows;
    q.cols = m->cols;
    q.wpr = m->cols * m->bits / 32;
    q.gpr = m->cols / 64;
    q.bits_ = m->bits;
    q.sb_ = raw_enum(m->sb_dtype);
    return q;
}

static constexpr size_t kLdsBudget = 64 * 1024;

// Work items after bucketing: at most ceil(n/kBatchTok) + (non-empty buckets).
static int max_work_items(int T, int K, int E) {
    const int n = T * K;
    const int buckets = n < E + 1 ? n : E + 1;
    return (n + kBatchTok - 1) / kBatchTok + buckets;
}

}  // namespace moe

using namespace moe;

extern "C" size_t moe_decode_expert_ffn_workspace_bytes(int32_t n_tokens, int32_t top_k, int32_t n_experts) {
    if (n_tokens <= 1 || top_k < 1 || n_experts < 1) return 0;
    const size_t mw = (size_t)max_work_items(n_tokens, top_k, n_experts);
    return align_up((1 + mw + (mw + 1) + (size_t)n_tokens * top_k) * sizeof(int32_t), 256);
}

namespace moe {

// Validated launch state shared by the three entry points.
struct Plan {
    FfnArgs a;
    hipStream_t s;
    int n_items;
    int maxt;
};

static moe_status check_tokens(const void *x, int n_tokens, int top_k) {
    if (!x) return MOE_EINVAL;
    if (n_tokens < 1 || n_tokens > MOE_MAX_TOKENS) return MOE_EINVAL;
    if (top_k < 1 || top_k > MOE_MAX_TOP_K) return MOE_EINVAL;
    if (!aligned16(x)) return MOE_EINVAL;
    return MOE_OK;
}

static moe_status plan_common(Plan &p, int n_tokens, int top_k, int E, const int32_t *ids,
                              void *workspace, size_t workspace_bytes, void *stream) {
    if (!ids) return MOE_EINVAL;
    const bool multi = n_tokens > 1;
    if (multi && (!workspace ||
                  workspace_bytes < moe_decode_expert_ffn_workspace_bytes(n_tokens, top_k, E)))
        return MOE_EINVAL;
    p.s = reinterpret_cast<hipStream_t>(stream);
    p.maxt = multi ? 8 : 1;
    p.a.T = n_tokens;
    p.a.K = top_k;
    p.a.E = E;
    p.a.ids = ids;
    p.n_items = top_k;
    if (multi) {
        const int mw = max_work_items(n_tokens, top_k, E);
        int32_t *ws = reinterpret_cast<int32_t *>(workspace);
        p.a.n_work = ws;
        p.a.work_expert = ws + 1;
        p.a.work_begin = ws + 1 + mw;
        p.a.pair_list = ws + 1 + mw + mw + 1;
        p.n_items = mw;
    }
    return MOE_OK;
}

static void launch_bucket(const Plan &p) {
    if (!p.a.pair_list) return;
    hipLaunchKernelGGL(bucket_kernel, dim3(1), dim3(kBucketThreads), 0, p.s, p.a.ids, p.a.T * p.a.K, p.a.K, p.a.E,
                       kBatchTok, const_cast<int32_t *>(p.a.work_expert), const_cast<int32_t *>(p.a.work_begin),
                       const_cast<int32_t *>(p.a.pair_list), const_cast<int32_t *>(p.a.n_work));
}

// Kernel launch geometry for a projection with `cols` inputs of `bits` bits.
static moe_status geometry(FfnArgs &a, int maxt, int cols, int bits, size_t &lds) {
    const int codes = codes_per_chunk(bits);
    const int cpr = cols / codes;
    a.lr_shift = pick_lr_shift(cpr);
    const int rpw = kWave >> a.lr_shift;
    a.rows_per_wg = 4 * rpw * kNR;
    if (maxt == 1) {
        a.tpp = 1;
        lds = 0;
        return MOE_OK;
    }
    const size_t per_tok = (size_t)cpr * (codes + 4) * sizeof(float);
    const int fit = (int)(kLdsBudget / per_tok);
    a.tpp = fit < maxt ? fit : maxt;
    if (a.tpp < 1) return MOE_EUNSUPPORTED;
    lds = a.tpp * per_tok;
    return MOE_OK;
}

// Lanes per row for the multi-token kernels: the largest power of two (8 to
// 64) that still gives every lane at least four chunks of a row per pass, so
// the cross-lane sums at the end of a pass (2 x rows x tokens values per
// lane group) are spread over enough codes; 8 when rows are shorter.  The
// kernels are VALU-bound at these sizes, and with 64 lanes on a 2048-input
// row (one chunk per lane, then a 64-lane reduction) the sums took about as
// many instructions as the dot products.  Measured on the 32-token
// Qwen3-shaped expert call (gate/up at 2048 inputs, one pass): 8 / 16 / 32
// / 64 lanes 99.6 / 92.4 / 96.3 / 101.3 us; down (768 inputs) keeps 8.
static int pick_lr_shift_batch(int cpr) {
    int s = 3;
    while (s < 6 && (cpr >> (s + 1)) >= 4) ++s;
    return s;
}

// The 4-bit multi-token kernels (batch.hip), when their LDS fits; rows_per_wg
// covers `passes` row passes of a workgroup.  More passes amortise a
// workgroup's staging of its tokens' inputs, but with 16 lanes per row one
// pass of gate/up is already 32 rows (2 passes measured 3% slower on the
// 32-token Qwen3-shaped call); down (768 inputs: 8 lanes per row, 2 rows per
// lane group) is fastest with a single pass: its workgroups are small and
// many, six per CU.
constexpr int kBatchPassesA = 1;
constexpr int kBatchPassesB = 1;
static KernelFn batch_geometry(FfnArgs &a, int cols, int bits, int nr, int passes, KernelFn k, size_t &lds) {
    if (bits != 4 || !k) return nullptr;
    lds = batch_lds_bytes(cols);
    if (lds > kLdsBudget) return nullptr;
    a.lr_shift = pick_lr_shift_batch(cols / 32);
    a.rows_per_wg = passes * 4 * (kWave >> a.lr_shift) * nr;
    a.tpp = kBatchTok;
    return k;
}

static moe_status launch_a(Plan &p) {
    size_t lds = 0;
    KernelFn k = nullptr;
    if (p.maxt > 1 && p.a.x_dt == MOE_BF16)
        k = batch_geometry(p.a, p.a.d_in, p.a.gate.bits_, kBatchNRA, kBatchPassesA, batch_gate_up_q4(p.a.gate.sb_), lds);
    if (!k) {
        k = select_gate_up(p.a.gate.bits_, p.a.gate.sb_, p.a.x_dt, p.maxt > 1);
        if (!k) return MOE_EUNSUPPORTED;
        const moe_status st = geometry(p.a, p.maxt, p.a.d_in, p.a.gate.bits_, lds);
        if (st != MOE_OK) return st;
    }
    dim3 grid((p.a.d_ff + p.a.rows_per_wg - 1) / p.a.rows_per_wg, p.n_items);
    hipLaunchKernelGGL(k, grid, dim3(kFfnThreads), lds, p.s, p.a);
    return MOE_OK;
}

static moe_status launch_b(Plan &p) {
    size_t lds = 0;
    KernelFn k = nullptr;
    if (p.maxt > 1) k = batch_geometry(p.a, p.a.d_ff, p.a.down.bits_, kBatchNRB, kBatchPassesB, batch_down_q4(p.a.down.sb_), lds);
    if (!k) {
        k = select_down(p.a.down.bits_, p.a.down.sb_, p.maxt > 1);
        if (!k) return MOE_EUNSUPPORTED;
        const moe_status st = geometry(p.a, p.maxt, p.a.d_ff, p.a.down.bits_, lds);
        if (st != MOE_OK) return st;
        if (p.maxt == 1) {       // down_kernel_t1 stages act as fp16 chunks
            const int bits = p.a.down.bits_;
            lds = (size_t)(p.a.d_ff / codes_per_chunk(bits)) *
                  (bits == 4 ? f16_chunk_bytes<4>() : f16_chunk_bytes<8>());
        }
    }
    dim3 grid((p.a.d_in + p.a.rows_per_wg - 1) / p.a.rows_per_wg, p.n_items);
    hipLaunchKernelGGL(k, grid, dim3(kFfnThreads), lds, p.s, p.a);
    return MOE_OK;
}

static moe_status finish() { return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP; }

}  // namespace moe

extern "C" moe_status moe_decode_gate_up(const void *x, moe_dtype x_dtype_arg, int32_t n_tokens,
                                         const moe_qmat *gate, const moe_qmat *up,
                                         const int32_t *expert_ids, int32_t top_k, float *act,
                                         void *workspace, size_t workspace_bytes, void *stream) {
    const int x_dtype = raw_enum(x_dtype_arg);
    moe_status st = check_tokens(x, n_tokens, top_k);
    if (st != MOE_OK) return st;
    for (const moe_qmat *m : {gate, up})
        if ((st = check_qmat(m)) != MOE_OK) return st;
    if (!valid_dtype(x_dtype)) return MOE_EUNSUPPORTED;
    if (up->rows != gate->rows || up->cols != gate->cols || up->n_experts != gate->n_experts) return MOE_EINVAL;
    if (raw_enum(up->sb_dtype) != raw_enum(gate->sb_dtype) || up->bits != gate->bits) return MOE_EUNSUPPORTED;
    if (!act || !aligned16(act)) return MOE_EINVAL;
    Plan p = {};
    if ((st = plan_common(p, n_tokens, top_k, gate->n_experts, expert_ids, workspace, workspace_bytes,
                          stream)) != MOE_OK)
        return st;
    p.a.x = x; p.a.x_dt = x_dtype; p.a.d_in = gate->cols; p.a.d_ff = gate->rows;
    p.a.gate = to_qm(gate); p.a.up = to_qm(up); p.a.act = act;
    size_t lds;
    FfnArgs probe = p.a;
    if ((st = geometry(probe, p.maxt, gate->cols, gate->bits, lds)) != MOE_OK) return st;
    launch_bucket(p);
    if ((st = launch_a(p)) != MOE_OK) return st;
    return finish();
}

extern "C" moe_status moe_decode_down(const float *act, int32_t n_tokens, const moe_qmat *down,
                                      const int32_t *expert_ids, const float *scores, int32_t top_k,
                                      float *partial, void *workspace, size_t workspace_bytes,
                                      void *stream) {
    moe_status st = check_tokens(act, n_tokens, top_k);
    if (st != MOE_OK) return st;
    if ((st = check_qmat(down)) != MOE_OK) return st;
    if (!partial || !aligned16(partial)) return MOE_EINVAL;
    Plan p = {};
    if ((st = plan_common(p, n_tokens, top_k, down->n_experts, expert_ids, workspace, workspace_bytes,
                          stream)) != MOE_OK)
        return st;
    p.a.d_in = down->rows; p.a.d_ff = down->cols;
    p.a.down = to_qm(down); p.a.act = const_cast<float *>(act); p.a.scores = scores; p.a.partial = partial;
    size_t lds;
    FfnArgs probe = p.a;
    if ((st = geometry(probe, p.maxt, down->cols, down->bits, lds)) != MOE_OK) return st;
    launch_bucket(p);
    if ((st = launch_b(p)) != MOE_OK) return st;
    return finish();
}

namespace moe {
static moe_status expert_ffn(const void *x, int x_dtype, int32_t n_tokens, const moe_qmat *gate, const moe_qmat *up,
                             const moe_qmat *down, const int32_t *expert_ids, const float *scores, int32_t top_k,
                             float *act, float *partial, void *workspace, size_t workspace_bytes, void *stream);
}  // namespace moe

extern "C" moe_status moe_decode_expert_ffn(const void *x, moe_dtype x_dtype, int32_t n_tokens,
                                            const moe_qmat *gate, const moe_qmat *up, const moe_qmat *down,
                                            const int32_t *expert_ids, const float *scores, int32_t top_k,
                                            float *act, float *partial,
                                            void *workspace, size_t workspace_bytes, void *stream) {
    return expert_ffn(x, raw_enum(x_dtype), n_tokens, gate, up, down, expert_ids, scores, top_k, act, partial,
                      workspace, workspace_bytes, stream);
}

static moe_status moe::expert_ffn(const void *x, int x_dtype, int32_t n_tokens, const moe_qmat *gate,
                                  const moe_qmat *up, const moe_qmat *down, const int32_t *expert_ids,
                                  const float *scores, int32_t top_k, float *act, float *partial, void *workspace,
                                  size_t workspace_bytes, void *stream) {
    moe_status st = check_tokens(x, n_tokens, top_k);
    if (st != MOE_OK) return st;
    for (const moe_qmat *m : {gate, up, down})
        if ((st = check_qmat(m)) != MOE_OK) return st;
    if (!valid_dtype(x_dtype)) return MOE_EUNSUPPORTED;
    const int d_in = gate->cols, d_ff = gate->rows, E = gate->n_experts;
    if (up->rows != d_ff || up->cols != d_in || down->rows != d_in || down->cols != d_ff) return MOE_EINVAL;
    if (up->n_experts != E || down->n_experts != E) return MOE_EINVAL;
    if (raw_enum(up->sb_dtype) != raw_enum(gate->sb_dtype) || raw_enum(down->sb_dtype) != raw_enum(gate->sb_dtype))
        return MOE_EUNSUPPORTED;
    if (up->bits != gate->bits) return MOE_EUNSUPPORTED;
    if (!act || !partial || !aligned16(act) || !aligned16(partial)) return MOE_EINVAL;
    Plan p = {};
    if ((st = plan_common(p, n_tokens, top_k, E, expert_ids, workspace, workspace_bytes, stream)) != MOE_OK)
        return st;
    p.a.x = x; p.a.x_dt = x_dtype; p.a.d_in = d_in; p.a.d_ff = d_ff;
    p.a.gate = to_qm(gate); p.a.up = to_qm(up); p.a.down = to_qm(down);
    p.a.scores = scores; p.a.act = act; p.a.partial = partial;
    // check both geometries before enqueueing anything
    size_t lds;
    FfnArgs probe = p.a;
    if ((st = geometry(probe, p.maxt, d_in, gate->bits, lds)) != MOE_OK) return st;
    if ((st = geometry(probe, p.maxt, d_ff, down->bits, lds)) != MOE_OK) return st;
    launch_bucket(p);
    if ((st = launch_a(p)) != MOE_OK) return st;
    if ((st = launch_b(p)) != MOE_OK) return st;
    return finish();
}

// ------------------------------------------------- the call that allocates nothing

namespace moe {

// The bucketing workspace of the largest call the limits allow (32 tokens,
// top-32, 1024 experts), as a device array: each device that the library
// runs on holds one until the process ends.
constexpr size_t kNoAllocScratchBytes =
    ((1 + 2 * (size_t)((MOE_MAX_TOKENS * MOE_MAX_TOP_K + kBatchTok - 1) / kBatchTok + MOE_MAX_EXPERTS + 1) + 1 +
      (size_t)MOE_MAX_TOKENS * MOE_MAX_TOP_K) * sizeof(int32_t) + 255) / 256 * 256;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex scratch_mu;
static void *scratch_ptr[kMaxDevices];

// The device address of `scratch` on the current device, looked up once per
// device (hipGetSymbolAddress with that device current); nullptr on failure.
static void *device_scratch() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        scratch_ptr[dev] = p;
    }
    return scratch_ptr[dev];
}

}  // namespace moe

extern "C" size_t moe_decode_expert_ffn_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

extern "C" moe_status moe_decode_expert_ffn_noalloc(const void *x, moe_dtype x_dtype_arg, int32_t n_tokens,
                                                    const moe_qmat *gate, const moe_qmat *up, const moe_qmat *down,
                                                    const int32_t *expert_ids, const float *scores, int32_t top_k,
                                                    float *act, float *partial, void *stream) {
    const int x_dtype = raw_enum(x_dtype_arg);
    if (n_tokens <= 1)        // one token needs no workspace
        return expert_ffn(x, x_dtype, n_tokens, gate, up, down, expert_ids, scores, top_k, act, partial, nullptr, 0,
                          stream);
    if (!gate || n_tokens > MOE_MAX_TOKENS || top_k < 1 || top_k > MOE_MAX_TOP_K || gate->n_experts < 1 ||
        gate->n_experts > MOE_MAX_EXPERTS)
        return MOE_EINVAL;
    const size_t need = moe_decode_expert_ffn_workspace_bytes(n_tokens, top_k, gate->n_experts);
    if (need == 0 || need > kNoAllocScratchBytes) return MOE_EINVAL;
    void *ws = device_scratch();
    if (!ws) return MOE_EHIP;
    return expert_ffn(x, x_dtype, n_tokens, gate, up, down, expert_ids, scores, top_k, act, partial, ws, need,
                      stream);
}
