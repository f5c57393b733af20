// The whole MoE decode layer for one token in a single launch.
//
// Steps (mlxcel PR #276, "What changed" step 2; Red Lite dev39, "Change"):
//   route   : logits = Wr x (+ shared-gate logit w_g . x)
//   select  : top-k by logit (ties to the lower id), softmax scores
//   kernel A: act[s][r] = silu(W_gate[e_s] x)_r * (W_up[e_s] x)_r   for every slot s
//   kernel B: partial[s][i] = score_s * (W_down[e_s] act[s])_i
//   tail    : out = resid + (sum_k partial[k] + (sum_j partial[K+j]) * gate)
// Slots 0..K-1 are the routed experts in rank order, slots K..K+S-1 the
// shared experts (score 1).
//
// Workgroup roles, by block index (producers before consumers):
//   [0, n_route)              router rows, four per workgroup (one per wave)
//   [.., + A units)           one (slot, row tile) of kernel A each
//   [.., + B units)           one (slot, row tile of d_in) of kernel B each
// A and B units of routed slots wait for every router logit and then rank
// them themselves, so each knows the selected experts without another round
// trip.  B units issue the loads of their weights before they wait for their
// slot's act vector, so the down-projection weights stream while kernel A
// runs.  The B unit of the last slot of each row tile (the
// highest block index of that tile) keeps its own partial rows in LDS, waits
// for the other slots' rows and runs the tail: it sums them in slot order
// and writes the output.
//
// Cross-workgroup values (logits, act, partial) are 64-bit words: the fp32
// value in the low half and a launch tag in the high half, each written with
// one device-scope atomic store.  A consumer polls the words it needs until
// they carry this launch's tag, so a value and its "ready" flag arrive
// together and no counter, store-completion wait or cache-wide fence sits on
// the critical path.  The tag is 1 + the launch epoch kept in the workspace;
// the last tail bumps the epoch, so values left by an earlier launch never
// match.  Every wait is bounded: on time-out the waiter raises the error word
// of the workspace and carries on, so the launch always drains.  Every wait
// targets a workgroup of lower block index, so in-order dispatch cannot
// deadlock even when the grid exceeds the co-resident capacity.
#pragma once

#include <math.h>

#include "api.hpp"
#include "common.hpp"
#include "qgemv.hpp"
#include "topk.hpp"

namespace moe {

// Addresses of the fused layer's weight loads are formed per lane in 64 bits
// (load_block without SBASE): scalar expert bases measured no faster here and
// 0.5-1% slower on the 60-expert layer.
constexpr bool kLayerSBase = false;
constexpr int kLayerNRA = 3;        // rows per lane group, kernel A units with a single stage: 12-row
                                    // units put exactly two on each CU at the Qwen3-30B-A3B shape
                                    // (16-row units put two on half of them, which finished last)
constexpr int kLayerNRA2 = 2;       // rows per lane group and stage, kernel A units with several (two in flight)
constexpr int kLayerNRB = 4;        // rows per lane group, kernel B units
// stages a kernel-B unit keeps in flight with 6- and 8-bit down projections
// (register buffers): all of them are loaded before act arrives, and each
// buffer is refilled as soon as its stage is done
constexpr int kLayerBDepth = 2;
constexpr int kLayerThreads = 256;  // threads per workgroup (the launch's block size)
constexpr int kLayerWaves = kLayerThreads / kWave;
constexpr int kCtrStride = 64;      // uint32 words between control words (256 bytes)
constexpr uint32_t kSpinLimit = 1u << 19;
constexpr int kLogitCopies = 16;    // copies of the router logits, each polled by 1/16 of the workgroups
constexpr int kActCopies = 8;       // copies of each slot's last act row (the kernel-B units' sentinel)
constexpr int kSentStride = 32;     // words between sentinel copies (256 bytes)
// s_sleep arguments (units of 64 cycles) between polls: with hundreds of
// pollers, sparse polls make the hand-off faster, not slower
constexpr int kLogitSleep = 24;     // the router logits (~900 polling workgroups over 16 copies)
constexpr int kActSleep = 2;        // a slot's act sentinel (64 pollers over 8 copies)
constexpr int kRetrySleep = 2;      // words still missing after a batch read
constexpr int kTailSleep = 2;       // the tail's reads of the other slots' partial rows

// control words (in units of kCtrStride)
constexpr int kCtrErr = 0;
constexpr int kCtrEpoch = 1;
constexpr int kCtrTilesDone = 2;
constexpr int kCtrCount = 3;

struct LayerArgs {
    const void *x;
    const void *resid;
    int resid_dt;
    const void *wr;                 // [E][d_in], dtype of x
    const void *wg;                 // [d_in] or null, dtype of x
    int E, K, renorm, S;
    int d_in, d_ff, d_ffs;
    QM gate, up, down;
    QM sgate, sup, sdown;
    void *out;                      // [d_in], dtype out_dt
    int out_dt;
    int32_t *ids_out;
    float *scores_out;
    float *gate_out;
    uint64_t *logits;               // [kLogitCopies][logit_stride] tagged, E + 1 used per copy
    int logit_stride;               // words between copies (a multiple of 512: 4 KiB)
    uint64_t *act;                  // [K + S][act_stride] tagged
    uint64_t *act_sent;             // [K + S][kActCopies][kSentStride] tagged copies of each slot's last act row
    int act_stride;
    uint64_t *partial;              // [K + S][d_in] tagged
    uint32_t *ctr;                  // control words
    // the next layer's RMSNorm of out, folded into the tail (norm_out null: none)
    const void *norm_w;             // [d_in], dtype norm_dt
    int norm_dt;
    float norm_eps;
    void *norm_out;                 // [d_in], dtype norm_out_dt
    int norm_out_dt;
    uint64_t *norm_part;            // [b_tiles] tagged: each tail tile's sum of squares
    int n_route;
    int by_xcd;                     // units in slot-interleaved order: slot s's units on XCD s (8 slots)
    int a_lr_shift, a_tile, a_tiles_r, a_tiles_s;
    int b_lr_shift_r, b_lr_shift_s, b_tile, b_tiles;
};

__device__ __forceinline__ uint32_t *ctr_at(const LayerArgs &a, int slot) { return a.ctr + slot * kCtrStride; }

__device__ __forceinline__ void st_tagged(uint64_t *p, float v, uint32_t tag) {
    const uint64_t w = ((uint64_t)tag << 32) | (uint64_t)__float_as_uint(v);
    __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t ld_tagged(const uint64_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A tagged word read past the CU's L1 but from the XCD's L2: a relaxed
// atomic load of workgroup scope, which this target serves from the L2 (the
// sc0 policy) where the device-scope ld_tagged goes to memory.  Units of one
// XCD that read the same words then share the lines their first reads
// brought in.  Nothing guarantees that such a read sees a word written by
// another workgroup, and a line cached before its words were written holds
// older tags, so the pollers that use it return to ld_tagged every eighth try.
__device__ __forceinline__ uint64_t ld_tagged_l2(const uint64_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

__device__ __forceinline__ void raise_error(const LayerArgs &a) {
    __hip_atomic_fetch_or(ctr_at(a, kCtrErr), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Poll one tagged word until it carries `tag`; returns its value (0 and the
// error word raised on time-out).  Polls are spaced out: with hundreds of
// workgroups polling, the polls themselves slow down the memory round trip
// that delivers the value.
template <int SLEEP>
__device__ __forceinline__ float wait_tagged(const LayerArgs &a, const uint64_t *p, uint32_t tag) {
    for (uint32_t i = 0; i < kSpinLimit; ++i) {
        const uint64_t w = ld_tagged(p);
        if ((uint32_t)(w >> 32) == tag) return __uint_as_float((uint32_t)w);
        __builtin_amdgcn_s_sleep(SLEEP);
    }
    raise_error(a);
    return 0.f;
}

// Per thread: read the tagged words addr(0), .., addr(cnt - 1) (cnt <= N) with
// all loads in flight together, then poll again only the ones not yet tagged,
// so a batch costs one round trip once its producers are done.  v[u] gets the
// values (0, and the error word raised, on time-out).
template <int N, int SLEEP = kRetrySleep, typename Addr>
__device__ __forceinline__ void poll_batch(const LayerArgs &a, uint32_t tag, int cnt, Addr addr, float *v) {
    uint64_t w[N];
    const uint64_t ready = (uint64_t)tag << 32;
#pragma unroll
    for (int u = 0; u < N; ++u) w[u] = u < cnt ? ld_tagged(addr(u)) : ready;
    for (uint32_t spin = 0;; ++spin) {
        bool all = true;
#pragma unroll
        for (int u = 0; u < N; ++u) all = all && (uint32_t)(w[u] >> 32) == tag;
        if (all) break;
        if (spin == kSpinLimit) {
            raise_error(a);
            break;
        }
        __builtin_amdgcn_s_sleep(SLEEP);
#pragma unroll
        for (int u = 0; u < N; ++u)
            if ((uint32_t)(w[u] >> 32) != tag) w[u] = ld_tagged(addr(u));
    }
#pragma unroll
    for (int u = 0; u < N; ++u) v[u] = (uint32_t)(w[u] >> 32) == tag ? __uint_as_float((uint32_t)w[u]) : 0.f;
}

constexpr int kGatherPer = 4;       // words per thread per gather batch

// Gather n tagged words addr(0..n) into f(i, value), in batches of
// kGatherPer words per thread, SLEEP between polls of missing words.  With a
// sentinel, thread 0 first waits for that one word (written when the
// producers are about done), so that while the producers run a workgroup
// polls one address rather than all n.
template <int SLEEP, typename Addr, typename Fn>
__device__ __forceinline__ void gather_tagged(const LayerArgs &a, int n, const uint64_t *sentinel, uint32_t tag,
                                              Addr addr, Fn f) {
    const int nt = blockDim.x, t = threadIdx.x;
    if (sentinel) {
        if (t == 0) (void)wait_tagged<SLEEP>(a, sentinel, tag);
        __syncthreads();
    }
    for (int base = 0; base < n; base += kGatherPer * nt) {
        const int left = n - base - t;
        const int cnt = left <= 0 ? 0 : min(kGatherPer, (left + nt - 1) / nt);
        float v[kGatherPer];
        poll_batch<kGatherPer, SLEEP>(a, tag, cnt, [&](int u) { return addr(base + u * nt + t); }, v);
#pragma unroll
        for (int u = 0; u < kGatherPer; ++u)
            if (u < cnt) f(base + u * nt + t, v[u]);
    }
}

// The act gather of a kernel-B unit: act[0, n) (n a multiple of the chunk
// size) into LDS as fp16 chunks placed as the packed dots read them
// (f16_stage_offset: 4-bit chunks of 32 values for dot_block_q4_f16, 6- and
// 8-bit chunks of 16 for dot_block_f16x16), each value times
// kActF16Prescale; with L2 the sentinel and the words are read through the
// XCD's L2 first (ld_tagged_l2).  Returns the factor by which the dot products of the
// staged values are to be multiplied: kActF16Postscale, unless some value
// would overflow fp16 that way (one compare per value; the waves' ballots
// meet in LDS over the barrier that ends the gather).  Then every thread
// reads its words again (all are present by then) and the vector is staged
// with the factor fitted to its largest magnitude (f16_stage_scale).
// wait_tagged and poll_batch with their reads through the L2 (L2:
// ld_tagged_l2, and ld_tagged every eighth try) or from memory (ld_tagged).
template <int SLEEP, bool L2>
__device__ __forceinline__ float wait_tagged_via(const LayerArgs &a, const uint64_t *p, uint32_t tag) {
    if constexpr (!L2) {
        return wait_tagged<SLEEP>(a, p, tag);
    } else {
        for (uint32_t i = 0; i < kSpinLimit; ++i) {
            const uint64_t w = (i & 7) != 7 ? ld_tagged_l2(p) : ld_tagged(p);
            if ((uint32_t)(w >> 32) == tag) return __uint_as_float((uint32_t)w);
            __builtin_amdgcn_s_sleep(SLEEP);
        }
        raise_error(a);
        return 0.f;
    }
}

template <int N, int SLEEP, bool L2, typename Addr>
__device__ __forceinline__ void poll_batch_via(const LayerArgs &a, uint32_t tag, int cnt, Addr addr, float *v) {
    if constexpr (!L2) {
        poll_batch<N, SLEEP>(a, tag, cnt, addr, v);
    } else {
        uint64_t w[N];
        const uint64_t ready = (uint64_t)tag << 32;
#pragma unroll
        for (int u = 0; u < N; ++u) w[u] = u < cnt ? ld_tagged_l2(addr(u)) : ready;
        for (uint32_t spin = 0;; ++spin) {
            bool all = true;
#pragma unroll
            for (int u = 0; u < N; ++u) all = all && (uint32_t)(w[u] >> 32) == tag;
            if (all) break;
            if (spin == kSpinLimit) {
                raise_error(a);
                break;
            }
            __builtin_amdgcn_s_sleep(SLEEP);
            if ((spin & 7) != 7) {
#pragma unroll
                for (int u = 0; u < N; ++u)
                    if ((uint32_t)(w[u] >> 32) != tag) w[u] = ld_tagged_l2(addr(u));
            } else {
#pragma unroll
                for (int u = 0; u < N; ++u)
                    if ((uint32_t)(w[u] >> 32) != tag) w[u] = ld_tagged(addr(u));
            }
        }
#pragma unroll
        for (int u = 0; u < N; ++u) v[u] = (uint32_t)(w[u] >> 32) == tag ? __uint_as_float((uint32_t)w[u]) : 0.f;
    }
}

template <int BB, bool L2>
__device__ __forceinline__ float gather_act_f16(const LayerArgs &a, int n, const uint64_t *sentinel, uint32_t tag,
                                                const uint64_t *act, char *lds) {
    static_assert(kLayerWaves == 4, "one flag word per wave, read as one 16-byte word");
    __shared__ __align__(16) uint32_t s_wave[2][kLayerWaves];   // per wave: overflow flag, largest magnitude
    constexpr int nt = kLayerThreads;
    const int t = threadIdx.x, lane = t & (kWave - 1), wave = t >> 6;
    auto place = [&](int i, float v) {
        *reinterpret_cast<_Float16 *>(lds + f16_stage_offset<BB>(i)) = (_Float16)v;
    };
    if (t == 0) (void)wait_tagged_via<kActSleep, L2>(a, sentinel, tag);
    __syncthreads();
    bool over = false;
    for (int base = 0; base < n; base += kGatherPer * nt) {
        const int left = n - base - t;
        const int cnt = left <= 0 ? 0 : min(kGatherPer, (left + nt - 1) / nt);
        float v[kGatherPer];
        poll_batch_via<kGatherPer, kActSleep, L2>(a, tag, cnt, [&](int u) { return act + base + u * nt + t; }, v);
#pragma unroll
        for (int u = 0; u < kGatherPer; ++u)
            if (u < cnt) {
                over |= !(__builtin_fabsf(v[u]) < kActF16Overflow);      // NaN counts as over
                place(base + u * nt + t, v[u] * kActF16Prescale);
            }
    }
    const uint64_t b_over = __builtin_amdgcn_ballot_w64(over);
    if (lane == 0) s_wave[0][wave] = b_over ? 1u : 0u;
    __syncthreads();
    const u32x4 f = *reinterpret_cast<const u32x4 *>(s_wave[0]);
    if (!(f.x | f.y | f.z | f.w)) return kActF16Postscale;
    // the slot's largest magnitude, then the values again, scaled to fit
    uint32_t mx = 0;
    for (int i = t; i < n; i += nt) mx = max(mx, (uint32_t)ld_tagged(act + i) & 0x7FFFFFFFu);
    const float wm = wave_max(__uint_as_float(mx));       // magnitudes as floats order like their bits
    if (lane == 0) s_wave[1][wave] = __float_as_uint(wm);
    __syncthreads();
    uint32_t m = 0;
#pragma unroll
    for (int w = 0; w < kLayerWaves; ++w) m = max(m, s_wave[1][w]);
    float inv;
    const float cs = f16_stage_scale(m, inv);
    for (int i = t; i < n; i += nt) place(i, __uint_as_float((uint32_t)ld_tagged(act + i)) * inv);
    __syncthreads();
    return cs;
}

__device__ __forceinline__ uint32_t launch_tag(const LayerArgs &a) {
    return __hip_atomic_load(ctr_at(a, kCtrEpoch), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
}

// Eight consecutive elements of a row as floats.
template <int DT>
__device__ __forceinline__ void load8(const void *base, int64_t elem, float *v) {
    if constexpr (DT == MOE_F32) {
        const f32x4 *p = reinterpret_cast<const f32x4 *>(reinterpret_cast<const float *>(base) + elem);
        const f32x4 u = p[0], w = p[1];
        v[0] = u.x; v[1] = u.y; v[2] = u.z; v[3] = u.w;
        v[4] = w.x; v[5] = w.y; v[6] = w.z; v[7] = w.w;
    } else {
        load_x_chunk<DT, 8>(base, elem, v);
    }
}

// Router row `row` of `w` (d_in long) dotted with x, reduced over the wave.
template <int XT>
__device__ __forceinline__ float layer_row_dot(const void *w, int64_t row, const void *x, int d_in, int lane) {
    const int nch = d_in / 8;
    float acc = 0.f;
    for (int base = 0; base < nch; base += 4 * kWave) {
        float wv[4][8], xv[4][8];
        bool ok[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int c = base + u * kWave + lane;
            ok[u] = c < nch;
            const int cc = ok[u] ? c : 0;
            load8<XT>(w, row * d_in + 8 * cc, wv[u]);
            load8<XT>(x, 8 * cc, xv[u]);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            float part = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) part += wv[u][i] * xv[u][i];
            acc += ok[u] ? part : 0.f;
        }
    }
    return wave_sum(acc);
}

// This workgroup's copy of the router logits.
__device__ __forceinline__ const uint64_t *my_logits(const LayerArgs &a) {
    return a.logits + (int64_t)(blockIdx.x % kLogitCopies) * a.logit_stride;
}

// Wait for every router logit (and the shared-gate logit) and stage them in
// LDS, padded with -inf for the rank count.  Each thread polls its words
// directly, with no sentinel first: the router rows all finish within about
// a memory round trip of each other, and one round trip fewer measured 0.3 us
// less per launch than a sentinel wait followed by the gather.
__device__ void gather_logits(const LayerArgs &a, uint32_t tag, float *s_logits, Selection *sel) {
    const int n = a.E + (a.wg ? 1 : 0);
    if (threadIdx.x == 0) {
        if (!a.wg) sel->gate = 1.0f;
        sel->n_over = 0;
    }
    if (threadIdx.x < kCandMax) sel->cand[threadIdx.x] = 0;
    for (int e = a.E + threadIdx.x; e < kRankMaxE; e += blockDim.x) s_logits[e] = -INFINITY;
    const uint64_t *lg = my_logits(a);
    gather_tagged<kLogitSleep>(a, n, nullptr, tag, [&](int i) { return lg + i; }, [&](int e, float v) {
        if (e < a.E) s_logits[e] = v == 0.f ? 0.f : v;      // -0 as +0
        else sel->gate = sigmoidf_(v);
    });
    __syncthreads();
}

__device__ __forceinline__ int n_slots(const LayerArgs &a) { return a.K + a.S; }

// Copies of a slot's last act row: the word its kernel-B units wait on
// before they read the whole vector.
__device__ __forceinline__ void store_act_sentinel(const LayerArgs &a, int slot, float v, uint32_t tag) {
    uint64_t *p = a.act_sent + (int64_t)slot * kActCopies * kSentStride;
#pragma unroll
    for (int c = 0; c < kActCopies; ++c) st_tagged(p + c * kSentStride, v, tag);
}

// Kernel-A epilogue: reduce the gate and up sums of NR rows over each lane
// group of width 1 << lrs and store the rows' SwiGLU values, rows r0 +
// n * rpw (r0 is the lane group's first row).  Wide groups reduce all 2 NR
// sums at once, and lane (n << SH) of a group stores row n with the up sum
// from the lane across the group's top bit; narrow groups reduce each sum
// on its own and the group's last lane stores every row.
template <int NR>
__device__ __forceinline__ void a_epilogue(const LayerArgs &a, int lrs, float (&acc)[2][NR], int r0, int rpw,
                                           int row_end, int dff, uint64_t *act, int slot, uint32_t tag) {
    const int lane = threadIdx.x & (kWave - 1);
    with_width(lrs, [&](auto w) {
        constexpr int W = decltype(w)::value;
        constexpr int NRP = NR <= 1 ? 1 : NR <= 2 ? 2 : NR <= 4 ? 4 : 8;    // NR rounded up to a power of two
        constexpr int V = 2 * NRP;
        if constexpr (W >= 16 && W >= V) {
            float sv[V];
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int n = 0; n < NRP; ++n) sv[m * NRP + n] = n < NR ? acc[m][n] : 0.f;
            group_multi_sum<W, V>(sv);
            const float u = group_partner<W>(sv[0]);
            constexpr int SH = ilog2(W) - ilog2(V);
            const int li = lane & (W - 1), n = li >> SH;
            if ((li & ((1 << SH) - 1)) == 0 && n < NR) {
                const int r = r0 + n * rpw;
                if (r < row_end) {
                    const float g = sv[0];
                    const float v = g * sigmoidf_(g) * u;
                    st_tagged(act + r, v, tag);
                    if (r == dff - 1) store_act_sentinel(a, slot, v, tag);
                }
            }
        } else {
#pragma unroll
            for (int n = 0; n < NR; ++n) {
                acc[0][n] = group_sum_last<W>(acc[0][n]);
                acc[1][n] = group_sum_last<W>(acc[1][n]);
            }
            if ((lane & (W - 1)) == W - 1) {
#pragma unroll
                for (int n = 0; n < NR; ++n) {
                    const int r = r0 + n * rpw;
                    if (r < row_end) {
                        const float g = acc[0][n], u = acc[1][n];
                        const float v = g * sigmoidf_(g) * u;
                        st_tagged(act + r, v, tag);
                        if (r == dff - 1) store_act_sentinel(a, slot, v, tag);
                    }
                }
            }
        }
    });
}

// Kernel A unit: rows [row0, row0 + a_tile) of slot `slot`, expert e (x
// already staged in LDS).
template <int BA, int SB, int XT>
__device__ void layer_a_unit_single(const LayerArgs &a, uint32_t tag, int slot, int tile, int e, void *xs) {
    constexpr int NR = kLayerNRA;
    using F = Fmt<BA>;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
    const bool routed = slot < a.K;
    const int dff = routed ? a.d_ff : a.d_ffs;
    const int E = routed ? a.E : a.S;
    const int row0 = tile * a.a_tile;
    const int row_end = min(row0 + a.a_tile, dff);
    uint64_t *act = a.act + (int64_t)slot * a.act_stride;
    if (e < 0 || e >= E) {
        for (int r = row0 + tid; r < row_end; r += blockDim.x) {
            st_tagged(act + r, 0.f, tag);
            if (r == dff - 1) store_act_sentinel(a, slot, 0.f, tag);
        }
        return;
    }
    const QM mats[2] = {routed ? a.gate : a.sgate, routed ? a.up : a.sup};
    const int64_t erow0 = (int64_t)e * dff;
    const int cpr = a.d_in / F::kCodes;
    const int lr = 1 << a.a_lr_shift, j = lane & (lr - 1), rsub = lane >> a.a_lr_shift, rpw = kWave >> a.a_lr_shift;
    // stages = (row pass, chunk position), each loaded and then consumed (a
    // unit of one stage is the common case: nothing to overlap)
    const int rb0 = row0 + wave * rpw * NR, pass_rows = 4 * rpw * NR;
    const int n_pass = rb0 < row_end ? (row_end - rb0 + pass_rows - 1) / pass_rows : 0;
    const int n_chunk = (cpr + lr - 1) / lr;
    const int n_stage = n_pass * n_chunk;
    float acc[2][NR];
    for (int st = 0; st < n_stage; ++st) {
        const int ps = st / n_chunk, ch = st - ps * n_chunk;
        const int r0 = rb0 + ps * pass_rows + rsub;
        if (ch == 0) {
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int n = 0; n < NR; ++n) acc[m][n] = 0.f;
        }
        const int cpos = ch * lr + j;
        XRaw<XT, F::kCodes> xr;
        read_x_raw<XT, F::kCodes>(xs, cpos < cpr ? cpos : 0, xr);
        BlockRegs<BA, 2, NR> cur;
        load_block<BA, 2, NR, kLayerSBase>(cur, mats, erow0, r0, rpw, row_end, cpos, cpr);
        if constexpr (BA == 4 && XT == MOE_BF16) {
            // raw bf16 inputs for the packed-dot path
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
            dot_block_q4_bf16<SB, 2, NR>(cur, xw, xsum, acc);
        } else {
            float xv[F::kCodes];
            convert_x<XT, F::kCodes>(xr, xv);
            dot_block<BA, SB, 2, NR>(cur, xv, sum_n<F::kCodes>(xv), acc);
        }
        if (ch == n_chunk - 1) a_epilogue<NR>(a, a.a_lr_shift, acc, r0, rpw, row_end, dff, act, slot, tag);
    }
}

// Kernel A unit of several stages, pipelined two deep (same work as
// layer_a_unit_single, kLayerNRA2 rows per lane group and stage).
template <int BA, int SB, int XT>
__device__ void layer_a_unit_pipelined(const LayerArgs &a, uint32_t tag, int slot, int tile, int e, void *xs) {
    using F = Fmt<BA>;
    constexpr int NR = kLayerNRA2;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
    const bool routed = slot < a.K;
    const int dff = routed ? a.d_ff : a.d_ffs;
    const int E = routed ? a.E : a.S;
    const int row0 = tile * a.a_tile;
    const int row_end = min(row0 + a.a_tile, dff);
    uint64_t *act = a.act + (int64_t)slot * a.act_stride;
    if (e < 0 || e >= E) {
        for (int r = row0 + tid; r < row_end; r += blockDim.x) {
            st_tagged(act + r, 0.f, tag);
            if (r == dff - 1) store_act_sentinel(a, slot, 0.f, tag);
        }
        return;
    }
    const QM mats[2] = {routed ? a.gate : a.sgate, routed ? a.up : a.sup};
    const int64_t erow0 = (int64_t)e * dff;
    const int cpr = a.d_in / F::kCodes;
    const int lr = 1 << a.a_lr_shift, j = lane & (lr - 1), rsub = lane >> a.a_lr_shift, rpw = kWave >> a.a_lr_shift;
    // stages = (row pass, chunk position).  Two of them live in registers:
    // the loads of stage st + 1 are in flight while stage st is consumed, so
    // a unit of several stages streams without a round trip per stage.
    const int rb0 = row0 + wave * rpw * NR, pass_rows = 4 * rpw * NR;
    const int n_pass = rb0 < row_end ? (row_end - rb0 + pass_rows - 1) / pass_rows : 0;
    const int n_chunk = (cpr + lr - 1) / lr;
    const int n_stage = n_pass * n_chunk;
    auto stage_row = [&](int st) { return rb0 + (st / n_chunk) * pass_rows + rsub; };
    auto load = [&](BlockRegs<BA, 2, NR> &R, int st) {
        load_block<BA, 2, NR, kLayerSBase>(R, mats, erow0, stage_row(st), rpw, row_end, (st % n_chunk) * lr + j, cpr);
    };
    float acc[2][NR];
    // a stage's inputs: chunk position c of x, staged in LDS
    auto read_x = [&](XRaw<XT, F::kCodes> &xr, int st) {
        const int c = (st % n_chunk) * lr + j;
        read_x_raw<XT, F::kCodes>(xs, c < cpr ? c : 0, xr);
    };
    auto consume = [&](const BlockRegs<BA, 2, NR> &cur, const XRaw<XT, F::kCodes> &xr, int st) {
        const int ch = st % n_chunk;
        if (ch == 0) {
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int n = 0; n < NR; ++n) acc[m][n] = 0.f;
        }
        if constexpr (BA == 4 && XT == MOE_BF16) {
            // raw bf16 inputs for the packed-dot path
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
            dot_block_q4_bf16<SB, 2, NR>(cur, xw, xsum, acc);
        } else {
            float xv[F::kCodes];
            convert_x<XT, F::kCodes>(xr, xv);
            dot_block<BA, SB, 2, NR>(cur, xv, sum_n<F::kCodes>(xv), acc);
        }
        if (ch == n_chunk - 1) a_epilogue<NR>(a, a.a_lr_shift, acc, stage_row(st), rpw, row_end, dff, act, slot, tag);
    };
    BlockRegs<BA, 2, NR> ra, rb;
    if (n_stage > 0) load(ra, 0);
    for (int st = 0; st < n_stage; st += 2) {
        if (st + 1 < n_stage) load(rb, st + 1);
        XRaw<XT, F::kCodes> xr;
        read_x(xr, st);
        consume(ra, xr, st);
        if (st + 1 < n_stage) {
            if (st + 2 < n_stage) load(ra, st + 2);
            read_x(xr, st + 1);
            consume(rb, xr, st + 1);
        }
    }
}

// Sum of v over the workgroup in a fixed order (DPP tree within each wave,
// then the waves' sums in wave order): the same bits on every run.  Every
// thread gets the sum.  Contains barriers.
__device__ __forceinline__ float block_sum_fixed(float v) {
    __shared__ float s_wsum[kLayerWaves];
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
    const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(group_sum_last<kWave>(v)), kWave - 1));
    __syncthreads();
    if (lane == 0) s_wsum[wave] = w;
    __syncthreads();
    float sum = s_wsum[0];
#pragma unroll
    for (int i = 1; i < kLayerWaves; ++i) sum += s_wsum[i];
    return sum;
}

// The next layer's RMSNorm of out, folded into the tail (Red Lite dev39,
// "Measurements": the tail that also computed the next layer's RMSNorm; there
// on one threadgroup, here spread over every tail tile).  Each tail tile
// publishes the sum of squares of its rows of out (a fixed-order workgroup
// sum) as a tagged word, gathers every tile's word, adds them in tile order
// (a fixed-order sum again), and writes its own rows of
//   norm_out[i] = out[i] / sqrt(sum_i out[i]^2 / d_in + eps) * weight[i]
// (rounded to norm_out's dtype).  own[k]: this thread's row row0 + tid +
// k * kLayerThreads of out as stored (0 past row_end).  s_part: LDS for every tile's sum (at least b_tiles floats; the
// unit's logits array, no longer needed).
template <int NROWS>
__device__ void tail_rmsnorm(const LayerArgs &a, uint32_t tag, int tile, int row0, int row_end,
                             const float (&own)[NROWS], float *s_part) {
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < NROWS; ++k) ss += own[k] * own[k];
    const float tile_ss = block_sum_fixed(ss);
    if (threadIdx.x == 0) st_tagged(a.norm_part + tile, tile_ss, tag);
    gather_tagged<kTailSleep>(a, a.b_tiles, nullptr, tag, [&](int i) { return a.norm_part + i; },
                              [&](int i, float v) { s_part[i] = v; });
    __syncthreads();
    float part = 0.f;                               // tiles tid, tid + 256, ... in order
    for (int i = threadIdx.x; i < a.b_tiles; i += blockDim.x) part += s_part[i];
    const float total = block_sum_fixed(part);
    const float inv = 1.0f / sqrtf(total / (float)a.d_in + a.norm_eps);
#pragma unroll
    for (int k = 0; k < NROWS; ++k) {
        const int r = row0 + threadIdx.x + k * kLayerThreads;
        if (r < row_end) store_act(a.norm_out, a.norm_out_dt, r, own[k] * inv * load_act(a.norm_w, a.norm_dt, r));
    }
}

// Kernel B unit: rows [row0, row0 + b_tile) of d_in for slot `slot`.  The
// unit of the last slot also runs the tail for those rows.  L2: act read
// through the XCD's L2 first (gather_act_f16).
template <int BB, int SB, bool L2>
__device__ void layer_b_unit(const LayerArgs &a, uint32_t tag, int slot, int tile, int e, float *s_logits,
                             Selection *sel, float *xs) {
    constexpr int NR = kLayerNRB;
    using F = Fmt<BB>;
    constexpr int CODES = F::kCodes;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
    const bool routed = slot < a.K;
    float score = 1.0f;
    const int dff = routed ? a.d_ff : a.d_ffs;
    const int E = routed ? a.E : a.S;
    const int row0 = tile * a.b_tile;
    const int row_end = min(row0 + a.b_tile, a.d_in);
    uint64_t *part = a.partial + (int64_t)slot * a.d_in;
    const int lrs = routed ? a.b_lr_shift_r : a.b_lr_shift_s;
    const int lr = 1 << lrs, j = lane & (lr - 1), rsub = lane >> lrs, rpw = kWave >> lrs;
    const int cpr = dff / CODES;
    const bool valid = e >= 0 && e < E;
    const QM mats[1] = {routed ? a.down : a.sdown};
    const int64_t erow0 = (int64_t)(valid ? e : 0) * a.d_in;
    const bool last_slot = slot == n_slots(a) - 1;
    // own partial rows, kept for the tail: a tile is at most 4 waves x 64 lane
    // groups of one lane x kLayerNRB rows
    __shared__ float s_own[4 * kWave * kLayerNRB];

    // stages = (row pass, chunk position); the first kDepth stages are loaded
    // before act is ready, into a ring of register buffers: stage st uses
    // buffer st % kDepth, which is refilled with stage st + kDepth once st is
    // done.  4-bit down projections keep one buffer (their first stage is
    // also unpacked before act arrives, which takes the registers).
    constexpr int kDepth = BB == 4 ? 1 : kLayerBDepth;
    const int rb0 = row0 + wave * rpw * NR, pass_rows = 4 * rpw * NR;
    const int n_pass = (valid && rb0 < row_end) ? (row_end - rb0 + pass_rows - 1) / pass_rows : 0;
    const int n_chunk = (cpr + lr - 1) / lr;
    const int n_stage = n_pass * n_chunk;
    auto load_stage = [&](BlockRegs<BB, 1, NR> &R, int st) __attribute__((always_inline)) {
        const int ps = st / n_chunk, ch = st - ps * n_chunk;
        load_block<BB, 1, NR, kLayerSBase>(R, mats, erow0, rb0 + ps * pass_rows + rsub, rpw, row_end, ch * lr + j,
                                           cpr);
    };
    static_assert(kDepth >= 1 && kDepth <= 3, "the stage loop below is written for up to three buffers");
    BlockRegs<BB, 1, NR> b0, b1, b2;        // separate variables: they stay in registers
    if (n_stage > 0) load_stage(b0, 0);
    if constexpr (kDepth >= 2) {
        if (n_stage > 1) load_stage(b1, 1);
    }
    if constexpr (kDepth >= 3) {
        if (n_stage > 2) load_stage(b2, 2);
    }

    if (routed && wave == 0) {   // scores while the weights and act are in flight
        with_per(a.E, [&](auto per) { softmax_scores<decltype(per)::value>(a.E, a.K, a.renorm, s_logits, lane, sel); });
        if (slot == 0 && tile == 0) {            // publish the routing result once
            if (lane < a.K) {
                if (a.ids_out) a.ids_out[lane] = sel->ids[lane];
                if (a.scores_out) a.scores_out[lane] = sel->scores[lane];
            }
            if (lane == 0 && a.gate_out && a.wg) a.gate_out[0] = sel->gate;
        }
    }

    if (valid) {
        const uint64_t *act = a.act + (int64_t)slot * a.act_stride;
        const int n_act = cpr * CODES;
        const uint64_t *sent = a.act_sent + ((int64_t)slot * kActCopies + tile % kActCopies) * kSentStride;
        // act as fp16 pairs for the packed dots, staged with a power-of-two
        // factor whose inverse joins the score (gather_act_f16).  With 4-bit
        // codes the first stage's codes are unpacked while act is on its way:
        // after it arrives only the dot products remain.
        [[maybe_unused]] uint32_t pre[1][NR][16];
        if constexpr (BB == 4) {
            if (n_stage > 0) unpack_q4_f16<1, NR>(b0, pre);
        }
        const float cs = gather_act_f16<BB, L2>(a, n_act, sent, tag, act, reinterpret_cast<char *>(xs));
        if (routed) score = sel->scores[slot];
        const float sc = score * cs;         // exact: cs is a power of two
        float acc[1][NR];
        auto run_stage = [&](BlockRegs<BB, 1, NR> &cur, int st) __attribute__((always_inline)) {
            const int ps = st / n_chunk, ch = st - ps * n_chunk;
            const int r0 = rb0 + ps * pass_rows + rsub;
            if (ch == 0) {
#pragma unroll
                for (int n = 0; n < NR; ++n) acc[0][n] = 0.f;
            }
            constexpr int NP = CODES / 2;           // staged pairs per chunk
            const u32x4 *src = reinterpret_cast<const u32x4 *>(reinterpret_cast<const char *>(xs) +
                                                               cur.cc * f16_chunk_bytes<BB>());
            uint32_t ap[NP];
#pragma unroll
            for (int i = 0; i < NP / 4; ++i) {
                const u32x4 v = src[i];
#pragma unroll
                for (int k = 0; k < 4; ++k) ap[4 * i + k] = v[k];
            }
            if constexpr (BB == 4) {
                if (st == 0) dot_pre_q4_f16<SB, 1, NR>(cur, pre, ap, f16_pairs_sum<NP>(ap), acc);
                else dot_block_q4_f16<SB, 1, NR>(cur, ap, f16_pairs_sum<NP>(ap), acc);
            } else {
                dot_block_f16x16<BB, SB, 1, NR>(cur, ap, f16_pairs_sum<NP>(ap), acc);
            }
            if (ch == n_chunk - 1) {
                auto put = [&](int r, float v) {
                    if (r < row_end) {
                        if (last_slot) s_own[r - row0] = sc * v;
                        else st_tagged(part + r, sc * v, tag);
                    }
                };
                with_width(lrs, [&](auto w) {
                    constexpr int W = decltype(w)::value;
                    if constexpr (W >= 16 && W >= NR) {
                        // all NR sums at once; lane (n << SH) of the group holds row n
                        float sv[NR];
#pragma unroll
                        for (int n = 0; n < NR; ++n) sv[n] = acc[0][n];
                        group_multi_sum<W, NR>(sv);
                        constexpr int SH = ilog2(W) - ilog2(NR);
                        const int li = lane & (W - 1);
                        if ((li & ((1 << SH) - 1)) == 0) put(r0 + (li >> SH) * rpw, sv[0]);
                    } else {
#pragma unroll
                        for (int n = 0; n < NR; ++n) acc[0][n] = group_sum_last<W>(acc[0][n]);
                        if (j == lr - 1) {
#pragma unroll
                            for (int n = 0; n < NR; ++n) put(r0 + n * rpw, acc[0][n]);
                        }
                    }
                });
            }
        };
        if constexpr (kDepth == 1) {
            for (int st = 0; st < n_stage; ++st) {
                if (st > 0) load_stage(b0, st);
                run_stage(b0, st);
            }
        } else {
            auto step = [&](BlockRegs<BB, 1, NR> &cur, int st) __attribute__((always_inline)) {
                if (st < n_stage) {
                    run_stage(cur, st);
                    if (st + kDepth < n_stage) load_stage(cur, st + kDepth);
                }
            };
            for (int st0 = 0; st0 < n_stage; st0 += kDepth) {
                step(b0, st0);
                step(b1, st0 + 1);
                if constexpr (kDepth >= 3) step(b2, st0 + 2);
            }
        }
    } else {
        for (int r = row0 + tid; r < row_end; r += blockDim.x) {
            if (last_slot) s_own[r - row0] = 0.f;
            else st_tagged(part + r, 0.f, tag);
        }
    }
    if (!last_slot) return;

    // Tail for rows [row0, row_end): wait for the other slots' partial rows and
    // sum in slot order: routed slots, then the shared experts times the gate.
    __syncthreads();
    __shared__ float s_gate;
    if (tid == 0)
        s_gate = a.wg ? sigmoidf_(wait_tagged<kLogitSleep>(a, my_logits(a) + a.E, tag)) : 1.0f;
    __syncthreads();
    const float g = s_gate;
    const int ns = n_slots(a);
    constexpr int kTailPer = 8;             // slots read together per batch
    // a tile has at most 4 waves x 64 lane groups x kLayerNRB rows: at most kTailRows per thread
    constexpr int kTailRows = 4 * kWave * kLayerNRB / kLayerThreads;
    float own[kTailRows];                   // this thread's rows of out, kept for the RMSNorm
#pragma unroll
    for (int k = 0; k < kTailRows; ++k) {
        const int r = row0 + tid + k * kLayerThreads;
        own[k] = 0.f;
        if (r >= row_end) continue;
        float routed_sum = 0.f, sh = 0.f;   // 0 + x == x: the sums start at slot 0 and slot K
        for (int s0 = 0; s0 < ns; s0 += kTailPer) {
            float v[kTailPer];
            const int cnt = min(kTailPer, ns - 1 - s0);     // the last slot's rows are in s_own
            poll_batch<kTailPer, kTailSleep>(
                a, tag, cnt, [&](int u) { return a.partial + (int64_t)(s0 + u) * a.d_in + r; }, v);
#pragma unroll
            for (int u = 0; u < kTailPer; ++u) {
                const int s2 = s0 + u;
                if (s2 < ns) {
                    const float pv = s2 == ns - 1 ? s_own[r - row0] : v[u];
                    if (s2 < a.K) routed_sum += pv;
                    else sh += pv;
                }
            }
        }
        const float o = round_to_dtype(a.out_dt, load_act(a.resid, a.resid_dt, r) + (routed_sum + sh * g));
        store_rounded(a.out, a.out_dt, r, o);
        own[k] = o;
    }
    if (a.norm_out) tail_rmsnorm<kTailRows>(a, tag, tile, row0, row_end, own, s_logits);
    // the last tile to finish moves the workspace to the next epoch
    __syncthreads();
    if (tid == 0) {
        const uint32_t done = __hip_atomic_fetch_add(ctr_at(a, kCtrTilesDone), 1u, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        if (done == (uint32_t)a.b_tiles - 1) {
            __hip_atomic_store(ctr_at(a, kCtrTilesDone), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(ctr_at(a, kCtrEpoch), tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// ANR: kLayerNRA (kernel-A units of one stage) or kLayerNRA2 (pipelined stages).
template <int BA, int BB, int SB, int XT, int ANR>
__global__ __launch_bounds__(kLayerThreads, 3) void layer_kernel(LayerArgs a) {
    __shared__ __align__(16) float s_logits[MOE_MAX_EXPERTS];
    __shared__ Selection sel;
    extern __shared__ float xs[];
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
    __shared__ uint32_t s_tag;
    if (tid == 0) s_tag = launch_tag(a);
    int b = blockIdx.x;
    if (b < a.n_route) {
        const int row = b * 4 + wave;
        const int n_log = a.E + (a.wg ? 1 : 0);
        float v = 0.f;
        if (row < n_log)
            v = row < a.E ? layer_row_dot<XT>(a.wr, row, a.x, a.d_in, lane)
                          : layer_row_dot<XT>(a.wg, 0, a.x, a.d_in, lane);
        v = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));   // one value for every copy
        __syncthreads();
        if (row < n_log && lane < kLogitCopies) st_tagged(a.logits + (int64_t)lane * a.logit_stride + row, v, s_tag);
        return;
    }
    __syncthreads();
    const uint32_t tag = s_tag;
    b -= a.n_route;
    const int n_a = a.K * a.a_tiles_r + a.S * a.a_tiles_s;
    bool is_a = b < n_a;
    int slot, tile;
    if (a.by_xcd) {
        // Workgroups go to the 8 XCDs round robin (block i to XCD i mod 8), and
        // the router blocks are a multiple of 8: in this order every unit of
        // slot s lands on XCD s, so the act hand-off between the slot's A and
        // B units stays within one XCD and its L2 (a round trip between two
        // workgroups measures ~1.0 us within an XCD, ~1.5 us across).  Every
        // slot has the same tile counts; the order still waits only on lower
        // block indices (A tiles of a slot, then its B tiles; the tail's slot
        // is the last of each group of 8).
        slot = b % 8;
        const int q = b / 8;
        is_a = q < a.a_tiles_r;
        tile = is_a ? q : q - a.a_tiles_r;
    } else if (!is_a) {
        b -= n_a;
        slot = b / a.b_tiles;
        tile = b % a.b_tiles;
    } else if (b < a.K * a.a_tiles_r) {
        slot = b / a.a_tiles_r;
        tile = b % a.a_tiles_r;
    } else {
        const int bs = b - a.K * a.a_tiles_r;
        slot = a.K + bs / a.a_tiles_s;
        tile = bs % a.a_tiles_s;
    }
    // kernel-A units stage x in LDS while the logits are on their way: the
    // weight stream then shares the memory pipeline with nothing else
    if (is_a) stage_x_raw<XT, Fmt<BA>::kCodes>(a.x, a.d_in / Fmt<BA>::kCodes, xs);
    // routed units rank the logits themselves (one copy of this code for both
    // roles): no extra hand-off
    int e = slot - a.K;
    if (slot < a.K) {
        gather_logits(a, tag, s_logits, &sel);
        select_all(a.E, a.K, s_logits, &sel);
        e = sel.ids[slot];
    } else {
        __syncthreads();
    }
    if (is_a) {
        if constexpr (ANR == kLayerNRA) layer_a_unit_single<BA, SB, XT>(a, tag, slot, tile, e, xs);
        else layer_a_unit_pipelined<BA, SB, XT>(a, tag, slot, tile, e, xs);
    }
    // the kernels with pipelined kernel-A units (the large layers) read act
    // through the L2 first: there each slot's act vector is read by a hundred
    // or more kernel-B units, and sharing the lines within an XCD took the
    // Qwen1.5- and dots.llm1-shaped layers from 31.1 / 36.5 to 30.6 / 35.7 us
    // per launch, while the Qwen3-shaped layer (single-stage units, 768-word
    // act vectors) measured 14.7 -> 14.9-15.2 us with it
    else layer_b_unit<BB, SB, ANR == kLayerNRA2>(a, tag, slot, tile, e, s_logits, &sel, xs);
}

using LayerFn = void (*)(LayerArgs);

// Instantiation tables, one translation unit per gate/up bit width and
// kernel-A unit kind (single stage, pipelined).
LayerFn layer_kernel_a4(int bb, int sb, int xt);
LayerFn layer_kernel_a6(int bb, int sb, int xt);
LayerFn layer_kernel_a8(int bb, int sb, int xt);
LayerFn layer_kernel_a4p(int bb, int sb, int xt);
LayerFn layer_kernel_a6p(int bb, int sb, int xt);
LayerFn layer_kernel_a8p(int bb, int sb, int xt);

template <int BA, int ANR>
LayerFn layer_kernel_pick(int bb, int sb, int xt) {
#define MOE_L(BB, S, X) \
    if (bb == BB && sb == S && xt == X) return layer_kernel<BA, BB, S, X, ANR>;
#define MOE_LX(BB, S) MOE_L(BB, S, MOE_F32) MOE_L(BB, S, MOE_F16) MOE_L(BB, S, MOE_BF16)
    MOE_LX(4, MOE_BF16) MOE_LX(4, MOE_F16)
    MOE_LX(6, MOE_BF16) MOE_LX(6, MOE_F16)
    MOE_LX(8, MOE_BF16) MOE_LX(8, MOE_F16)
#undef MOE_LX
#undef MOE_L
    return nullptr;
}

}  // namespace moe
