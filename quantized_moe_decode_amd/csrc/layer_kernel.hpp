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
// trip.  B units issue the loads of their first weight chunks before they
// wait for their slot's act vector, so the down-projection weights stream
// while kernel A runs.  The B unit of the last slot of each row tile (the
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

namespace moe {

constexpr int kLayerNRA = 4;        // rows per lane group, kernel A units
constexpr int kLayerNRB = 4;        // rows per lane group, kernel B units
constexpr int kCtrStride = 64;      // uint32 words between control words (256 bytes)
constexpr uint32_t kSpinLimit = 1u << 19;

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
    float *out;
    int32_t *ids_out;
    float *scores_out;
    float *gate_out;
    uint64_t *logits;               // [E + 1] tagged
    uint64_t *act;                  // [K + S][act_stride] tagged
    int act_stride;
    uint64_t *partial;              // [K + S][d_in] tagged
    uint32_t *ctr;                  // control words
    int n_route;
    int a_lr_shift, a_tile, a_tiles_r, a_tiles_s;
    int b_lr_shift_r, b_lr_shift_s, b_tile, b_tiles;
};

__device__ __forceinline__ uint32_t *ctr_at(const LayerArgs &a, int slot) { return a.ctr + slot * kCtrStride; }

__device__ __forceinline__ void st_tagged(uint64_t *p, float v, uint32_t tag) {
    const uint64_t w = ((uint64_t)tag << 32) | (uint64_t)__float_as_uint(v);
    __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Poll one tagged word until it carries `tag`; returns its value (0 and the
// error word raised on time-out).
__device__ __forceinline__ float wait_tagged(const LayerArgs &a, const uint64_t *p, uint32_t tag) {
    for (uint32_t i = 0; i < kSpinLimit; ++i) {
        const uint64_t w = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if ((uint32_t)(w >> 32) == tag) return __uint_as_float((uint32_t)w);
        __builtin_amdgcn_s_sleep(2);
    }
    __hip_atomic_fetch_or(ctr_at(a, kCtrErr), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return 0.f;
}

// Gather n tagged words p[0..n): thread 0 first polls the last one (producers
// finish at about the same time), then every thread reads its words, and only
// words not yet tagged are polled again.  f(i, value) consumes word i.  This
// keeps the polling traffic of a workgroup to one address instead of n.
template <typename Fn>
__device__ __forceinline__ void gather_tagged(const LayerArgs &a, const uint64_t *p, int n, uint32_t tag, Fn f) {
    if (threadIdx.x == 0) (void)wait_tagged(a, p + n - 1, tag);
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += blockDim.x) f(i, wait_tagged(a, p + i, tag));
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

struct Selection {
    int ids[MOE_MAX_TOP_K];
    float scores[MOE_MAX_TOP_K];
    float gate;
};

// Top-k in one wave, PER logits per lane (expert lane + 64*i in l[i]): rounds
// of "largest untaken logit" (a DPP wave maximum), each taking the lowest
// expert id that holds that value (a ballot), i.e. descending logit with ties
// to the lower id.  Lane k ends with the k-th id and logit.  Rounds [k0, k1)
// run per call, so a caller can stop at the rank it needs and resume later.
template <int PER>
struct TopK {
    float l[PER];
    uint32_t taken;
    int my_id;
    float my_logit, mx;

    __device__ __forceinline__ void init(const float *s_logits, int E, int lane) {
        taken = 0;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int e = lane + i * kWave;
            l[i] = e < E ? s_logits[e] : -INFINITY;
            if (e >= E) taken |= 1u << i;
        }
        my_id = -1;
        my_logit = 0.f;
        mx = 0.f;
    }

    __device__ __forceinline__ void rounds(int k0, int k1, int lane) {
        for (int k = k0; k < k1; ++k) {
            float best = -INFINITY;
#pragma unroll
            for (int i = 0; i < PER; ++i) best = ((taken >> i) & 1u) ? best : fmaxf(best, l[i]);
            const float m = wave_max(best);
            int e = -1;
#pragma unroll
            for (int i = 0; i < PER; ++i) {
                const uint64_t hit = __ballot(!((taken >> i) & 1u) && l[i] == m);
                if (e < 0 && hit) e = i * kWave + (int)__ffsll((unsigned long long)hit) - 1;
            }
            if (k == 0) mx = m;
            if (lane == k) {
                my_id = e;
                my_logit = m;
            }
            if ((e & (kWave - 1)) == lane) taken |= 1u << ((e / kWave) & 31);
        }
    }

    // softmax over all E logits; lanes < K get their selection's score
    __device__ __forceinline__ float score(int E, int K, bool renorm, int lane) const {
        float zz = 0.f;
#pragma unroll
        for (int i = 0; i < PER; ++i) zz += (lane + i * kWave < E) ? __expf(l[i] - mx) : 0.f;
        const float z = wave_sum(zz);
        const float p = lane < K ? __expf(my_logit - mx) / z : 0.f;
        const float psum = wave_sum(p);
        return renorm ? p / psum : p;
    }
};

// Wave 0 runs the selection; the other waves wait at the barriers.  With
// need_scores == false only the ids of ranks [0, upto] are produced; a later
// finish_selection() completes the ranks and the scores.
template <int PER>
__device__ void select_impl(const LayerArgs &a, const float *s_logits, Selection *sel, int upto, bool all,
                            TopK<PER> &tk) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
    if (wave == 0) {
        tk.init(s_logits, a.E, lane);
        const int k1 = all ? a.K : upto + 1;
        tk.rounds(0, k1, lane);
        if (lane < k1) sel->ids[lane] = tk.my_id;
        if (all) {
            const float sc = tk.score(a.E, a.K, a.renorm, lane);
            if (lane < a.K) sel->scores[lane] = sc;
        }
    }
    __syncthreads();
}

template <int PER>
__device__ void finish_impl(const LayerArgs &a, Selection *sel, int done, TopK<PER> &tk) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
    if (wave == 0) {
        tk.rounds(done, a.K, lane);
        const float sc = tk.score(a.E, a.K, a.renorm, lane);
        if (lane < a.K) {
            sel->ids[lane] = tk.my_id;
            sel->scores[lane] = sc;
        }
    }
    __syncthreads();
}

// Wait for every router logit and stage them in LDS (plus the shared gate).
__device__ void gather_logits(const LayerArgs &a, uint32_t tag, float *s_logits, Selection *sel) {
    gather_tagged(a, a.logits, a.E, tag, [&](int e, float v) { s_logits[e] = v; });
    if (threadIdx.x == 0) sel->gate = a.wg ? sigmoidf_(wait_tagged(a, a.logits + a.E, tag)) : 1.0f;
    __syncthreads();
}

// Dispatch on the number of logits per lane of the selection wave.
template <typename Fn>
__device__ __forceinline__ void with_per(int E, Fn fn) {
    const int per = (E + kWave - 1) / kWave;
    if (per <= 1) fn(TopK<1>{});
    else if (per <= 2) fn(TopK<2>{});
    else if (per <= 4) fn(TopK<4>{});
    else if (per <= 8) fn(TopK<8>{});
    else fn(TopK<16>{});
}

__device__ __forceinline__ int n_slots(const LayerArgs &a) { return a.K + a.S; }

// Kernel A unit: rows [row0, row0 + a_tile) of slot `slot`.
template <int BA, int SB, int XT>
__device__ void layer_a_unit(const LayerArgs &a, uint32_t tag, int slot, int tile, float *s_logits,
                             Selection *sel) {
    constexpr int NR = kLayerNRA;
    using F = Fmt<BA>;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
    const bool routed = slot < a.K;
    int e;
    if (routed) {
        gather_logits(a, tag, s_logits, sel);
        with_per(a.E, [&](auto tk) { select_impl(a, s_logits, sel, slot, false, tk); });
        e = sel->ids[slot];
    } else {
        e = slot - a.K;
    }
    const int dff = routed ? a.d_ff : a.d_ffs;
    const int E = routed ? a.E : a.S;
    const int row0 = tile * a.a_tile;
    const int row_end = min(row0 + a.a_tile, dff);
    uint64_t *act = a.act + (int64_t)slot * a.act_stride;
    if (e < 0 || e >= E) {
        for (int r = row0 + tid; r < row_end; r += blockDim.x) st_tagged(act + r, 0.f, tag);
        return;
    }
    const QM mats[2] = {routed ? a.gate : a.sgate, routed ? a.up : a.sup};
    const int64_t erow0 = (int64_t)e * dff;
    const int cpr = a.d_in / F::kCodes;
    const int lr = 1 << a.a_lr_shift, j = lane & (lr - 1), rsub = lane >> a.a_lr_shift, rpw = kWave >> a.a_lr_shift;
    // stages = (row pass, chunk position), each loaded and then consumed
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
        BlockRegs<BA, 2, NR> cur;
        load_block<BA, 2, NR>(cur, mats, erow0, r0, rpw, row_end, ch * lr + j, cpr);
        if constexpr (BA == 4 && XT == MOE_BF16) {
            // raw bf16 inputs for the packed-dot path
            const u32x4 *xp = reinterpret_cast<const u32x4 *>(reinterpret_cast<const uint16_t *>(a.x) +
                                                               (int64_t)cur.cc * F::kCodes);
            uint32_t xw[16];
            float xsum = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const u32x4 v = xp[i];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    xw[4 * i + k] = v[k];
                    xsum += __uint_as_float(v[k] << 16) + __uint_as_float(v[k] & 0xFFFF0000u);
                }
            }
            dot_block_q4_bf16<SB, 2, NR>(cur, xw, xsum, acc);
        } else {
            float xv[F::kCodes];
            load_x_chunk<XT, F::kCodes>(a.x, (int64_t)cur.cc * F::kCodes, xv);
            dot_block<BA, SB, 2, NR>(cur, xv, sum_n<F::kCodes>(xv), acc);
        }
        if (ch == n_chunk - 1) {
#pragma unroll
            for (int n = 0; n < NR; ++n) {
                acc[0][n] = group_sum(acc[0][n], lr);
                acc[1][n] = group_sum(acc[1][n], lr);
            }
            if (j == 0) {
#pragma unroll
                for (int n = 0; n < NR; ++n) {
                    const int r = r0 + n * rpw;
                    if (r < row_end) {
                        const float g = acc[0][n], u = acc[1][n];
                        st_tagged(act + r, g * sigmoidf_(g) * u, tag);
                    }
                }
            }
        }
    }
}

// Kernel B unit: rows [row0, row0 + b_tile) of d_in for slot `slot`.  The
// unit of the last slot also runs the tail for those rows.
template <int BB, int SB>
__device__ void layer_b_unit(const LayerArgs &a, uint32_t tag, int slot, int tile, float *s_logits,
                             Selection *sel, float *xs) {
    constexpr int NR = kLayerNRB;
    using F = Fmt<BB>;
    constexpr int CODES = F::kCodes;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
    const bool routed = slot < a.K;
    int e;
    float score = 1.0f;
    if (routed) {            // ranks up to this slot first: enough to start loading weights
        gather_logits(a, tag, s_logits, sel);
        with_per(a.E, [&](auto tk) { select_impl(a, s_logits, sel, slot, false, tk); });
        e = sel->ids[slot];
    } else {
        e = slot - a.K;
    }
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
    __shared__ float s_own[MOE_MAX_DIM / 4];      // own partial rows, kept for the tail

    // stages = (row pass, chunk position); stage 0 is loaded before act is ready
    const int rb0 = row0 + wave * rpw * NR, pass_rows = 4 * rpw * NR;
    const int n_pass = (valid && rb0 < row_end) ? (row_end - rb0 + pass_rows - 1) / pass_rows : 0;
    const int n_chunk = (cpr + lr - 1) / lr;
    const int n_stage = n_pass * n_chunk;
    BlockRegs<BB, 1, NR> cur;
    if (n_stage > 0) load_block<BB, 1, NR>(cur, mats, erow0, rb0 + rsub, rpw, row_end, j, cpr);

    if (routed) {            // full selection and scores while the weights and act are in flight
        with_per(a.E, [&](auto tk) { select_impl(a, s_logits, sel, 0, true, tk); });
        score = sel->scores[slot];
        if (slot == 0 && tile == 0) {            // publish the routing result once
            if (tid < a.K) {
                if (a.ids_out) a.ids_out[tid] = sel->ids[tid];
                if (a.scores_out) a.scores_out[tid] = sel->scores[tid];
            }
            if (tid == 0 && a.gate_out && a.wg) a.gate_out[0] = sel->gate;
        }
    }

    if (valid) {
        const uint64_t *act = a.act + (int64_t)slot * a.act_stride;
        gather_tagged(a, act, cpr * CODES, tag, [&](int i, float v) {
            const int c = i / CODES;
            xs[c * (CODES + 4) + (i - c * CODES)] = v;
        });
        __syncthreads();
        float acc[1][NR];
        for (int st = 0; st < n_stage; ++st) {
            const int ps = st / n_chunk, ch = st - ps * n_chunk;
            const int r0 = rb0 + ps * pass_rows + rsub;
            if (ch == 0) {
#pragma unroll
                for (int n = 0; n < NR; ++n) acc[0][n] = 0.f;
            }
            if (st > 0) load_block<BB, 1, NR>(cur, mats, erow0, r0, rpw, row_end, ch * lr + j, cpr);
            float xv[CODES];
            read_staged<CODES>(staged_chunk<CODES>(xs, 0, cpr, cur.cc), xv);
            dot_block<BB, SB, 1, NR>(cur, xv, sum_n<CODES>(xv), acc);
            if (ch == n_chunk - 1) {
#pragma unroll
                for (int n = 0; n < NR; ++n) acc[0][n] = group_sum(acc[0][n], lr);
                if (j == 0) {
#pragma unroll
                    for (int n = 0; n < NR; ++n) {
                        const int r = r0 + n * rpw;
                        if (r < row_end) {
                            const float v = score * acc[0][n];
                            if (last_slot) s_own[r - row0] = v;
                            else st_tagged(part + r, v, tag);
                        }
                    }
                }
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
        s_gate = a.wg ? sigmoidf_(wait_tagged(a, a.logits + a.E, tag)) : 1.0f;
    __syncthreads();
    const float g = s_gate;
    const int ns = n_slots(a);
    for (int r = row0 + tid; r < row_end; r += blockDim.x) {
        auto pv = [&](int s2) {
            return s2 == ns - 1 ? s_own[r - row0] : wait_tagged(a, a.partial + (int64_t)s2 * a.d_in + r, tag);
        };
        float routed_sum = pv(0);
        for (int k = 1; k < a.K; ++k) routed_sum += pv(k);
        float sh = 0.f;
        if (a.S > 0) {
            sh = pv(a.K);
            for (int s2 = a.K + 1; s2 < ns; ++s2) sh += pv(s2);
        }
        a.out[r] = load_act(a.resid, a.resid_dt, r) + (routed_sum + sh * g);
    }
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

template <int BA, int BB, int SB, int XT>
__global__ __launch_bounds__(256, 3) void layer_kernel(LayerArgs a) {
    __shared__ float s_logits[MOE_MAX_EXPERTS];
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
        __syncthreads();
        if (row < n_log && lane == 0) st_tagged(a.logits + row, v, s_tag);
        return;
    }
    __syncthreads();
    const uint32_t tag = s_tag;
    b -= a.n_route;
    const int n_a = a.K * a.a_tiles_r + a.S * a.a_tiles_s;
    if (b < n_a) {
        int slot, tile;
        if (b < a.K * a.a_tiles_r) {
            slot = b / a.a_tiles_r;
            tile = b % a.a_tiles_r;
        } else {
            const int bs = b - a.K * a.a_tiles_r;
            slot = a.K + bs / a.a_tiles_s;
            tile = bs % a.a_tiles_s;
        }
        layer_a_unit<BA, SB, XT>(a, tag, slot, tile, s_logits, &sel);
    } else {
        b -= n_a;
        layer_b_unit<BB, SB>(a, tag, b / a.b_tiles, b % a.b_tiles, s_logits, &sel, xs);
    }
}

using LayerFn = void (*)(LayerArgs);

// Instantiation tables, one translation unit per gate/up bit width.
LayerFn layer_kernel_a4(int bb, int sb, int xt);
LayerFn layer_kernel_a6(int bb, int sb, int xt);
LayerFn layer_kernel_a8(int bb, int sb, int xt);

template <int BA>
LayerFn layer_kernel_pick(int bb, int sb, int xt) {
#define MOE_L(BB, S, X) \
    if (bb == BB && sb == S && xt == X) return layer_kernel<BA, BB, S, X>;
#define MOE_LX(BB, S) MOE_L(BB, S, MOE_F32) MOE_L(BB, S, MOE_F16) MOE_L(BB, S, MOE_BF16)
    MOE_LX(4, MOE_BF16) MOE_LX(4, MOE_F16)
    MOE_LX(6, MOE_BF16) MOE_LX(6, MOE_F16)
    MOE_LX(8, MOE_BF16) MOE_LX(8, MOE_F16)
#undef MOE_LX
#undef MOE_L
    return nullptr;
}

}  // namespace moe
