// Top-k expert selection and the routing softmax for one token, by one
// 256-thread workgroup from logits staged in LDS (Red Lite dev39, "Change":
// routing runs on the GPU; the order is descending logit with ties to the
// lower expert id, the scores are the softmax over all experts of the
// selected ones, renormalised over the K when asked).
#pragma once

#include <math.h>

#include "api.hpp"
#include "common.hpp"

namespace moe {

// LDS state of one workgroup's selection: the result (ids in rank order,
// their scores, the shared-expert gate) and the selection's scratch.
struct Selection {
    int ids[MOE_MAX_TOP_K];
    float scores[MOE_MAX_TOP_K];
    float gate;
    uint32_t n_over;                                  // a first-round wave had too many candidates
    __align__(16) uint64_t cand[kWave / 2];           // their (logit, id) keys, zero-padded
    __align__(16) uint32_t cand_key[MOE_MAX_TOP_K];   // the one-wave path's selected keys and ids
    int cand_id[MOE_MAX_TOP_K];                       // in id order, before ranking
};

template <int N>
struct IntC {
    static constexpr int value = N;
};

// Dispatch on the number of logit words per lane of a one-wave pass over E
// logits: two for up to 128 experts, else sixteen (the largest count); words
// past E hold nothing.  Two instantiations keep the kernel's code small.
template <typename Fn>
__device__ __forceinline__ void with_per(int E, Fn fn) {
    if (E <= 2 * kWave) fn(IntC<2>{});
    else fn(IntC<MOE_MAX_EXPERTS / kWave>{});
}

// Order-preserving image of an fp32 logit as an unsigned key (larger logit,
// larger key); -0 maps to the key of +0 so that equal values tie.
__device__ __forceinline__ uint32_t logit_key(float v) {
    const uint32_t u = __float_as_uint(v == 0.f ? 0.f : v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Number of keys >= c over the wave's PER key words (one ballot per word).
template <int PER>
__device__ __forceinline__ int count_ge(const uint32_t *key, uint32_t c) {
    int n = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) n += __popcll(__ballot(key[i] >= c));
    return n;
}

// Exact top-k in one wave, PER logits per lane (expert lane + 64*i in key i):
// descending logit, ties to the lower expert id.  It serves ties and large
// expert counts; its cost is one wave's serial instruction stream.
//  1. A threshold t with at least K keys >= t, raised two bits at a time from
//     the top: of the three candidates that set the next two bits, the largest
//     one that still has K keys at or above it is kept (three independent
//     ballot counts per step).  The search stops as soon as exactly K keys are
//     >= t, which the gap between the K-th and (K+1)-th logit usually allows
//     after a dozen bits; otherwise it ends with t equal to the K-th key.
//  2. The selection: every key above t, plus the lowest-id keys equal to t
//     until there are K.
//  3. The K selected (key, id) pairs are packed in id order into LDS, and the
//     first K lanes rank one pair each against all of them: larger keys, and
//     equal keys of lower id, come first.  Rank r stores its id in ids[r].
template <int PER>
__device__ __forceinline__ void topk_radix(const float *s_logits, int E, int K, int lane, Selection *sel) {
    uint32_t key[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = lane + i * kWave;
        key[i] = e < E ? logit_key(s_logits[e]) : 0u;    // 0 is below every finite logit's key
    }
    uint32_t t = 0;
    for (int b = 30; b >= 0; b -= 2) {
        const uint32_t c1 = t | (1u << b), c2 = t | (2u << b), c3 = t | (3u << b);
        const int n1 = count_ge<PER>(key, c1), n2 = count_ge<PER>(key, c2), n3 = count_ge<PER>(key, c3);
        int n;
        if (n3 >= K) { t = c3; n = n3; }
        else if (n2 >= K) { t = c2; n = n2; }
        else if (n1 >= K) { t = c1; n = n1; }
        else n = K + 1;
        if (n == K) break;
    }
    int need = K;
    uint64_t selm[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        selm[i] = __ballot(key[i] > t);
        need -= __popcll(selm[i]);
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {             // keys equal to t: lowest ids first
        uint64_t eq = __ballot(key[i] == t);
        const int c = __popcll(eq);
        if (c <= need) {
            selm[i] |= eq;
            need -= c;
        } else {
            for (; need > 0; --need) {
                selm[i] |= eq & (~eq + 1);      // lowest remaining set bit
                eq &= eq - 1;
            }
        }
    }
    int base = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        if ((selm[i] >> lane) & 1u) {
            const int pos = base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(selm[i] >> 32),
                                                                 __builtin_amdgcn_mbcnt_lo((uint32_t)selm[i], 0u));
            sel->cand_key[pos] = key[i];
            sel->cand_id[pos] = lane + i * kWave;
        }
        base += __popcll(selm[i]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (lane < K) {
        const uint32_t kt = sel->cand_key[lane];
        const uint4 *ck = reinterpret_cast<const uint4 *>(sel->cand_key);
        int rank = 0;
        for (int u0 = 0; u0 < K; u0 += 4) {
            const uint4 v = ck[u0 >> 2];
            const uint32_t kv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int u = u0 + q;
                rank += (u < K && (kv[q] > kt || (kv[q] == kt && u < lane))) ? 1 : 0;
            }
        }
        sel->ids[rank] = sel->cand_id[lane];
    }
}

// Softmax over all E logits in one wave, then the selected ranks'
// probabilities, renormalised over the K when asked; lane k writes scores[k].
template <int PER>
__device__ void softmax_scores(int E, int K, int renorm, const float *s_logits, int lane, Selection *sel) {
    const float mx = s_logits[sel->ids[0]];
    float zz = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = lane + i * kWave;
        zz += e < E ? __expf(s_logits[e] - mx) : 0.f;
    }
    const float z = wave_sum(zz);
    const float p = lane < K ? __expf(s_logits[sel->ids[lane]] - mx) / z : 0.f;
    const float psum = wave_sum(p);
    if (lane < K) sel->scores[lane] = renorm ? p / psum : p;
}

constexpr int kRankMaxE = 2 * kWave;    // the two-round selection handles E up to this
constexpr int kCandMax = kWave / 2;     // candidates the second round ranks
constexpr int kCandPerWave = kCandMax / 4;

// Stage one token's E logits for select_all (every thread of the block
// calls this, then a barrier must follow): -0 is stored as +0, the list is
// padded with -inf to kRankMaxE entries, and the selection's scratch cleared.
// logit(e) gives logit e.
template <typename Logit>
__device__ __forceinline__ void stage_logits(int E, float *s_logits, Selection *sel, Logit logit) {
    const int n = E > kRankMaxE ? E : kRankMaxE;
    for (int e = threadIdx.x; e < n; e += blockDim.x) {
        const float v = e < E ? logit(e) : -INFINITY;
        s_logits[e] = v == 0.f ? 0.f : v;
    }
    if (threadIdx.x == 0) sel->n_over = 0;
    if (threadIdx.x < kCandMax) sel->cand[threadIdx.x] = 0;
}

// All K ids, in rank order, in sel->ids.  The vector work of one selection
// is shared by every workgroup on the CU that selects at the same moment, so
// the fast path keeps it small and spread over all four waves:
//  1. wave w ranks logits 32w..32w+31 among themselves (two lanes per logit,
//     sixteen comparisons each: the sign of l_i - l_j, exact for finite
//     values once -0 is stored as +0).  A logit with fewer than K larger ones
//     in its group is a candidate; every true top-K logit is one.
//  2. if no group has more than 8 candidates (K <= 8 without ties at a
//     group's cut), wave 0 ranks the (at most 32) candidates by the key
//     (logit, then lower id first), unique per expert, and rank r < K stores
//     its id in ids[r].
// Otherwise (more experts, larger K, ties at the cut), the exact one-wave
// selection decides.  s_logits must hold -0 as +0 and be padded with -inf to
// kRankMaxE entries; n_over and cand[] must be zeroed before the preceding
// barrier.
__device__ __forceinline__ void select_all(int E, int K, const float *s_logits, Selection *sel) {
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
    bool exact = false;
    if (E <= kRankMaxE) {
        const int i = 32 * wave + (lane >> 1), h = lane & 1;
        const float li = s_logits[i];
        const f32x4 *row = reinterpret_cast<const f32x4 *>(s_logits + 32 * wave + 16 * h);
        f32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = row[u];
        uint32_t c4[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int u = 0; u < 4; ++u) {                   // l_j > l_i  <=>  l_i - l_j < 0
            c4[0] += __float_as_uint(li - v[u].x) >> 31;
            c4[1] += __float_as_uint(li - v[u].y) >> 31;
            c4[2] += __float_as_uint(li - v[u].z) >> 31;
            c4[3] += __float_as_uint(li - v[u].w) >> 31;
        }
        int cnt = (int)(c4[0] + c4[1] + c4[2] + c4[3]);
        cnt += __builtin_amdgcn_mov_dpp(cnt, 0xB1, 0xf, 0xf, false);    // quad_perm [1,0,3,2]
        const bool is_cand = h == 0 && i < E && cnt < K;
        const uint64_t bal = __ballot(is_cand);
        // wave w owns candidate places 8w..8w+7; a wave with more candidates
        // (K > 8, or ties) sends the selection to the exact path
        const int pos = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                      __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
        if (is_cand && pos < kCandPerWave)
            sel->cand[kCandPerWave * wave + pos] = ((uint64_t)logit_key(li) << 32) | (0xFFFFFFFFu - (uint32_t)i);
        if (lane == 0 && __popcll(bal) > kCandPerWave) sel->n_over = 1;
        __syncthreads();
        if (sel->n_over == 0) {
            if (wave == 0) {
                const int c = lane >> 1, hh = lane & 1;
                const uint64_t kc = sel->cand[c];           // 0 past the last candidate
                const uint64_t *cr = sel->cand + 16 * hh;
                int r = 0;
#pragma unroll
                for (int u = 0; u < 16; ++u) r += cr[u] > kc ? 1 : 0;
                r += __builtin_amdgcn_mov_dpp(r, 0xB1, 0xf, 0xf, false);
                if (hh == 0 && kc != 0 && r < K) sel->ids[r] = (int)(0xFFFFFFFFu - (uint32_t)kc);
            }
            __syncthreads();
            exact = true;
        }
    }
    if (!exact) {
        if (wave == 0)
            with_per(E, [&](auto per) { topk_radix<decltype(per)::value>(s_logits, E, K, lane, sel); });
        __syncthreads();
    }
}

}  // namespace moe
