// Routing: router GEMV, softmax over all experts, top-k and scores, and the
// optional shared-expert gate (Red Lite dev39, "Change": the layer is
// GPU-routed; the shared expert's output is scaled by a scalar gate).
//
// One launch.  Workgroups of four waves each compute four router logits of
// one token (one wave per router row, fp32 accumulation over the contraction
// with a wave64 butterfly reduction).  The router matrix is read once, spread
// over many CUs.  Each logit is published as one 64-bit word, the fp32 value
// and above it the launch's tag (1 + the launch epoch kept in the workspace),
// written with one device-scope store.  The last workgroup of each token's
// row of the grid (every other one has a lower index, so in-order dispatch
// cannot deadlock) polls that token's words until all carry the tag, stages
// the logits in LDS, selects the top-k with the whole block (topk.hpp) and
// computes the scores.  The last selector to finish moves the workspace to
// the next epoch, once every workgroup of the launch has read the tag, so a
// word left by an earlier launch (or written late by one whose wait ran out)
// never matches a later launch's tag.  Every wait is bounded; on time-out the
// workspace's error word is raised and stays raised.  No cache-wide fence is
// involved.
//
// Many tokens (a prefill chunk, more than MOE_MAX_TOKENS) with bf16 x, router
// and gate vector take two launches instead: the logits of every token as one
// matrix product on the matrix cores (route_logits_mfma: each workgroup a
// tile of 16 tokens x 16 router rows, its four waves splitting the
// contraction, v_mfma_f32_16x16x32_bf16, products exact and fp32 sums), so
// the router matrix is read once per 16 tokens instead of once per token; then one workgroup per token selects and scores
// (route_select_kernel), stream-ordered after the first, so no tags or waits.
// Its logits go to the same workspace words with tag 0, which no tagged
// launch ever expects (tags are 1 + the epoch).
#include <hip/hip_runtime.h>
#include <math.h>

#include "api.hpp"
#include "common.hpp"
#include "topk.hpp"

namespace moe {

constexpr int kRouteWaves = 4;

struct RouteArgs {
    const void *x;
    const void *wr;
    const void *wg;          // shared gate vector or null
    int x_dt, wr_dt, wg_dt;
    int T, d_in, E, K, renorm;
    int32_t *ids;
    float *scores;
    float *gate;
    uint64_t *logits;        // workspace [T][E + 1] tagged words
    uint32_t *ctr;           // workspace control words, kRouteCtrStride apart: error, epoch, selectors done
};

// Eight consecutive elements of a row as floats (one 16-byte load for 16-bit
// dtypes, two for fp32).
template <int DT>
__device__ __forceinline__ void load8(const void *base, int64_t elem, float *v) {
    if constexpr (DT == MOE_F32) {
        const f32x4 *p = reinterpret_cast<const f32x4 *>(reinterpret_cast<const float *>(base) + elem);
        const f32x4 a = p[0], b = p[1];
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
        const u32x4 w = *reinterpret_cast<const u32x4 *>(reinterpret_cast<const uint16_t *>(base) + elem);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if constexpr (DT == MOE_BF16) {
                v[2 * k] = __uint_as_float(w[k] << 16);
                v[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
            } else {
                _Float16 lo, hi;
                const uint16_t l16 = (uint16_t)(w[k] & 0xFFFFu), h16 = (uint16_t)(w[k] >> 16);
                __builtin_memcpy(&lo, &l16, 2);
                __builtin_memcpy(&hi, &h16, 2);
                v[2 * k] = (float)lo;
                v[2 * k + 1] = (float)hi;
            }
        }
    }
}

// One router (or shared-gate) row dotted with x: lane l takes the 8-element
// chunks l, l+64, ...; up to four chunks' loads are in flight before use.
template <int XT, int WT>
__device__ float row_dot(const void *w, int64_t row, const void *x, int64_t xrow, int d_in, int lane) {
    const int nch = d_in / 8;
    float acc = 0.f;
    for (int base = 0; base < nch; base += 4 * kWave) {
        float wv[4][8], xv[4][8];
        bool ok[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int c = base + u * kWave + lane;
            ok[u] = c < nch;
            const int cc = ok[u] ? c : 0;     // in-bounds address; masked below
            load8<WT>(w, row * d_in + 8 * cc, wv[u]);
            load8<XT>(x, xrow * d_in + 8 * cc, xv[u]);
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

constexpr uint32_t kRouteSpinLimit = 1u << 22;
constexpr int kRouteCtrStride = 64;          // uint32 words between control words (256 bytes)
constexpr int kRouteCtrErr = 0, kRouteCtrEpoch = 1, kRouteCtrDone = 2;
constexpr size_t kRouteHeadBytes = 1024;     // control words, then the tagged logits

// Wait for one tagged logit word and return its value (0, with the error word
// raised, if the wait runs out).
__device__ __forceinline__ float wait_logit(const RouteArgs &a, const uint64_t *w, uint32_t tag) {
    for (uint32_t i = 0; i < kRouteSpinLimit; ++i) {
        const uint64_t v = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if ((uint32_t)(v >> 32) == tag) return __uint_as_float((uint32_t)v);
        __builtin_amdgcn_s_sleep(1);
    }
    __hip_atomic_fetch_or(a.ctr + kRouteCtrErr * kRouteCtrStride, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return 0.f;
}

template <int XT, int WT, int GT>
__global__ __launch_bounds__(256) void route_kernel(RouteArgs a) {
    const int t = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
    const int n_rows = a.E + (a.wg ? 1 : 0);
    uint64_t *logits = a.logits + (int64_t)t * (a.E + 1);
    __shared__ uint32_t s_tag;
    if (tid == 0)
        s_tag = __hip_atomic_load(a.ctr + kRouteCtrEpoch * kRouteCtrStride, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT) + 1u;
    __syncthreads();
    const uint32_t tag = s_tag;

    const int row = blockIdx.x * kRouteWaves + wave;
    if (row < n_rows) {
        const float v = (row < a.E) ? row_dot<XT, WT>(a.wr, row, a.x, t, a.d_in, lane)
                                    : row_dot<XT, GT>(a.wg, 0, a.x, t, a.d_in, lane);
        if (lane == 0)
            __hip_atomic_store(logits + row, ((uint64_t)tag << 32) | __float_as_uint(v), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
    if (blockIdx.x != gridDim.x - 1) return;

    // The token's selector: its logits into LDS as they are flagged, then the
    // block-wide top-k and, in one wave, the softmax scores.
    __shared__ __align__(16) float s_logits[MOE_MAX_EXPERTS];
    __shared__ Selection sel;
    __shared__ float s_gate_logit;
    stage_logits(a.E, s_logits, &sel, [&](int e) { return wait_logit(a, logits + e, tag); });
    if (tid == 0 && a.wg) s_gate_logit = wait_logit(a, logits + a.E, tag);
    __syncthreads();
    // every word of the token has been read, so every workgroup of this token
    // has read the tag: the last token's selector moves the workspace to the
    // next epoch
    if (tid == 0) {
        uint32_t *done = a.ctr + kRouteCtrDone * kRouteCtrStride;
        if (__hip_atomic_fetch_add(done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)a.T - 1) {
            __hip_atomic_store(done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(a.ctr + kRouteCtrEpoch * kRouteCtrStride, tag, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    select_all(a.E, a.K, s_logits, &sel);
    if (wave != 0) return;
    with_per(a.E, [&](auto per) { softmax_scores<decltype(per)::value>(a.E, a.K, a.renorm, s_logits, lane, &sel); });
    if (lane < a.K) {
        a.ids[t * a.K + lane] = sel.ids[lane];
        a.scores[t * a.K + lane] = sel.scores[lane];
    }
    if (lane == 0 && a.wg) a.gate[t] = 1.0f / (1.0f + expf(-s_gate_logit));
}

// ------------------------------------------------------------ many tokens
typedef __bf16 bf16x8r_t __attribute__((ext_vector_type(8)));
constexpr int kRouteMfmaRing = 8;                // k-steps of loads in flight per lane
constexpr int kRouteKSplit = 4;                  // waves per tile, each a share of the contraction

// logits[t][row] (tag 0) for rows < E + (wg ? 1 : 0), one 16-token x 16-row
// tile per workgroup: wave w takes the 32-wide k-steps w, w + 4, ...; lane
// (j, g) loads 8 inputs of token 16 by + j (the A operand) and 8 weights of
// row 16 bx + j (B) per k-step and ends with D[4 g + r][j]: token 4 g + r of
// the tile, row j.  The four waves' partial tiles are added through LDS in
// wave order.  Rows and tokens past the end are read clamped and not written.
__global__ __launch_bounds__(kRouteKSplit * kWave) void route_logits_mfma(RouteArgs a) {
    __shared__ f32x4 s_part[kRouteKSplit - 1][kWave];
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
    const int g = lane >> 4, j = lane & 15;
    const int n_rows = a.E + (a.wg ? 1 : 0);
    const int row = blockIdx.x * 16 + j, t0 = blockIdx.y * 16;
    const int rc = min(row, n_rows - 1);
    const uint16_t *w = rc < a.E ? reinterpret_cast<const uint16_t *>(a.wr) + (int64_t)rc * a.d_in
                                 : reinterpret_cast<const uint16_t *>(a.wg);
    const uint16_t *x = reinterpret_cast<const uint16_t *>(a.x) + (int64_t)min(t0 + j, a.T - 1) * a.d_in;
    const int n_step = a.d_in / 32;                  // this wave's k-steps: wave, wave + 4, ... < n_step
    const int n_mine = (n_step - wave + kRouteKSplit - 1) / kRouteKSplit;
    u32x4 xa[kRouteMfmaRing], wb[kRouteMfmaRing];
#pragma unroll
    for (int d = 0; d < kRouteMfmaRing; ++d) {
        const int sd = min(wave + kRouteKSplit * d, n_step - 1);
        xa[d] = *reinterpret_cast<const u32x4 *>(x + 32 * sd + 8 * g);
        wb[d] = *reinterpret_cast<const u32x4 *>(w + 32 * sd + 8 * g);
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int i0 = 0; i0 < n_mine; i0 += kRouteMfmaRing) {
#pragma unroll
        for (int d = 0; d < kRouteMfmaRing; ++d) {
            const u32x4 av = xa[d], bv = wb[d];
            const int sn = min(wave + kRouteKSplit * (i0 + d + kRouteMfmaRing), n_step - 1);   // refill (clamped)
            xa[d] = *reinterpret_cast<const u32x4 *>(x + 32 * sn + 8 * g);
            wb[d] = *reinterpret_cast<const u32x4 *>(w + 32 * sn + 8 * g);
            if (i0 + d < n_mine)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8r_t, av),
                                                              __builtin_bit_cast(bf16x8r_t, bv), acc, 0, 0, 0);
        }
    }
    if (wave > 0) s_part[wave - 1][lane] = acc;
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int q = 0; q < kRouteKSplit - 1; ++q) {
        const f32x4 p = s_part[q][lane];
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] += p[r];
    }
    if (row < n_rows) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = t0 + 4 * g + r;
            if (t < a.T) a.logits[(int64_t)t * (a.E + 1) + row] = (uint64_t)__float_as_uint(acc[r]);
        }
    }
}

// One workgroup per token: the token's logits (left by route_logits_mfma on
// the same stream) staged in LDS, the block-wide top-k, the scores and the
// shared gate, as in route_kernel's selector.
__global__ __launch_bounds__(256) void route_select_kernel(RouteArgs a) {
    const int t = blockIdx.x, tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
    const uint64_t *logits = a.logits + (int64_t)t * (a.E + 1);
    __shared__ __align__(16) float s_logits[MOE_MAX_EXPERTS];
    __shared__ Selection sel;
    stage_logits(a.E, s_logits, &sel, [&](int e) { return __uint_as_float((uint32_t)logits[e]); });
    __syncthreads();
    select_all(a.E, a.K, s_logits, &sel);
    if (wave != 0) return;
    with_per(a.E, [&](auto per) { softmax_scores<decltype(per)::value>(a.E, a.K, a.renorm, s_logits, lane, &sel); });
    if (lane < a.K) {
        a.ids[t * a.K + lane] = sel.ids[lane];
        a.scores[t * a.K + lane] = sel.scores[lane];
    }
    if (lane == 0 && a.wg) a.gate[t] = 1.0f / (1.0f + expf(-__uint_as_float((uint32_t)logits[a.E])));
}

using RouteFn = void (*)(RouteArgs);

template <int XT, int WT>
static RouteFn pick_route_g(int gt) {
    switch (gt) {
    case MOE_F32: return route_kernel<XT, WT, MOE_F32>;
    case MOE_F16: return route_kernel<XT, WT, MOE_F16>;
    default: return route_kernel<XT, WT, MOE_BF16>;
    }
}

template <int XT>
static RouteFn pick_route_w(int wt, int gt) {
    switch (wt) {
    case MOE_F32: return pick_route_g<XT, MOE_F32>(gt);
    case MOE_F16: return pick_route_g<XT, MOE_F16>(gt);
    default: return pick_route_g<XT, MOE_BF16>(gt);
    }
}

static RouteFn pick_route(int xt, int wt, int gt) {
    switch (xt) {
    case MOE_F32: return pick_route_w<MOE_F32>(wt, gt);
    case MOE_F16: return pick_route_w<MOE_F16>(wt, gt);
    default: return pick_route_w<MOE_BF16>(wt, gt);
    }
}

}  // namespace moe

using namespace moe;

extern "C" size_t moe_decode_route_workspace_bytes(int32_t n_tokens, int32_t n_experts) {
    if (n_tokens < 1 || n_experts < 1) return 0;
    return kRouteHeadBytes + align_up((size_t)n_tokens * (n_experts + 1) * sizeof(uint64_t), 256);
}

extern "C" moe_status moe_decode_workspace_status(const void *head, size_t head_bytes) {
    if (!head || head_bytes < MOE_WORKSPACE_HEAD_BYTES) return MOE_EINVAL;
    uint32_t err;
    __builtin_memcpy(&err, head, sizeof err);
    return err ? MOE_ETIMEOUT : MOE_OK;
}

extern "C" moe_status moe_decode_route(const void *x, moe_dtype x_dtype_arg, int32_t n_tokens, int32_t d_in,
                                       const void *w_router, moe_dtype w_router_dtype_arg,
                                       int32_t n_experts, int32_t top_k, int32_t renormalize,
                                       const void *w_shared_gate, moe_dtype w_shared_gate_dtype_arg,
                                       int32_t *expert_ids, float *scores, float *shared_gate,
                                       void *workspace, size_t workspace_bytes, void *stream) {
    const int x_dtype = raw_enum(x_dtype_arg), w_router_dtype = raw_enum(w_router_dtype_arg),
              w_shared_gate_dtype = raw_enum(w_shared_gate_dtype_arg);
    if (!x || !w_router || !expert_ids || !scores || !workspace) return MOE_EINVAL;
    if ((w_shared_gate == nullptr) != (shared_gate == nullptr)) return MOE_EINVAL;
    if (n_tokens < 1 || n_tokens > MOE_MAX_GROUPED_TOKENS) return MOE_EINVAL;
    if (n_experts < 1 || n_experts > MOE_MAX_EXPERTS) return MOE_EINVAL;
    if (top_k < 1 || top_k > MOE_MAX_TOP_K || top_k > n_experts) return MOE_EINVAL;
    if (d_in < kGroup || d_in > MOE_MAX_DIM || d_in % kGroup) return MOE_EINVAL;
    if (!valid_dtype(x_dtype) || !valid_dtype(w_router_dtype) ||
        (w_shared_gate && !valid_dtype(w_shared_gate_dtype)))
        return MOE_EUNSUPPORTED;
    if (!aligned16(x) || !aligned16(w_router) || (w_shared_gate && !aligned16(w_shared_gate)) ||
        !aligned16(workspace))
        return MOE_EINVAL;
    if (workspace_bytes < moe_decode_route_workspace_bytes(n_tokens, n_experts)) return MOE_EINVAL;

    RouteArgs a;
    a.x = x; a.wr = w_router; a.wg = w_shared_gate;
    a.x_dt = x_dtype; a.wr_dt = w_router_dtype; a.wg_dt = w_shared_gate_dtype;
    a.T = n_tokens; a.d_in = d_in; a.E = n_experts; a.K = top_k; a.renorm = renormalize ? 1 : 0;
    a.ids = expert_ids; a.scores = scores; a.gate = shared_gate;
    a.ctr = reinterpret_cast<uint32_t *>(workspace);
    a.logits = reinterpret_cast<uint64_t *>(reinterpret_cast<char *>(workspace) + kRouteHeadBytes);

    const int n_rows = n_experts + (w_shared_gate ? 1 : 0);
    if (n_tokens > MOE_MAX_TOKENS && x_dtype == MOE_BF16 && w_router_dtype == MOE_BF16 &&
        (!w_shared_gate || w_shared_gate_dtype == MOE_BF16)) {
        hipStream_t s = reinterpret_cast<hipStream_t>(stream);
        hipLaunchKernelGGL(route_logits_mfma, dim3((n_rows + 15) / 16, (n_tokens + 15) / 16), dim3(kRouteKSplit * kWave),
                           0, s, a);
        hipLaunchKernelGGL(route_select_kernel, dim3(n_tokens), dim3(256), 0, s, a);
        return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
    }
    dim3 grid((n_rows + kRouteWaves - 1) / kRouteWaves, n_tokens);
    RouteFn k = pick_route(x_dtype, w_router_dtype, w_shared_gate ? w_shared_gate_dtype : MOE_BF16);
    hipLaunchKernelGGL(k, grid, dim3(256), 0, reinterpret_cast<hipStream_t>(stream), a);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}
