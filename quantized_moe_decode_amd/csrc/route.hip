// Routing: router GEMV, softmax over all experts, top-k and scores, and the
// optional shared-expert gate (Red Lite dev39, "Change": the layer is
// GPU-routed; the shared expert's output is scaled by a scalar gate).
//
// One launch.  Workgroups of four waves each compute four router logits
// (one wave per router row, fp32 accumulation over the contraction with a
// wave64 butterfly reduction).  The router matrix is read once, spread over
// many CUs.  The last workgroup to finish a token (device-scope counter)
// selects the top-k from that token's logits and computes its scores; the
// counter is reset to zero by that workgroup, so the workspace stays clean
// for the next call (and for graph replays).
#include <hip/hip_runtime.h>
#include <math.h>

#include "api.hpp"
#include "common.hpp"

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
    float *logits;           // workspace [T][E + 1]
    uint32_t *counters;      // workspace [T]
};

// Dot product of a d_in-long row (dtype dt) with x staged as fp32 in LDS.
__device__ float row_dot(const void *w, int dt, int64_t row, int d_in, const float *xs, int lane) {
    float acc = 0.f;
    if (dt == MOE_F32) {
        const f32x4 *p = reinterpret_cast<const f32x4 *>(reinterpret_cast<const float *>(w) + row * d_in);
        for (int c = lane; c < d_in / 4; c += kWave) {
            const f32x4 v = p[c];
            acc += v.x * xs[4 * c] + v.y * xs[4 * c + 1] + v.z * xs[4 * c + 2] + v.w * xs[4 * c + 3];
        }
    } else {
        const u32x4 *p = reinterpret_cast<const u32x4 *>(reinterpret_cast<const uint16_t *>(w) + row * d_in);
        for (int c = lane; c < d_in / 8; c += kWave) {
            const u32x4 v = p[c];
            float part = 0.f;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                float a, b;
                if (dt == MOE_BF16) {
                    a = __uint_as_float(v[k] << 16);
                    b = __uint_as_float(v[k] & 0xFFFF0000u);
                } else {
                    _Float16 ha, hb;
                    const uint16_t la = (uint16_t)(v[k] & 0xFFFFu), lb = (uint16_t)(v[k] >> 16);
                    __builtin_memcpy(&ha, &la, 2);
                    __builtin_memcpy(&hb, &lb, 2);
                    a = (float)ha;
                    b = (float)hb;
                }
                part += a * xs[8 * c + 2 * k] + b * xs[8 * c + 2 * k + 1];
            }
            acc += part;
        }
    }
    return wave_sum(acc);
}

__global__ __launch_bounds__(256) void route_kernel(RouteArgs a) {
    extern __shared__ float xs[];   // [d_in] fp32
    __shared__ int s_last;
    const int t = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
    const int n_rows = a.E + (a.wg ? 1 : 0);

    for (int j = tid; j < a.d_in; j += blockDim.x)
        xs[j] = load_act(a.x, a.x_dt, (int64_t)t * a.d_in + j);
    __syncthreads();

    const int row = blockIdx.x * kRouteWaves + wave;
    if (row < n_rows) {
        float v = (row < a.E) ? row_dot(a.wr, a.wr_dt, row, a.d_in, xs, lane)
                              : row_dot(a.wg, a.wg_dt, 0, a.d_in, xs, lane);
        if (lane == 0) a.logits[(int64_t)t * (a.E + 1) + row] = v;
    }

    // Last-arriving workgroup of this token does the selection.
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        const uint32_t prev = atomicAdd(&a.counters[t], 1u);
        s_last = (prev == gridDim.x - 1);
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    if (wave != 0) return;

    const float *l = a.logits + (int64_t)t * (a.E + 1);
    // Each lane owns experts lane, lane+64, ... (at most 16 of them).
    constexpr int kPer = MOE_MAX_EXPERTS / kWave;
    float mine[kPer];
    uint32_t taken = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int e = lane + i * kWave;
        mine[i] = (e < a.E) ? l[e] : -INFINITY;
    }
    int my_id = -1;           // lane k keeps the k-th selection
    float my_logit = 0.f, mx = 0.f;
    for (int k = 0; k < a.K; ++k) {
        float bv = -INFINITY;
        int bi = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int e = lane + i * kWave;
            if (e < a.E && !((taken >> i) & 1u) && (mine[i] > bv || (mine[i] == bv && e < bi))) {
                bv = mine[i];
                bi = e;
            }
        }
        // wave argmax: larger logit wins, ties go to the lower index
#pragma unroll
        for (int m = 32; m > 0; m >>= 1) {
            const float ov = __shfl_xor(bv, m, kWave);
            const int oi = __shfl_xor(bi, m, kWave);
            if (ov > bv || (ov == bv && oi < bi)) {
                bv = ov;
                bi = oi;
            }
        }
        if (k == 0) mx = bv;
        if (lane == k) {
            my_id = bi;
            my_logit = bv;
        }
        if ((bi & (kWave - 1)) == lane) taken |= 1u << (bi / kWave);
    }
    // softmax over all experts, max-subtracted (the maximum is the first selection)
    float z = 0.f;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int e = lane + i * kWave;
        if (e < a.E) z += expf(mine[i] - mx);
    }
    z = wave_sum(z);
    const float p = (lane < a.K) ? expf(my_logit - mx) / z : 0.f;
    const float psum = wave_sum(p);
    if (lane < a.K) {
        a.ids[t * a.K + lane] = my_id;
        a.scores[t * a.K + lane] = a.renorm ? p / psum : p;
    }
    if (lane == 0) {
        if (a.wg) a.gate[t] = 1.0f / (1.0f + expf(-l[a.E]));
        a.counters[t] = 0u;   // leave the workspace zeroed for the next call
    }
}

}  // namespace moe

using namespace moe;

extern "C" size_t moe_decode_route_workspace_bytes(int32_t n_tokens, int32_t n_experts) {
    if (n_tokens < 1 || n_experts < 1) return 0;
    const size_t logits = (size_t)n_tokens * (n_experts + 1) * sizeof(float);
    return align_up(logits, 256) + align_up((size_t)n_tokens * sizeof(uint32_t), 256);
}

extern "C" moe_status moe_decode_route(const void *x, moe_dtype x_dtype, int32_t n_tokens, int32_t d_in,
                                       const void *w_router, moe_dtype w_router_dtype,
                                       int32_t n_experts, int32_t top_k, int32_t renormalize,
                                       const void *w_shared_gate, moe_dtype w_shared_gate_dtype,
                                       int32_t *expert_ids, float *scores, float *shared_gate,
                                       void *workspace, size_t workspace_bytes, void *stream) {
    if (!x || !w_router || !expert_ids || !scores || !workspace) return MOE_EINVAL;
    if ((w_shared_gate == nullptr) != (shared_gate == nullptr)) return MOE_EINVAL;
    if (n_tokens < 1 || n_tokens > MOE_MAX_TOKENS) return MOE_EINVAL;
    if (n_experts < 1 || n_experts > MOE_MAX_EXPERTS) return MOE_EINVAL;
    if (top_k < 1 || top_k > MOE_MAX_TOP_K || top_k > n_experts) return MOE_EINVAL;
    if (d_in < kGroup || d_in > MOE_MAX_DIM || d_in % kGroup) return MOE_EINVAL;
    if (!valid_dtype(x_dtype) || !valid_dtype(w_router_dtype) ||
        (w_shared_gate && !valid_dtype(w_shared_gate_dtype)))
        return MOE_EUNSUPPORTED;
    if (!aligned16(x) || !aligned16(w_router) || (w_shared_gate && !aligned16(w_shared_gate)))
        return MOE_EINVAL;
    if (workspace_bytes < moe_decode_route_workspace_bytes(n_tokens, n_experts)) return MOE_EINVAL;

    RouteArgs a;
    a.x = x; a.wr = w_router; a.wg = w_shared_gate;
    a.x_dt = x_dtype; a.wr_dt = w_router_dtype; a.wg_dt = w_shared_gate_dtype;
    a.T = n_tokens; a.d_in = d_in; a.E = n_experts; a.K = top_k; a.renorm = renormalize ? 1 : 0;
    a.ids = expert_ids; a.scores = scores; a.gate = shared_gate;
    char *ws = reinterpret_cast<char *>(workspace);
    a.logits = reinterpret_cast<float *>(ws);
    a.counters = reinterpret_cast<uint32_t *>(
        ws + align_up((size_t)n_tokens * (n_experts + 1) * sizeof(float), 256));

    const int n_rows = n_experts + (w_shared_gate ? 1 : 0);
    dim3 grid((n_rows + kRouteWaves - 1) / kRouteWaves, n_tokens);
    hipLaunchKernelGGL(route_kernel, grid, dim3(256), d_in * sizeof(float),
                       reinterpret_cast<hipStream_t>(stream), a);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}
