// Tail: out = resid + (routed + shared * gate), one thread per hidden element
// (Red Lite dev39, "Change": the pool's weighted sum, the scale-add and the
// layer-output copy fused into one dispatch).  The expert scores were
// already applied by the down projection, so `routed` is the plain sum of the
// per-expert partial rows, taken left to right in slot order.
#include <hip/hip_runtime.h>

#include "api.hpp"
#include "common.hpp"

namespace moe {

struct TailArgs {
    const float *partial;
    const float *shared;
    const float *gate;
    const void *resid;
    float *out;
    int resid_dt, T, K, D, S;
};

// p[0] + p[D] + ... + p[(n-1) D], added in that order; the loads are issued
// eight at a time so that they are in flight together.
__device__ __forceinline__ float sum_rows(const float *p, int n, int D) {
    float sum = 0.f;
    for (int k0 = 0; k0 < n; k0 += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = k0 + u < n ? p[(int64_t)(k0 + u) * D] : 0.f;
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (k0 + u < n) sum = k0 + u == 0 ? v[u] : sum + v[u];
    }
    return sum;
}

__global__ __launch_bounds__(256) void tail_kernel(TailArgs a) {
    const int64_t n = (int64_t)a.T * a.D;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= n) return;
    const int t = (int)(idx / a.D), i = (int)(idx % a.D);
    const float routed = sum_rows(a.partial + (int64_t)t * a.K * a.D + i, a.K, a.D);
    const float sh = a.S > 0 ? sum_rows(a.shared + (int64_t)t * a.S * a.D + i, a.S, a.D) : 0.f;
    const float g = a.gate ? a.gate[t] : 1.0f;
    a.out[idx] = load_act(a.resid, a.resid_dt, idx) + (routed + sh * g);
}

}  // namespace moe

using namespace moe;

extern "C" moe_status moe_decode_tail(const float *partial, int32_t n_tokens, int32_t top_k, int32_t d_in,
                                      const float *shared, int32_t n_shared, const float *shared_gate,
                                      const void *residual, moe_dtype residual_dtype_arg, float *out,
                                      void *stream) {
    if (!partial || !residual || !out) return MOE_EINVAL;
    if (n_tokens < 1 || n_tokens > MOE_MAX_TOKENS) return MOE_EINVAL;
    if (top_k < 1 || top_k > MOE_MAX_TOP_K) return MOE_EINVAL;
    if (d_in < kGroup || d_in > MOE_MAX_DIM || d_in % kGroup) return MOE_EINVAL;
    if (n_shared < 0 || n_shared > MOE_MAX_TOP_K) return MOE_EINVAL;
    if ((n_shared == 0) != (shared == nullptr)) return MOE_EINVAL;
    const int residual_dtype = raw_enum(residual_dtype_arg);
    if (!valid_dtype(residual_dtype)) return MOE_EUNSUPPORTED;
    TailArgs a;
    a.partial = partial; a.shared = shared; a.gate = shared_gate; a.resid = residual; a.out = out;
    a.resid_dt = residual_dtype; a.T = n_tokens; a.K = top_k; a.D = d_in; a.S = n_shared;
    const int64_t n = (int64_t)n_tokens * d_in;
    hipLaunchKernelGGL(tail_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                       reinterpret_cast<hipStream_t>(stream), a);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

extern "C" const char *moe_decode_status_string(moe_status s_arg) {
    switch (raw_enum(s_arg)) {
    case MOE_OK: return "MOE_OK";
    case MOE_EINVAL: return "MOE_EINVAL: invalid argument (null pointer, shape, size or alignment)";
    case MOE_EUNSUPPORTED: return "MOE_EUNSUPPORTED: bit width, group size or dtype not built";
    case MOE_EHIP: return "MOE_EHIP: HIP launch error";
    case MOE_ETIMEOUT: return "MOE_ETIMEOUT: a wait inside a launch ran out; its results are invalid";
    }
    return "unknown moe_status";
}

extern "C" int32_t moe_decode_abi_version(void) { return MOE_DECODE_ABI_VERSION; }
