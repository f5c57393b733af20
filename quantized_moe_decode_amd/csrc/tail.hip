// Tail: out = resid + (routed + shared * gate), one thread per hidden element
// (Red Lite dev39, "Change": the pool's weighted sum, the scale-add and the
// layer-output copy fused into one dispatch).  The expert scores were
// already applied by the down projection, so `routed` is the plain sum of the
// per-expert partial rows, taken left to right in slot order.
#include <hip/hip_runtime.h>

#include <mutex>

#include "api.hpp"
#include "common.hpp"

namespace moe {

struct TailArgs {
    const float *partial;
    const float *shared;
    const float *gate;
    const void *resid;
    void *out;
    int resid_dt, out_dt, T, K, D, S;
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
    store_act(a.out, a.out_dt, idx, load_act(a.resid, a.resid_dt, idx) + (routed + sh * g));
}

// ---------------------------------------------- tail + the next layer's RMSNorm

// The tail of moe_decode_tail_rmsnorm: the workgroup (bx, t) computes token
// t's elements [256 bx, 256 bx + 256) of out as tail_kernel does, publishes
// their sum of squares (a fixed-order workgroup sum) as a word tagged with
// the launch's epoch, gathers token t's words of every chunk, adds them in
// chunk order, and writes its elements of
//   normed = out / sqrt(sum out^2 / D + eps) * weight,
// out taken as stored (rounded to its dtype), normed rounded to its own.
// The workspace: control words (error, epoch, finished workgroups), 256 bytes
// apart, then [T][chunks] tagged words.  Every workgroup waits only on
// workgroups of its own token, all of which are resident (the host checks that
// the grid fits the device).  Every wait is bounded: on time-out the error
// word is raised and the launch drains.
constexpr int kTailNormThreads = 256;
constexpr int kTailCtrStride = 64;
constexpr int kTailCtrErr = 0, kTailCtrEpoch = 1, kTailCtrDone = 2;
constexpr size_t kTailHeadBytes = 1024;
constexpr uint32_t kTailSpinLimit = 1u << 22;

struct TailNormArgs {
    TailArgs t;
    const void *norm_w;
    int norm_dt;
    float eps;
    void *normed;
    int normed_dt;
    uint32_t *ctr;
    uint64_t *part;         // [T][chunks]
    int chunks;
};

__device__ __forceinline__ float block_sum_fixed256(float v, float *s_w) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
    const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(group_sum_last<kWave>(v)), kWave - 1));
    __syncthreads();
    if (lane == 0) s_w[wave] = w;
    __syncthreads();
    return ((s_w[0] + s_w[1]) + s_w[2]) + s_w[3];
}

__global__ __launch_bounds__(kTailNormThreads) void tail_norm_kernel(TailNormArgs a) {
    __shared__ uint32_t s_tag;
    __shared__ float s_w[kTailNormThreads / kWave];
    __shared__ float s_part[MOE_MAX_DIM / kTailNormThreads];
    const int t = blockIdx.y, bx = blockIdx.x, tid = threadIdx.x;
    const int D = a.t.D;
    if (tid == 0)
        s_tag = __hip_atomic_load(a.ctr + kTailCtrEpoch * kTailCtrStride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
    __syncthreads();
    const uint32_t tag = s_tag;
    const int i = bx * kTailNormThreads + tid;
    float o = 0.f;
    if (i < D) {
        const int64_t idx = (int64_t)t * D + i;
        const float routed = sum_rows(a.t.partial + (int64_t)t * a.t.K * D + i, a.t.K, D);
        const float sh = a.t.S > 0 ? sum_rows(a.t.shared + (int64_t)t * a.t.S * D + i, a.t.S, D) : 0.f;
        const float g = a.t.gate ? a.t.gate[t] : 1.0f;
        o = round_to_dtype(a.t.out_dt, load_act(a.t.resid, a.t.resid_dt, idx) + (routed + sh * g));
        store_rounded(a.t.out, a.t.out_dt, idx, o);
    }
    const float ss = block_sum_fixed256(o * o, s_w);
    uint64_t *part = a.part + (int64_t)t * a.chunks;
    if (tid == 0)
        __hip_atomic_store(part + bx, ((uint64_t)tag << 32) | __float_as_uint(ss), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    if (tid < a.chunks) {
        float v = 0.f;
        uint32_t spin = 0;
        for (;; ++spin) {
            const uint64_t w = __hip_atomic_load(part + tid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if ((uint32_t)(w >> 32) == tag) {
                v = __uint_as_float((uint32_t)w);
                break;
            }
            if (spin == kTailSpinLimit) {
                __hip_atomic_fetch_or(a.ctr + kTailCtrErr * kTailCtrStride, 1u, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        s_part[tid] = v;
    }
    __syncthreads();
    float total = 0.f;
    for (int c = 0; c < a.chunks; ++c) total += s_part[c];      // chunk order
    const float inv = 1.0f / sqrtf(total / (float)D + a.eps);
    if (i < D) store_act(a.normed, a.normed_dt, (int64_t)t * D + i, o * inv * load_act(a.norm_w, a.norm_dt, i));
    // every word of this token was read: the last workgroup moves the workspace to the next epoch
    __syncthreads();
    if (tid == 0) {
        uint32_t *done = a.ctr + kTailCtrDone * kTailCtrStride;
        const uint32_t total_wg = gridDim.x * gridDim.y;
        if (__hip_atomic_fetch_add(done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == total_wg - 1) {
            __hip_atomic_store(done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(a.ctr + kTailCtrEpoch * kTailCtrStride, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// Plain RMSNorm, one workgroup per token: normed[t] = y[t] / sqrt(mean(y[t]^2)
// + eps) * weight, the sum of squares in a fixed order (each thread's
// elements in order, then the fixed workgroup tree).
__global__ __launch_bounds__(kTailNormThreads) void rmsnorm_kernel(const void *y, int y_dt, int D, const void *w,
                                                                   int w_dt, float eps, void *normed, int normed_dt) {
    __shared__ float s_w[kTailNormThreads / kWave];
    const int64_t t0 = (int64_t)blockIdx.x * D;
    float ss = 0.f;
    for (int i = threadIdx.x; i < D; i += kTailNormThreads) {
        const float v = load_act(y, y_dt, t0 + i);
        ss += v * v;
    }
    const float total = block_sum_fixed256(ss, s_w);
    const float inv = 1.0f / sqrtf(total / (float)D + eps);
    for (int i = threadIdx.x; i < D; i += kTailNormThreads)
        store_act(normed, normed_dt, t0 + i, load_act(y, y_dt, t0 + i) * inv * load_act(w, w_dt, i));
}

// Workgroups of tail_norm_kernel that can be resident at once on the current
// device, looked up once per device (0 if the runtime cannot tell).
static int tail_norm_capacity() {
    static std::mutex mu;
    static int cap[64];
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    std::lock_guard<std::mutex> lock(mu);
    if (!cap[dev]) {
        int cus = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void *>(tail_norm_kernel),
                                                         kTailNormThreads, 0) != hipSuccess)
            return 0;
        cap[dev] = cus * per_cu;
    }
    return cap[dev];
}

}  // namespace moe

using namespace moe;

extern "C" size_t moe_decode_tail_rmsnorm_workspace_bytes(int32_t n_tokens, int32_t d_in) {
    if (n_tokens < 1 || d_in < 1) return 0;
    const size_t chunks = (size_t)(d_in + kTailNormThreads - 1) / kTailNormThreads;
    return kTailHeadBytes + align_up((size_t)n_tokens * chunks * sizeof(uint64_t), 256);
}

extern "C" moe_status moe_decode_tail(const float *partial, int32_t n_tokens, int32_t top_k, int32_t d_in,
                                      const float *shared, int32_t n_shared, const float *shared_gate,
                                      const void *residual, moe_dtype residual_dtype_arg, void *out,
                                      moe_dtype out_dtype_arg, void *stream) {
    if (!partial || !residual || !out) return MOE_EINVAL;
    if (n_tokens < 1 || n_tokens > MOE_MAX_GROUPED_TOKENS) return MOE_EINVAL;
    if (top_k < 1 || top_k > MOE_MAX_TOP_K) return MOE_EINVAL;
    if (d_in < kGroup || d_in > MOE_MAX_DIM || d_in % kGroup) return MOE_EINVAL;
    if (n_shared < 0 || n_shared > MOE_MAX_TOP_K) return MOE_EINVAL;
    if ((n_shared == 0) != (shared == nullptr)) return MOE_EINVAL;
    const int residual_dtype = raw_enum(residual_dtype_arg), out_dtype = raw_enum(out_dtype_arg);
    if (!valid_dtype(residual_dtype) || !valid_dtype(out_dtype)) return MOE_EUNSUPPORTED;
    if (!aligned_elem(out, out_dtype)) return MOE_EINVAL;
    TailArgs a;
    a.partial = partial; a.shared = shared; a.gate = shared_gate; a.resid = residual; a.out = out;
    a.resid_dt = residual_dtype; a.out_dt = out_dtype; a.T = n_tokens; a.K = top_k; a.D = d_in; a.S = n_shared;
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

extern "C" moe_status moe_decode_tail_rmsnorm(const float *partial, int32_t n_tokens, int32_t top_k, int32_t d_in,
                                              const float *shared, int32_t n_shared, const float *shared_gate,
                                              const void *residual, moe_dtype residual_dtype_arg, void *out,
                                              moe_dtype out_dtype_arg, const moe_rmsnorm *norm, void *workspace,
                                              size_t workspace_bytes, void *stream) {
    const int residual_dtype = raw_enum(residual_dtype_arg), out_dtype = raw_enum(out_dtype_arg);
    if (!partial || !residual || !out || !norm || !workspace) return MOE_EINVAL;
    if (n_tokens < 1 || n_tokens > MOE_MAX_GROUPED_TOKENS) return MOE_EINVAL;
    if (top_k < 1 || top_k > MOE_MAX_TOP_K) return MOE_EINVAL;
    if (d_in < kGroup || d_in > MOE_MAX_DIM || d_in % kGroup) return MOE_EINVAL;
    if (n_shared < 0 || n_shared > MOE_MAX_TOP_K) return MOE_EINVAL;
    if ((n_shared == 0) != (shared == nullptr)) return MOE_EINVAL;
    if (!valid_dtype(residual_dtype) || !valid_dtype(out_dtype)) return MOE_EUNSUPPORTED;
    if (!aligned_elem(out, out_dtype)) return MOE_EINVAL;
    const moe_status nst = check_rmsnorm(norm);
    if (nst != MOE_OK) return nst;
    if (!aligned16(workspace)) return MOE_EINVAL;
    if (workspace_bytes < moe_decode_tail_rmsnorm_workspace_bytes(n_tokens, d_in)) return MOE_EINVAL;
    const int chunks = (d_in + kTailNormThreads - 1) / kTailNormThreads;
    const int cap = tail_norm_capacity();
    if (cap > 0 && n_tokens * chunks > cap) return MOE_EUNSUPPORTED;
    TailNormArgs a;
    a.t.partial = partial; a.t.shared = shared; a.t.gate = shared_gate; a.t.resid = residual; a.t.out = out;
    a.t.resid_dt = residual_dtype; a.t.out_dt = out_dtype;
    a.t.T = n_tokens; a.t.K = top_k; a.t.D = d_in; a.t.S = n_shared;
    a.norm_w = norm->weight; a.norm_dt = raw_enum(norm->dtype); a.eps = norm->eps;
    a.normed = norm->normed; a.normed_dt = raw_enum(norm->normed_dtype);
    a.ctr = reinterpret_cast<uint32_t *>(workspace);
    a.part = reinterpret_cast<uint64_t *>(reinterpret_cast<char *>(workspace) + kTailHeadBytes);
    a.chunks = chunks;
    hipLaunchKernelGGL(tail_norm_kernel, dim3(chunks, n_tokens), dim3(kTailNormThreads), 0,
                       reinterpret_cast<hipStream_t>(stream), a);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

extern "C" moe_status moe_decode_rmsnorm(const void *y, moe_dtype y_dtype_arg, int32_t n_tokens, int32_t d,
                                         const moe_rmsnorm *norm, void *stream) {
    const int y_dtype = raw_enum(y_dtype_arg);
    if (!y) return MOE_EINVAL;
    const moe_status nst = check_rmsnorm(norm);
    if (nst != MOE_OK) return nst;
    if (n_tokens < 1 || n_tokens > MOE_MAX_GROUPED_TOKENS || d < 1 || d > MOE_MAX_DIM) return MOE_EINVAL;
    if (!valid_dtype(y_dtype)) return MOE_EUNSUPPORTED;
    if (!aligned_elem(y, y_dtype)) return MOE_EINVAL;
    hipLaunchKernelGGL(rmsnorm_kernel, dim3(n_tokens), dim3(kTailNormThreads), 0, reinterpret_cast<hipStream_t>(stream),
                       y, y_dtype, d, norm->weight, raw_enum(norm->dtype), norm->eps, norm->normed,
                       raw_enum(norm->normed_dtype));
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}
