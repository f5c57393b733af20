// Grouped expert FFN for larger batches and prefill (many tokens per expert)
// on the matrix cores.
//
// The pages' method is a pair of GEMVs per selected expert (mlxcel PR #276,
// "What changed" step 2); with a few tokens per expert the multi-token
// kernels apply each streamed weight chunk to every token with packed dots.
// With tens of tokens per expert the same work becomes a small GEMM per
// expert, and the point at which a GEMM path starts to beat the GEMV path is
// the one meTile PR #30 measures (its GB/s table: parity at 8 rows, a win
// only from 32 rows, batch or prefill).  Here a work item is one expert and up
// to 16 of its (token, slot) pairs; a workgroup takes 64 weight rows of it,
// each wave 16 rows x 16 tokens, and multiplies with v_mfma_f32_16x16x32
// (lane l holds A[l % 16][8 (l / 16) + i], B[8 (l / 16) + i][l % 16] for
// i = 0..7, and D[4 (l / 16) + r][l % 16] for r = 0..3).
//
// Codes stay exact: kernel A turns a 4-bit code q into the bf16 number 128 + q
// (nibble_pairs), kernel B into the fp16 number q (1024 + q, minus 1024 in a
// packed fp16 subtraction), so every product in the matrix core is exact and
// the affine scale and bias are applied per group of 64 inputs afterwards:
//   sum_i (s q_i + b) x_i = s * sum_i (128 + q_i) x_i + (b - 128 s) * sum_i x_i.
// A lane's 8 values of a k-step are one code word; its nibble pairs come in
// the order (q0, q4, q1, q5, q2, q6, q3, q7), and the inputs are permuted to
// the same order (pair_words), which leaves the dot products unchanged.  Each
// k-step stays inside one group: lane group g takes code words 2g and 2g + 1
// of the group, one per k-step.  act enters kernel B as fp16 multiplied by a
// power of two fitted to each token's largest magnitude (f16_stage_scale);
// the inverse joins the score.
#include <hip/hip_runtime.h>

#include "api.hpp"
#include "common.hpp"
#include "qgemv.hpp"

namespace moe {

constexpr int kGrpTok = 16;          // pairs per work item (the MFMA's N)
constexpr int kGrpRows = 64;         // weight rows per workgroup: 4 waves x 16
constexpr int kGrpThreads = 256;
constexpr int kGrpDepth = 4;         // groups of code words in flight per lane
constexpr int kGrpActChunk = 512;    // act inputs staged in LDS at a time (kernel B)
constexpr int kGrpBucketThreads = 1024;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

struct GroupedArgs {
    const void *x;                   // [T][d_in] bf16
    int T, K, E, d_in, d_ff;
    QM gate, up, down;
    const int32_t *ids;
    const float *scores;
    float *act;                      // [T*K][d_ff]
    float *partial;                  // [T*K][d_in]
    const int32_t *n_work;
    const int32_t *work_expert;      // [max_work]: expert, or -1 for the out-of-range ids
    const int32_t *work_begin;       // [max_work]: first index into pair_list
    const int32_t *work_count;       // [max_work]: pairs (1..16)
    const int32_t *pair_list;        // [T*K] pair indices t*K + k, grouped by expert
};

// Pairs (v[8k+p], v[8k+p+4]) of 8 consecutive 16-bit inputs held as 4 words:
// the order nibble_pairs gives the codes.
__device__ __forceinline__ void pair_inputs(const u32x4 &w, uint32_t (&o)[4]) {
    o[0] = __builtin_amdgcn_perm(w[2], w[0], 0x05040100u);
    o[1] = __builtin_amdgcn_perm(w[2], w[0], 0x07060302u);
    o[2] = __builtin_amdgcn_perm(w[3], w[1], 0x05040100u);
    o[3] = __builtin_amdgcn_perm(w[3], w[1], 0x07060302u);
}

// Sum over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (every lane gets the same bits).
__device__ __forceinline__ float sum_lane_groups(float v) {
    float r0, r1;
    swap_across<4>(v, v, r0, r1);
    v = r0 + r1;
    swap_across<5>(v, v, r0, r1);
    return r0 + r1;
}

// ------------------------------------------------------------------ bucketing
// One workgroup: the (token, slot) pairs grouped by expert (bucket E collects
// the ids outside [0, E)), each bucket cut into work items of at most
// kGrpTok pairs.  The order of pairs inside a bucket does not matter: every
// pair's results depend only on its own inputs.
__global__ __launch_bounds__(kGrpBucketThreads) void grouped_bucket_kernel(const int32_t *ids, int n_pairs, int E,
                                                                          int32_t *n_work, int32_t *work_expert,
                                                                          int32_t *work_begin, int32_t *work_count,
                                                                          int32_t *pair_list) {
    __shared__ int cnt[MOE_MAX_EXPERTS + 1], base[MOE_MAX_EXPERTS + 1], tiles[MOE_MAX_EXPERTS + 1];
    __shared__ int s_total[2];
    const int tid = threadIdx.x, nb = E + 1;
    for (int b = tid; b < nb; b += kGrpBucketThreads) cnt[b] = 0;
    __syncthreads();
    for (int p = tid; p < n_pairs; p += kGrpBucketThreads) {
        const int e = ids[p];
        atomicAdd(&cnt[e >= 0 && e < E ? e : E], 1);
    }
    __syncthreads();
    if (tid == 0) {                  // exclusive scans of pair and work-item counts (E + 1 <= 1025 entries)
        int pb = 0, tb = 0;
        for (int b = 0; b < nb; ++b) {
            base[b] = pb;
            tiles[b] = tb;
            pb += cnt[b];
            tb += (cnt[b] + kGrpTok - 1) / kGrpTok;
        }
        s_total[0] = tb;
    }
    __syncthreads();
    for (int b = tid; b < nb; b += kGrpBucketThreads) {
        const int n = cnt[b];
        for (int i = 0; i * kGrpTok < n; ++i) {
            const int w = tiles[b] + i;
            work_expert[w] = b < E ? b : -1;
            work_begin[w] = base[b] + i * kGrpTok;
            work_count[w] = min(kGrpTok, n - i * kGrpTok);
        }
        cnt[b] = 0;                  // reused as the placement cursor
    }
    __syncthreads();
    for (int p = tid; p < n_pairs; p += kGrpBucketThreads) {
        const int e = ids[p];
        const int b = e >= 0 && e < E ? e : E;
        pair_list[base[b] + atomicAdd(&cnt[b], 1)] = p;
    }
    if (tid == 0) *n_work = s_total[0];
}

// Zero rows [row0, row_end) of the item's pairs in out ([pairs][n]).
__device__ __forceinline__ void zero_rows(float *out, int n, const GroupedArgs &a, int begin, int count, int row0,
                                          int row_end) {
    for (int i = 0; i < count; ++i) {
        float *o = out + (int64_t)a.pair_list[begin + i] * n;
        for (int r = row0 + (int)threadIdx.x; r < row_end; r += kGrpThreads) o[r] = 0.f;
    }
}

// ------------------------------------------------------------------ kernel A
// act[pair][r] = silu(g_r) u_r for the item's pairs and rows [64 bx, 64 bx + 64).
template <int SB>
__global__ __launch_bounds__(kGrpThreads) void gate_up_grouped(GroupedArgs a) {
    const int w = blockIdx.y;
    if (w >= *a.n_work) return;
    const int e = a.work_expert[w], begin = a.work_begin[w], count = a.work_count[w];
    const int row0 = blockIdx.x * kGrpRows;
    if (e < 0) {
        zero_rows(a.act, a.d_ff, a, begin, count, row0, min(row0 + kGrpRows, a.d_ff));
        return;
    }
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
    const int g = lane >> 4, j = lane & 15;
    const int rw = row0 + wave * 16;                      // the wave's first row
    const int ra = min(rw + j, a.d_ff - 1);               // the lane's A row (clamped; results masked)
    const int pair_j = a.pair_list[begin + (j < count ? j : 0)];
    const uint16_t *xr = reinterpret_cast<const uint16_t *>(a.x) + (int64_t)(pair_j / a.K) * a.d_in + 16 * g;
    const int64_t erow = (int64_t)e * a.d_ff;
    const uint32_t *qg = a.gate.q + (erow + ra) * a.gate.wpr + 2 * g;
    const uint32_t *qu = a.up.q + (erow + ra) * a.up.wpr + 2 * g;
    // the lane's D rows rw + 4 g + r: their scales and biases per group
    int64_t srow[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) srow[r] = (erow + min(rw + 4 * g + r, a.d_ff - 1)) * a.gate.gpr;
    const int n_grp = a.d_in / kGroup;
    f32x4 acc_g = {0.f, 0.f, 0.f, 0.f}, acc_u = {0.f, 0.f, 0.f, 0.f};
    u32x2 wg[kGrpDepth], wu[kGrpDepth];
#pragma unroll
    for (int d = 0; d < kGrpDepth; ++d) {
        if (d < n_grp) {
            wg[d] = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(qg + d * 8));
            wu[d] = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(qu + d * 8));
        }
    }
    for (int G0 = 0; G0 < n_grp; G0 += kGrpDepth) {
#pragma unroll
        for (int d = 0; d < kGrpDepth; ++d) {
            const int G = G0 + d;
            if (G >= n_grp) break;
            const u32x4 x0 = *reinterpret_cast<const u32x4 *>(xr + G * kGroup);
            const u32x4 x1 = *reinterpret_cast<const u32x4 *>(xr + G * kGroup + 8);
            float sg[4], bg[4], su[4], bu[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                sg[r] = load_sb<SB>(a.gate.s, srow[r] + G);
                bg[r] = load_sb<SB>(a.gate.b, srow[r] + G);
                su[r] = load_sb<SB>(a.up.s, srow[r] + G);
                bu[r] = load_sb<SB>(a.up.b, srow[r] + G);
            }
            f32x4 tg = {0.f, 0.f, 0.f, 0.f}, tu = {0.f, 0.f, 0.f, 0.f};
            float xs = 0.f;
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const u32x4 xw = s == 0 ? x0 : x1;
                uint32_t xp[4], pg[4], pu[4];
                pair_inputs(xw, xp);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    xs += __uint_as_float(xw[i] << 16) + __uint_as_float(xw[i] & 0xFFFF0000u);
                nibble_pairs<0x43u>(wg[d][s], pg);
                nibble_pairs<0x43u>(wu[d][s], pu);
                const bf16x8_t B = __builtin_bit_cast(bf16x8_t, u32x4{xp[0], xp[1], xp[2], xp[3]});
                tg = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, u32x4{pg[0], pg[1], pg[2], pg[3]}),
                                                             B, tg, 0, 0, 0);
                tu = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, u32x4{pu[0], pu[1], pu[2], pu[3]}),
                                                             B, tu, 0, 0, 0);
            }
            if (G + kGrpDepth < n_grp) {             // refill this slot of the ring
                wg[d] = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(qg + (G + kGrpDepth) * 8));
                wu[d] = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(qu + (G + kGrpDepth) * 8));
            }
            const float xsum = sum_lane_groups(xs);  // token j's inputs of group G
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                acc_g[r] += sg[r] * tg[r] + (bg[r] - 128.0f * sg[r]) * xsum;
                acc_u[r] += su[r] * tu[r] + (bu[r] - 128.0f * su[r]) * xsum;
            }
        }
    }
    if (j < count) {
        float *o = a.act + (int64_t)pair_j * a.d_ff;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = rw + 4 * g + r;
            if (row < a.d_ff) o[row] = acc_g[r] * sigmoidf_(acc_g[r]) * acc_u[r];
        }
    }
}

// ------------------------------------------------------------------ kernel B
// partial[pair][i] = score * (W_down[e] act[pair])_i for the item's pairs and
// rows [64 bx, 64 bx + 64).  act is staged kGrpActChunk inputs at a time as
// fp16 rows of 16 tokens (8 halves of padding per row: the 16 lanes of a
// k-step read 16 different rows without bank conflicts).
template <int SB>
__global__ __launch_bounds__(kGrpThreads) void down_grouped(GroupedArgs a) {
    constexpr int kRow = kGrpActChunk + 8;            // halves per staged row
    __shared__ __align__(16) _Float16 s_act[kGrpTok * kRow];
    __shared__ float s_inv[kGrpTok], s_cs[kGrpTok];
    __shared__ uint32_t s_max[kGrpTok];
    const int w = blockIdx.y;
    if (w >= *a.n_work) return;
    const int e = a.work_expert[w], begin = a.work_begin[w], count = a.work_count[w];
    const int row0 = blockIdx.x * kGrpRows;
    if (e < 0) {
        zero_rows(a.partial, a.d_in, a, begin, count, row0, min(row0 + kGrpRows, a.d_in));
        return;
    }
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
    const int g = lane >> 4, j = lane & 15;
    const int n = a.d_ff;
    // each token's largest act magnitude: wave w scans token rows w, w + 4, ...
    for (int t = wave; t < kGrpTok; t += kGrpThreads / kWave) {
        uint32_t mx = 0;
        if (t < count) {
            const float *src = a.act + (int64_t)a.pair_list[begin + t] * n;
            for (int i = lane; i < n; i += kWave) mx = max(mx, __float_as_uint(src[i]) & 0x7FFFFFFFu);
        }
        const float wm = wave_max(__uint_as_float(mx));
        if (lane == 0) s_max[t] = __float_as_uint(wm);
    }
    __syncthreads();
    if (tid < kGrpTok) {
        float inv;
        s_cs[tid] = f16_stage_scale(s_max[tid], inv);
        s_inv[tid] = inv;
    }
    const int rw = row0 + wave * 16;
    const int ra = min(rw + j, a.d_in - 1);
    const int64_t erow = (int64_t)e * a.d_in;
    const uint32_t *qd = a.down.q + (erow + ra) * a.down.wpr + 2 * g;
    int64_t srow[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) srow[r] = (erow + min(rw + 4 * g + r, a.d_in - 1)) * a.down.gpr;
    const int pair_j = a.pair_list[begin + (j < count ? j : 0)];
    const f16x2_t off = {(_Float16)1024.0f, (_Float16)1024.0f};
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < n; k0 += kGrpActChunk) {
        const int kn = min(kGrpActChunk, n - k0);
        __syncthreads();                                 // the previous chunk's readers are done
        for (int idx = tid; idx < kGrpTok * (kn / 4); idx += kGrpThreads) {
            const int t = idx / (kn / 4), c = (idx - t * (kn / 4)) * 4;
            f32x4 v = {0.f, 0.f, 0.f, 0.f};
            if (t < count)
                v = *reinterpret_cast<const f32x4 *>(a.act + (int64_t)a.pair_list[begin + t] * n + k0 + c);
            const float inv = s_inv[t];
            _Float16 *d = s_act + t * kRow + c;
            d[0] = (_Float16)(v.x * inv);
            d[1] = (_Float16)(v.y * inv);
            d[2] = (_Float16)(v.z * inv);
            d[3] = (_Float16)(v.w * inv);
        }
        __syncthreads();
        const int g0 = k0 / kGroup, n_grp = kn / kGroup;
        for (int G = 0; G < n_grp; ++G) {
            const u32x2 wd = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(qd + (g0 + G) * 8));
            float sd[4], bd[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                sd[r] = load_sb<SB>(a.down.s, srow[r] + g0 + G);
                bd[r] = load_sb<SB>(a.down.b, srow[r] + g0 + G);
            }
            f32x4 t4 = {0.f, 0.f, 0.f, 0.f};
            float as = 0.f;
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const u32x4 aw = *reinterpret_cast<const u32x4 *>(s_act + j * kRow + G * kGroup + 16 * g + 8 * s);
                uint32_t ap[4], pq[4];
                pair_inputs(aw, ap);
                as += f16_pairs_sum<4>(ap);              // products by 1 exact, fp32 sums
                nibble_pairs<0x64u>(wd[s], pq);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    pq[i] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, pq[i]) - off);
                t4 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, u32x4{pq[0], pq[1], pq[2], pq[3]}),
                                                            __builtin_bit_cast(f16x8_t, u32x4{ap[0], ap[1], ap[2], ap[3]}),
                                                            t4, 0, 0, 0);
            }
            const float asum = sum_lane_groups(as);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] += sd[r] * t4[r] + bd[r] * asum;
        }
    }
    if (j < count) {
        const float sc = (a.scores ? a.scores[pair_j] : 1.0f) * s_cs[j];     // exact: s_cs is a power of two
        float *o = a.partial + (int64_t)pair_j * a.d_in;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = rw + 4 * g + r;
            if (row < a.d_in) o[row] = sc * acc[r];
        }
    }
}

static int grouped_max_work(int n_pairs, int E) { return (n_pairs + kGrpTok - 1) / kGrpTok + E + 1; }

}  // namespace moe

using namespace moe;

extern "C" size_t moe_decode_expert_ffn_grouped_workspace_bytes(int32_t n_tokens, int32_t top_k, int32_t n_experts) {
    if (n_tokens < 1 || top_k < 1 || n_experts < 1) return 0;
    const size_t n_pairs = (size_t)n_tokens * top_k, mw = (size_t)grouped_max_work((int)n_pairs, n_experts);
    return align_up((1 + 3 * mw + n_pairs) * sizeof(int32_t), 256);
}

extern "C" moe_status moe_decode_expert_ffn_grouped(const void *x, moe_dtype x_dtype_arg, int32_t n_tokens,
                                                    const moe_qmat *gate, const moe_qmat *up, const moe_qmat *down,
                                                    const int32_t *expert_ids, const float *scores, int32_t top_k,
                                                    float *act, float *partial, void *workspace,
                                                    size_t workspace_bytes, void *stream) {
    if (!x || !gate || !up || !down || !expert_ids || !act || !partial || !workspace) return MOE_EINVAL;
    if (n_tokens < 1 || n_tokens > MOE_MAX_GROUPED_TOKENS) return MOE_EINVAL;
    if (top_k < 1 || top_k > MOE_MAX_TOP_K) return MOE_EINVAL;
    moe_status st;
    for (const moe_qmat *m : {gate, up, down})
        if ((st = check_qmat(m)) != MOE_OK) return st;
    if (raw_enum(x_dtype_arg) != MOE_BF16) return MOE_EUNSUPPORTED;
    if (gate->bits != 4 || up->bits != 4 || down->bits != 4) return MOE_EUNSUPPORTED;
    const int sb = raw_enum(gate->sb_dtype);
    if (raw_enum(up->sb_dtype) != sb || raw_enum(down->sb_dtype) != sb) return MOE_EUNSUPPORTED;
    const int d_in = gate->cols, d_ff = gate->rows, E = gate->n_experts;
    if (up->rows != d_ff || up->cols != d_in || down->rows != d_in || down->cols != d_ff) return MOE_EINVAL;
    if (up->n_experts != E || down->n_experts != E) return MOE_EINVAL;
    if (!aligned16(x) || !aligned16(act) || !aligned16(partial) || !aligned16(workspace)) return MOE_EINVAL;
    if (workspace_bytes < moe_decode_expert_ffn_grouped_workspace_bytes(n_tokens, top_k, E)) return MOE_EINVAL;
    const int n_pairs = n_tokens * top_k, mw = grouped_max_work(n_pairs, E);
    GroupedArgs a;
    a.x = x; a.T = n_tokens; a.K = top_k; a.E = E; a.d_in = d_in; a.d_ff = d_ff;
    auto qm = [](const moe_qmat *m) {
        QM q;
        q.q = m->q;
        q.s = reinterpret_cast<const uint16_t *>(m->scales);
        q.b = reinterpret_cast<const uint16_t *>(m->biases);
        q.rows = m->rows; q.cols = m->cols;
        q.wpr = m->cols * m->bits / 32; q.gpr = m->cols / 64;
        q.bits_ = m->bits; q.sb_ = raw_enum(m->sb_dtype);
        return q;
    };
    a.gate = qm(gate); a.up = qm(up); a.down = qm(down);
    a.ids = expert_ids; a.scores = scores; a.act = act; a.partial = partial;
    int32_t *ws = reinterpret_cast<int32_t *>(workspace);
    a.n_work = ws;
    a.work_expert = ws + 1;
    a.work_begin = ws + 1 + mw;
    a.work_count = ws + 1 + 2 * mw;
    a.pair_list = ws + 1 + 3 * mw;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(grouped_bucket_kernel, dim3(1), dim3(kGrpBucketThreads), 0, s, expert_ids, n_pairs, E, ws,
                       ws + 1, ws + 1 + mw, ws + 1 + 2 * mw, ws + 1 + 3 * mw);
    const auto ka = sb == MOE_BF16 ? gate_up_grouped<MOE_BF16> : gate_up_grouped<MOE_F16>;
    const auto kb = sb == MOE_BF16 ? down_grouped<MOE_BF16> : down_grouped<MOE_F16>;
    hipLaunchKernelGGL(ka, dim3((d_ff + kGrpRows - 1) / kGrpRows, mw), dim3(kGrpThreads), 0, s, a);
    hipLaunchKernelGGL(kb, dim3((d_in + kGrpRows - 1) / kGrpRows, mw), dim3(kGrpThreads), 0, s, a);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}
