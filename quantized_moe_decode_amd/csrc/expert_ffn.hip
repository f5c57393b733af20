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

#include "api.hpp"
#include "common.hpp"

namespace moe {

struct QM {
    const uint32_t *q;
    const uint16_t *s;
    const uint16_t *b;
    int rows, cols, wpr, gpr;   // words and groups per row
    int bits_, sb_;             // host-side kernel selection only
};

struct FfnArgs {
    const void *x;
    int x_dt;
    int T, K, E, d_in, d_ff;
    QM gate, up, down;
    const int32_t *ids;
    const float *scores;
    float *act;
    float *partial;
    // multi-token work list, built by bucket_kernel (all null when T == 1)
    const int32_t *work_expert;   // [max_work] expert id, or -1 for the out-of-range ids
    const int32_t *work_begin;    // [max_work + 1] offsets into pair_list
    const int32_t *pair_list;     // [T*K] pair index t*K + k, grouped by expert
    const int32_t *n_work;        // number of work items
    int lr_shift;                 // log2(lanes per row)
    int rows_per_wg;
    int tpp;                      // tokens per LDS pass
};

struct Work {
    int e, npairs, single;
    const int32_t *pairs;
};

__device__ __forceinline__ bool get_work(const FfnArgs &a, int w, Work &wk) {
    if (!a.pair_list) {
        wk.e = a.ids[w];
        wk.npairs = 1;
        wk.single = w;
        wk.pairs = nullptr;
        return true;
    }
    if (w >= *a.n_work) return false;
    wk.e = a.work_expert[w];
    const int b = a.work_begin[w];
    wk.npairs = a.work_begin[w + 1] - b;
    wk.pairs = a.pair_list + b;
    wk.single = 0;
    return true;
}

__device__ __forceinline__ int pair_at(const Work &wk, int i) { return wk.pairs ? wk.pairs[i] : wk.single; }

// Stage nt input vectors of `cols` floats into LDS plus their per-chunk sums.
// src(tt, c) gives element c of the tt-th vector of this pass.
template <int CODES, typename Src>
__device__ __forceinline__ void stage_inputs(float *xs, float *xsum, int nt, int cols, Src src) {
    const int tid = threadIdx.x;
    for (int i = tid; i < nt * cols; i += blockDim.x) xs[i] = src(i / cols, i % cols);
    __syncthreads();
    const int cpr = cols / CODES;
    for (int i = tid; i < nt * cpr; i += blockDim.x) {
        const float *p = xs + (i / cpr) * cols + (i % cpr) * CODES;
        float s = 0.f;
#pragma unroll
        for (int q = 0; q < CODES; ++q) s += p[q];
        xsum[i] = s;
    }
    __syncthreads();
}

// Kernel A: gate and up projections of one expert over a tile of rows, then SwiGLU.
template <int BITS, int SB, int MAXT>
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
    const int cols = a.d_in, cpr = cols / F::kCodes;
    float *xs = lds;
    float *xsum = lds + a.tpp * cols;
    const int LR = 1 << a.lr_shift, j = lane & (LR - 1), rsub = lane >> a.lr_shift, RPW = kWave >> a.lr_shift;
    const int64_t ebase_q = (int64_t)wk.e * a.d_ff;   // row index of the expert's first row
    const uint32_t *gq = a.gate.q + ebase_q * a.gate.wpr;
    const uint32_t *uq = a.up.q + ebase_q * a.up.wpr;
    const uint16_t *gs = a.gate.s + ebase_q * a.gate.gpr, *gb = a.gate.b + ebase_q * a.gate.gpr;
    const uint16_t *us = a.up.s + ebase_q * a.up.gpr, *ub = a.up.b + ebase_q * a.up.gpr;

    for (int pb = 0; pb < wk.npairs; pb += a.tpp) {
        const int nt = min(a.tpp, wk.npairs - pb);
        __syncthreads();
        stage_inputs<F::kCodes>(xs, xsum, nt, cols, [&](int tt, int c) {
            const int64_t tok = pair_at(wk, pb + tt) / a.K;
            return load_act(a.x, a.x_dt, tok * cols + c);
        });
        for (int rb = row0 + wave * RPW; rb < row_end; rb += 4 * RPW) {
            const int r = rb + rsub;
            const bool live = r < row_end;
            float g[MAXT], u[MAXT];
#pragma unroll
            for (int t = 0; t < MAXT; ++t) g[t] = u[t] = 0.f;
            if (live) {
                const uint32_t *grow = gq + (int64_t)r * a.gate.wpr;
                const uint32_t *urow = uq + (int64_t)r * a.up.wpr;
                for (int c = j; c < cpr; c += LR) {
                    const Chunk<BITS> cg = load_chunk<BITS>(grow + c * F::kWords);
                    const Chunk<BITS> cu = load_chunk<BITS>(urow + c * F::kWords);
                    const int64_t gi = (int64_t)r * a.gate.gpr + c / F::kChunksPerGroup;
                    const float sg = load_sb<SB>(gs, gi), bg = load_sb<SB>(gb, gi);
                    const float su = load_sb<SB>(us, gi), bu = load_sb<SB>(ub, gi);
                    float qg[F::kCodes], qu[F::kCodes];
                    unpack<BITS>(cg, qg);
                    unpack<BITS>(cu, qu);
#pragma unroll
                    for (int t = 0; t < MAXT; ++t) {
                        if (t < nt) {
                            const float *xv = xs + t * cols + c * F::kCodes;
                            float dg = 0.f, du = 0.f;
#pragma unroll
                            for (int q = 0; q < F::kCodes; ++q) {
                                dg += qg[q] * xv[q];
                                du += qu[q] * xv[q];
                            }
                            const float xsm = xsum[t * cpr + c];
                            g[t] += sg * dg + bg * xsm;
                            u[t] += su * du + bu * xsm;
                        }
                    }
                }
            }
#pragma unroll
            for (int t = 0; t < MAXT; ++t) {
                if (t < nt) {
                    g[t] = group_sum(g[t], LR);
                    u[t] = group_sum(u[t], LR);
                }
            }
            if (live && j == 0) {
#pragma unroll
                for (int t = 0; t < MAXT; ++t)
                    if (t < nt) {
                        const int64_t p = pair_at(wk, pb + t);
                        a.act[p * a.d_ff + r] = g[t] * sigmoidf_(g[t]) * u[t];
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
    const int cols = a.d_ff, cpr = cols / F::kCodes;
    float *xs = lds;
    float *xsum = lds + a.tpp * cols;
    const int LR = 1 << a.lr_shift, j = lane & (LR - 1), rsub = lane >> a.lr_shift, RPW = kWave >> a.lr_shift;
    const int64_t ebase = (int64_t)wk.e * a.d_in;
    const uint32_t *dq = a.down.q + ebase * a.down.wpr;
    const uint16_t *ds = a.down.s + ebase * a.down.gpr, *db = a.down.b + ebase * a.down.gpr;

    for (int pb = 0; pb < wk.npairs; pb += a.tpp) {
        const int nt = min(a.tpp, wk.npairs - pb);
        __syncthreads();
        stage_inputs<F::kCodes>(xs, xsum, nt, cols, [&](int tt, int c) {
            const int64_t p = pair_at(wk, pb + tt);
            return a.act[p * cols + c];
        });
        for (int rb = row0 + wave * RPW; rb < row_end; rb += 4 * RPW) {
            const int r = rb + rsub;
            const bool live = r < row_end;
            float acc[MAXT];
#pragma unroll
            for (int t = 0; t < MAXT; ++t) acc[t] = 0.f;
            if (live) {
                const uint32_t *row = dq + (int64_t)r * a.down.wpr;
                for (int c = j; c < cpr; c += LR) {
                    const Chunk<BITS> cd = load_chunk<BITS>(row + c * F::kWords);
                    const int64_t gi = (int64_t)r * a.down.gpr + c / F::kChunksPerGroup;
                    const float s = load_sb<SB>(ds, gi), b = load_sb<SB>(db, gi);
                    float qd[F::kCodes];
                    unpack<BITS>(cd, qd);
#pragma unroll
                    for (int t = 0; t < MAXT; ++t) {
                        if (t < nt) {
                            const float *xv = xs + t * cols + c * F::kCodes;
                            float d = 0.f;
#pragma unroll
                            for (int q = 0; q < F::kCodes; ++q) d += qd[q] * xv[q];
                            acc[t] += s * d + b * xsum[t * cpr + c];
                        }
                    }
                }
            }
#pragma unroll
            for (int t = 0; t < MAXT; ++t)
                if (t < nt) acc[t] = group_sum(acc[t], LR);
            if (live && j == 0) {
#pragma unroll
                for (int t = 0; t < MAXT; ++t)
                    if (t < nt) {
                        const int64_t p = pair_at(wk, pb + t);
                        const float sc = a.scores ? a.scores[p] : 1.0f;
                        a.partial[p * a.d_in + r] = sc * acc[t];
                    }
            }
        }
    }
}

// Small-batch bucketing: groups the (token, slot) pairs by expert with a
// stable counting sort (pairs stay in ascending t*K + k order inside an
// expert).  Work items list the touched experts in ascending id order, then
// one item (expert -1) collecting every out-of-range id.  One workgroup.
__global__ __launch_bounds__(256) void bucket_kernel(const int32_t *ids, int n_pairs, int E,
                                                     int32_t *work_expert, int32_t *work_begin,
                                                     int32_t *pair_list, int32_t *n_work) {
    __shared__ int cnt[MOE_MAX_EXPERTS + 1];
    __shared__ int cur[MOE_MAX_EXPERTS + 1];
    const int tid = threadIdx.x;
    for (int i = tid; i <= E; i += blockDim.x) cnt[i] = 0;
    __syncthreads();
    for (int p = tid; p < n_pairs; p += blockDim.x) {
        const int e = ids[p];
        atomicAdd(&cnt[(e >= 0 && e < E) ? e : E], 1);
    }
    __syncthreads();
    if (tid == 0) {
        int off = 0, w = 0;
        for (int e = 0; e <= E; ++e) {
            cur[e] = off;
            if (cnt[e]) {
                work_expert[w] = (e < E) ? e : -1;
                work_begin[w] = off;
                ++w;
                off += cnt[e];
            }
        }
        work_begin[w] = off;
        *n_work = w;
        for (int p = 0; p < n_pairs; ++p) {
            const int e = ids[p];
            const int b = (e >= 0 && e < E) ? e : E;
            pair_list[cur[b]++] = p;
        }
    }
}

// ------------------------------------------------------------------ host side

using KernelFn = void (*)(FfnArgs);

template <int BITS, int SB, int MAXT>
static KernelFn pick_gate_up() { return gate_up_kernel<BITS, SB, MAXT>; }
template <int BITS, int SB, int MAXT>
static KernelFn pick_down() { return down_kernel<BITS, SB, MAXT>; }

template <bool GATE_UP, int MAXT>
static KernelFn select_kernel(int bits, int sb) {
#define MOE_PICK(B, S) \
    if (bits == B && sb == S) return GATE_UP ? pick_gate_up<B, S, MAXT>() : pick_down<B, S, MAXT>();
    MOE_PICK(4, MOE_BF16) MOE_PICK(4, MOE_F16)
    MOE_PICK(6, MOE_BF16) MOE_PICK(6, MOE_F16)
    MOE_PICK(8, MOE_BF16) MOE_PICK(8, MOE_F16)
#undef MOE_PICK
    return nullptr;
}

static int codes_per_chunk(int bits) { return bits == 4 ? 32 : 16; }

// Lanes per row: the largest power of two <= 64 dividing the chunk count,
// unless that leaves more than 16 chunks per lane.
static int pick_lr_shift(int cpr) {
    int s = 0;
    while (s < 6 && (cpr % (2 << s)) == 0) ++s;
    while (s < 6 && (cpr >> s) > 16) ++s;
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
    q.sb_ = m->sb_dtype;
    return q;
}

static constexpr size_t kLdsBudget = 64 * 1024;

static int max_work_items(int T, int K, int E) { return (T * K < E ? T * K : E) + 1; }

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
    hipLaunchKernelGGL(bucket_kernel, dim3(1), dim3(256), 0, p.s, p.a.ids, p.a.T * p.a.K, p.a.E,
                       const_cast<int32_t *>(p.a.work_expert), const_cast<int32_t *>(p.a.work_begin),
                       const_cast<int32_t *>(p.a.pair_list), const_cast<int32_t *>(p.a.n_work));
}

// Kernel launch geometry for a projection with `cols` inputs of `bits` bits and `rows` outputs.
static moe_status geometry(FfnArgs &a, int maxt, int cols, int bits, size_t &lds) {
    const int cpr = cols / codes_per_chunk(bits);
    a.lr_shift = pick_lr_shift(cpr);
    const int rpw = kWave >> a.lr_shift;
    a.rows_per_wg = 4 * rpw * 2;
    const size_t per_tok = (size_t)(cols + cpr) * sizeof(float);
    const int fit = (int)(kLdsBudget / per_tok);
    a.tpp = fit < maxt ? fit : maxt;
    if (a.tpp < 1) return MOE_EUNSUPPORTED;
    lds = a.tpp * per_tok;
    return MOE_OK;
}

static moe_status launch_a(Plan &p) {
    KernelFn k = p.maxt > 1 ? select_kernel<true, 8>(p.a.gate.bits_, p.a.gate.sb_)
                            : select_kernel<true, 1>(p.a.gate.bits_, p.a.gate.sb_);
    if (!k) return MOE_EUNSUPPORTED;
    size_t lds;
    const moe_status st = geometry(p.a, p.maxt, p.a.d_in, p.a.gate.bits_, lds);
    if (st != MOE_OK) return st;
    dim3 grid((p.a.d_ff + p.a.rows_per_wg - 1) / p.a.rows_per_wg, p.n_items);
    hipLaunchKernelGGL(k, grid, dim3(256), lds, p.s, p.a);
    return MOE_OK;
}

static moe_status launch_b(Plan &p) {
    KernelFn k = p.maxt > 1 ? select_kernel<false, 8>(p.a.down.bits_, p.a.down.sb_)
                            : select_kernel<false, 1>(p.a.down.bits_, p.a.down.sb_);
    if (!k) return MOE_EUNSUPPORTED;
    size_t lds;
    const moe_status st = geometry(p.a, p.maxt, p.a.d_ff, p.a.down.bits_, lds);
    if (st != MOE_OK) return st;
    dim3 grid((p.a.d_in + p.a.rows_per_wg - 1) / p.a.rows_per_wg, p.n_items);
    hipLaunchKernelGGL(k, grid, dim3(256), lds, p.s, p.a);
    return MOE_OK;
}

static moe_status finish() { return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP; }

}  // namespace moe

extern "C" moe_status moe_decode_gate_up(const void *x, moe_dtype x_dtype, int32_t n_tokens,
                                         const moe_qmat *gate, const moe_qmat *up,
                                         const int32_t *expert_ids, int32_t top_k, float *act,
                                         void *workspace, size_t workspace_bytes, void *stream) {
    moe_status st = check_tokens(x, n_tokens, top_k);
    if (st != MOE_OK) return st;
    for (const moe_qmat *m : {gate, up})
        if ((st = check_qmat(m)) != MOE_OK) return st;
    if (!valid_dtype(x_dtype)) return MOE_EUNSUPPORTED;
    if (up->rows != gate->rows || up->cols != gate->cols || up->n_experts != gate->n_experts) return MOE_EINVAL;
    if (up->sb_dtype != gate->sb_dtype || up->bits != gate->bits) return MOE_EUNSUPPORTED;
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

extern "C" moe_status moe_decode_expert_ffn(const void *x, moe_dtype x_dtype, int32_t n_tokens,
                                            const moe_qmat *gate, const moe_qmat *up, const moe_qmat *down,
                                            const int32_t *expert_ids, const float *scores, int32_t top_k,
                                            float *act, float *partial,
                                            void *workspace, size_t workspace_bytes, void *stream) {
    moe_status st = check_tokens(x, n_tokens, top_k);
    if (st != MOE_OK) return st;
    for (const moe_qmat *m : {gate, up, down})
        if ((st = check_qmat(m)) != MOE_OK) return st;
    if (!valid_dtype(x_dtype)) return MOE_EUNSUPPORTED;
    const int d_in = gate->cols, d_ff = gate->rows, E = gate->n_experts;
    if (up->rows != d_ff || up->cols != d_in || down->rows != d_in || down->cols != d_ff) return MOE_EINVAL;
    if (up->n_experts != E || down->n_experts != E) return MOE_EINVAL;
    if (up->sb_dtype != gate->sb_dtype || down->sb_dtype != gate->sb_dtype) return MOE_EUNSUPPORTED;
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
