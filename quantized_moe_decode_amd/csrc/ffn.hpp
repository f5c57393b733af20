// Launch arguments and work items shared by the expert-FFN kernels (one
// token per launch, and the multi-token paths of small-batch decode).
#pragma once

#include "common.hpp"
#include "qgemv.hpp"

namespace moe {

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

// Rows of one lane group processed together: the loads of all of them are
// issued before any is consumed, so each lane keeps several 16-byte loads in
// flight.
constexpr int kNR = 3;          // rows per lane group, single- and multi-token kernels (12-row workgroups:
                                // two per CU for the Qwen3-shaped gate/up)

// Small-batch decode: the bucketing splits an expert's token list into work
// items of at most kBatchTok tokens, so a workgroup stages its tokens' inputs
// once and streams the expert's rows once for all of them.
constexpr int kBatchTok = 4;

using KernelFn = void (*)(FfnArgs);

constexpr int kFfnThreads = 256;     // threads per workgroup of every expert-FFN kernel

// Multi-token kernels for 4-bit weights (batch.hip): kernel A with bf16 x,
// kernel B with any act; scale dtype sb.  LDS bytes for `cols` inputs.
KernelFn batch_gate_up_q4(int sb);
KernelFn batch_down_q4(int sb);
size_t batch_lds_bytes(int cols);
constexpr int kBatchNRA = 2;     // rows per lane group, kernel A (2 matrices x 4 tokens of accumulators)
constexpr int kBatchNRB = 2;     // rows per lane group, kernel B

}  // namespace moe
