// Grouped expert FFN for larger batches and prefill (many tokens per expert)
// on the matrix cores.
//
// The pages' method is a pair of GEMVs per selected expert (mlxcel PR #276,
// "What changed" step 2); with a few tokens per expert the multi-token
// kernels apply each streamed weight chunk to every token with packed dots.
// With tens of tokens per expert the same work becomes a small GEMM per
// expert, and the point at which a GEMM path starts to beat the GEMV path is
// the one meTile PR #30 measures (its GB/s table: parity at 8 rows, a win
// only from 32 rows, batch or prefill).
//
// Work decomposition.  The (token, slot) pairs are grouped by expert and each
// expert's list is cut into work items of up to NT = 16 NB pairs (NB = 1 or
// 2, chosen from the average number of pairs per expert).  A workgroup of
// eight waves takes one work item and 128 weight rows of it; each wave owns
// 16 rows and multiplies them with every 16-pair block of the item using
// v_mfma_f32_16x16x32 (lane l holds A[l % 16][8 (l / 16) + i],
// B[8 (l / 16) + i][l % 16] for i = 0..7, and D[4 (l / 16) + r][l % 16] for
// r = 0..3), so a weight row is read once per work item whatever NB is.  The
// item's inputs (x for kernel A, act for kernel B) and the row block's scales
// and biases are staged in LDS four groups of 64 inputs at a time, double
// buffered, and shared by the eight waves; each lane keeps the code words of
// the next four groups in flight.  Workgroups are placed so that the row
// blocks of one work item run on one XCD and share its L2 copy of the inputs.
//
// Codes stay exact: kernel A turns a 4-bit code q into the bf16 number 128 + q
// (nibble_pairs), kernel B into the fp16 number 1024 + q, so every product in
// the matrix core is exact and the affine scale and bias are applied per group
// of 64 inputs afterwards, with the offset folded into the bias term:
//   sum_i (s q_i + b) x_i = s * sum_i (128 + q_i) x_i + (b - 128 s) * sum_i x_i
// (1024 and b - 1024 s for kernel B; its group sums are those of the fp16
// values it multiplies, so the offset cancels up to fp32 rounding).
// A lane's 8 values of a k-step are one code word; its nibble pairs come in
// the order (q0, q4, q1, q5, q2, q6, q3, q7) and the inputs are permuted to
// the same order (pair_inputs), which leaves the dot products unchanged.  Each
// k-step stays inside one group, and the four lane groups take four different
// words of it per k-step (spread_code_pair).
//
// Kernel A writes act in fp32 (the call's output) and, for kernel B, in fp16
// multiplied by a power of two fitted to the largest magnitude of each pair's
// 128 values in the workgroup's row block (f16_stage_scale); the factor's
// inverse is kept per (pair, block) and applied to each group's dot products
// in kernel B (exact: a power of two).
//
// Launches: a bucketing workgroup, then (when act fits a down unit's LDS) one
// launch of gate/up units followed by down units that wait per work item for
// its gate/up units (ffn_grouped_fused), else a gate/up launch and a chunked
// down launch.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <map>
#include <mutex>
#include <tuple>

#include "api.hpp"
#include "common.hpp"
#include "qgemv.hpp"

namespace moe {

constexpr int kGW = 8;                           // waves per workgroup
constexpr int kGThreads = kGW * kWave;           // 512
constexpr int kGRows = kGW * 16;                 // weight rows per workgroup (also the act16 block)
constexpr int kGChunkGroups = 4;                 // groups of 64 inputs per staged chunk
constexpr int kGChunk = kGChunkGroups * kGroup;  // 256 inputs
constexpr int kGPad = kGChunk + 8;               // 16-bit values per staged token row
constexpr int kGMinTok = 16;                     // smallest work item tile (sizes the workspace)
constexpr int kGBucketThreads = 1024;
constexpr int kGResIters = 8;                    // staging loads per thread, at most (resident x / act16, scales)

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

struct GroupedArgs {
    const uint16_t *x;               // [T][d_in] bf16
    int T, K, E, d_in, d_ff, n_blk;  // n_blk = ceil(d_ff / 128)
    QM gate, up, down;
    const float *scores;
    float *act;                      // [T*K][d_ff]
    float *partial;                  // [T*K][d_in]
    uint16_t *act16;                 // [T*K][d_ff] fp16 bits, scaled per (pair, block)
    float *act_cs;                   // [T*K][n_blk] the factor that undoes the scaling
    const int32_t *n_work;
    const int32_t *work_expert;      // [max_work]: expert, or -1 for the out-of-range ids
    const int32_t *work_begin;       // [max_work]: first index into pair_list
    const int32_t *work_count;       // [max_work]: pairs (1..NT)
    const int32_t *pair_list;        // [T*K] pair indices t*K + k, grouped by expert
    int row_blocks;                  // workgroups (units) per work item: gate/up kernel / unit
    int res_rb;                      // resident down units: row blocks per unit
    // the one-launch path (ffn_grouped_fused)
    int row_blocks_b;                // down units per work item
    int grid_a;                      // workgroups of gate/up units (a multiple of 8)
    int32_t *err;                    // raised when a wait runs out
    int32_t *done;                   // [max_work]: gate/up units finished per work item
};

// Pairs (v[p], v[p+4]) of 8 consecutive 16-bit inputs held as 4 words: the
// order nibble_pairs gives the codes.
__device__ __forceinline__ void pair_inputs(const uint32_t (&w)[4], uint32_t (&o)[4]) {
    o[0] = __builtin_amdgcn_perm(w[2], w[0], 0x05040100u);
    o[1] = __builtin_amdgcn_perm(w[2], w[0], 0x07060302u);
    o[2] = __builtin_amdgcn_perm(w[3], w[1], 0x05040100u);
    o[3] = __builtin_amdgcn_perm(w[3], w[1], 0x07060302u);
}

__device__ __forceinline__ void words_of(const u32x4 &v, uint32_t (&w)[4]) {
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
}

// Maximum over the four lanes l, l ^ 16, l ^ 32, l ^ 48.
__device__ __forceinline__ float max_lane_groups(float v) {
    float r0, r1;
    swap_across<4>(v, v, r0, r1);
    v = fmaxf(r0, r1);
    swap_across<5>(v, v, r0, r1);
    return fmaxf(r0, r1);
}

// Code words of two groups G and G + 1 of a weight row: one 16-byte load
// per lane gives lane group g words 4 (g & 1) .. 4 (g & 1) + 3 of group
// G + (g >> 1) (a group past the row's end is clamped to the last one; its
// words are never used), and two swaps across the wave halves leave every lane
// with words w[0], w[1] of group G and w[2], w[3] of group G + 1: word
// 4 (g & 1) + 2 (g >> 1) + s of the group for k-step s (code_word_input
// gives the inputs of that word).  Each load instruction reads 64 contiguous
// bytes of each of the wave's 16 rows.
__device__ __forceinline__ const u32x4 *code_pair_addr(const uint32_t *row, int G, int n_grp, int g) {
    return reinterpret_cast<const u32x4 *>(row + min(G + (g >> 1), n_grp - 1) * 8 + 4 * (g & 1));
}

// The same words addressed from the expert's first code word (uniform: in
// scalar registers) plus a 32-bit byte offset per lane, so a load costs a few
// 32-bit vector operations instead of a 64-bit address: off = the lane's row
// * bytes per row + 16 (g & 1), lim = n_grp - 1 - (g >> 1).  Rows of at most
// 8192 codes of at most 8192 rows per expert keep the offset within 32 bits.
struct CodeLane {
    uint32_t off;
    int lim, gh;
};
__device__ __forceinline__ CodeLane code_lane(int row, int wpr, int n_grp, int g) {
    return CodeLane{(uint32_t)__umul24((uint32_t)row, 4u * (uint32_t)wpr) + 16u * (uint32_t)(g & 1),
                    n_grp - 1 - (g >> 1), g >> 1};
}
__device__ __forceinline__ u32x4 load_code_pair(const uint32_t *base, const CodeLane &l, int G) {
    const uint32_t byte = l.off + 32u * (uint32_t)(min(G, l.lim) + l.gh);
    return *reinterpret_cast<const u32x4 *>(reinterpret_cast<const char *>(base) + byte);
}

// A register copy the compiler keeps (a DPP move with the identity pattern).
__device__ __forceinline__ uint32_t kept_copy(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xE4, 0xF, 0xF, false);
}

// KEEP: the swaps act on copies of the loaded words.  v_permlane32_swap
// overwrites both its operands, and on the words themselves it led the
// register allocator (in the down units) to keep a ring in other registers
// than the ones its loads write, with a copy at the loop's end that waits for
// the loads just issued; the gate/up units do without the copies.
template <bool KEEP>
__device__ __forceinline__ void spread_code_pair(const u32x4 &v, uint32_t (&w)[4]) {
    // v_permlane32_swap: lanes 32..63 of the first operand trade places with
    // lanes 0..31 of the second
    const uint32_t x = KEEP ? kept_copy(v.x) : v.x, y = KEEP ? kept_copy(v.y) : v.y;
    const uint32_t z = KEEP ? kept_copy(v.z) : v.z, ww = KEEP ? kept_copy(v.w) : v.w;
    const auto r02 = __builtin_amdgcn_permlane32_swap(x, z, false, false);
    const auto r13 = __builtin_amdgcn_permlane32_swap(y, ww, false, false);
    w[0] = r02[0];
    w[2] = r02[1];
    w[1] = r13[0];
    w[3] = r13[1];
}

// Offset (in inputs) within a group of the 8 inputs lane group g multiplies
// in k-step 0 (k-step 1: the next 8).
__device__ __forceinline__ int code_word_input(int g) { return 32 * (g & 1) + 16 * (g >> 1); }

// Sum of 8 bf16 (BF16) or fp16 values held as 4 words: products by one are
// exact, the sums are fp32.
template <bool BF16>
__device__ __forceinline__ float sum8(const uint32_t (&w)[4]) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if constexpr (BF16) {
            const bf16x2_t one = {(__bf16)1.0f, (__bf16)1.0f};
            s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[i]), one, s, false);
        } else {
            const f16x2_t one = {(_Float16)1.0f, (_Float16)1.0f};
            s = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, w[i]), one, s, false);
        }
    }
    return s;
}

// Workgroup -> (work item, row block): the row blocks of one item are eight
// linear workgroup indices apart, so they share an XCD (workgroups are
// dealt to the eight XCDs in turn).
__device__ __forceinline__ void item_and_block(int row_blocks, int &w, int &rb, int b = blockIdx.x) {
    const int lane8 = b & 7, q = b >> 3;
    rb = q % row_blocks;
    w = (q / row_blocks) * 8 + lane8;
}

// ------------------------------------------------------------------ bucketing
// One workgroup: the (token, slot) pairs grouped by expert (bucket E collects
// the ids outside [0, E)), each bucket cut into work items of at most nt
// pairs.  The order of pairs inside a bucket does not matter: every pair's
// results depend only on its own inputs.
// It also clears the words the one-launch path counts with (the error word
// and the per-item counters, max_work of them), so every call starts from
// zero without a separate fill.
__global__ __launch_bounds__(kGBucketThreads) void grouped_bucket_kernel(const int32_t *ids, int n_pairs, int E,
                                                                        int nt, int32_t *n_work,
                                                                        int32_t *work_expert, int32_t *work_begin,
                                                                        int32_t *work_count, int32_t *pair_list,
                                                                        int32_t *err, int32_t *done, int max_work) {
    constexpr int kWaves = kGBucketThreads / kWave;
    constexpr int kPer = MOE_MAX_GROUPED_TOKENS * MOE_MAX_TOP_K / kGBucketThreads;   // ids per thread, at most
    __shared__ int cnt[2 * kGBucketThreads], base[2 * kGBucketThreads], tiles[2 * kGBucketThreads];
    __shared__ int s_wp[kWaves], s_wt[kWaves];
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave, nb = E + 1;
    const int per = (n_pairs + kGBucketThreads - 1) / kGBucketThreads;
    cnt[2 * tid] = 0;
    cnt[2 * tid + 1] = 0;
    if (tid == 0) *err = 0;
    for (int i = tid; i < max_work; i += kGBucketThreads) done[i] = 0;
    // this thread's pairs tid + i * kGBucketThreads: their buckets, all loads in flight at once
    int bk[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        bk[i] = -1;
        if (i < per) {
            const int p = tid + i * kGBucketThreads;
            const int e = ids[min(p, n_pairs - 1)];
            bk[i] = p < n_pairs ? (e >= 0 && e < E ? e : E) : -1;
        }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kPer; ++i)
        if (bk[i] >= 0) atomicAdd(&cnt[bk[i]], 1);
    __syncthreads();
    // exclusive scans of the pair and work-item counts: thread t owns buckets
    // 2t and 2t + 1 (nb <= 1025 <= 2048), wave prefix sums, then the waves'
    const int c0 = cnt[2 * tid], c1 = cnt[2 * tid + 1];
    const int t0 = (c0 + nt - 1) / nt, t1 = (c1 + nt - 1) / nt;
    int ip = c0 + c1, it = t0 + t1;                        // inclusive within the wave
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int up = __shfl_up(ip, d), ut = __shfl_up(it, d);
        if (lane >= d) {
            ip += up;
            it += ut;
        }
    }
    if (lane == kWave - 1) {
        s_wp[wave] = ip;
        s_wt[wave] = it;
    }
    __syncthreads();
    int op = 0, ot = 0;
    for (int w = 0; w < wave; ++w) {
        op += s_wp[w];
        ot += s_wt[w];
    }
    const int ep = op + ip - (c0 + c1), et = ot + it - (t0 + t1);   // exclusive
    base[2 * tid] = ep;
    base[2 * tid + 1] = ep + c0;
    tiles[2 * tid] = et;
    tiles[2 * tid + 1] = et + t0;
    if (tid == kGBucketThreads - 1) *n_work = ot + it;
    __syncthreads();
    for (int b = tid; b < nb; b += kGBucketThreads) {
        const int n = cnt[b];
        for (int i = 0; i * nt < n; ++i) {
            const int w = tiles[b] + i;
            work_expert[w] = b < E ? b : -1;
            work_begin[w] = base[b] + i * nt;
            work_count[w] = min(nt, n - i * nt);
        }
    }
    __syncthreads();
    for (int b = tid; b < nb; b += kGBucketThreads) cnt[b] = 0;   // reused as the placement cursor
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kPer; ++i)
        if (bk[i] >= 0) pair_list[base[bk[i]] + atomicAdd(&cnt[bk[i]], 1)] = tid + i * kGBucketThreads;
}

// Zero rows [row0, row_end) of the item's pairs in out ([pairs][n]).
__device__ __forceinline__ void zero_rows(float *out, int n, const GroupedArgs &a, int begin, int count, int row0,
                                          int row_end) {
    for (int i = 0; i < count; ++i) {
        float *o = out + (int64_t)a.pair_list[begin + i] * n;
        for (int r = row0 + (int)threadIdx.x; r < row_end; r += kGThreads) o[r] = 0.f;
    }
}

// ------------------------------------------------------------ input staging
// The item's NT 16-bit input rows (x rows of the pairs' tokens, or the pairs'
// act16 rows), kGChunk values at a time: thread i loads 16 bytes (piece
// i % 32) of slots i / 32 + 16 r, r < NB; slots past the item's count and
// pieces past the row's end stage zeros.  Each 8-value piece is one lane's
// k-step operand and is stored already in the codes' pair order
// (pair_inputs), with the per-group sums beside the rows.
template <int NB>
struct InStage {
    u32x4 v[NB];
    bool ok[NB];
};

// row[r]: element offset of the slot's row in src (a valid row for an empty
// slot: the load always happens, an address clamped into range, and its value
// is replaced by zeros when the slot is empty or the piece lies past n.  No
// load sits behind a branch, so the wait counts stay exact and the code word
// ring stays in flight across the chunk's end).
// (row[r]: the row's first element as a 32-bit offset from src, which is
// uniform, so the loads take src from scalar registers and a 32-bit byte
// offset per lane; the inputs of a call stay far below 2^31 elements)
template <int NB>
__device__ __forceinline__ void in_load(InStage<NB> &st, const uint16_t *src, const uint32_t (&row)[NB],
                                        const bool (&live)[NB], int k0, int n) {
    const int c = 8 * (threadIdx.x & 31);
    const bool in_range = k0 + c < n;
    const uint32_t kc = (uint32_t)(in_range ? k0 + c : n - 8);
#pragma unroll
    for (int r = 0; r < NB; ++r) {
        st.v[r] = *reinterpret_cast<const u32x4 *>(reinterpret_cast<const char *>(src) + 2u * (row[r] + kc));
        st.ok[r] = live[r] && in_range;
    }
}

// buf: [NT][kGPad] 16-bit values; sums: [kGChunkGroups][NT] fp32.
template <int NB, bool BF16>
__device__ __forceinline__ void in_store(const InStage<NB> &st, uint16_t *buf, float *sums) {
    const int p = threadIdx.x & 31, t0 = threadIdx.x >> 5;
#pragma unroll
    for (int r = 0; r < NB; ++r) {
        const int t = t0 + 16 * r;
        uint32_t w[4], wp[4];
        words_of(st.v[r], w);
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = st.ok[r] ? w[i] : 0u;
        pair_inputs(w, wp);
        *reinterpret_cast<u32x4 *>(buf + t * kGPad + 8 * p) = u32x4{wp[0], wp[1], wp[2], wp[3]};
        float s = sum8<BF16>(w);
        s = group_sum_last<8>(s);                    // DPP: every lane of the 8 gets the sum
        if ((p & 7) == 0) sums[(p >> 3) * (16 * NB) + t] = s;
    }
}

// Maximum over the 16 lanes of each DPP row (lanes 16 g .. 16 g + 15); the
// result is valid in the row's last lane.
__device__ __forceinline__ float row16_max(float v) {
    v = fmax_dpp<0x111, 0xf>(v);   // row_shr:1
    v = fmax_dpp<0x112, 0xf>(v);   // row_shr:2
    v = fmax_dpp<0x114, 0xf>(v);   // row_shr:4
    return fmax_dpp<0x118, 0xf>(v);   // row_shr:8
}

// ------------------------------------------------------------------ kernel A
// act[pair][r] = silu(g_r) u_r for the item's pairs and the workgroup's 128
// rows; act16 and act_cs as described at the top.  The inputs are the MFMA's
// A operand and the codes its B operand, so lane (j, g) of wave w ends with
// D[4 g + r][j]: pairs 16 n + 4 g + r of weight row 16 w + j, and needs the
// scales of that one row.

// Where act_cs goes (act16 likewise, see the end of gate_up_unit): plain
// stores when the down projection is a later launch; device-scope (sc1)
// stores, which another XCD's device-scope loads see, when a down unit of the
// same launch reads them.
template <bool AGENT>
__device__ __forceinline__ void put_f32(float *p, float v) {
    if constexpr (AGENT)
        __hip_atomic_store(reinterpret_cast<uint32_t *>(p), __float_as_uint(v), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    else *p = v;
}

// LDS of a gate/up unit.
template <int NB>
struct GUSmem {
    static constexpr int NT = 16 * NB;
    static constexpr size_t kX = 2 * NT * kGPad * 2, kSb = 2 * kGChunkGroups * kGRows * 4 * 4,
                            kXs = 2 * kGChunkGroups * NT * 4, kMax = kGW * NT * 4, kInv = NT * 4, kPair = NT * 4;
    static constexpr size_t kBytes = kX + kSb + kXs + kMax + kInv + kPair;
    uint16_t *x;     // [2][NT][kGPad] staged inputs, pair order
    float *sb;       // [2][group][row][sg, cg, su, cu]
    float *xs;       // [2][group][slot] input group sums
    float *mx;       // [wave][slot]
    float *inv;      // [slot]
    int *pair;       // [slot]
    __device__ explicit GUSmem(unsigned char *p)
        : x(reinterpret_cast<uint16_t *>(p)), sb(reinterpret_cast<float *>(p + kX)),
          xs(reinterpret_cast<float *>(p + kX + kSb)), mx(reinterpret_cast<float *>(p + kX + kSb + kXs)),
          inv(reinterpret_cast<float *>(p + kX + kSb + kXs + kMax)),
          pair(reinterpret_cast<int *>(p + kX + kSb + kXs + kMax + kInv)) {}
};

// One gate/up unit: work item w, row block rb.  AGENT: act16 and act_cs with
// device-scope stores (read by a down unit of the same launch).
template <int SB, int NB, bool AGENT>
__device__ __forceinline__ void gate_up_unit(const GroupedArgs &a, int w, int rb, GUSmem<NB> sm) {
    constexpr int NT = 16 * NB;
    constexpr int kXBuf = NT * kGPad, kSbBuf = kGChunkGroups * kGRows * 4, kXsBuf = kGChunkGroups * NT;
    const int e = a.work_expert[w], begin = a.work_begin[w], count = a.work_count[w];
    const int row0 = rb * kGRows;
    if (e < 0) {
        zero_rows(a.act, a.d_ff, a, begin, count, row0, min(row0 + kGRows, a.d_ff));
        return;
    }
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
    const int g = lane >> 4, j = lane & 15;
    const int n_grp = a.d_in / kGroup, n_chunk = (n_grp + kGChunkGroups - 1) / kGChunkGroups;
    const int64_t erow = (int64_t)e * a.d_ff;
    if (tid < NT) sm.pair[tid] = tid < count ? a.pair_list[begin + tid] : -1;
    // staging roles: x rows of the slots this thread loads; scale row and kind
    uint32_t xrow[NB];
    bool xlive[NB];
#pragma unroll
    for (int r = 0; r < NB; ++r) {
        const int t = (tid >> 5) + 16 * r;
        xlive[r] = t < count;
        xrow[r] = (uint32_t)(a.pair_list[begin + (xlive[r] ? t : 0)] / a.K) * (uint32_t)a.d_in;
    }
    // scale staging: thread -> (row, matrix, pair of groups), a 32-bit byte
    // offset per lane from the expert's scales; c = b - 128 s (one matrix per
    // wave instead, so that its base stayed scalar, measured 3-6% slower)
    const int sb_row = tid >> 2, sb_m = (tid >> 1) & 1, sb_h = tid & 1;
    const uint16_t *sb_s = (sb_m ? a.up.s : a.gate.s) + erow * a.gate.gpr;
    const uint16_t *sb_b = (sb_m ? a.up.b : a.gate.b) + erow * a.gate.gpr;
    const uint32_t sb_off = 2u * (uint32_t)__umul24((uint32_t)min(row0 + sb_row, a.d_ff - 1), (uint32_t)a.gate.gpr);
    // the lane's weight row and its code words
    const int rowl = wave * 16 + j;
    const int ra = min(row0 + rowl, a.d_ff - 1);
    const uint32_t *qg = a.gate.q + erow * a.gate.wpr, *qu = a.up.q + erow * a.up.wpr;   // the expert's codes
    const CodeLane cl = code_lane(ra, a.gate.wpr, n_grp, g);                             // (same layout for up)
    const int xo = code_word_input(g);
    // The code words of a chunk (two groups per entry) are requested one
    // chunk before they are used, into two named register sets taken in turn
    // (chunk c reads one and loads chunk c + 1 into the other), so no register
    // copy at the loop's end waits for loads in flight.
    u32x4 rg0[2], ru0[2], rg1[2], ru1[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        rg0[p] = load_code_pair(qg, cl, 2 * p);
        ru0[p] = load_code_pair(qu, cl, 2 * p);
    }
    InStage<NB> st;
    uint16_t sbv[4];                                         // s, b of groups 2h and 2h + 1
    int sb_g0 = 0;                                           // first group of the staged chunk
    auto load_chunk = [&](int c) {
        in_load<NB>(st, a.x, xrow, xlive, c * kGChunk, a.d_in);
        sb_g0 = c * kGChunkGroups + 2 * sb_h;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint32_t o = sb_off + 2u * (uint32_t)min(sb_g0 + i, n_grp - 1);
            sbv[2 * i] = *reinterpret_cast<const uint16_t *>(reinterpret_cast<const char *>(sb_s) + o);
            sbv[2 * i + 1] = *reinterpret_cast<const uint16_t *>(reinterpret_cast<const char *>(sb_b) + o);
        }
    };
    auto store_chunk = [&](int buf) {
        in_store<NB, true>(st, sm.x + buf * kXBuf, sm.xs + buf * kXsBuf);
#pragma unroll
        for (int i = 0; i < 2; ++i) {           // groups past the end: zero scale and bias
            const bool ok = sb_g0 + i < n_grp;
            const float sv = ok ? sb_to_float<SB>(sbv[2 * i]) : 0.f, bv = ok ? sb_to_float<SB>(sbv[2 * i + 1]) : 0.f;
            *reinterpret_cast<float2 *>(&sm.sb[buf * kSbBuf + ((2 * sb_h + i) * kGRows + sb_row) * 4 + 2 * sb_m]) =
                make_float2(sv, bv - 128.0f * sv);
        }
    };
    // The inputs and scales of chunk c + 1 are requested at the end of chunk
    // c - 1 and stored to LDS at the end of chunk c: a whole chunk in flight.
    load_chunk(0);
    store_chunk(0);
    load_chunk(1);                                           // past the last chunk: clamped, unused
    __syncthreads();

    f32x4 acc_g[NB], acc_u[NB];
#pragma unroll
    for (int n = 0; n < NB; ++n) {
        acc_g[n] = f32x4{0.f, 0.f, 0.f, 0.f};
        acc_u[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    auto chunk = [&](int c, u32x4(&rg)[2], u32x4(&ru)[2], u32x4(&ng)[2], u32x4(&nu)[2]) {
        const int buf = c & 1;
        const uint16_t *sx = sm.x + buf * kXBuf;
        const float *ssb = sm.sb + buf * kSbBuf, *sxs = sm.xs + buf * kXsBuf;
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            uint32_t wg[4], wu[4];
            spread_code_pair<false>(rg[p], wg);
            spread_code_pair<false>(ru[p], wu);
            // the next chunk's words (past the end: clamped, unused): no load
            // sits behind a branch, so the wait counts stay exact
            ng[p] = load_code_pair(qg, cl, (c + 1) * kGChunkGroups + 2 * p);
            nu[p] = load_code_pair(qu, cl, (c + 1) * kGChunkGroups + 2 * p);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int d = 2 * p + h, G = c * kGChunkGroups + d;
                if (G >= n_grp) continue;                    // the last chunk of a ragged d_in
                const float2 sc = make_float2(ssb[(d * kGRows + rowl) * 4], ssb[(d * kGRows + rowl) * 4 + 2]);
                uint32_t pg[2][4], pu[2][4];
                nibble_pairs<0x43u>(wg[2 * h], pg[0]);
                nibble_pairs<0x43u>(wg[2 * h + 1], pg[1]);
                nibble_pairs<0x43u>(wu[2 * h], pu[0]);
                nibble_pairs<0x43u>(wu[2 * h + 1], pu[1]);
#pragma unroll
                for (int n = 0; n < NB; ++n) {
                    const uint16_t *xr = sx + (16 * n + j) * kGPad + d * kGroup + xo;
                    f32x4 tg = {0.f, 0.f, 0.f, 0.f}, tu = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < 2; ++s) {
                        const bf16x8_t A =
                            __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4 *>(xr + 8 * s));
                        tg = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            A, __builtin_bit_cast(bf16x8_t, u32x4{pg[s][0], pg[s][1], pg[s][2], pg[s][3]}), tg, 0, 0,
                            0);
                        tu = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            A, __builtin_bit_cast(bf16x8_t, u32x4{pu[s][0], pu[s][1], pu[s][2], pu[s][3]}), tu, 0, 0,
                            0);
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        acc_g[n][r] += sc.x * tg[r];
                        acc_u[n][r] += sc.y * tu[r];
                    }
                }
            }
        }
        // the chunk's bias terms, sum over its groups d of xsum[d][pair] c[d][row],
        // as one fp32 matrix product per 16-pair block (16x16x4: lane (j, g)
        // supplies xsum of pair 16 n + j and c of row j, both of group g; a
        // group past the end has both zero)
        {
            const float cgv = ssb[(g * kGRows + rowl) * 4 + 1], cuv = ssb[(g * kGRows + rowl) * 4 + 3];
#pragma unroll
            for (int n = 0; n < NB; ++n) {
                const float xv = sxs[g * NT + 16 * n + j];
                acc_g[n] = __builtin_amdgcn_mfma_f32_16x16x4f32(xv, cgv, acc_g[n], 0, 0, 0);
                acc_u[n] = __builtin_amdgcn_mfma_f32_16x16x4f32(xv, cuv, acc_u[n], 0, 0, 0);
            }
        }
        if (c + 1 < n_chunk) store_chunk(buf ^ 1);
        load_chunk(c + 2);                                   // past the last chunk: clamped, unused
        __syncthreads();
    };
    int c = 0;
    for (; c + 1 < n_chunk; c += 2) {
        chunk(c, rg0, ru0, rg1, ru1);
        chunk(c + 1, rg1, ru1, rg0, ru0);
    }
    if (c < n_chunk) chunk(c, rg0, ru0, rg1, ru1);

    // act in fp32, then the block's fp16 copy
    const int row = row0 + rowl;
    const bool row_ok = row < a.d_ff;
    f32x4 v[NB];
#pragma unroll
    for (int n = 0; n < NB; ++n) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            v[n][r] = acc_g[n][r] * sigmoidf_(acc_g[n][r]) * acc_u[n][r];
            const int t = 16 * n + 4 * g + r;
            const float m = row16_max(row_ok ? fabsf(v[n][r]) : 0.f);
            if (j == 15) sm.mx[wave * NT + t] = m;
            if (t < count && row_ok) a.act[(int64_t)sm.pair[t] * a.d_ff + row] = v[n][r];
        }
    }
    __syncthreads();
    if (tid < NT) {
        float m = 0.f;
#pragma unroll
        for (int q = 0; q < kGW; ++q) m = fmaxf(m, sm.mx[q * NT + tid]);
        float inv;
        const float cs = f16_stage_scale(__float_as_uint(m), inv);
        sm.inv[tid] = inv;
        if (tid < count) put_f32<AGENT>(a.act_cs + (int64_t)sm.pair[tid] * a.n_blk + rb, cs);
    }
    __syncthreads();
    if constexpr (!AGENT) {
        if (row_ok) {
#pragma unroll
            for (int n = 0; n < NB; ++n)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 16 * n + 4 * g + r;
                    if (t < count)
                        a.act16[(int64_t)sm.pair[t] * a.d_ff + row] = (uint16_t)f32_to_f16_bits(v[n][r] * sm.inv[t]);
                }
        }
    } else {
        // through LDS ([slot][128 rows], in the staging buffer, free by now),
        // then out as 8-byte device-scope stores: each slot's 128 rows are
        // 256 contiguous bytes, written as whole lines
        uint16_t *tile = sm.x;
#pragma unroll
        for (int n = 0; n < NB; ++n)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * n + 4 * g + r;
                tile[t * kGRows + rowl] = (uint16_t)f32_to_f16_bits(v[n][r] * sm.inv[t]);
            }
        __syncthreads();
#pragma unroll
        for (int n = 0; n < NB; ++n) {
            const int t = 16 * n + (tid >> 5), q = tid & 31;          // slot, 4-row piece
            if (t < count && row0 + 4 * q < a.d_ff)
                __hip_atomic_store(reinterpret_cast<uint64_t *>(a.act16 + (int64_t)sm.pair[t] * a.d_ff + row0 + 4 * q),
                                   *reinterpret_cast<const uint64_t *>(tile + t * kGRows + 4 * q), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// At most 128 VGPRs (four waves per SIMD: two workgroups per CU); the
// compiler otherwise takes a few more with 32-pair items.
template <int SB, int NB>
__global__ __launch_bounds__(kGThreads) __attribute__((amdgpu_waves_per_eu(4))) void gate_up_grouped(GroupedArgs a) {
    __shared__ __align__(16) unsigned char s_mem[GUSmem<NB>::kBytes];
    int w, rb;
    item_and_block(a.row_blocks, w, rb);
    if (w >= *a.n_work) return;
    gate_up_unit<SB, NB, false>(a, w, rb, GUSmem<NB>(s_mem));
}

// ------------------------------------------------------------------ kernel B
// partial[pair][i] = score * (W_down[e] act[pair])_i for the item's pairs and
// the workgroup's 128 rows, from act16 and act_cs; the same operand roles as
// kernel A.
template <int SB, int NB>
__global__ __launch_bounds__(kGThreads) void down_grouped(GroupedArgs a) {
    constexpr int NT = 16 * NB;
    constexpr int kBlkPerChunk = kGChunk / kGRows;           // act16 blocks per chunk (2)
    __shared__ __align__(16) uint16_t s_a[2][NT * kGPad];
    __shared__ __align__(16) float s_sb[2][kGChunkGroups * kGRows * 2];      // [group][row][s, b]
    __shared__ __align__(16) float s_as[2][kGChunkGroups * NT];             // [group][slot]
    __shared__ __align__(16) float s_cs[2][kBlkPerChunk * NT];              // [block][slot]
    __shared__ int s_pair[NT];
    __shared__ float s_score[NT];
    int w, rb;
    item_and_block(a.row_blocks, w, rb);
    if (w >= *a.n_work) return;
    const int e = a.work_expert[w], begin = a.work_begin[w], count = a.work_count[w];
    const int row0 = rb * kGRows;
    if (e < 0) {
        zero_rows(a.partial, a.d_in, a, begin, count, row0, min(row0 + kGRows, a.d_in));
        return;
    }
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
    const int g = lane >> 4, j = lane & 15;
    const int n = a.d_ff, n_grp = n / kGroup, n_chunk = (n_grp + kGChunkGroups - 1) / kGChunkGroups;
    const int64_t erow = (int64_t)e * a.d_in;
    if (tid < NT) {
        const int p = tid < count ? a.pair_list[begin + tid] : -1;
        s_pair[tid] = p;
        s_score[tid] = p >= 0 && a.scores ? a.scores[p] : 1.0f;
    }
    uint32_t arow[NB];
    bool alive[NB];
#pragma unroll
    for (int r = 0; r < NB; ++r) {
        const int t = (tid >> 5) + 16 * r;
        alive[r] = t < count;
        arow[r] = (uint32_t)a.pair_list[begin + (alive[r] ? t : 0)] * (uint32_t)n;
    }
    // scale staging, threads < 256: (row, pair of groups)
    const int sb_row = (tid >> 1) & (kGRows - 1), sb_h = tid & 1;
    const int64_t sb_off = (erow + min(row0 + sb_row, a.d_in - 1)) * a.down.gpr;
    const int cs_t = (tid >> 1) & (NT - 1), cs_k = tid & 1;           // threads < 2 NT: (slot, block)
    const bool cs_live = cs_t < count;
    const int64_t cs_row = (int64_t)a.pair_list[begin + (cs_live ? cs_t : 0)] * a.n_blk;
    const int rowl = wave * 16 + j;
    const int ra = min(row0 + rowl, a.d_in - 1);
    const uint32_t *qd = a.down.q + (erow + ra) * a.down.wpr;
    const int xo = code_word_input(g);
    u32x4 rw[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) rw[p] = *code_pair_addr(qd, 2 * p, n_grp, g);
    InStage<NB> st;
    uint16_t sbv[4];
    float csv = 1.f;
    int sb_g0 = 0, blk = 0;
    // every thread loads (clamped addresses); only the staging threads store
    auto load_chunk = [&](int c) {
        in_load<NB>(st, a.act16, arow, alive, c * kGChunk, n);
        sb_g0 = c * kGChunkGroups + 2 * sb_h;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int G = min(sb_g0 + i, n_grp - 1);
            sbv[2 * i] = a.down.s[sb_off + G];
            sbv[2 * i + 1] = a.down.b[sb_off + G];
        }
        blk = c * kBlkPerChunk + cs_k;
        csv = a.act_cs[cs_row + min(blk, a.n_blk - 1)];
    };
    auto store_chunk = [&](int buf) {
        in_store<NB, false>(st, s_a[buf], s_as[buf]);
        if (tid < 2 * kGRows) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {       // groups past the end: zero scale and bias
                const bool ok = sb_g0 + i < n_grp;
                const float sv = ok ? sb_to_float<SB>(sbv[2 * i]) : 0.f;
                const float bv = ok ? sb_to_float<SB>(sbv[2 * i + 1]) : 0.f;
                *reinterpret_cast<float2 *>(&s_sb[buf][((2 * sb_h + i) * kGRows + sb_row) * 2]) =
                    make_float2(sv, bv - 1024.0f * sv);      // the codes enter as 1024 + q
            }
        }
        if (tid < kBlkPerChunk * NT) s_cs[buf][cs_k * NT + cs_t] = cs_live && blk < a.n_blk ? csv : 0.f;
    };
    load_chunk(0);
    store_chunk(0);
    __syncthreads();

    f32x4 acc[NB];
#pragma unroll
    for (int m = 0; m < NB; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int c = 0; c < n_chunk; ++c) {
        const int buf = c & 1;
        if (c + 1 < n_chunk) load_chunk(c + 1);
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            uint32_t wd[4];
            spread_code_pair<true>(rw[p], wd);
            rw[p] = *code_pair_addr(qd, (c + 1) * kGChunkGroups + 2 * p, n_grp, g);   // as in kernel A
            // groups 2p and 2p + 1 are act16 block p of the chunk
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int d = 2 * p + h, G = c * kGChunkGroups + d;
                if (G >= n_grp) continue;
                const float sd = s_sb[buf][(d * kGRows + rowl) * 2];
                uint32_t pq[2][4];
                nibble_pairs<0x64u>(wd[2 * h], pq[0]);
                nibble_pairs<0x64u>(wd[2 * h + 1], pq[1]);
#pragma unroll
                for (int m = 0; m < NB; ++m) {
                    const uint16_t *ar = s_a[buf] + (16 * m + j) * kGPad + d * kGroup + xo;
                    f32x4 t4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < 2; ++s)
                        t4 = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                            __builtin_bit_cast(f16x8_t, *reinterpret_cast<const u32x4 *>(ar + 8 * s)),
                            __builtin_bit_cast(f16x8_t, u32x4{pq[s][0], pq[s][1], pq[s][2], pq[s][3]}), t4, 0, 0, 0);
                    const f32x4 cs = *reinterpret_cast<const f32x4 *>(&s_cs[buf][p * NT + 16 * m + 4 * g]);
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[m][r] += (cs[r] * sd) * t4[r];
                }
            }
        }
        // the chunk's bias terms, sum over its groups d of b[d][row] asum[d][pair]
        // times the block factor, as one fp32 matrix product per 16-pair block
        // (as in kernel A; lane (j, g): pair 16 m + j, row j, group g)
        {
            const float bv = s_sb[buf][(g * kGRows + rowl) * 2 + 1];
#pragma unroll
            for (int m = 0; m < NB; ++m) {
                const float av = s_as[buf][g * NT + 16 * m + j] * s_cs[buf][(g >> 1) * NT + 16 * m + j];
                acc[m] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, acc[m], 0, 0, 0);
            }
        }
        if (c + 1 < n_chunk) store_chunk(buf ^ 1);
        __syncthreads();
    }
    const int row = row0 + rowl;
    if (row < a.d_in) {
#pragma unroll
        for (int m = 0; m < NB; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * m + 4 * g + r;
                if (t < count) a.partial[(int64_t)s_pair[t] * a.d_in + row] = s_score[t] * acc[m][r];
            }
    }
}

// Down units with the item's whole act resident in LDS (when it fits):
// act16, its group sums and block factors staged once per unit, then res_rb
// row blocks of 128 rows in turn, each with all its groups' scales staged at
// once, so the contraction runs without a barrier per chunk.  Same operand
// roles and arithmetic as down_grouped.  Dynamic LDS: [NT][d_ff + 8] act16,
// [n_grp][NT] sums, [n_blk][NT] factors, [n_grp][128][2] scales.
constexpr size_t kGResLdsMax = 64 * 1024 - 512;    // dynamic LDS within the default per-workgroup limit

__host__ __device__ constexpr int res_row_pad(int d_ff) { return d_ff + 8; }

static size_t res_lds_bytes(int nt, int d_ff) {
    const int n_grp = d_ff / kGroup, n_blk = (d_ff + kGRows - 1) / kGRows;
    return align_up((size_t)nt * res_row_pad(d_ff) * 2, 16) + (size_t)n_grp * nt * 4 + (size_t)n_blk * nt * 4 +
           (size_t)n_grp * kGRows * 8;
}

// The resident kernel applies: its LDS within the limit, and its staging
// within kGResIters loads per thread and one block factor per thread.
static bool res_fits(int nt, int d_ff) {
    const int n_grp = d_ff / kGroup, n_blk = (d_ff + kGRows - 1) / kGRows;
    return res_lds_bytes(nt, d_ff) <= kGResLdsMax && nt * (d_ff / 8) <= kGResIters * kGThreads &&
           n_grp * kGRows <= kGResIters * kGThreads && n_blk * nt <= kGThreads;
}

constexpr uint32_t kGSpinLimit = 1u << 20;       // polls of a per-item counter before giving up

// A 16-byte piece of act16 and a block factor: plain loads when act16 was
// written by an earlier launch; device-scope (sc1) loads, which see the sc1
// stores of another XCD, when a gate/up unit of the same launch wrote them.
template <bool AGENT>
__device__ __forceinline__ u32x4 get_piece(const uint16_t *p) {
    if constexpr (AGENT) {
        const uint64_t *q = reinterpret_cast<const uint64_t *>(p);
        const uint64_t lo = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint64_t hi = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return u32x4{(uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32)};
    } else {
        return *reinterpret_cast<const u32x4 *>(p);
    }
}
template <bool AGENT>
__device__ __forceinline__ float get_f32(const float *p) {
    if constexpr (AGENT)
        return __uint_as_float(
            __hip_atomic_load(reinterpret_cast<const uint32_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    else return *p;
}

// One resident down unit: work item w, row blocks res_rb * rbb .. (up to
// n_rb).  dyn: the dynamic LDS (res_lds_bytes); pair, score: [NT].  AGENT:
// act16 and act_cs come from gate/up units of the same launch; thread 0 first
// waits until all row_blocks of them have finished the item (bounded: on
// time-out the error word is raised and the unit goes on, its results
// invalid).
template <int SB, int NB, bool AGENT>
__device__ __forceinline__ void down_unit(const GroupedArgs &a, int w, int rbb, unsigned char *dyn, int *s_pair,
                                          float *s_score) {
    constexpr int NT = 16 * NB;
    const int e = a.work_expert[w], begin = a.work_begin[w], count = a.work_count[w];
    const int n_rb = (a.d_in + kGRows - 1) / kGRows;
    if (e < 0) {
        zero_rows(a.partial, a.d_in, a, begin, count, rbb * a.res_rb * kGRows,
                  min((rbb + 1) * a.res_rb * kGRows, a.d_in));
        return;
    }
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
    const int g = lane >> 4, j = lane & 15;
    const int n = a.d_ff, n_grp = n / kGroup, n_chunk = (n_grp + kGChunkGroups - 1) / kGChunkGroups;
    const int pad = res_row_pad(n);
    uint16_t *s_a = reinterpret_cast<uint16_t *>(dyn);
    float *s_as = reinterpret_cast<float *>(dyn + ((size_t)NT * pad * 2 + 15) / 16 * 16);
    float *s_cs = s_as + n_grp * NT;
    float *s_sb = s_cs + a.n_blk * NT;
    if (tid < NT) {
        const int p = tid < count ? a.pair_list[begin + tid] : -1;
        s_pair[tid] = p;
        s_score[tid] = p >= 0 && a.scores ? a.scores[p] : 1.0f;
    }
    const int64_t erow = (int64_t)e * a.d_in;
    const int rowl = wave * 16 + j, xo = code_word_input(g);
    const int rb0 = rbb * a.res_rb, n_rbw = min(a.res_rb, n_rb - rb0);   // this unit's row blocks (>= 1)
    const uint32_t *qd = a.down.q + erow * a.down.wpr;      // the expert's codes
    auto code_lane_of = [&](int rbi) { return code_lane(min((rb0 + rbi) * kGRows + rowl, a.d_in - 1), a.down.wpr, n_grp, g); };
    // Steps (row block, chunk) in order.  The code words of a step are
    // requested LEAD steps before they are used (past the last step: the
    // last one again, unused), into LEAD + 1 named register sets taken in
    // turn, so no register copy at a loop's end waits for loads in flight and
    // the next row block's first words are in flight while this one ends.
    // Three steps ahead with 16-pair items, two with 32-pair items (what the
    // registers allow at four waves per SIMD).  The first steps' words are
    // requested before act is staged.
    constexpr int LEAD = NB == 1 ? 3 : 2;
    const int n_steps = n_rbw * n_chunk;
    int l_rb = 0, l_c = 0;                                   // the next step whose words are requested
    auto load_words = [&](u32x4(&dst)[2]) {
        const CodeLane cl = code_lane_of(l_rb);
#pragma unroll
        for (int p = 0; p < 2; ++p) dst[p] = load_code_pair(qd, cl, l_c * kGChunkGroups + 2 * p);
        if (++l_c == n_chunk) {
            l_c = 0;
            l_rb = min(l_rb + 1, n_rbw - 1);
        }
    };
    u32x4 rw0[2], rw1[2], rw2[2], rw3[2];
    load_words(rw0);
    load_words(rw1);
    if constexpr (LEAD == 3) load_words(rw2);
    if constexpr (AGENT) {
        if (tid == 0) {
            for (uint32_t spin = 0;
                 __hip_atomic_load(a.done + w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < a.row_blocks; ++spin) {
                if (spin == kGSpinLimit) {
                    __hip_atomic_fetch_or(a.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    break;
                }
                __builtin_amdgcn_s_sleep(2);
            }
        }
    }
    __syncthreads();
    // the item's act16 rows: 16-byte pieces q = tid + 512 i, slot q / (n / 8),
    // piece q % (n / 8) (eight consecutive lanes hold one group of 64), stored
    // in the codes' pair order with their group sums.  Every thread issues
    // kGResIters loads (indices past the end clamped to the last piece: one
    // address for the whole wave) before the first store, so none waits for
    // another (the host checks that kGResIters loads per thread cover act16)
    {
        const int ppr = n / 8, n_pc = NT * ppr, iters = (n_pc + kGThreads - 1) / kGThreads;
        u32x4 v[kGResIters];
#pragma unroll
        for (int i = 0; i < kGResIters; ++i) {
            const int q = min(tid + kGThreads * i, n_pc - 1), t = q / ppr, c = q - t * ppr;
            const int64_t row = (int64_t)s_pair[t < count ? t : 0] * n;
            v[i] = get_piece<AGENT>(a.act16 + row + 8 * c);
        }
        const int n_cs = a.n_blk * NT, ics = min(tid, n_cs - 1), t_cs = ics % NT;
        const float csv = get_f32<AGENT>(a.act_cs + (int64_t)s_pair[t_cs < count ? t_cs : 0] * a.n_blk + ics / NT);
#pragma unroll
        for (int i = 0; i < kGResIters; ++i) {
            if (i < iters) {
                const int q = tid + kGThreads * i, t = min(q / ppr, NT - 1), c = q % ppr;
                const bool live = q < n_pc && t < count;
                uint32_t wv[4], wp[4];
                words_of(v[i], wv);
#pragma unroll
                for (int k = 0; k < 4; ++k) wv[k] = live ? wv[k] : 0u;
                pair_inputs(wv, wp);
                if (q < n_pc) *reinterpret_cast<u32x4 *>(s_a + t * pad + 8 * c) = u32x4{wp[0], wp[1], wp[2], wp[3]};
                const float sm = group_sum_last<8>(sum8<false>(wv));
                if (q < n_pc && (c & 7) == 0) s_as[(c >> 3) * NT + t] = sm;
            }
        }
        if (tid < n_cs) s_cs[tid] = t_cs < count ? csv : 0.f;
    }
    // a row block's scales and biases, [group][row][s, b]: kGResIters loads
    // of each per thread (clamped as above) before the first store (the group
    // index runs fastest, so a wave reads whole rows of the scale matrices)
    auto stage_scales = [&](int row0) {
        const int tot = n_grp * kGRows, iters = (tot + kGThreads - 1) / kGThreads;
        uint32_t sv[kGResIters], bv[kGResIters];            // 16-bit values, one per register
#pragma unroll
        for (int i = 0; i < kGResIters; ++i) {
            const int idx = min(tid + kGThreads * i, tot - 1), r = idx / n_grp, G = idx - r * n_grp;
            const int64_t o = (erow + min(row0 + r, a.d_in - 1)) * a.down.gpr + G;
            sv[i] = a.down.s[o];
            bv[i] = a.down.b[o];
        }
#pragma unroll
        for (int i = 0; i < kGResIters; ++i) {
            const int idx = tid + kGThreads * i, r = idx / n_grp, G = idx - r * n_grp;
            if (i < iters && idx < tot) {
                const float sf = sb_to_float<SB>((uint16_t)sv[i]);
                *reinterpret_cast<float2 *>(&s_sb[(G * kGRows + r) * 2]) =
                    make_float2(sf, sb_to_float<SB>((uint16_t)bv[i]) - 1024.0f * sf);   // codes as 1024 + q
            }
        }
    };
    f32x4 acc[NB];
    int rbi = 0, c = 0;                                      // the step being computed
    auto step = [&](u32x4(&cur)[2], u32x4(&nxt)[2]) {
        const int row0 = (rb0 + rbi) * kGRows;
        if (c == 0) {
            __syncthreads();                                 // act staged / the previous block's scale readers done
            stage_scales(row0);
            __syncthreads();
#pragma unroll
            for (int m = 0; m < NB; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        uint32_t wd2[2][4];
        spread_code_pair<true>(cur[0], wd2[0]);
        spread_code_pair<true>(cur[1], wd2[1]);
        load_words(nxt);
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const uint32_t(&wd)[4] = wd2[p];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int G = c * kGChunkGroups + 2 * p + h;
                if (G >= n_grp) continue;
                const float sd = s_sb[(G * kGRows + rowl) * 2];
                uint32_t pq[2][4];
                nibble_pairs<0x64u>(wd[2 * h], pq[0]);
                nibble_pairs<0x64u>(wd[2 * h + 1], pq[1]);
#pragma unroll
                for (int m = 0; m < NB; ++m) {
                    const uint16_t *ar = s_a + (16 * m + j) * pad + G * kGroup + xo;
                    f32x4 t4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2)
                        t4 = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                            __builtin_bit_cast(f16x8_t, *reinterpret_cast<const u32x4 *>(ar + 8 * s2)),
                            __builtin_bit_cast(f16x8_t, u32x4{pq[s2][0], pq[s2][1], pq[s2][2], pq[s2][3]}), t4,
                            0, 0, 0);
                    const f32x4 cs = *reinterpret_cast<const f32x4 *>(&s_cs[(G * kGroup / kGRows) * NT + 16 * m + 4 * g]);
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[m][r] += (cs[r] * sd) * t4[r];
                }
            }
        }
        // the chunk's bias terms as one fp32 16x16x4 MFMA per pair block (a
        // group past the end: zero sum and zero bias)
        const int Gb = c * kGChunkGroups + g;
        const bool gok = Gb < n_grp;
        const float bv = gok ? s_sb[(Gb * kGRows + rowl) * 2 + 1] : 0.f;
#pragma unroll
        for (int m = 0; m < NB; ++m) {
            const float av = gok ? s_as[Gb * NT + 16 * m + j] * s_cs[(Gb * kGroup / kGRows) * NT + 16 * m + j] : 0.f;
            acc[m] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, acc[m], 0, 0, 0);
        }
        if (c == n_chunk - 1) {
            const int row = row0 + rowl;
            if (row < a.d_in) {
#pragma unroll
                for (int m = 0; m < NB; ++m)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int t = 16 * m + 4 * g + r;
                        if (t < count) a.partial[(int64_t)s_pair[t] * a.d_in + row] = s_score[t] * acc[m][r];
                    }
            }
        }
        if (++c == n_chunk) {
            c = 0;
            ++rbi;
        }
    };
    int st = 0;
    if constexpr (LEAD == 2) {
        for (; st + 2 < n_steps; st += 3) {
            step(rw0, rw2);
            step(rw1, rw0);
            step(rw2, rw1);
        }
        if (st < n_steps) step(rw0, rw2);
        if (st + 1 < n_steps) step(rw1, rw0);
    } else {
        for (; st + 3 < n_steps; st += 4) {
            step(rw0, rw3);
            step(rw1, rw0);
            step(rw2, rw1);
            step(rw3, rw2);
        }
        if (st < n_steps) step(rw0, rw3);
        if (st + 1 < n_steps) step(rw1, rw0);
        if (st + 2 < n_steps) step(rw2, rw1);
    }
}

// ------------------------------------------------------- the one-launch path
// Gate/up and down of the whole call in one launch: workgroups 0 ..
// grid_a - 1 are gate/up units (work item, row block), the rest down units
// (work item, res_rb row blocks), both placed as the separate kernels place
// them (an item's units on one XCD).  A down unit first waits until the
// gate/up units of its item have finished (a per-item counter), so the last
// gate/up units of the launch run beside the first down units instead of
// leaving most of the chip idle at the end of a separate gate/up launch, and
// only the last down units end alone.  Workgroups start in index order, so
// every gate/up unit a down unit waits for has started before it, and gate/up
// units never wait; the waits are bounded all the same (error word).  act16
// and act_cs travel with device-scope stores and loads; each wave waits for
// its stores before the item's counter moves.
template <int SB, int NB>
__global__ __launch_bounds__(kGThreads) __attribute__((amdgpu_waves_per_eu(4))) void ffn_grouped_fused(GroupedArgs a) {
    extern __shared__ __align__(16) unsigned char g_lds[];
    __shared__ int s_pair[16 * NB];
    __shared__ float s_score[16 * NB];
    const int n_work = *a.n_work;
    if ((int)blockIdx.x < a.grid_a) {
        int w, rb;
        item_and_block(a.row_blocks, w, rb);
        if (w >= n_work) return;
        gate_up_unit<SB, NB, true>(a, w, rb, GUSmem<NB>(g_lds));
        __builtin_amdgcn_s_waitcnt(0x0F70);                  // vmcnt(0): this wave's act16 / act_cs stores are done
        __syncthreads();
        if (threadIdx.x == 0) __hip_atomic_fetch_add(a.done + w, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
        int w, rbb;
        item_and_block(a.row_blocks_b, w, rbb, blockIdx.x - a.grid_a);
        if (w >= n_work) return;
        down_unit<SB, NB, true>(a, w, rbb, g_lds, s_pair, s_score);
    }
}

static int grouped_max_work(int n_pairs, int E, int nt) { return (n_pairs + nt - 1) / nt + E + 1; }

// Pairs per work item: 16 NB, from the average number of pairs per expert.
// Measured on the Qwen3-shaped layer: 16-pair items are faster up to about 8
// pairs per expert (128 tokens: 108 against 116 us per call), 32-pair items
// above (192 tokens: 117 against 129 us); 64-pair items (each expert read
// once up to 64 pairs, but 166 VGPRs: two waves per SIMD) were never faster
// (256 tokens 203 against 136 us, 1024 tokens 308 against 292 us).
static int grouped_nb(int n_pairs, int E) { return n_pairs / E <= 9 ? 1 : 2; }

// Workspace: the head (error word, n_work, two spare words),
// the work lists and per-item counters (int32), then act16, then act_cs,
// each 256-byte aligned.
constexpr int kGHeadWords = 4;

struct GroupedLayout {
    size_t act16, act_cs, total;
};

static GroupedLayout grouped_layout(int n_tokens, int top_k, int n_experts, int d_ff) {
    GroupedLayout L;
    const size_t n_pairs = (size_t)n_tokens * top_k;
    const size_t mw = (size_t)grouped_max_work((int)n_pairs, n_experts, kGMinTok);
    L.act16 = align_up((kGHeadWords + 4 * mw + n_pairs) * sizeof(int32_t), 256);
    L.act_cs = L.act16 + align_up(n_pairs * d_ff * sizeof(uint16_t), 256);
    L.total = L.act_cs + align_up(n_pairs * ((d_ff + kGRows - 1) / kGRows) * sizeof(float), 256);
    return L;
}

// Dynamic LDS above the default 64 KB per workgroup is allowed per kernel
// once (the largest size asked so far is remembered per kernel; gfx950 gives
// a workgroup up to 160 KB).
static void allow_dynamic_lds(const void *kernel, size_t bytes) {
    if (bytes <= 64 * 1024) return;
    static std::mutex mu;
    static std::map<const void *, size_t> allowed;
    std::lock_guard<std::mutex> lock(mu);
    size_t &have = allowed[kernel];
    if (have >= bytes) return;
    if (hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes) == hipSuccess) have = bytes;
}

// Row blocks per down unit of the one-launch path: 4 when the call is
// expected to touch at least 64 work items (expected distinct experts under
// uniform routing, plus the items beyond 16 NB pairs), else 1 (with few items,
// longer units leave CUs idle).  Measured on the Qwen3-shaped layer at 4, 2
// and 1 row blocks: 32 tokens 97.9 / 100.3 / 105.7 us per call, 256 tokens
// 115.1 / 122.3 / 134.9 us; 1 token 43 us at 4.
static int fused_rb(int n_pairs, int E, int nt) {
    const double items = E * (1.0 - std::exp(n_pairs * std::log1p(-1.0 / E))) + (double)n_pairs / nt;
    return items >= 64.0 ? 4 : 1;
}

template <int SB, int NB>
static void launch_grouped(const GroupedArgs &a, int mw, hipStream_t s) {
    const int items8 = (mw + 7) / 8 * 8;
    const int ra = (a.d_ff + kGRows - 1) / kGRows, n_rb = (a.d_in + kGRows - 1) / kGRows;
    if (res_fits(16 * NB, a.d_ff)) {
        GroupedArgs f = a;
        f.row_blocks = ra;
        f.res_rb = fused_rb(a.T * a.K, a.E, 16 * NB);
        f.row_blocks_b = (n_rb + f.res_rb - 1) / f.res_rb;
        f.grid_a = items8 * ra;
        const size_t lds = std::max(GUSmem<NB>::kBytes, res_lds_bytes(16 * NB, a.d_ff));
        allow_dynamic_lds(reinterpret_cast<const void *>(&ffn_grouped_fused<SB, NB>), lds);
        hipLaunchKernelGGL((ffn_grouped_fused<SB, NB>), dim3(items8 * (ra + f.row_blocks_b)), dim3(kGThreads), lds, s,
                           f);
        return;
    }
    GroupedArgs ga = a, gb = a;
    ga.row_blocks = ra;
    hipLaunchKernelGGL((gate_up_grouped<SB, NB>), dim3(items8 * ga.row_blocks), dim3(kGThreads), 0, s, ga);
    gb.row_blocks = n_rb;
    hipLaunchKernelGGL((down_grouped<SB, NB>), dim3(items8 * gb.row_blocks), dim3(kGThreads), 0, s, gb);
}

}  // namespace moe

using namespace moe;

extern "C" size_t moe_decode_expert_ffn_grouped_workspace_bytes(int32_t n_tokens, int32_t top_k, int32_t n_experts,
                                                                int32_t d_ff) {
    if (n_tokens < 1 || top_k < 1 || n_experts < 1 || d_ff < 1) return 0;
    return grouped_layout(n_tokens, top_k, n_experts, d_ff).total;
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
    const GroupedLayout L = grouped_layout(n_tokens, top_k, E, d_ff);
    if (workspace_bytes < L.total) return MOE_EINVAL;
    const int n_pairs = n_tokens * top_k, nb = grouped_nb(n_pairs, E), nt = 16 * nb;
    const int mw = grouped_max_work(n_pairs, E, nt), mw_ws = grouped_max_work(n_pairs, E, kGMinTok);
    GroupedArgs a;
    a.x = reinterpret_cast<const uint16_t *>(x);
    a.T = n_tokens; a.K = top_k; a.E = E; a.d_in = d_in; a.d_ff = d_ff;
    a.n_blk = (d_ff + kGRows - 1) / kGRows;
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
    a.scores = scores; a.act = act; a.partial = partial;
    char *wsb = reinterpret_cast<char *>(workspace);
    int32_t *ws = reinterpret_cast<int32_t *>(wsb);
    a.err = ws;
    a.n_work = ws + 1;
    a.work_expert = ws + kGHeadWords;
    a.work_begin = ws + kGHeadWords + mw_ws;
    a.work_count = ws + kGHeadWords + 2 * mw_ws;
    a.done = ws + kGHeadWords + 3 * mw_ws;
    a.pair_list = ws + kGHeadWords + 4 * mw_ws;
    a.act16 = reinterpret_cast<uint16_t *>(wsb + L.act16);
    a.act_cs = reinterpret_cast<float *>(wsb + L.act_cs);
    a.row_blocks = 1;
    a.res_rb = 1;
    a.row_blocks_b = 1;
    a.grid_a = 0;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(grouped_bucket_kernel, dim3(1), dim3(kGBucketThreads), 0, s, expert_ids, n_pairs, E, nt,
                       ws + 1, ws + kGHeadWords, ws + kGHeadWords + mw_ws, ws + kGHeadWords + 2 * mw_ws,
                       ws + kGHeadWords + 4 * mw_ws, a.err, a.done, mw_ws);
    const bool bf = sb == MOE_BF16;
    if (nb == 1)
        bf ? launch_grouped<MOE_BF16, 1>(a, mw, s) : launch_grouped<MOE_F16, 1>(a, mw, s);
    else
        bf ? launch_grouped<MOE_BF16, 2>(a, mw, s) : launch_grouped<MOE_F16, 2>(a, mw, s);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}
