/*
 * moe_decode.h -- C ABI of the MI355X (gfx950) quantized MoE decode layer.
 *
 * One decode step of a mixture-of-experts layer over group-wise
 * affine-quantized expert weights, split into the three calls the layer is
 * made of:
 *
 *   moe_decode_route       router logits, softmax, top-k, scores (+ shared gate)
 *   moe_decode_expert_ffn  per selected expert: gate/up GEMV + SwiGLU -> act
 *                          ("kernel A"), down GEMV * score -> partial ("kernel B")
 *   moe_decode_tail        out = resid + (sum_k partial_k + shared * gate)
 *
 * Sources: mlxcel PR #276, "two-kernel decode-MoE that beats gather_qmm",
 * section "What changed" step 2 (the act/partial split), "Scope / flags"
 * (4- and 8-bit affine weights) and "Next" (6-bit and mixed-bit weights);
 * Red Lite dev39, "fused expert tail (GPU-routed decode)", section "Change"
 * (GPU routing, per-expert outputs exposed by the pool, the one-dispatch
 * tail).
 *
 * Conventions for every call:
 *  - All tensor pointers are DEVICE pointers owned by the caller; moe_qmat
 *    and the call arguments themselves live on the host.  The library never
 *    allocates, frees, copies to or from the host, synchronises, or prints.
 *  - All work is enqueued on `stream` (a hipStream_t; NULL = the legacy
 *    default stream).  Buffers must stay valid until the stream reaches the
 *    enqueued work.  Calls may be captured into a HIP graph.
 *  - Arguments are validated on the host before anything is enqueued; an
 *    invalid call returns a status and enqueues nothing.  MOE_EHIP reports a
 *    failed launch.
 *  - Tensors are dense, row-major, with the shapes given below.
 *  - Results are deterministic: repeated calls on the same inputs give
 *    bit-identical outputs (no floating-point atomics are used).
 */
#ifndef MOE_DECODE_H
#define MOE_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_DECODE_ABI_VERSION 4

typedef enum {
    MOE_OK = 0,
    MOE_EINVAL = 1,        /* null pointer, inconsistent shape, out-of-range size, misalignment */
    MOE_EUNSUPPORTED = 2,  /* bit width, group size or dtype combination that is not built */
    MOE_EHIP = 3,          /* the HIP runtime reported an error when launching */
    MOE_ETIMEOUT = 4       /* recorded in a workspace: a wait inside a launch ran out (moe_decode_workspace_status) */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_F16 = 1, MOE_BF16 = 2 } moe_dtype;

/*
 * One stack of quantized projection matrices, one per expert.
 * Expert e's matrix W_e has `rows` outputs and `cols` inputs (the
 * contraction dimension).  Its weight is w[r][j] = scale[r][j/64] * q[r][j]
 * + bias[r][j/64] (groups of 64 along the contraction dimension; mlxcel PR
 * #276, "Scope / flags": affine quantization).
 *   q       : uint32 [n_experts][rows][cols*bits/32]; code j of a row occupies
 *             bits [bits*j, bits*j+bits) of the row's little-endian, LSB-first
 *             bit stream (6-bit codes straddle words; 16 codes per 3 words).
 *             Must be 16-byte aligned.
 *   scales, biases : sb_dtype [n_experts][rows][cols/64].
 *   bits       : 4, 6 or 8.      group_size : must be 64.
 *   sb_dtype   : MOE_F16 or MOE_BF16.
 *   cols must be a multiple of 64.
 */
typedef struct {
    const uint32_t *q;
    const void *scales;
    const void *biases;
    int32_t n_experts;
    int32_t rows;
    int32_t cols;
    int32_t bits;
    int32_t group_size;
    moe_dtype sb_dtype;
} moe_qmat;

/* Limits checked by every call.  MOE_MAX_TOKENS: tokens per call of the
 * fused layer and of moe_decode_expert_ffn, moe_decode_gate_up and
 * moe_decode_down (and their variants). */
#define MOE_MAX_TOKENS 32
#define MOE_MAX_TOP_K 32
#define MOE_MAX_EXPERTS 1024
/* tokens per call of moe_decode_expert_ffn_grouped, and of moe_decode_route,
 * moe_decode_tail and the RMSNorm calls that feed or follow it */
#define MOE_MAX_GROUPED_TOKENS 1024
#define MOE_MAX_DIM 8192

/*
 * Routing (Red Lite dev39, "Change": the layer is GPU-routed).  Per token t:
 *   logits[e] = sum_j w_router[e][j] * x[t][j]           (fp32 accumulation)
 *   p = softmax(logits) over all n_experts
 *   expert_ids[t][0..top_k) = experts by descending logit, ties to the lower id
 *   scores[t][k] = p[id_k] / sum_k' p[id_k']  if renormalize, else p[id_k]
 *   shared_gate[t] = sigmoid(sum_j w_shared_gate[j] * x[t][j])  if w_shared_gate
 * Arguments:
 *   x           [n_tokens][d_in], dtype x_dtype (F32, F16 or BF16)
 *   w_router    [n_experts][d_in], dtype w_router_dtype
 *   w_shared_gate [d_in] or NULL, dtype w_shared_gate_dtype
 *   expert_ids  out int32 [n_tokens][top_k]
 *   scores      out float [n_tokens][top_k]
 *   shared_gate out float [n_tokens]; must be NULL iff w_shared_gate is NULL
 *   workspace   device scratch of at least moe_decode_route_workspace_bytes(),
 *               16-byte aligned; zero-filled before its first use and not
 *               written by the caller afterwards: it carries a launch epoch
 *               from call to call, and each call leaves it in the state the
 *               next call expects.  The router logits travel between the
 *               launch's workgroups as words tagged with that epoch, so no
 *               word of an earlier call can be taken for one of this call.
 *               Every internal wait is bounded; if one runs out (possible only
 *               when other work starves the launch for a long time) the
 *               workspace's error word is raised, stays raised, and
 *               moe_decode_workspace_status reports MOE_ETIMEOUT.  Calls that
 *               may run concurrently need separate workspaces.
 * Limits: 1 <= n_tokens <= MOE_MAX_GROUPED_TOKENS, 1 <= top_k <= min(n_experts, 32),
 *         n_experts <= 1024, d_in a multiple of 64 and <= 8192.
 */
moe_status moe_decode_route(const void *x, moe_dtype x_dtype, int32_t n_tokens, int32_t d_in,
                            const void *w_router, moe_dtype w_router_dtype,
                            int32_t n_experts, int32_t top_k, int32_t renormalize,
                            const void *w_shared_gate, moe_dtype w_shared_gate_dtype,
                            int32_t *expert_ids, float *scores, float *shared_gate,
                            void *workspace, size_t workspace_bytes, void *stream);

size_t moe_decode_route_workspace_bytes(int32_t n_tokens, int32_t n_experts);

/*
 * Status recorded in the workspace of moe_decode_route, moe_decode_layer or
 * moe_decode_expert_ffn_grouped.
 * `head` is a host copy of the first MOE_WORKSPACE_HEAD_BYTES bytes of the
 * workspace, taken after the stream has passed the calls of interest (the
 * library itself never copies device memory).  Returns MOE_OK, or
 * MOE_ETIMEOUT when a wait inside some launch that used the workspace ran out
 * since the workspace was last zero-filled (route, layer) or within the last
 * call (grouped expert FFN, whose calls clear the word); that launch's
 * results are invalid.  MOE_EINVAL for a null `head` or head_bytes <
 * MOE_WORKSPACE_HEAD_BYTES.  Host-only; no device access.
 */
#define MOE_WORKSPACE_HEAD_BYTES 4
moe_status moe_decode_workspace_status(const void *head, size_t head_bytes);

/*
 * Expert FFN (mlxcel PR #276, "What changed" step 2).  For every token t and
 * slot k with e = expert_ids[t][k]:
 *   act[t][k][r]     = silu(g_r) * u_r,  g = W_gate[e] x_t,  u = W_up[e] x_t   (kernel A)
 *   partial[t][k][i] = score[t][k] * (W_down[e] act[t][k])[i]                  (kernel B)
 * where silu(z) = z * sigmoid(z) and score = 1 when `scores` is NULL.
 * An id outside [0, n_experts) yields all-zero act and partial rows.
 * With n_tokens > 1, the pairs are regrouped by expert and an expert's weights
 * are streamed once per work item of up to 4 of its tokens (an expert with
 * more tokens is streamed again, mostly from cache).
 * A shared expert is run through this same call with its own stacks,
 * expert_ids[t][s] = s and scores = NULL; its partial is the `shared` input
 * of moe_decode_tail.
 * Arithmetic: fp32 sums throughout.  Kernel A with 4-bit codes and bf16 x
 * uses the packed bf16 dot (the code q as the exact bf16 128 + q, products
 * exact); other gate/up formats convert codes and inputs to fp32.  Kernel B
 * stages each act row as fp16 after an exact power-of-two scaling (2^8, or
 * the factor fitted to the row's largest magnitude when 2^8 would overflow)
 * and uses the packed fp16 dot (codes as exact fp16 values).  The result
 * stays within 2e-3 of its infinity norm.
 * Arguments:
 *   x        [n_tokens][d_in], dtype x_dtype; d_in = gate->cols
 *   gate, up : stacks with rows = d_ff, cols = d_in; down: rows = d_in, cols = d_ff;
 *              the same n_experts and sb_dtype; gate->bits == up->bits
 *   expert_ids int32 [n_tokens][top_k]; scores float [n_tokens][top_k] or NULL
 *   act      out float [n_tokens][top_k][d_ff]   (also read back by kernel B)
 *   partial  out float [n_tokens][top_k][d_in]
 *   workspace device scratch of moe_decode_expert_ffn_workspace_bytes() bytes
 *             (0 bytes, and NULL allowed, when n_tokens == 1); no zeroing needed.
 * Limits: as for moe_decode_route; d_in and d_ff multiples of 64, <= 8192.
 */
moe_status moe_decode_expert_ffn(const void *x, moe_dtype x_dtype, int32_t n_tokens,
                                 const moe_qmat *gate, const moe_qmat *up, const moe_qmat *down,
                                 const int32_t *expert_ids, const float *scores, int32_t top_k,
                                 float *act, float *partial,
                                 void *workspace, size_t workspace_bytes, void *stream);

size_t moe_decode_expert_ffn_workspace_bytes(int32_t n_tokens, int32_t top_k, int32_t n_experts);

/*
 * moe_decode_expert_ffn for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same computation, kernels and results, with the
 * workspace taken from a fixed device array the library holds, one per
 * device, for the life of the process (moe_decode_expert_ffn_noalloc_max_bytes()
 * bytes, enough for every call within the limits: up to 32 tokens, top-32,
 * 1024 experts).  Nothing is allocated or freed; the array's device address
 * is looked up once per device, on the first call made with that device
 * current.  The caller still passes every input and output.
 * Calls that overlap on one device (concurrent streams, or host threads)
 * share that device's array and race: order them on one stream.  The array
 * keeps the last call's contents; every call writes what it reads, so no
 * clearing is needed.  Returns MOE_EINVAL for anything moe_decode_expert_ffn
 * rejects or a workspace need beyond the array (not reachable within the
 * limits), MOE_EHIP if the array's address cannot be obtained.
 */
moe_status moe_decode_expert_ffn_noalloc(const void *x, moe_dtype x_dtype, int32_t n_tokens,
                                         const moe_qmat *gate, const moe_qmat *up, const moe_qmat *down,
                                         const int32_t *expert_ids, const float *scores, int32_t top_k,
                                         float *act, float *partial, void *stream);

size_t moe_decode_expert_ffn_noalloc_max_bytes(void);

/*
 * moe_decode_expert_ffn for larger batches and prefill, on the matrix cores:
 * the same outputs (act and partial, same layouts, same zero rows for ids
 * outside [0, n_experts)) for up to MOE_MAX_GROUPED_TOKENS tokens.  The
 * (token, slot) pairs are grouped by expert into work items of up to 16 or
 * 32 pairs, and each work item is a small GEMM per expert (meTile PR #30,
 * the GB/s table and its reading: a GEMM path pays only from about 32 rows,
 * i.e. batch or prefill, not single-token decode).  Supported: 4-bit gate,
 * up and down codes with bf16 or fp16 scales, bf16 x; anything else is
 * MOE_EUNSUPPORTED.  scores may be NULL (every pair weighted 1).
 * Arithmetic: codes exact in the products (bf16 128 + q for gate/up, fp16 q
 * for down), fp32 accumulation, the affine scale and bias applied per group
 * of 64 inputs; act enters the down projection as fp16 after a power of two
 * fitted to the largest magnitude of each block of 128 of a pair's values
 * (exact, undone per group).  Within 2e-3 of the result's infinity norm.
 * workspace: moe_decode_expert_ffn_grouped_workspace_bytes() bytes (the work
 * lists, per-item counters and the fp16 copy of act), 16-byte aligned, no
 * zeroing needed; asynchronous on `stream`.  Its first
 * MOE_WORKSPACE_HEAD_BYTES bytes are an error word that each call clears:
 * when act fits the down units' LDS the call runs gate/up and down in one
 * launch, where a down unit waits (bounded) for the gate/up units of its
 * work item; if such a wait ran out, that call's results are invalid and
 * moe_decode_workspace_status on a host copy of the head reports
 * MOE_ETIMEOUT.  Calls that may overlap need separate workspaces.
 */
moe_status moe_decode_expert_ffn_grouped(const void *x, moe_dtype x_dtype, int32_t n_tokens,
                                         const moe_qmat *gate, const moe_qmat *up, const moe_qmat *down,
                                         const int32_t *expert_ids, const float *scores, int32_t top_k,
                                         float *act, float *partial, void *workspace, size_t workspace_bytes,
                                         void *stream);

/* d_ff: rows of gate (columns of down).  0 for a size below 1. */
size_t moe_decode_expert_ffn_grouped_workspace_bytes(int32_t n_tokens, int32_t top_k, int32_t n_experts,
                                                     int32_t d_ff);

/*
 * The two halves of moe_decode_expert_ffn as separate calls, for callers that
 * schedule kernel A and kernel B themselves (mlxcel PR #276, "What changed"
 * step 2: two dispatches with act staged in global memory between them).
 * moe_decode_gate_up writes act exactly as moe_decode_expert_ffn does;
 * moe_decode_down reads act [n_tokens][top_k][down->cols] and writes partial.
 * Same limits, ownership and workspace rules as moe_decode_expert_ffn; with
 * n_tokens > 1 each call regroups the pairs by expert in its workspace.
 */
moe_status moe_decode_gate_up(const void *x, moe_dtype x_dtype, int32_t n_tokens,
                              const moe_qmat *gate, const moe_qmat *up,
                              const int32_t *expert_ids, int32_t top_k, float *act,
                              void *workspace, size_t workspace_bytes, void *stream);

moe_status moe_decode_down(const float *act, int32_t n_tokens, const moe_qmat *down,
                           const int32_t *expert_ids, const float *scores, int32_t top_k,
                           float *partial, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Tail (Red Lite dev39, "Change": one dispatch, one thread per hidden
 * element).  For every token t and hidden index i:
 *   routed = (((partial[t][0][i] + partial[t][1][i]) + ...) + partial[t][top_k-1][i])
 *   shared = shared[t][0][i] + ... + shared[t][n_shared-1][i]   (0 when n_shared == 0)
 *   out[t][i] = residual[t][i] + (routed + shared * g),  g = shared_gate[t] or 1
 * The sums run left to right in slot order in fp32.
 * Arguments:
 *   partial  [n_tokens][top_k][d_in] float
 *   shared   [n_tokens][n_shared][d_in] float, or NULL iff n_shared == 0
 *   shared_gate [n_tokens] float or NULL (gate 1)
 *   residual [n_tokens][d_in], dtype residual_dtype
 *   out      out [n_tokens][d_in], dtype out_dtype, aligned to its element
 *            size; may not alias the inputs
 * Output dtype: the fp32 sum above is what F32 stores; BF16 and F16 store it
 * rounded once to the nearest value of that type, ties to even (overflow to
 * infinity), so the layer drops into an engine that keeps its hidden state in
 * 16 bits (mlxcel PR #276, "Validation": the fused path checked inside the
 * engine's own decode loop; Red Lite dev39, "Scope boundary": parity checked
 * by error bounds rather than bit identity).  Everything before the store
 * (partial, shared, the sums) stays at least as precise as with F32 output.
 */
moe_status moe_decode_tail(const float *partial, int32_t n_tokens, int32_t top_k, int32_t d_in,
                           const float *shared, int32_t n_shared, const float *shared_gate,
                           const void *residual, moe_dtype residual_dtype, void *out, moe_dtype out_dtype,
                           void *stream);

/*
 * The whole layer for ONE token in a single launch: route, kernel A and
 * kernel B for the K selected experts and the S shared experts, and the tail:
 * the same computation as moe_decode_route + moe_decode_expert_ffn (routed,
 * then shared) + moe_decode_tail (sources as cited above), the same routing
 * bit for bit and the same summation order, but not the same rounding: with
 * 4-bit weights and bf16 x the gate/up dot products use the packed bf16 dot
 * (128 + q as exact bf16 pairs, one rounding per pair sum), and the down
 * projections take act staged as fp16 after an exact power-of-two scaling
 * (2^8, or a factor fitted to the slot's largest magnitude when that would
 * overflow, as in moe_decode_expert_ffn), with fp32 sums throughout.  Both stay within 2e-3 of the result's infinity norm.
 * Workgroups hand results to each other through the workspace instead of
 * kernel boundaries, so the down-projection weights stream while the gate/up
 * projections run (the dependency mlxcel PR #276 "What changed" step 1
 * describes, resolved inside one launch).
 *
 * moe_layer_weights (host struct; every pointer in it is a device pointer):
 *   w_router [n_experts][d_in] in the dtype of x; n_experts == gate.n_experts
 *   top_k, renormalize         as in moe_decode_route
 *   gate, up, down             routed stacks (as in moe_decode_expert_ffn)
 *   n_shared                   0..MOE_MAX_SHARED shared experts, summed in order
 *   shared_gate/_up/_down      shared stacks (n_experts = n_shared; their own
 *                              d_ff; same bit widths and scale dtype as the
 *                              routed stacks); ignored when n_shared == 0
 *   w_shared_gate              [d_in] in the dtype of x, or NULL (gate 1); only
 *                              with n_shared > 0
 * Arguments: x [d_in] and residual [d_in] (one token); out [d_in] of dtype
 * out_dtype, rounded as moe_decode_tail's;
 * expert_ids [top_k], scores [top_k], shared_gate [1]: optional outputs (NULL
 * to skip); workspace of moe_decode_layer_workspace_bytes() bytes, 16-byte
 * aligned, zero-filled before its first use and not written by the caller
 * afterwards (each launch leaves it ready for the next).  Its first 4 bytes
 * become nonzero, and stay so, if an internal wait ever timed out (results of
 * that launch invalid; moe_decode_workspace_status reports MOE_ETIMEOUT); this
 * cannot happen unless the device is shared with work that starves the launch
 * for a long time.  Launches that may run concurrently need separate
 * workspaces; launches in order on one stream may share one workspace, also
 * across layers of different shapes, if it has the largest layer's size.
 */
#define MOE_MAX_SHARED 8

typedef struct {
    const void *w_router;
    moe_dtype w_router_dtype;
    int32_t n_experts;
    int32_t top_k;
    int32_t renormalize;
    moe_qmat gate, up, down;
    int32_t n_shared;
    moe_qmat shared_gate, shared_up, shared_down;
    const void *w_shared_gate;
} moe_layer_weights;

moe_status moe_decode_layer(const moe_layer_weights *weights, const void *x, moe_dtype x_dtype,
                            const void *residual, moe_dtype residual_dtype, void *out, moe_dtype out_dtype,
                            int32_t *expert_ids, float *scores, float *shared_gate,
                            void *workspace, size_t workspace_bytes, void *stream);

/* 0 when the weights are invalid or unsupported. */
size_t moe_decode_layer_workspace_bytes(const moe_layer_weights *weights);

/*
 * The next layer's RMSNorm of the layer output, folded into the tail (Red
 * Lite dev39, "fused expert tail (GPU-routed decode)", section
 * "Measurements": a tail that also computed the next layer's RMSNorm; there it
 * ran on one threadgroup and lost to the separate dispatches, here the sum of
 * squares is spread over the tail's workgroups).  For every token t:
 *   normed[t][i] = out[t][i] / sqrt((1/d_in) sum_i out[t][i]^2 + eps) * weight[i]
 * computed from out as stored (after its rounding to out's dtype), in fp32,
 * and rounded to normed_dtype as out is.  Each tail workgroup sums the
 * squares of its own elements in a fixed order and the workgroups' sums are
 * added in workgroup order, so repeated calls give the same bits.
 *   weight        [d_in] device pointer, dtype `dtype` (F32, F16 or BF16),
 *                 aligned to its element size
 *   eps           >= 0 and finite
 *   normed        out [n_tokens][d_in] device pointer, dtype normed_dtype,
 *                 aligned to its element size; may not alias out
 *   normed_dtype  F32, F16 or BF16
 */
typedef struct {
    const void *weight;
    moe_dtype dtype;
    float eps;
    void *normed;
    moe_dtype normed_dtype;
} moe_rmsnorm;

/*
 * moe_decode_tail, also writing norm->normed (norm must not be NULL).  The
 * workspace (moe_decode_tail_rmsnorm_workspace_bytes() bytes, 16-byte aligned)
 * is zero-filled before its first use and not written by the caller
 * afterwards: like moe_decode_route's, it carries a launch epoch from call
 * to call, its first MOE_WORKSPACE_HEAD_BYTES bytes are the error word
 * (moe_decode_workspace_status), and calls that may overlap need separate
 * workspaces.  MOE_EUNSUPPORTED if the device cannot hold all
 * n_tokens * ceil(d_in / 256) workgroups at once.
 */
moe_status moe_decode_tail_rmsnorm(const float *partial, int32_t n_tokens, int32_t top_k, int32_t d_in,
                                   const float *shared, int32_t n_shared, const float *shared_gate,
                                   const void *residual, moe_dtype residual_dtype, void *out,
                                   moe_dtype out_dtype, const moe_rmsnorm *norm, void *workspace,
                                   size_t workspace_bytes, void *stream);

size_t moe_decode_tail_rmsnorm_workspace_bytes(int32_t n_tokens, int32_t d_in);

/*
 * The same RMSNorm as a call of its own, one workgroup per token: normed =
 * y / sqrt(mean(y^2) + eps) * weight for y [n_tokens][d] of dtype y_dtype
 * (device, aligned to its element size), computed in fp32 and rounded to
 * norm->normed_dtype.  The separate dispatch the folded forms are measured
 * against.
 */
moe_status moe_decode_rmsnorm(const void *y, moe_dtype y_dtype, int32_t n_tokens, int32_t d,
                              const moe_rmsnorm *norm, void *stream);

/* moe_decode_layer, also writing norm->normed (norm must not be NULL); the
 * same workspace as moe_decode_layer. */
moe_status moe_decode_layer_rmsnorm(const moe_layer_weights *weights, const void *x, moe_dtype x_dtype,
                                    const void *residual, moe_dtype residual_dtype, void *out,
                                    moe_dtype out_dtype, const moe_rmsnorm *norm, int32_t *expert_ids, float *scores,
                                    float *shared_gate, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Streaming-read probe: a measurement aid, not part of the layer.  Reads
 * `bytes` bytes at `data` (device memory, 16-byte aligned, bytes a nonzero
 * multiple of 16) exactly once with 16-byte loads and writes one fp32 partial
 * sum of the buffer's fp32 values per workgroup to partial_sums[0..n) (device
 * memory), n = moe_decode_read_probe_blocks(bytes); n_partial must be at least
 * n (MOE_EINVAL otherwise).  Its launch time gives the machine's practical
 * HBM read rate for a read of that size, the ceiling the decode kernels are
 * compared with (meTile PR #30: decode GEMVs measured against streaming).
 * Asynchronous on `stream`; allocates nothing.
 */
moe_status moe_decode_read_probe(const void *data, size_t bytes, float *partial_sums, int32_t n_partial,
                                 void *stream);
int32_t moe_decode_read_probe_blocks(size_t bytes);

/* Human-readable name of a status code (static storage). */
const char *moe_decode_status_string(moe_status s);

/* MOE_DECODE_ABI_VERSION of the built library. */
int32_t moe_decode_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_DECODE_H */
