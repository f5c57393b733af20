// moe_decode_layer: the fused single-launch decode layer (layer_kernel.hpp).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <tuple>

#include "api.hpp"
#include "layer_kernel.hpp"

namespace moe {

static int codes_of(int bits) { return bits == 4 ? 32 : 16; }

static int lr_shift_for(int cpr) {
    int s = 0;
    while (s < 6 && (1 << s) < cpr) ++s;
    return s;
}

struct LayerPlan {
    LayerArgs a;
    int a_nr;                       // kLayerNRA: kernel-A units of one stage; kLayerNRA2: pipelined stages
    int grid;
    size_t lds;
    size_t ws_bytes;
    size_t off_logits, off_act, off_act_sent, off_partial, off_norm;
};

static moe_status plan_layer(const moe_layer_weights *w, int d_in_check, LayerPlan &p) {
    if (!w || !w->w_router) return MOE_EINVAL;
    moe_status st;
    for (const moe_qmat *m : {&w->gate, &w->up, &w->down})
        if ((st = check_qmat(m)) != MOE_OK) return st;
    const int d_in = w->gate.cols, d_ff = w->gate.rows, E = w->gate.n_experts;
    if (w->up.rows != d_ff || w->up.cols != d_in || w->down.rows != d_in || w->down.cols != d_ff)
        return MOE_EINVAL;
    if (w->up.n_experts != E || w->down.n_experts != E || w->n_experts != E) return MOE_EINVAL;
    if (w->up.bits != w->gate.bits) return MOE_EUNSUPPORTED;
    const int sb = raw_enum(w->gate.sb_dtype);
    if (raw_enum(w->up.sb_dtype) != sb || raw_enum(w->down.sb_dtype) != sb) return MOE_EUNSUPPORTED;
    if (d_in_check >= 0 && d_in_check != d_in) return MOE_EINVAL;
    if (w->top_k < 1 || w->top_k > MOE_MAX_TOP_K || w->top_k > E) return MOE_EINVAL;
    if (w->n_shared < 0 || w->n_shared > MOE_MAX_SHARED) return MOE_EINVAL;
    if (!valid_dtype(raw_enum(w->w_router_dtype))) return MOE_EUNSUPPORTED;
    if (!aligned16(w->w_router)) return MOE_EINVAL;
    int d_ffs = 0;
    if (w->n_shared > 0) {
        for (const moe_qmat *m : {&w->shared_gate, &w->shared_up, &w->shared_down})
            if ((st = check_qmat(m)) != MOE_OK) return st;
        d_ffs = w->shared_gate.rows;
        if (w->shared_gate.cols != d_in || w->shared_up.cols != d_in || w->shared_up.rows != d_ffs ||
            w->shared_down.rows != d_in || w->shared_down.cols != d_ffs)
            return MOE_EINVAL;
        if (w->shared_gate.n_experts != w->n_shared || w->shared_up.n_experts != w->n_shared ||
            w->shared_down.n_experts != w->n_shared)
            return MOE_EINVAL;
        if (w->shared_gate.bits != w->gate.bits || w->shared_up.bits != w->gate.bits ||
            w->shared_down.bits != w->down.bits)
            return MOE_EUNSUPPORTED;
        if (raw_enum(w->shared_gate.sb_dtype) != sb || raw_enum(w->shared_up.sb_dtype) != sb ||
            raw_enum(w->shared_down.sb_dtype) != sb)
            return MOE_EUNSUPPORTED;
    } else if (w->w_shared_gate) {
        return MOE_EINVAL;       // a shared gate needs shared experts
    }
    if (w->w_shared_gate && !aligned16(w->w_shared_gate)) return MOE_EINVAL;

    LayerArgs &a = p.a;
    a = LayerArgs{};
    a.wr = w->w_router;
    a.wg = w->w_shared_gate;
    a.E = E; a.K = w->top_k; a.renorm = w->renormalize ? 1 : 0; a.S = w->n_shared;
    a.d_in = d_in; a.d_ff = d_ff; a.d_ffs = d_ffs;
    auto qm = [](const moe_qmat &m) {
        QM q;
        q.q = m.q;
        q.s = reinterpret_cast<const uint16_t *>(m.scales);
        q.b = reinterpret_cast<const uint16_t *>(m.biases);
        q.rows = m.rows; q.cols = m.cols;
        q.wpr = m.cols * m.bits / 32; q.gpr = m.cols / 64;
        q.bits_ = m.bits; q.sb_ = raw_enum(m.sb_dtype);
        return q;
    };
    a.gate = qm(w->gate); a.up = qm(w->up); a.down = qm(w->down);
    if (a.S > 0) { a.sgate = qm(w->shared_gate); a.sup = qm(w->shared_up); a.sdown = qm(w->shared_down); }

    const int slots = a.K + a.S;
    a.n_route = (E + (a.wg ? 1 : 0) + 3) / 4;
    a.a_lr_shift = lr_shift_for(d_in / codes_of(w->gate.bits));
    a.a_tile = 4 * (64 >> a.a_lr_shift) * kLayerNRA;
    a.a_tiles_r = (d_ff + a.a_tile - 1) / a.a_tile;
    a.a_tiles_s = a.S > 0 ? (d_ffs + a.a_tile - 1) / a.a_tile : 0;
    const int cb = codes_of(w->down.bits);
    a.b_lr_shift_r = lr_shift_for(d_ff / cb);
    a.b_lr_shift_s = a.S > 0 ? lr_shift_for(d_ffs / cb) : a.b_lr_shift_r;
    a.b_tile = 4 * (64 >> a.b_lr_shift_r) * kLayerNRB;
    a.b_tiles = (d_in + a.b_tile - 1) / a.b_tile;
    const int dmax = d_ffs > d_ff ? d_ffs : d_ff;
    a.act_stride = dmax;
    p.grid = a.n_route + a.K * a.a_tiles_r + a.S * a.a_tiles_s + slots * a.b_tiles;
    // dynamic LDS: kernel-B units stage act as fp16 chunks (f16_chunk_bytes),
    // kernel-A units stage x raw (+16 bytes per chunk)
    const int ca = codes_of(w->gate.bits);
    const size_t x_elem = raw_enum(w->w_router_dtype) == MOE_F32 ? 4 : 2;     // x has the router's dtype
    const size_t lds_b = (size_t)(dmax / cb) * (cb == 32 ? f16_chunk_bytes<4>() : f16_chunk_bytes<8>());
    const size_t lds_a = (size_t)(d_in / ca) * ((size_t)ca * x_elem + 16);
    p.lds = lds_b > lds_a ? lds_b : lds_a;
    if (p.lds > 64 * 1024) return MOE_EUNSUPPORTED;

    size_t off = align_up((size_t)kCtrCount * kCtrStride * sizeof(uint32_t), 256);
    p.off_logits = off;
    a.logit_stride = (int)(align_up((size_t)(E + 1) * sizeof(uint64_t), 4096) / sizeof(uint64_t));
    off += (size_t)kLogitCopies * a.logit_stride * sizeof(uint64_t);
    p.off_act = off;
    off = align_up(off + (size_t)slots * dmax * sizeof(uint64_t), 256);
    p.off_act_sent = off;
    off = align_up(off + (size_t)slots * kActCopies * kSentStride * sizeof(uint64_t), 256);
    p.off_partial = off;
    off = align_up(off + (size_t)slots * d_in * sizeof(uint64_t), 256);
    p.off_norm = off;                       // one tagged word per tail tile (a tile has >= 16 rows)
    off = align_up(off + (size_t)(d_in / 16) * sizeof(uint64_t), 256);
    p.ws_bytes = off;
    return MOE_OK;
}

// Workgroups of `k` that can be resident at once on the current device (0 if
// the runtime cannot tell).
// Workgroups of kernel k with lds bytes of dynamic LDS that fit on the
// current device at once, asked of the runtime once per (kernel, LDS size,
// device) and remembered; 0 if the runtime cannot tell.
static int resident_capacity(LayerFn k, size_t lds) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    static std::mutex mu;
    static std::map<std::tuple<const void *, size_t, int>, int> known;
    const auto key = std::make_tuple(reinterpret_cast<const void *>(k), lds, dev);
    {
        std::lock_guard<std::mutex> lock(mu);
        const auto it = known.find(key);
        if (it != known.end()) return it->second;
    }
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void *>(k), kLayerThreads, lds) !=
        hipSuccess)
        return 0;
    std::lock_guard<std::mutex> lock(mu);
    known[key] = cus * per_cu;
    return cus * per_cu;
}

// Size the kernel-A and kernel-B units.  A kernel-A unit is either one stage
// (kLayerNRA rows per lane group at one chunk position; only when the rows'
// inputs fit the lane group) or several, pipelined two deep (kLayerNRA2 rows
// per lane group and stage, `passes` row passes of every chunk position).  A
// kernel-B unit covers `bp` row passes of kLayerNRB rows per lane group at
// every chunk position; only its first stage is loaded before act arrives.
// Among the layouts whose grid fits the resident capacity (every unit
// issues its loads from the start of the launch, and no unit waits for a
// slot to free up; the router workgroups' slots count, as they free up
// early), take the one with the fewest serial stages: a kernel-A unit's
// stages plus a kernel-B unit's stages after act (measured: the
// dots.llm1-shaped layer 50.7 us with single-pass B units that do not all
// fit, 37.8 us with 4-pass B units and 2-pass A units; the Qwen1.5-shaped
// layer is best with single-pass B units).  Ties go to single-stage A
// units, then to fewer B passes; if nothing fits, or the capacity is
// unknown, the smallest grid.  cap1, cap2: resident capacity with
// single-stage and with pipelined units (0 if unknown).
static void fit_a_passes(LayerPlan &p, int cap1, int cap2) {
    LayerArgs &a = p.a;
    const int slots = a.K + a.S;
    const int dff_s = a.S > 0 ? a.d_ffs : 0;
    const int rpw = 64 >> a.a_lr_shift;
    auto n_a_for = [&](int t) { return a.K * ((a.d_ff + t - 1) / t) + a.S * ((dff_s + t - 1) / t); };
    const int cpr = a.d_in / (a.gate.bits_ == 4 ? 32 : 16);
    const int n_chunk_a = (cpr + (1 << a.a_lr_shift) - 1) >> a.a_lr_shift;
    const int single = 4 * rpw * kLayerNRA, piped = 4 * rpw * kLayerNRA2;
    const int cb = a.down.bits_ == 4 ? 32 : 16;
    auto chunks_b = [&](int dff, int lrs) { return (dff / cb + (1 << lrs) - 1) >> lrs; };
    int n_chunk_b = chunks_b(a.d_ff, a.b_lr_shift_r);
    if (a.S > 0) n_chunk_b = std::max(n_chunk_b, chunks_b(a.d_ffs, a.b_lr_shift_s));
    const int b_pass = a.b_tile;                     // one pass of a kernel-B unit
    struct Layout { int a_nr, a_tile, bp, grid, cost; };
    Layout best{0, 0, 0, 0, 0}, smallest{0, 0, 0, 0, 0};
    bool have = false, have_small = false;
    auto consider = [&](int a_nr, int a_tile, int bp, int stages_a, int cap) {
        const int n_b = slots * ((a.d_in + b_pass * bp - 1) / (b_pass * bp));
        const int grid = a.n_route + n_a_for(a_tile) + n_b;
        const Layout l{a_nr, a_tile, bp, grid, stages_a + bp * n_chunk_b - 1};
        if (!have_small || grid < smallest.grid) { smallest = l; have_small = true; }
        // the router workgroups exit within ~2 us, long before routing is
        // done, so up to n_route units past the capacity start in their place
        if (cap <= 0 || grid > cap + a.n_route) return false;
        if (!have || l.cost < best.cost) { best = l; have = true; }
        return true;
    };
    for (int bp = 1; bp <= 16 && b_pass * bp <= 4 * kWave * kLayerNRB; bp *= 2) {
        if (bp > 1 && b_pass * (bp / 2) >= a.d_in) break;     // one tile already covers d_in
        if (cpr <= (1 << a.a_lr_shift)) consider(kLayerNRA, single, bp, 1, cap1);
        for (int passes = 1; passes <= 8; ++passes)
            if (consider(kLayerNRA2, piped * passes, bp, passes * n_chunk_a, cap2)) break;
    }
    const Layout &l = have ? best : smallest;
    p.a_nr = l.a_nr;
    a.a_tile = l.a_tile;
    a.a_tiles_r = (a.d_ff + a.a_tile - 1) / a.a_tile;
    a.a_tiles_s = a.S > 0 ? (dff_s + a.a_tile - 1) / a.a_tile : 0;
    a.b_tile = b_pass * l.bp;
    a.b_tiles = (a.d_in + a.b_tile - 1) / a.b_tile;
    p.grid = a.n_route + a.K * a.a_tiles_r + a.S * a.a_tiles_s + slots * a.b_tiles;
    a.by_xcd = slots == 8 && a.n_route % 8 == 0 && (a.S == 0 || a.a_tiles_s == a.a_tiles_r) ? 1 : 0;
}

static LayerFn pick_layer(int ba, int bb, int sb, int xt, int anr) {
    const bool single = anr == kLayerNRA;
    switch (ba) {
    case 4: return single ? layer_kernel_a4(bb, sb, xt) : layer_kernel_a4p(bb, sb, xt);
    case 6: return single ? layer_kernel_a6(bb, sb, xt) : layer_kernel_a6p(bb, sb, xt);
    case 8: return single ? layer_kernel_a8(bb, sb, xt) : layer_kernel_a8p(bb, sb, xt);
    }
    return nullptr;
}

}  // namespace moe

using namespace moe;

extern "C" size_t moe_decode_layer_workspace_bytes(const moe_layer_weights *weights) {
    LayerPlan p;
    return plan_layer(weights, -1, p) == MOE_OK ? p.ws_bytes : 0;
}

namespace moe {

static moe_status layer_impl(const moe_layer_weights *weights, const void *x, int x_dtype, const void *residual,
                             int residual_dtype, void *out, int out_dtype, int32_t *expert_ids, float *scores,
                             float *shared_gate, const moe_rmsnorm *norm, void *workspace, size_t workspace_bytes,
                             void *stream) {
    if (!x || !residual || !out || !workspace) return MOE_EINVAL;
    if (!valid_dtype(x_dtype) || !valid_dtype(residual_dtype) || !valid_dtype(out_dtype)) return MOE_EUNSUPPORTED;
    if (!aligned16(x) || !aligned16(workspace) || !aligned_elem(out, out_dtype)) return MOE_EINVAL;
    moe_status st = norm ? check_rmsnorm(norm) : MOE_OK;
    if (st != MOE_OK) return st;
    LayerPlan p;
    st = plan_layer(weights, -1, p);
    if (st != MOE_OK) return st;
    if (raw_enum(weights->w_router_dtype) != x_dtype) return MOE_EUNSUPPORTED;
    if (workspace_bytes < p.ws_bytes) return MOE_EINVAL;
    const int sb = raw_enum(weights->gate.sb_dtype);
    LayerFn k1 = pick_layer(weights->gate.bits, weights->down.bits, sb, x_dtype, kLayerNRA);
    LayerFn k2 = pick_layer(weights->gate.bits, weights->down.bits, sb, x_dtype, kLayerNRA2);
    if (!k1 || !k2) return MOE_EUNSUPPORTED;
    fit_a_passes(p, resident_capacity(k1, p.lds), resident_capacity(k2, p.lds));
    LayerFn k = p.a_nr == kLayerNRA ? k1 : k2;
    LayerArgs &a = p.a;
    a.x = x; a.resid = residual; a.resid_dt = residual_dtype; a.out = out; a.out_dt = out_dtype;
    a.ids_out = expert_ids; a.scores_out = scores; a.gate_out = shared_gate;
    char *ws = reinterpret_cast<char *>(workspace);
    a.ctr = reinterpret_cast<uint32_t *>(ws);
    a.logits = reinterpret_cast<uint64_t *>(ws + p.off_logits);
    a.act = reinterpret_cast<uint64_t *>(ws + p.off_act);
    a.act_sent = reinterpret_cast<uint64_t *>(ws + p.off_act_sent);
    a.partial = reinterpret_cast<uint64_t *>(ws + p.off_partial);
    a.norm_part = reinterpret_cast<uint64_t *>(ws + p.off_norm);
    if (norm) {
        a.norm_w = norm->weight;
        a.norm_dt = raw_enum(norm->dtype);
        a.norm_eps = norm->eps;
        a.norm_out = norm->normed;
        a.norm_out_dt = raw_enum(norm->normed_dtype);
    }
    hipLaunchKernelGGL(k, dim3(p.grid), dim3(kLayerThreads), p.lds, reinterpret_cast<hipStream_t>(stream), a);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

}  // namespace moe

extern "C" moe_status moe_decode_layer(const moe_layer_weights *weights, const void *x, moe_dtype x_dtype_arg,
                                       const void *residual, moe_dtype residual_dtype_arg, void *out,
                                       moe_dtype out_dtype_arg, int32_t *expert_ids, float *scores,
                                       float *shared_gate, void *workspace, size_t workspace_bytes, void *stream) {
    return layer_impl(weights, x, raw_enum(x_dtype_arg), residual, raw_enum(residual_dtype_arg), out,
                      raw_enum(out_dtype_arg), expert_ids, scores, shared_gate, nullptr, workspace, workspace_bytes,
                      stream);
}

extern "C" moe_status moe_decode_layer_rmsnorm(const moe_layer_weights *weights, const void *x,
                                               moe_dtype x_dtype_arg, const void *residual,
                                               moe_dtype residual_dtype_arg, void *out, moe_dtype out_dtype_arg,
                                               const moe_rmsnorm *norm, int32_t *expert_ids, float *scores,
                                               float *shared_gate, void *workspace, size_t workspace_bytes,
                                               void *stream) {
    if (!norm) return MOE_EINVAL;
    return layer_impl(weights, x, raw_enum(x_dtype_arg), residual, raw_enum(residual_dtype_arg), out,
                      raw_enum(out_dtype_arg), expert_ids, scores, shared_gate, norm, workspace, workspace_bytes,
                      stream);
}
