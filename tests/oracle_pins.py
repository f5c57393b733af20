"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
a closed form, a library routine (numpy, scipy, torch), brute force on tiny
inputs, or an exact invariant of the layer.  ``test_oracle_pins.py`` runs
them against the oracle; ``test_oracle_mutations.py`` runs them against
deliberately broken copies of the oracle and requires that each copy fails at
least one pin.

The layer being pinned (mlxcel PR #276, "What changed", step 2; Red Lite
dev39, "Change"): router logits, softmax over all experts, top-k with
optional renormalisation; per selected expert act = SwiGLU(W_g x, W_u x) and
partial = score * W_d act over affine-quantized weights
w = scale * q + bias (groups of 64 along the contraction index); then
out = resid + (sum_k partial_k + shared * gate).
"""
from __future__ import annotations

import itertools

import numpy as np
import scipy.special
import torch

import moe_inputs as mi
import oracle
from helpers import (bigint_pack, dense, make_stack, np_decode, np_unpack,
                     stack_from_arrays)


def _rng(k):
    return np.random.default_rng([7707, k])


def _small_cfg(**kw):
    base = dict(name="pin", cfg_id=90, weight_cfg_id=90, d_in=128, d_ff=64, n_experts=6,
                top_k=2, renormalize=True, bits_gate_up=4, bits_down=4, sb_dtype=mi.BF16,
                x_dtype=mi.BF16, router_dtype=mi.BF16, resid_dtype=mi.BF16)
    base.update(kw)
    return mi.LayerConfig(**base)


def _torch_mlp(x64, Wg, Wu, Wd):
    """Dense SwiGLU MLP with torch's library routines in float64."""
    x = torch.from_numpy(x64)
    g = torch.from_numpy(Wg) @ x
    u = torch.from_numpy(Wu) @ x
    h = torch.nn.functional.silu(g) * u
    return (torch.from_numpy(Wd) @ h).numpy(), h.numpy()


# --------------------------------------------------------------- unpacking
def pin_unpack_matches_bigint():
    """Oracle unpacking == an independent big-integer packer, random rows, bits 4/6/8."""
    r = _rng(1)
    for bits in (4, 6, 8):
        for cols in (64, 192, 1408 // 64 * 64):
            codes = r.integers(0, 1 << bits, size=(3, cols))
            words = bigint_pack(codes, bits)
            for i in range(3):
                got = oracle.unpack_row(words[i], bits, cols)
                assert np.array_equal(got, codes[i]), (bits, cols, i)


def pin_unpack_exhaustive():
    """Every code value at every position class of a group (incl. 6-bit straddles)."""
    for bits in (4, 6, 8):
        n = 1 << bits
        codes = (np.arange(n)[:, None] + 7 * np.arange(64)[None, :]) % n
        words = bigint_pack(codes, bits)
        for v in range(n):
            assert np.array_equal(oracle.unpack_row(words[v], bits, 64), codes[v]), (bits, v)


# ---------------------------------------------------------------- decoding
def pin_decode_all_half_and_bf16_patterns():
    """Exact decoding of every finite fp16 and bf16 bit pattern vs numpy's conversions."""
    pats = np.arange(1 << 16, dtype=np.uint16)
    h = pats.view(np.float16)
    fin = np.isfinite(h)
    got = oracle.decode(pats[fin], mi.F16)
    assert np.array_equal(got, h[fin].astype(np.float64))
    bf = (pats.astype(np.uint32) << 16).view(np.float32)
    finb = np.isfinite(bf)
    sel = pats[finb][::7]  # every 7th pattern keeps the ctypes loop short
    got = oracle.decode(sel, mi.BF16)
    assert np.array_equal(got, np_decode(sel, mi.BF16))
    f = _rng(2).standard_normal(50).astype(np.float32)
    assert np.array_equal(oracle.decode(f, mi.F32), f.astype(np.float64))


# ----------------------------------------------------------------- dequant
def pin_dequant_closed_form():
    """w = scale*q + bias with known codes and dyadic scale/bias, every bit width and dtype."""
    for bits in (4, 6, 8):
        for sbd in (mi.F16, mi.BF16):
            E, rows, cols = 2, 5, 192
            e_, r_, j_ = np.meshgrid(np.arange(E), np.arange(rows), np.arange(cols), indexing="ij")
            codes = (3 * r_ + 5 * j_ + e_) % (1 << bits)
            G = cols // 64
            eg, rg, gg = np.meshgrid(np.arange(E), np.arange(rows), np.arange(G), indexing="ij")
            scales = 2.0 ** -(5 + (rg + gg + eg) % 4)
            biases = -(gg + 1) * 2.0 ** -6 + eg * 2.0 ** -3
            st = make_stack(codes, scales, biases, bits, sbd)
            for e in range(E):
                for r in range(rows):
                    want = (np.repeat(scales[e, r], 64) * codes[e, r]
                            + np.repeat(biases[e, r], 64))
                    got = oracle.dequant_row(st, e, r)
                    assert np.array_equal(got, want), (bits, sbd, e, r)
            # zero codes or zero scales leave the bias
            z = make_stack(np.zeros_like(codes), scales, biases, bits, sbd)
            z2 = make_stack(codes, np.zeros_like(scales), biases, bits, sbd)
            for st2 in (z, z2):
                got = oracle.dequant_row(st2, 1, 3)
                assert np.array_equal(got, np.repeat(biases[1, 3], 64))


def _onehot_stacks(bits_gu, bits_d, d_in, d_ff, j0, r0, g0_code, sbd=mi.BF16):
    """Gate with known codes, up = e_{r0} e_{j0}^T, down with known codes."""
    Gi, Gf = d_in // 64, d_ff // 64
    cg = (np.arange(d_ff)[:, None] * 3 + np.arange(d_in)[None, :]) % (1 << bits_gu)
    cg[r0, j0] = g0_code
    sg = np.full((d_ff, Gi), 2.0 ** -4)
    bg = np.full((d_ff, Gi), -(2.0 ** (bits_gu - 1)) * 2.0 ** -4)
    gate = make_stack(cg[None], sg[None], bg[None], bits_gu, sbd)
    cu = np.zeros((d_ff, d_in), np.int64)
    cu[r0, j0] = 1
    up = make_stack(cu[None], np.ones((1, d_ff, Gi)), np.zeros((1, d_ff, Gi)), bits_gu, sbd)
    cd = (np.arange(d_in)[:, None] * 5 + 2 * np.arange(d_ff)[None, :] + 1) % (1 << bits_d)
    sd = np.full((d_in, Gf), 2.0 ** -5) * (1 + (np.arange(d_in)[:, None] % 3))
    bd = np.full((d_in, Gf), -(2.0 ** (bits_d - 1)) * 2.0 ** -5)
    down = make_stack(cd[None], sd[None], bd[None], bits_d, sbd)
    g0 = 2.0 ** -4 * g0_code - (2.0 ** (bits_gu - 1)) * 2.0 ** -4
    wd_col = np.repeat(sd, 64, axis=1)[:, r0] * cd[:, r0] + np.repeat(bd, 64, axis=1)[:, r0]
    return gate, up, down, g0, wd_col


def pin_onehot_x_probes_every_index():
    """x = e_j, up = e_r0 e_j^T: act = silu(W_g[r0, j]) e_r0 and partial = W_d[:, r0] * act[r0]."""
    for bits_gu, bits_d in ((4, 4), (8, 8), (4, 6)):
        d_in, d_ff = 256, 128
        for j0, r0 in ((0, 0), (63, 5), (64, 127), (101, 64), (255, 33)):
            code = (j0 * 7 + r0) % (1 << bits_gu)
            gate, up, down, g0, wd_col = _onehot_stacks(bits_gu, bits_d, d_in, d_ff, j0, r0, code)
            x = np.zeros(d_in, np.float32)
            x[j0] = 1.0
            res = oracle.expert_ffn(x, mi.F32, gate, up, down, np.array([[0]]), None)
            act = res["act"][0, 0]
            want_act = np.zeros(d_ff)
            want_act[r0] = torch.nn.functional.silu(torch.tensor(g0, dtype=torch.float64)).item()
            assert np.allclose(act, want_act, rtol=1e-15, atol=0), (bits_gu, j0, r0)
            want_p = wd_col * want_act[r0]
            assert np.allclose(res["partial"][0, 0], want_p, rtol=1e-14, atol=1e-300), (bits_d, j0, r0)


# ---------------------------------------------------- library special cases
def pin_k1_equals_dense_swiglu_mlp():
    """top-1 with renormalisation gives score exactly 1, and out - resid is the chosen
    expert's dense dequantised SwiGLU MLP (torch matmul + silu, float64)."""
    for jitter in (False, True):
        for cfgkw in (dict(), dict(bits_gate_up=8, bits_down=8, d_ff=128),
                      dict(bits_gate_up=4, bits_down=6, d_in=192, sb_dtype=mi.F16)):
            cfg = _small_cfg(top_k=1, **cfgkw)
            w = mi.gen_layer_weights(cfg, 0, jitter_bias=jitter, threads=1)
            x, resid = mi.gen_token(cfg, 0, 0)
            r = oracle.route(x, cfg.x_dtype, w["router"], cfg.router_dtype, 1, True)
            assert r["scores"][0, 0] == 1.0
            e = int(r["ids"][0, 0])
            f = oracle.expert_ffn(x, cfg.x_dtype, w["gate"], w["up"], w["down"], r["ids"], r["scores"])
            out = oracle.tail(f["partial"], resid, cfg.resid_dtype)
            x64 = np_decode(x, cfg.x_dtype)
            y, h = _torch_mlp(x64, dense(w["gate"], [e])[0], dense(w["up"], [e])[0],
                              dense(w["down"], [e])[0])
            y_or = out[0] - np_decode(resid, cfg.resid_dtype)
            scale = np.max(np.abs(y))
            assert np.max(np.abs(y_or - y)) <= 1e-12 * scale, cfgkw
            assert np.max(np.abs(f["act"][0, 0] - h)) <= 1e-12 * np.max(np.abs(h))


def pin_slots_equal_scaled_dense_mlps():
    """Each slot's partial is score_k times the dense MLP of its expert (K = 3, real scores)."""
    cfg = _small_cfg(top_k=3, n_experts=7)
    w = mi.gen_layer_weights(cfg, 1, threads=1)
    x, _ = mi.gen_token(cfg, 1, 0)
    r = oracle.route(x, cfg.x_dtype, w["router"], cfg.router_dtype, 3, True)
    f = oracle.expert_ffn(x, cfg.x_dtype, w["gate"], w["up"], w["down"], r["ids"], r["scores"])
    x64 = np_decode(x, cfg.x_dtype)
    for k in range(3):
        e = int(r["ids"][0, k])
        y, _ = _torch_mlp(x64, dense(w["gate"], [e])[0], dense(w["up"], [e])[0],
                          dense(w["down"], [e])[0])
        got = f["partial"][0, k]
        assert np.max(np.abs(got - r["scores"][0, k] * y)) <= 1e-12 * np.max(np.abs(y)), k


def pin_router_logits_softmax_library():
    """Logits == numpy matmul; probabilities == scipy softmax; E=2 gives sigmoid(l0 - l1)."""
    for E, xdt, wdt in ((60, mi.BF16, mi.BF16), (8, mi.F32, mi.F32), (2, mi.BF16, mi.BF16)):
        cfg = _small_cfg(n_experts=E, x_dtype=xdt, router_dtype=wdt, top_k=1)
        wr = mi.gen_router(cfg, 3)
        x, _ = mi.gen_token(cfg, 3, 0)
        r = oracle.route(x, xdt, wr, wdt, 1, False)
        l_np = np_decode(wr, wdt) @ np_decode(x, xdt)
        assert np.allclose(r["logits"][0], l_np, rtol=1e-13, atol=1e-13)
        p_sp = scipy.special.softmax(l_np)
        assert np.allclose(r["probs"][0], p_sp, rtol=1e-12, atol=1e-15)
        assert abs(r["probs"][0].sum() - 1.0) < 1e-12
        if E == 2:
            p0 = scipy.special.expit(l_np[0] - l_np[1])
            assert abs(r["probs"][0, 0] - p0) < 1e-15
            assert r["scores"][0, 0] == r["probs"][0, int(r["ids"][0, 0])]


def pin_topk_bruteforce():
    """The selected ids are the unique subset beating every other expert, in descending order."""
    for K in (1, 2, 3, 5):
        for seed in range(4):
            cfg = _small_cfg(n_experts=8, top_k=K, cfg_id=91 + seed)
            wr = mi.gen_router(cfg, seed)
            x, _ = mi.gen_token(cfg, seed, 0)
            r = oracle.route(x, cfg.x_dtype, wr, cfg.router_dtype, K, True)
            l = r["logits"][0]
            winners = [S for S in itertools.combinations(range(8), K)
                       if min(l[list(S)]) > max(np.delete(l, list(S)), default=-np.inf)]
            assert len(winners) == 1
            best = sorted(winners[0], key=lambda e: -l[e])
            assert list(r["ids"][0]) == best, (K, seed)
            assert abs(r["scores"][0].sum() - 1.0) < 1e-12
            sc = r["probs"][0, best] / r["probs"][0, best].sum()
            assert np.allclose(r["scores"][0], sc, rtol=1e-14)


def pin_exact_tie_prefers_lower_index():
    """Duplicate router rows give equal logits; the lower expert index is taken first."""
    cfg = _small_cfg(n_experts=8, x_dtype=mi.F32, router_dtype=mi.F32)
    x = np.ones(cfg.d_in, np.float32)
    wr = np.zeros((8, cfg.d_in), np.float32)
    wr[5] = wr[3] = 0.01        # tie for first place
    wr[6] = 0.005               # third
    wr[1] = wr[2] = 0.002       # tie for the last place of top-4
    r = oracle.route(x, mi.F32, wr, mi.F32, 4, True)
    assert list(r["ids"][0]) == [3, 5, 6, 1]
    r3 = oracle.route(x, mi.F32, wr, mi.F32, 2, True)
    assert list(r3["ids"][0]) == [3, 5]
    assert abs(r3["scores"][0, 0] - 0.5) < 1e-15


def pin_shared_gate():
    """w_g = 0 gives gate = 1/2 exactly; otherwise gate = expit(w_g . x)."""
    cfg = _small_cfg()
    wr = mi.gen_router(cfg, 0)
    x, _ = mi.gen_token(cfg, 0, 0)
    r = oracle.route(x, cfg.x_dtype, wr, cfg.router_dtype, 2, True,
                     w_shared_gate=mi.encode(np.zeros(cfg.d_in), mi.BF16))
    assert r["gate"][0] == 0.5
    wg = mi.encode(_rng(5).normal(0, 0.1, cfg.d_in), mi.BF16)
    r = oracle.route(x, cfg.x_dtype, wr, cfg.router_dtype, 2, True, w_shared_gate=wg)
    want = scipy.special.expit(np_decode(wg, mi.BF16) @ np_decode(x, cfg.x_dtype))
    assert abs(r["gate"][0] - want) < 1e-15


# -------------------------------------------------------------- invariants
def _layer_out(cfg, w, x, resid):
    return oracle.layer(cfg, w, x, resid)


def pin_expert_relabeling_invariance():
    """Relabelling experts by a permutation maps ids through it and leaves out unchanged."""
    cfg = _small_cfg(n_experts=6, top_k=3)
    w = mi.gen_layer_weights(cfg, 2, threads=1)
    x, resid = mi.gen_token(cfg, 2, 0)
    base = _layer_out(cfg, w, x, resid)
    perm = _rng(6).permutation(cfg.n_experts)      # new index of old expert e is perm[e]
    inv = np.argsort(perm)
    w2 = dict(w)
    w2["router"] = w["router"][inv]
    for p in ("gate", "up", "down"):
        s = w[p]
        w2[p] = stack_from_arrays(s.q[inv], s.scales[inv], s.biases[inv], s)
    moved = _layer_out(cfg, w2, x, resid)
    assert np.array_equal(moved["route"]["ids"], perm[base["route"]["ids"]])
    scale = np.max(np.abs(base["out"]))
    assert np.max(np.abs(moved["out"] - base["out"])) <= 1e-12 * scale


def pin_slot_order_only_changes_rounding():
    """Shuffling the K slots (ids with their scores) changes out only by rounding."""
    cfg = _small_cfg(n_experts=6, top_k=4)
    w = mi.gen_layer_weights(cfg, 4, threads=1)
    x, resid = mi.gen_token(cfg, 4, 0)
    base = _layer_out(cfg, w, x, resid)
    order = np.array([2, 0, 3, 1])
    ids = base["route"]["ids"][:, order]
    sc = base["route"]["scores"][:, order]
    sh = oracle.layer(cfg, w, x, resid, ids=ids, scores=sc)
    assert np.max(np.abs(sh["out"] - base["out"])) <= 1e-13 * np.max(np.abs(base["out"]))
    assert not np.array_equal(ids, base["route"]["ids"])


def pin_down_linearity_exact():
    """Doubling the down projection's scales and biases doubles every partial exactly."""
    cfg = _small_cfg(top_k=2)
    w = mi.gen_layer_weights(cfg, 5, threads=1)
    x, _ = mi.gen_token(cfg, 5, 0)
    r = oracle.route(x, cfg.x_dtype, w["router"], cfg.router_dtype, 2, True)
    d = w["down"]
    d2 = stack_from_arrays(d.q, mi.encode(2 * np_decode(d.scales, d.sb_dtype), d.sb_dtype),
                           mi.encode(2 * np_decode(d.biases, d.sb_dtype), d.sb_dtype), d)
    a = oracle.expert_ffn(x, cfg.x_dtype, w["gate"], w["up"], d, r["ids"], r["scores"])
    b = oracle.expert_ffn(x, cfg.x_dtype, w["gate"], w["up"], d2, r["ids"], r["scores"])
    assert np.array_equal(b["partial"], 2 * a["partial"])
    assert np.array_equal(b["act"], a["act"])


def pin_zero_gate_projection_gives_residual():
    """Gate scales and biases zero: g = 0, act = 0, partial = 0, out == resid exactly."""
    cfg = _small_cfg(top_k=2)
    w = mi.gen_layer_weights(cfg, 6, threads=1)
    g = w["gate"]
    zero = mi.encode(np.zeros(g.scales.shape), g.sb_dtype)
    w["gate"] = stack_from_arrays(g.q, zero, zero, g)
    x, resid = mi.gen_token(cfg, 6, 0)
    res = _layer_out(cfg, w, x, resid)
    assert np.all(res["ffn"]["act"] == 0) and np.all(res["ffn"]["partial"] == 0)
    assert np.array_equal(res["out"][0], np_decode(resid, cfg.resid_dtype))


def pin_out_of_range_ids_contribute_zero():
    cfg = _small_cfg(top_k=3, n_experts=6)
    w = mi.gen_layer_weights(cfg, 7, threads=1)
    x, _ = mi.gen_token(cfg, 7, 0)
    ids = np.array([[2, -1, 6]], np.int32)
    f = oracle.expert_ffn(x, cfg.x_dtype, w["gate"], w["up"], w["down"], ids, np.ones((1, 3)))
    assert np.all(f["act"][0, 1:] == 0) and np.all(f["partial"][0, 1:] == 0)
    assert np.any(f["partial"][0, 0] != 0)


def pin_tail_exact_small_integers():
    """Integer-valued partials/shared and dyadic gates: the tail is exact arithmetic."""
    r = _rng(8)
    T, K, S, D = 2, 3, 2, 64
    partial = r.integers(-50, 50, size=(T, K, D)).astype(np.float64)
    shared = r.integers(-50, 50, size=(T, S, D)).astype(np.float64)
    resid = r.integers(-50, 50, size=(T, D)).astype(np.float32)
    gate = np.array([0.5, 0.25])
    out = oracle.tail(partial, resid, mi.F32, shared, gate)
    want = resid + (partial.sum(1) + shared.sum(1) * gate[:, None])
    assert np.array_equal(out, want)
    out1 = oracle.tail(partial, resid, mi.F32, shared, None)
    assert np.array_equal(out1, resid + (partial.sum(1) + shared.sum(1)))
    out0 = oracle.tail(partial, resid, mi.F32)
    assert np.array_equal(out0, resid + partial.sum(1))


def pin_two_shared_experts_equal_one_concatenated():
    """Two shared experts of width d sum to one shared expert of width 2d (rows/cols concatenated)."""
    cfg = _small_cfg(n_shared=2, d_ff_shared=64, bits_down=6)
    w = mi.gen_layer_weights(cfg, 8, threads=1)
    x, resid = mi.gen_token(cfg, 8, 0)
    two = oracle.expert_ffn(x, cfg.x_dtype, w["shared_gate_proj"], w["shared_up"],
                            w["shared_down"], np.array([[0, 1]]), None)
    g, u, d = w["shared_gate_proj"], w["shared_up"], w["shared_down"]

    def cat_rows(s):
        return mi.QStack(s.q.reshape(1, -1, s.q.shape[2]), s.scales.reshape(1, -1, s.scales.shape[2]),
                         s.biases.reshape(1, -1, s.biases.shape[2]), 2 * s.rows, s.cols, s.bits, s.sb_dtype)

    dq = np.concatenate([d.q[0], d.q[1]], axis=1)[None]
    ds = np.concatenate([d.scales[0], d.scales[1]], axis=1)[None]
    db = np.concatenate([d.biases[0], d.biases[1]], axis=1)[None]
    d1 = mi.QStack(dq, ds, db, d.rows, 2 * d.cols, d.bits, d.sb_dtype)
    one = oracle.expert_ffn(x, cfg.x_dtype, cat_rows(g), cat_rows(u), d1, np.array([[0]]), None)
    s2 = two["partial"][0].sum(0)
    assert np.max(np.abs(one["partial"][0, 0] - s2)) <= 1e-12 * np.max(np.abs(s2))
    # zero shared weights leave resid + routed
    zq = [stack_from_arrays(s.q, mi.encode(np.zeros(s.scales.shape), s.sb_dtype),
                            mi.encode(np.zeros(s.biases.shape), s.sb_dtype), s) for s in (g, u, d)]
    w0 = dict(w, shared_gate_proj=zq[0], shared_up=zq[1], shared_down=zq[2])
    full = oracle.layer(cfg, w0, x, resid)
    routed_only = oracle.tail(full["ffn"]["partial"], resid, cfg.resid_dtype)
    assert np.array_equal(full["out"], routed_only)


def pin_sampled_rows_real_shapes():
    """Sampled rows of the large workloads: oracle act/partial vs dense torch MLP."""
    for cfg, layer in ((mi.QWEN3, 0), (mi.QWEN15, 0), (mi.DOTS, 0)):
        e = 5
        gate = mi.gen_proj_stack(cfg, layer, "gate", [e], threads=1)
        up = mi.gen_proj_stack(cfg, layer, "up", [e], threads=1)
        down = mi.gen_proj_stack(cfg, layer, "down", [e], threads=1)
        x, _ = mi.gen_token(cfg, layer, 0)
        f = oracle.expert_ffn(x, cfg.x_dtype, gate, up, down, np.array([[0]]), np.array([[0.25]]))
        y, h = _torch_mlp(np_decode(x, cfg.x_dtype), dense(gate)[0], dense(up)[0], dense(down)[0])
        assert np.max(np.abs(f["act"][0, 0] - h)) <= 1e-12 * np.max(np.abs(h)), cfg.name
        assert np.max(np.abs(f["partial"][0, 0] - 0.25 * y)) <= 1e-12 * np.max(np.abs(y)), cfg.name


def pin_tokens_are_independent():
    """With T = 3 tokens, each token's slots equal its own dense MLPs (no cross-token mixing)."""
    cfg = _small_cfg(top_k=2, n_experts=5)
    w = mi.gen_layer_weights(cfg, 9, threads=1)
    x, resid = mi.gen_tokens(cfg, 9, 3)
    r = oracle.route(x, cfg.x_dtype, w["router"], cfg.router_dtype, 2, True)
    f = oracle.expert_ffn(x, cfg.x_dtype, w["gate"], w["up"], w["down"], r["ids"], r["scores"])
    for t in range(3):
        rt = oracle.route(x[t], cfg.x_dtype, w["router"], cfg.router_dtype, 2, True)
        assert np.array_equal(rt["ids"][0], r["ids"][t])
        for k in range(2):
            e = int(r["ids"][t, k])
            y, _ = _torch_mlp(np_decode(x[t], cfg.x_dtype), dense(w["gate"], [e])[0],
                              dense(w["up"], [e])[0], dense(w["down"], [e])[0])
            got = f["partial"][t, k]
            assert np.max(np.abs(got - r["scores"][t, k] * y)) <= 1e-12 * np.max(np.abs(y))
    out = oracle.tail(f["partial"], resid, cfg.resid_dtype)
    for t in range(3):
        o1 = oracle.tail(f["partial"][t:t + 1], resid[t], cfg.resid_dtype)
        assert np.array_equal(o1[0], out[t])


def _gamma(d, seed):
    """A non-symmetric RMSNorm weight in bf16 (exactly decodable)."""
    g = np.random.default_rng([seed, d]).uniform(0.5, 1.5, d)
    return mi.encode(g, mi.BF16), np_decode(mi.encode(g, mi.BF16), mi.BF16)


def pin_rmsnorm_closed_forms():
    """Constant vectors: y = c 1 gives ms = c^2, so normed = c / sqrt(c^2 + eps) * w
    (sign(c) * w at eps = 0); a +-1 vector with eps = 0 gives y * w exactly."""
    d = 96
    wb, w = _gamma(d, 1)
    for c, eps in ((3.0, 0.0), (-0.25, 0.0), (2.0, 1e-6), (1e-3, 1e-6), (0.5, 0.75)):
        got = oracle.rmsnorm(np.full((1, d), c), wb, mi.BF16, eps)[0]
        want = c / np.sqrt(c * c + eps) * w
        assert np.max(np.abs(got - want)) <= 1e-15 * np.max(np.abs(want)), (c, eps)
    y = np.where(np.random.default_rng(2).integers(0, 2, d) == 1, 1.0, -1.0)
    assert np.array_equal(oracle.rmsnorm(y[None], wb, mi.BF16, 0.0)[0], y * w)


def pin_rmsnorm_equals_l2_normalisation():
    """At eps = 0, y / sqrt(mean(y^2)) = sqrt(d) * y / ||y||_2 (numpy's L2 norm);
    with eps the scale is 1 / sqrt(||y||^2 / d + eps)."""
    rng = np.random.default_rng(3)
    for d in (64, 2048, 4096):
        wb, w = _gamma(d, 4)
        y = rng.standard_normal((3, d)) * rng.uniform(0.01, 10.0, (3, 1))
        got = oracle.rmsnorm(y, wb, mi.BF16, 0.0)
        want = np.sqrt(d) * y / np.linalg.norm(y, axis=1, keepdims=True) * w
        assert np.max(np.abs(got - want)) <= 1e-13 * np.max(np.abs(want))
        eps = 1e-2
        got = oracle.rmsnorm(y, wb, mi.BF16, eps)
        want = y / np.sqrt(np.linalg.norm(y, axis=1, keepdims=True) ** 2 / d + eps) * w
        assert np.max(np.abs(got - want)) <= 1e-13 * np.max(np.abs(want))


def pin_rmsnorm_scale_invariance_and_sum_of_squares():
    """rmsnorm(a y, a^2 eps) = rmsnorm(y, eps) for a > 0, and with unit weight the
    normed vector's sum of squares is d * ms / (ms + eps)."""
    rng = np.random.default_rng(5)
    d = 768
    wb, _ = _gamma(d, 6)
    one = mi.encode(np.ones(d), mi.F32)
    y = rng.standard_normal((2, d))
    for a, eps in ((7.0, 1e-6), (1e-3, 0.25), (1e4, 3.0)):
        ref = oracle.rmsnorm(y, wb, mi.BF16, eps)
        got = oracle.rmsnorm(a * y, wb, mi.BF16, eps * a * a)
        assert np.max(np.abs(got - ref)) <= 1e-13 * np.max(np.abs(ref)), (a, eps)
        n = oracle.rmsnorm(y, one, mi.F32, eps)
        ms = np.mean(y * y, axis=1)
        assert np.allclose(np.sum(n * n, axis=1), d * ms / (ms + eps), rtol=1e-13, atol=0)


def pin_rmsnorm_tokens_independent():
    """Each token is normalised by its own mean square."""
    rng = np.random.default_rng(7)
    d = 128
    wb, _ = _gamma(d, 8)
    y = rng.standard_normal((4, d)) * np.array([[1.0], [100.0], [1e-3], [5.0]])
    both = oracle.rmsnorm(y, wb, mi.BF16, 1e-6)
    for t in range(4):
        assert np.array_equal(oracle.rmsnorm(y[t], wb, mi.BF16, 1e-6)[0], both[t])


def _bf16_table():
    """Every finite bf16 value in increasing order, with its bit pattern."""
    bits = np.arange(1 << 16, dtype=np.uint32)
    vals = (bits << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    ok = np.isfinite(vals) & ~((bits == 0x8000))           # one zero
    order = np.argsort(vals[ok], kind="stable")
    return vals[ok][order], bits[ok][order]


def _round_bf16_bruteforce(x):
    """Nearest finite bf16 value by search over the sorted table; on a tie the
    one with an even pattern; beyond the largest finite value by at least half
    its spacing, infinity."""
    vals, bits = _bf16_table()
    vmax, half = vals[-1], (vals[-1] - vals[-2]) / 2
    out = np.empty_like(x)
    for n, v in enumerate(x):
        if abs(v) >= vmax + half:
            out[n] = np.copysign(np.inf, v)
            continue
        i = int(np.searchsorted(vals, v))
        cand = [j for j in (i - 1, i) if 0 <= j < len(vals)]
        dist = [abs(vals[j] - v) for j in cand]
        best = [cand[k] for k in range(len(cand)) if dist[k] == min(dist)]
        if len(best) > 1:
            best = [j for j in best if bits[j] % 2 == 0]
        out[n] = vals[best[0]] if vals[best[0]] != 0 else np.copysign(0.0, v)
    return out


def _round_samples(rng, table):
    """Values spread over the whole range (subnormals to overflow), exact ties
    (midpoints of neighbouring table values, exact in double) and values just
    beside them."""
    pos = table[table > 0]
    i = rng.integers(0, len(pos) - 1, 300)
    mids = (pos[i] + pos[i + 1]) / 2
    near = np.concatenate([np.nextafter(mids, np.inf), np.nextafter(mids, -np.inf)])
    mag = np.exp2(rng.uniform(-150, 140, 400)) * rng.uniform(1, 2, 400)
    x = np.concatenate([mids, near, mag, pos[i]])
    return x * np.where(rng.integers(0, 2, x.size) == 1, 1.0, -1.0)


def pin_round_bf16_bruteforce():
    """bf16 rounding equals the brute-force nearest value (ties to an even
    pattern), over ties, their neighbours, subnormals and overflow."""
    rng = np.random.default_rng(11)
    vals, _ = _bf16_table()
    x = _round_samples(rng, vals)
    x = x[np.abs(x) < 1e39]
    got = oracle.round_to(x, mi.BF16)
    want = _round_bf16_bruteforce(x)
    assert np.array_equal(got, want), np.flatnonzero(got != want)[:5]


def pin_round_f16_library():
    """binary16 rounding equals numpy's float64 -> float16 conversion (IEEE
    round to nearest even, done from the double directly)."""
    rng = np.random.default_rng(12)
    table = np.arange(1 << 16, dtype=np.uint16).view(np.float16).astype(np.float64)
    table = np.unique(table[np.isfinite(table)])
    x = _round_samples(rng, table)
    x = x[np.abs(x) < 1e6]
    got = oracle.round_to(x, mi.F16)
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).astype(np.float64)
    assert np.array_equal(got, want), np.flatnonzero(got != want)[:5]


def pin_round_closed_forms():
    """Hand-worked cases: ties to even at 1 (bf16 spacing 2^-7, binary16 2^-10),
    the largest finite values and the overflow tie, the smallest subnormals,
    and f32 leaving values alone."""
    e = np.exp2
    cases = [
        (mi.BF16, 1 + e(-8), 1.0), (mi.BF16, 1 + 3 * e(-8), 1 + e(-6)), (mi.BF16, -(1 + e(-8)), -1.0),
        (mi.BF16, 1 + e(-8) + e(-30), 1 + e(-7)), (mi.BF16, 3.0 + e(-7), 3.0),
        (mi.BF16, (2 - e(-7)) * e(127), (2 - e(-7)) * e(127)),
        (mi.BF16, (2 - e(-8)) * e(127), np.inf), (mi.BF16, (2 - e(-8)) * e(127) - e(100), (2 - e(-7)) * e(127)),
        (mi.BF16, e(-133), e(-133)), (mi.BF16, e(-134), 0.0), (mi.BF16, 3 * e(-134), e(-132)),
        (mi.F16, 1 + e(-11), 1.0), (mi.F16, 1 + 3 * e(-11), 1 + e(-9)), (mi.F16, 65504.0, 65504.0),
        (mi.F16, 65519.0, 65504.0), (mi.F16, 65520.0, np.inf), (mi.F16, -65520.0, -np.inf),
        (mi.F16, e(-24), e(-24)), (mi.F16, e(-25), 0.0), (mi.F16, 3 * e(-25), e(-23)),
        (mi.F16, 2049.0, 2048.0), (mi.F16, 2051.0, 2052.0),
        (mi.F32, 1 + e(-40), 1 + e(-40)),
    ]
    for dt, v, want in cases:
        got = float(oracle.round_to(np.array([v]), dt)[0])
        assert got == want, (dt, v, got, want)


def pin_round_idempotent_monotone():
    """Rounding a rounded value changes nothing, and rounding keeps order."""
    rng = np.random.default_rng(13)
    x = np.sort(rng.standard_normal(5000) * np.exp2(rng.uniform(-20, 20, 5000)))
    for dt in (mi.BF16, mi.F16):
        r = oracle.round_to(x, dt)
        assert np.array_equal(oracle.round_to(r, dt), r)
        assert np.all(r[1:] >= r[:-1])


# cheap pins first, so that a broken oracle is usually rejected within a second
_SLOW = ("pin_onehot_x_probes_every_index", "pin_decode_all_half_and_bf16_patterns",
         "pin_round_bf16_bruteforce", "pin_sampled_rows_real_shapes")
ALL_PINS = ([v for k, v in sorted(globals().items())
             if k.startswith("pin_") and callable(v) and k not in _SLOW]
            + [globals()[k] for k in _SLOW])
