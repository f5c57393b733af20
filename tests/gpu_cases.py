"""Shared helpers for the GPU parity tests: build a layer on the device from the
seeded generator, run it through the C ABI, and compare with the oracle.

Comparison rules (the layer's own bar): expert ids bit-exact; scores within
1e-5 absolute; act, partial and out within 2e-3 of their infinity norm, and
out - resid within 2e-3 of the MoE term's infinity norm, so that a large
residual cannot hide a wrong expert sum.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import moe_inputs as mi
import oracle
from helpers import np_decode, oracle_layer_selected, pick_tokens, rel_err  # noqa: F401
from quantized_moe_decode_amd.layer import layer_from_host, tensor_from_encoded

DEV = torch.device("cuda:0")
TOL = 2e-3
SCORE_TOL = 1e-5


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_gpu_layer(cfg, w, x, resid, graph: bool = False, layer=None, fused: bool = False):
    """The layer for the tokens in x on the GPU; returns host copies.

    fused=False: route + expert FFN + tail (three calls); fused=True: the
    single-launch moe_decode_layer (one token; act and partial are not exposed).
    """
    if layer is None:
        layer = layer_from_host(cfg, w, DEV, n_tokens=x.shape[0])
    xd = tensor_from_encoded(x, cfg.x_dtype, DEV)
    rd = tensor_from_encoded(resid, cfg.resid_dtype, DEV)
    out = torch.empty(x.shape[0], cfg.d_in, device=DEV, dtype=torch.float32)
    fwd = layer.forward_fused if fused else layer.forward
    if graph:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fwd(xd, rd, out)          # warm-up outside the capture
        torch.cuda.current_stream().wait_stream(s)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fwd(xd, rd, out)
        out.zero_()
        g.replay()
    else:
        fwd(xd, rd, out)
    torch.cuda.synchronize()
    res = dict(ids=layer.ids.cpu().numpy(), scores=layer.scores.cpu().numpy(),
               act=None if fused else layer.act.cpu().numpy(),
               partial=None if fused else layer.partial.cpu().numpy(),
               out=out.cpu().numpy())
    if fused:
        res["error_word"] = layer.fused_error_word()
    else:
        import quantized_moe_decode_amd as q
        res["error_word"] = int(q.workspace_status(layer.route_ws) != q.MOE_OK)
    if layer.shared_gate is not None:
        res["gate"] = layer.shared_gate.cpu().numpy()
    if layer.n_shared:
        res["shared_partial"] = layer.shared_partial.cpu().numpy()
    return res, layer


def compare_layer(cfg, w, x, resid, gpu, label="", ref=None):
    """Assert the GPU result matches the oracle on the same inputs; returns the
    errors.  `ref` is the oracle's result when already computed (then `w` is
    not used)."""
    if ref is None:
        ref = oracle.layer(cfg, w, x, resid)
    ids_ref = ref["route"]["ids"]
    assert np.array_equal(gpu["ids"], ids_ref), f"{label}: ids {gpu['ids']} vs {ids_ref}"
    ds = float(np.max(np.abs(gpu["scores"] - ref["route"]["scores"])))
    assert ds <= SCORE_TOL, f"{label}: scores off by {ds}"
    if gpu.get("error_word"):
        raise AssertionError(f"{label}: a launch reported a wait time-out")
    if cfg.shared_gate:
        dg = float(np.max(np.abs(gpu["gate"] - ref["route"]["gate"])))
        assert dg <= SCORE_TOL, f"{label}: shared gate off by {dg}"
    errs = {}
    T = x.shape[0]
    for t in range(T if gpu["act"] is not None else 0):
        for k in range(cfg.top_k):
            errs.setdefault("act", []).append(rel_err(gpu["act"][t, k], ref["ffn"]["act"][t, k]))
            errs.setdefault("partial", []).append(
                rel_err(gpu["partial"][t, k], ref["ffn"]["partial"][t, k]))
    resid64 = np_decode(resid, cfg.resid_dtype).reshape(T, cfg.d_in)
    for t in range(T):
        errs.setdefault("out", []).append(rel_err(gpu["out"][t], ref["out"][t]))
        errs.setdefault("moe", []).append(rel_err(gpu["out"][t] - resid64[t], ref["out"][t] - resid64[t]))
    worst = {k: max(v) for k, v in errs.items()}
    say(f"  {label}: worst relative errors {worst}")
    for k, v in worst.items():
        assert v <= TOL, f"{label}: {k} relative error {v} > {TOL}"
    return worst


def margin_tokens(cfg, layer_idx, w, n_tokens):
    x, resid, attempts = pick_tokens(cfg, layer_idx, n_tokens, w["router"])
    return x, resid


def small_cfg(**kw):
    base = dict(name="small", cfg_id=60, weight_cfg_id=60, d_in=192, d_ff=320, n_experts=5,
                top_k=3, renormalize=True, bits_gate_up=4, bits_down=4, sb_dtype=mi.BF16,
                x_dtype=mi.BF16, router_dtype=mi.BF16, resid_dtype=mi.BF16)
    base.update(kw)
    return mi.LayerConfig(**base)
