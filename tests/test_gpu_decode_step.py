"""The decode step as the benchmark runs it, against the oracle: several
full-size layers in order on one stream, each distinct token's step captured
once into a HIP graph and replayed in rotated order, the fused launches of all
layers sharing one workspace (quantized_moe_decode_amd.layer.DecodeStep, the
class the benchmark uses).  Every layer's output and routing is compared with
the oracle after every replay.  Every case prints its name before it runs.
"""
import numpy as np
import pytest
import torch

import moe_inputs as mi
from gpu_cases import DEV, compare_layer, say
from helpers import oracle_layer_selected, pick_tokens

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_moe_decode_amd  # noqa: F401
    yield


def build_step(specs, n_distinct, path, n_tokens=1, norm=False):
    """Layers (cfg, layer index) on the device, margin tokens per layer, and the
    oracle's result for every (token, layer).  norm: every layer's tail also
    computes the next layer's RMSNorm (weight gen_norm_weight, the workload's eps)."""
    from quantized_moe_decode_amd.layer import DecodeStep, layer_from_host, tensor_from_encoded
    layers, host_x, host_r = [], [], []
    for cfg, li in specs:
        w = mi.gen_layer_weights(cfg, li)
        layers.append(layer_from_host(cfg, w, DEV, n_tokens=n_tokens))
        if norm:
            layers[-1].set_next_norm(tensor_from_encoded(mi.gen_norm_weight(cfg, li), mi.BF16, DEV), cfg.norm_eps)
        x, r, _ = pick_tokens(cfg, li, n_distinct * n_tokens, w["router"])
        host_x.append(x.reshape(n_distinct, n_tokens, -1))
        host_r.append(r.reshape(n_distinct, n_tokens, -1))
        del w
    xs = [[tensor_from_encoded(host_x[l][t], specs[l][0].x_dtype, DEV) for l in range(len(specs))]
          for t in range(n_distinct)]
    rs = [[tensor_from_encoded(host_r[l][t], specs[l][0].resid_dtype, DEV) for l in range(len(specs))]
          for t in range(n_distinct)]
    step = DecodeStep(layers, xs, rs, path=path)
    refs = {(t, l): oracle_layer_selected(specs[l][0], specs[l][1], host_x[l][t], host_r[l][t])
            for t in range(n_distinct) for l in range(len(specs))}
    return step, host_x, host_r, refs


def check_replays(step, specs, host_x, host_r, refs, order, label):
    step.capture()
    for i, t in enumerate(order):
        for o in step.outs:
            o.fill_(-1.0)                  # eager work on the step's buffers between replays
        for lay in step.layers:
            lay.ids.fill_(-1)
        step.replay(t)
        torch.cuda.synchronize()
        assert step.error_words() == 0, f"{label}: a fused wait timed out"
        for l, (cfg, li) in enumerate(specs):
            lay = step.layers[l]
            gpu = dict(ids=lay.ids.cpu().numpy(), scores=lay.scores.cpu().numpy(),
                       act=None, partial=None, out=step.outs[l].cpu().numpy())
            if lay.shared_gate is not None:
                gpu["gate"] = lay.shared_gate.cpu().numpy()
            compare_layer(cfg, None, host_x[l][t], host_r[l][t], gpu,
                          f"{label} replay {i} token {t} layer {l} ({cfg.name} L{li})", ref=refs[(t, l)])
            if lay.normed is not None:
                import oracle
                from helpers import rel_err
                want = oracle.rmsnorm(refs[(t, l)]["out"], mi.gen_norm_weight(cfg, li), mi.BF16, cfg.norm_eps)
                e = rel_err(lay.normed.cpu().numpy(), want)
                assert e <= 2e-3, f"{label} replay {i} token {t} layer {l}: normed relative error {e}"


MIXED = [(mi.QWEN3, 0), (mi.QWEN3, 1), (mi.QWEN3, 2), (mi.QWEN3, 3), (mi.QWEN15, 0), (mi.QWEN15, 1)]


def test_fused_step_shared_workspace():
    say("case decode step: fused, 4 Qwen3 + 2 Qwen1.5 layers, one shared workspace, 3 tokens")
    step, hx, hr, refs = build_step(MIXED, 3, "fused")
    ptrs = {l.fused_ws.data_ptr() for l in step.layers}
    assert len(ptrs) == 1 and step.fused_ws is not None, "layers do not share one fused workspace"
    check_replays(step, MIXED, hx, hr, refs, [0, 1, 2, 1, 0, 2, 2], "fused step")


def test_three_call_step():
    say("case decode step: three-call, 4 Qwen3 + 2 Qwen1.5 layers, 2 tokens")
    step, hx, hr, refs = build_step(MIXED, 2, "three-call")
    check_replays(step, MIXED, hx, hr, refs, [0, 1, 1, 0], "three-call step")


def test_batch32_step():
    specs = [(mi.QWEN3_B32, 0), (mi.QWEN3_B32, 1), (mi.QWEN3_B32, 2)]
    say("case decode step: 32 tokens per step, 3 Qwen3 layers, 2 token batches")
    step, hx, hr, refs = build_step(specs, 2, "three-call", n_tokens=32)
    check_replays(step, specs, hx, hr, refs, [0, 1, 0], "batch-32 step")


def test_fused_step_with_folded_rmsnorm():
    say("case decode step: fused, 4 Qwen3 + 2 Qwen1.5 layers, next-layer RMSNorm folded, 2 tokens")
    step, hx, hr, refs = build_step(MIXED, 2, "fused", norm=True)
    check_replays(step, MIXED, hx, hr, refs, [0, 1, 1, 0], "fused step + rmsnorm")


def test_three_call_step_with_folded_rmsnorm():
    specs = [(mi.QWEN3_B32, 0), (mi.QWEN3_B32, 1)]
    say("case decode step: 32 tokens, 2 Qwen3 layers, next-layer RMSNorm folded, 2 batches")
    step, hx, hr, refs = build_step(specs, 2, "three-call", n_tokens=32, norm=True)
    check_replays(step, specs, hx, hr, refs, [0, 1, 0], "batch-32 step + rmsnorm")


def test_prefill_step_grouped():
    """256 tokens per step on 2 Qwen3-shaped layers: batched routing, the
    grouped expert FFN and the tail captured in one graph per batch, replayed
    in rotated order; sampled tokens of every layer against the oracle after
    every replay."""
    from quantized_moe_decode_amd.layer import DecodeStep, layer_from_host, tensor_from_encoded
    cfg, T, n_b = mi.QWEN3_P256, 256, 2
    say("case decode step: 256 tokens per step (grouped), 2 Qwen3 layers, 2 batches")
    sample = np.array([0, 37, 128, 255])
    layers, hx, hr, refs = [], [], [], {}
    for li in range(2):
        w = mi.gen_layer_weights(cfg, li)
        lay = layer_from_host(cfg, w, DEV, n_tokens=T)
        assert lay.grouped
        layers.append(lay)
        x, r, _ = pick_tokens(cfg, li, n_b * T, w["router"])
        hx.append(x.reshape(n_b, T, -1))
        hr.append(r.reshape(n_b, T, -1))
        for b in range(n_b):
            refs[(b, li)] = oracle_layer_selected(cfg, li, hx[li][b][sample], hr[li][b][sample])
        del w
    xs = [[tensor_from_encoded(hx[l][b], cfg.x_dtype, DEV) for l in range(2)] for b in range(n_b)]
    rs = [[tensor_from_encoded(hr[l][b], cfg.resid_dtype, DEV) for l in range(2)] for b in range(n_b)]
    step = DecodeStep(layers, xs, rs, path="three-call")
    step.capture()
    for i, b in enumerate([0, 1, 1, 0]):
        for o in step.outs:
            o.fill_(-1.0)
        for lay in step.layers:
            lay.ids.fill_(-1)
        step.replay(b)
        torch.cuda.synchronize()
        for l in range(2):
            lay = step.layers[l]
            gpu = dict(ids=lay.ids.cpu().numpy()[sample], scores=lay.scores.cpu().numpy()[sample],
                       act=None, partial=None, out=step.outs[l].cpu().numpy()[sample])
            compare_layer(cfg, None, hx[l][b][sample], hr[l][b][sample], gpu,
                          f"prefill step replay {i} batch {b} layer {l}", ref=refs[(b, l)])


def test_steps_repeated_in_one_graph_give_the_single_step():
    """DecodeStep(repeat=4): each replay runs the step four times on the same
    token; the outputs equal those of the one-step graph bit for bit and the
    oracle's (the tiny layer, fused and three-call)."""
    from quantized_moe_decode_amd.layer import DecodeStep
    specs = [(mi.TINY, 0)]
    for path in ("fused", "three-call"):
        say(f"case decode step: tiny layer, 4 steps per graph, {path}")
        step, hx, hr, refs = build_step(specs, 2, path)
        step.capture()
        single = []
        for t in range(2):
            step.replay(t)
            torch.cuda.synchronize()
            single.append(step.outs[0].clone())
        rstep = DecodeStep(step.layers, step.xs, step.rs, path=path, repeat=4)
        check_replays(rstep, specs, hx, hr, refs, [0, 1, 1, 0], f"{path} x4")
        for t in range(2):
            rstep.replay(t)
            torch.cuda.synchronize()
            assert torch.equal(rstep.outs[0], single[t]), f"{path}: repeated step differs from one step"
