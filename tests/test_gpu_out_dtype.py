"""The layer output and the folded RMSNorm stored in 16 bits (bf16 or fp16), as
an engine that keeps its hidden state in bf16 holds them, on both paths,
against the oracle under a bound that accounts for the rounding.

Bound for out (per element i, oracle result y in fp64): the fp32 result the
kernels compute is within tau = 2e-3 * max|y| of y (the layer's own bar), and
one rounding to a dtype with p significand bits moves a value v by at most
h * |v|, h = 2^-p (bf16 2^-8, fp16 2^-11), so
    |out_i - y_i| <= tau + h * (|y_i| + tau).
Bound for normed: the oracle rounds y itself (oracle.round_to) to u and
normalises u.  The stored out s differs from u by at most
    d_i = tau + h * (|y_i| + tau) + h * |y_i|,
so the root mean squares differ by at most D = rms(d) (the triangle
inequality of the RMS norm, which eps inside the root only shrinks), and
    |w_i s_i / r_s - w_i u_i / r_u| <= |w_i| (d_i / (r_u - D) + |u_i| D / ((r_u - D) r_u)) = b_i,
plus the final rounding h_n * (|n_i| + b_i) and 1e-5 * max|n| for the fp32
arithmetic.  Besides the bound: with the same inputs, the 16-bit out is
exactly the fp32 out rounded to nearest even (torch's conversion), because
the store is the only step that changes.  Every case prints its name first.
"""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from gpu_cases import DEV, SCORE_TOL, margin_tokens, say, small_cfg
from helpers import np_decode

pytestmark = pytest.mark.gpu
TOL = 2e-3
HALF_ULP = {torch.float32: 0.0, torch.bfloat16: 2.0 ** -8, torch.float16: 2.0 ** -11}
NAME = {torch.float32: mi.F32, torch.bfloat16: mi.BF16, torch.float16: mi.F16}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_moe_decode_amd  # noqa: F401
    yield


def run(cfg, w, x, resid, fused, out_dt, norm_dt=None, fold=True, layer=None):
    """The layer on the GPU with out of out_dt (and normed of norm_dt when given)."""
    import quantized_moe_decode_amd as q
    from quantized_moe_decode_amd.layer import layer_from_host, tensor_from_encoded
    T = x.shape[0]
    if layer is None:
        layer = layer_from_host(cfg, w, DEV, n_tokens=T)
        if norm_dt is not None:
            nw = mi.gen_norm_weight(cfg, 0)
            layer.set_next_norm(tensor_from_encoded(nw, mi.BF16, DEV), cfg.norm_eps, fold=fold, dtype=norm_dt)
    xd = tensor_from_encoded(x, cfg.x_dtype, DEV)
    rd = tensor_from_encoded(resid, cfg.resid_dtype, DEV)
    out = torch.zeros(T, cfg.d_in, device=DEV, dtype=out_dt)
    (layer.forward_fused if fused else layer.forward)(xd, rd, out)
    torch.cuda.synchronize()
    err = (layer.fused_error_word() if fused else
           int(q.workspace_status(layer.route_ws) != q.MOE_OK or
               (layer.normed is not None and fold and q.workspace_status(layer.tail_ws) != q.MOE_OK)))
    res = dict(ids=layer.ids.cpu().numpy(), scores=layer.scores.cpu().numpy(), error_word=err,
               out=out.float().cpu().numpy().astype(np.float64), out_raw=out.cpu())
    if layer.normed is not None:
        res["normed"] = layer.normed.float().cpu().numpy().astype(np.float64)
    return res, layer


def out_bound(y, dt):
    h, tau = HALF_ULP[dt], TOL * float(np.max(np.abs(y)))
    return tau + h * (np.abs(y) + tau)


def normed_bound(y, wd, eps, out_dt, norm_dt):
    """Per-element bound of the GPU's normed against the oracle's normalisation
    of y rounded to out_dt (derivation in the module docstring); returns the
    oracle's normed and the bound."""
    h, hn, tau = HALF_ULP[out_dt], HALF_ULP[norm_dt], TOL * float(np.max(np.abs(y)))
    u = oracle.round_to(y, NAME[out_dt])
    n = oracle.rmsnorm(u, mi.encode(wd, mi.F32), mi.F32, eps)
    d = tau + h * (np.abs(y) + tau) + h * np.abs(u)
    r_u = np.sqrt(np.mean(u * u, axis=-1, keepdims=True) + eps)
    D = np.sqrt(np.mean(d * d, axis=-1, keepdims=True))
    assert np.all(D < r_u / 2), "bound not applicable: rounding error comparable to the norm"
    b = np.abs(wd) * (d / (r_u - D) + np.abs(u) * D / ((r_u - D) * r_u))
    return n, b + hn * (np.abs(n) + b) + 1e-5 * np.max(np.abs(n))


def check(cfg, w, x, resid, gpu, out_dt, norm_dt, label):
    ref = oracle.layer(cfg, w, x, resid)
    assert not gpu["error_word"], f"{label}: a wait timed out"
    assert np.array_equal(gpu["ids"], ref["route"]["ids"]), f"{label}: ids differ"
    assert np.max(np.abs(gpu["scores"] - ref["route"]["scores"])) <= SCORE_TOL, f"{label}: scores"
    y = ref["out"]
    excess = np.abs(gpu["out"] - y) / out_bound(y, out_dt)
    say(f"  {label}: out error / bound {excess.max():.3f}")
    assert excess.max() <= 1.0, f"{label}: out outside the bound at {np.unravel_index(excess.argmax(), y.shape)}"
    if norm_dt is not None:
        wd = np_decode(mi.gen_norm_weight(cfg, 0), mi.BF16)
        n, bound = normed_bound(y, wd, cfg.norm_eps, out_dt, norm_dt)
        excess = np.abs(gpu["normed"] - n) / bound
        say(f"  {label}: normed error / bound {excess.max():.3f}")
        assert excess.max() <= 1.0, f"{label}: normed outside the bound"


SMALL = [dict(), dict(d_in=1088, d_ff=704, n_experts=9, top_k=4, bits_down=6),
         dict(n_shared=1, d_ff_shared=256, shared_gate=True)]


@pytest.mark.parametrize("out_dt", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
@pytest.mark.parametrize("kw", SMALL, ids=["base", "ragged-6bit", "shared"])
@pytest.mark.parametrize("fused", [True, False], ids=["fused", "three-call"])
def test_small_layers_16bit_out(kw, fused, out_dt):
    cfg = small_cfg(**kw)
    say(f"case 16-bit out {'fused' if fused else 'three-call'} {kw} {out_dt}")
    w = mi.gen_layer_weights(cfg, 0, threads=4)
    x, resid = margin_tokens(cfg, 0, w, 1)
    for norm_dt in (None, out_dt):
        gpu, _ = run(cfg, w, x, resid, fused, out_dt, norm_dt)
        check(cfg, w, x, resid, gpu, out_dt, norm_dt, f"{kw} out {out_dt} normed {norm_dt}")


@pytest.mark.parametrize("fused", [True, False], ids=["fused", "three-call"])
def test_16bit_out_is_the_fp32_out_rounded(fused):
    """Same inputs, same launch shape: the 16-bit outputs equal torch's
    round-to-nearest-even conversion of the fp32 output, bit for bit."""
    cfg = small_cfg(d_in=1088, d_ff=704, n_experts=9, top_k=4)
    say(f"case 16-bit out exact rounding fused={fused}")
    w = mi.gen_layer_weights(cfg, 3, threads=4)
    x, resid = margin_tokens(cfg, 3, w, 1)
    f32, layer = run(cfg, w, x, resid, fused, torch.float32)
    for dt in (torch.bfloat16, torch.float16):
        g, _ = run(cfg, w, x, resid, fused, dt, layer=layer)
        want = f32["out_raw"].to(dt)
        assert torch.equal(g["out_raw"].view(torch.int16), want.view(torch.int16)), f"{dt}: not one rounding"


def test_three_call_32_tokens_bf16_with_folded_and_separate_norm():
    cfg = small_cfg(d_in=512, d_ff=384, n_experts=12, top_k=4)
    w = mi.gen_layer_weights(cfg, 1, threads=4)
    x, resid = margin_tokens(cfg, 1, w, 32)
    for fold in (True, False):
        say(f"case 16-bit out three-call T=32 fold={fold}")
        gpu, _ = run(cfg, w, x, resid, False, torch.bfloat16, torch.bfloat16, fold=fold)
        check(cfg, w, x, resid, gpu, torch.bfloat16, torch.bfloat16, f"T=32 fold={fold}")


@pytest.mark.parametrize("name", ["qwen3_30b_a3b_moe", "dots_llm1_mixed_bit"])
def test_full_size_bf16(name):
    cfg = mi.CONFIGS[name]
    w = mi.gen_layer_weights(cfg, 0)
    x, resid = margin_tokens(cfg, 0, w, 1)
    for fused in (True, False):
        say(f"case 16-bit out {name} fused={fused}")
        gpu, _ = run(cfg, w, x, resid, fused, torch.bfloat16, torch.bfloat16)
        check(cfg, w, x, resid, gpu, torch.bfloat16, torch.bfloat16, f"{name} fused={fused}")


def test_decode_step_bf16_graph_replays():
    """Several layers in one captured step with bf16 outputs and bf16 normed:
    every replay equals the eager step bit for bit and matches the oracle."""
    from quantized_moe_decode_amd.layer import DecodeStep, layer_from_host, tensor_from_encoded
    cfg = small_cfg(d_in=1024, d_ff=512, n_experts=16, top_k=4)
    say("case 16-bit out decode step, 3 layers, 2 tokens, graph replays")
    n_layers, n_tok = 3, 2
    ws = [mi.gen_layer_weights(cfg, l, threads=4) for l in range(n_layers)]
    layers, toks = [], []
    for l in range(n_layers):
        lay = layer_from_host(cfg, ws[l], DEV, n_tokens=1)
        lay.set_next_norm(tensor_from_encoded(mi.gen_norm_weight(cfg, 0), mi.BF16, DEV), cfg.norm_eps,
                          dtype=torch.bfloat16)
        layers.append(lay)
        x, r = margin_tokens(cfg, l, ws[l], n_tok)
        toks.append((x, r))
    xs = [[tensor_from_encoded(toks[l][0][t:t + 1], cfg.x_dtype, DEV) for l in range(n_layers)]
          for t in range(n_tok)]
    rs = [[tensor_from_encoded(toks[l][1][t:t + 1], cfg.resid_dtype, DEV) for l in range(n_layers)]
          for t in range(n_tok)]
    for path in ("fused", "three-call"):
        step = DecodeStep(layers, xs, rs, path=path, out_dtype=torch.bfloat16)
        step.capture()
        for t in range(n_tok):
            step.eager(t)
            torch.cuda.synchronize()
            eager = [(o.clone(), l.normed.clone()) for o, l in zip(step.outs, layers)]
            for _ in range(3):
                for o in step.outs:
                    o.zero_()
                step.replay(t)
                torch.cuda.synchronize()
                for (eo, en), o, l in zip(eager, step.outs, layers):
                    assert torch.equal(o.view(torch.int16), eo.view(torch.int16)), f"{path} token {t}: out"
                    assert torch.equal(l.normed.view(torch.int16), en.view(torch.int16)), f"{path}: normed"
            assert step.error_words() == 0
            for l in range(n_layers):
                x, r = toks[l][0][t:t + 1], toks[l][1][t:t + 1]
                gpu = dict(ids=layers[l].ids.cpu().numpy(), scores=layers[l].scores.cpu().numpy(),
                           error_word=0, out=step.outs[l].float().cpu().numpy().astype(np.float64),
                           normed=layers[l].normed.float().cpu().numpy().astype(np.float64))
                check(cfg, ws[l], x, r, gpu, torch.bfloat16, torch.bfloat16, f"{path} layer {l} token {t}")
