"""GPU parity of the fused single-launch layer (moe_decode_layer) against the oracle,
and against the three-call path.  Every case prints its name before it runs."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
from gpu_cases import DEV, compare_layer, margin_tokens, run_gpu_layer, say, small_cfg
from helpers import rel_err
from test_gpu_parity import SMALL

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_moe_decode_amd  # noqa: F401
    yield


@pytest.mark.parametrize("kw", SMALL + [dict(n_shared=1, d_ff_shared=256, shared_gate=True),
                                        dict(n_shared=2, d_ff_shared=128, bits_down=6),
                                        dict(n_shared=1, d_ff_shared=1152, shared_gate=True,
                                             bits_gate_up=8, bits_down=8)],
                         ids=lambda d: ",".join(f"{k}={v}" for k, v in d.items()) or "base")
def test_fused_small_layers(kw):
    cfg = small_cfg(**kw)
    say(f"case fused small {kw}")
    w = mi.gen_layer_weights(cfg, 0, threads=4)
    x, resid = margin_tokens(cfg, 0, w, 2)
    for t in range(2):
        gpu, layer = run_gpu_layer(cfg, w, x[t:t + 1], resid[t:t + 1], fused=True)
        compare_layer(cfg, w, x[t:t + 1], resid[t:t + 1], gpu, f"fused small {kw} t{t}")
        ws = layer.fused_ws.cpu().numpy()
        assert not np.any(ws[:4]), "error word set"


# Eight slots at d_in = 2048 (units in the XCD-aligned slot order; top-8
# routed, or top-6 plus two shared experts), a ragged d_ff (704 = 44 x 16),
# each input dtype's dot path and 6-bit down projections.
@pytest.mark.parametrize("kw", [
    dict(d_ff=704, n_experts=12, top_k=8),
    dict(d_ff=768, n_experts=10, top_k=8, x_dtype=mi.F16, router_dtype=mi.F16, resid_dtype=mi.F16),
    dict(d_ff=768, n_experts=9, top_k=8, x_dtype=mi.F32, router_dtype=mi.F32, resid_dtype=mi.F32,
         sb_dtype=mi.F16),
    dict(d_ff=768, n_experts=11, top_k=8, bits_down=6),
    dict(d_ff=768, n_experts=10, top_k=6, n_shared=2, d_ff_shared=704),
], ids=lambda d: ",".join(f"{k}={v}" for k, v in d.items()))
def test_fused_eight_slots(kw):
    cfg = small_cfg(d_in=2048, **kw)
    say(f"case fused eight slots {kw}")
    w = mi.gen_layer_weights(cfg, 5, threads=4)
    x, resid = margin_tokens(cfg, 5, w, 2)
    for t in range(2):
        gpu, layer = run_gpu_layer(cfg, w, x[t:t + 1], resid[t:t + 1], fused=True)
        compare_layer(cfg, w, x[t:t + 1], resid[t:t + 1], gpu, f"fused eight slots {kw} t{t}")
        ws = layer.fused_ws.cpu().numpy()
        assert not np.any(ws[:4]), "error word set"


def test_fused_jittered_bias():
    for bits in ((4, 4), (8, 8), (4, 6)):
        cfg = small_cfg(bits_gate_up=bits[0], bits_down=bits[1])
        say(f"case fused jitter {bits}")
        w = mi.gen_layer_weights(cfg, 2, jitter_bias=True, threads=4)
        x, resid = margin_tokens(cfg, 2, w, 1)
        gpu, _ = run_gpu_layer(cfg, w, x, resid, fused=True)
        compare_layer(cfg, w, x, resid, gpu, f"fused jitter {bits}")


@pytest.mark.parametrize("name,layers,T", [
    ("tiny_e8_top2", (0,), 3),
    ("qwen3_30b_a3b_moe", (0, 31), 2),
    ("qwen1.5_moe_a2.7b", (0,), 2),
    ("dots_llm1_mixed_bit", (0,), 1),
])
def test_fused_full_size_layers(name, layers, T):
    cfg = mi.CONFIGS[name]
    for li in layers:
        say(f"case fused {name} layer {li}")
        w = mi.gen_layer_weights(cfg, li)
        x, resid = margin_tokens(cfg, li, w, T)
        for t in range(T):
            gpu, layer = run_gpu_layer(cfg, w, x[t:t + 1], resid[t:t + 1], graph=True, fused=True)
            compare_layer(cfg, w, x[t:t + 1], resid[t:t + 1], gpu, f"fused {name} L{li} t{t}")
            three, _ = run_gpu_layer(cfg, w, x[t:t + 1], resid[t:t + 1], layer=layer)
            assert np.array_equal(three["ids"], gpu["ids"])
            # the fused launch rounds act to fp16 before 4-bit down projections
            # (relative 2^-11 per element; about 2.3e-4 of |out|_inf measured on these
            # layers), the three-call path keeps fp32: both sit within the oracle's bar
            assert rel_err(gpu["out"], three["out"]) <= 1e-3


def test_fused_determinism_graph_replays_and_clean_workspace():
    cfg = mi.QWEN3
    say("case fused determinism + graph replays")
    w = mi.gen_layer_weights(cfg, 3)
    x, resid = margin_tokens(cfg, 3, w, 1)
    a, layer = run_gpu_layer(cfg, w, x, resid, fused=True)
    for rep in range(3):
        b, _ = run_gpu_layer(cfg, w, x, resid, layer=layer, fused=True)
        assert np.array_equal(a["out"], b["out"]) and np.array_equal(a["ids"], b["ids"])
    from quantized_moe_decode_amd.layer import tensor_from_encoded
    xd = tensor_from_encoded(x, cfg.x_dtype, DEV)
    rd = tensor_from_encoded(resid, cfg.resid_dtype, DEV)
    out = torch.zeros(1, cfg.d_in, device=DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        layer.forward_fused(xd, rd, out)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.forward_fused(xd, rd, out)
    for rep in range(5):
        out.fill_(-1.0)
        layer.forward(xd, rd, torch.empty_like(out))       # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), a["out"]), rep
    # every counter is back at zero and no wait timed out
    ws = layer.fused_ws.view(torch.int32).cpu().numpy()
    # control words 64 apart: error word, launch epoch, finished-tile counter
    launches = 1 + 3 + 1 + 5
    assert ws[0] == 0, "a wait timed out"
    assert ws[64] == launches, f"epoch {ws[64]} after {launches} launches"
    assert ws[128] == 0, "finished-tile counter not reset"


@pytest.mark.parametrize("top_k,rows,want", [
    # exact tie inside the top-k: the lower id takes the higher rank
    (3, {6: 0.05, 2: 0.05, 5: 0.04, 1: 0.01}, [2, 6, 5]),
    # ties only below the top-k (four zero logits)
    (4, {6: 0.05, 2: 0.04, 5: 0.03, 1: 0.02}, [6, 2, 5, 1]),
    # the k-th place is a tie of four zero logits: the lowest id wins it
    (5, {6: 0.05, 2: 0.04, 5: 0.03, 1: 0.02}, [6, 2, 5, 1, 0]),
    # tie across the k-th place between two positive logits
    (2, {3: 0.05, 5: 0.04, 1: 0.04}, [3, 1]),
], ids=["inside", "below", "at-k-zeros", "at-k"])
def test_fused_tie_prefers_lower_index(top_k, rows, want):
    """Router rows that tie exactly: descending logit, ties to the lower id, as the oracle."""
    cfg = small_cfg(n_experts=8, top_k=top_k, x_dtype=mi.F32, router_dtype=mi.F32, resid_dtype=mi.F32)
    say(f"case fused router tie k={top_k} {rows}")
    w = mi.gen_layer_weights(cfg, 4, threads=4)
    x, resid = mi.gen_tokens(cfg, 4, 1)
    wr = np.zeros_like(w["router"])
    r = x[0].astype(np.float32)
    for e, c in rows.items():
        wr[e] = r * np.float32(c)
    w["router"] = wr
    gpu, _ = run_gpu_layer(cfg, w, x, resid, fused=True)
    assert gpu["ids"].tolist() == [want]
    import oracle
    ref = oracle.route(x, cfg.x_dtype, w["router"], cfg.router_dtype, top_k, cfg.renormalize)
    assert ref["ids"].tolist() == [want]
    np.testing.assert_allclose(gpu["scores"], ref["scores"], rtol=1e-5, atol=1e-7)


@pytest.mark.parametrize("n_experts,top_k,rows,want", [
    # ties between ids held in different lane words of the selecting wave (ids 64 apart)
    (200, 6, {150: 0.05, 3: 0.04, 70: 0.04, 199: 0.03, 66: 0.03, 130: 0.03, 10: 0.02},
     [150, 3, 70, 66, 130, 199]),
    # the k-th place split inside a three-way tie spread over three lane words
    (200, 5, {150: 0.05, 3: 0.04, 70: 0.04, 199: 0.03, 66: 0.03, 130: 0.03, 10: 0.02},
     [150, 3, 70, 66, 130]),
    # every logit zero: the lowest ids, in id order
    (200, 8, {}, list(range(8))),
    # a negative-only router: the zero logits outrank the negative ones
    (130, 4, {5: -0.02, 129: -0.01}, [0, 1, 2, 3]),
], ids=["across-words", "split-at-k", "all-zero", "negatives"])
def test_fused_ties_many_experts(n_experts, top_k, rows, want):
    """Exact ties with more experts than one wave has lanes: descending logit, ties to the lower id."""
    cfg = small_cfg(n_experts=n_experts, top_k=top_k, x_dtype=mi.F32, router_dtype=mi.F32, resid_dtype=mi.F32)
    say(f"case fused router ties E={n_experts} k={top_k}")
    w = mi.gen_layer_weights(cfg, 6, threads=8)
    x, resid = mi.gen_tokens(cfg, 6, 1)
    wr = np.zeros_like(w["router"])
    r = x[0].astype(np.float32)
    for e, c in rows.items():
        wr[e] = r * np.float32(c)
    w["router"] = wr
    gpu, _ = run_gpu_layer(cfg, w, x, resid, fused=True)
    import oracle
    ref = oracle.route(x, cfg.x_dtype, w["router"], cfg.router_dtype, top_k, cfg.renormalize)
    assert ref["ids"].tolist() == [want]
    assert gpu["ids"].tolist() == [want]
    np.testing.assert_allclose(gpu["scores"], ref["scores"], rtol=1e-5, atol=1e-7)


@pytest.mark.parametrize("n_experts,top_k", [(160, 6), (1000, 8), (64, 32)])
def test_fused_expert_counts(n_experts, top_k):
    """Expert counts from one lane word to sixteen in the selecting wave, and k = 32."""
    cfg = small_cfg(n_experts=n_experts, top_k=top_k)
    say(f"case fused E={n_experts} K={top_k}")
    w = mi.gen_layer_weights(cfg, 5, threads=8)
    x, resid = margin_tokens(cfg, 5, w, 1)
    gpu, layer = run_gpu_layer(cfg, w, x, resid, fused=True)
    compare_layer(cfg, w, x, resid, gpu, f"fused E={n_experts} K={top_k}")
    assert not np.any(layer.fused_ws.cpu().numpy()[:4]), "error word set"
