"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Every case prints its name before it touches the GPU.  Inputs come from the
seeded generator; tokens are drawn with a routing margin of 1e-3 between
consecutive top-(K+1) logits so that the expert ids are fixed.
"""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from gpu_cases import (DEV, compare_layer, margin_tokens, run_gpu_layer, say, small_cfg)
from helpers import np_decode, stack_from_arrays

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_moe_decode_amd  # noqa: F401  (raises if the library is not built)
    yield


# ------------------------------------------------------------ small shapes
SMALL = [
    dict(),                                                   # 4-bit, bf16, ragged row tiles
    dict(bits_gate_up=8, bits_down=8),
    dict(bits_gate_up=4, bits_down=6),
    dict(bits_gate_up=6, bits_down=6, sb_dtype=mi.F16),
    dict(bits_gate_up=8, bits_down=4, x_dtype=mi.F32, router_dtype=mi.F32, resid_dtype=mi.F32),
    dict(x_dtype=mi.F16, router_dtype=mi.F16, resid_dtype=mi.F16, renormalize=False),
    dict(d_in=64, d_ff=64, n_experts=3, top_k=1),             # smallest legal shapes
    dict(d_in=1088, d_ff=704, n_experts=9, top_k=4, bits_down=6),  # odd group counts
    dict(d_in=1088, d_ff=704, n_experts=9, top_k=4),          # 4-bit, rows of 34 and 22 chunks
]


@pytest.mark.parametrize("kw", SMALL, ids=lambda d: ",".join(f"{k}={v}" for k, v in d.items()) or "base")
@pytest.mark.parametrize("T", [1, 3])
def test_small_layers(kw, T):
    cfg = small_cfg(**kw)
    say(f"case small {kw} T={T}")
    w = mi.gen_layer_weights(cfg, 0, threads=4)
    x, resid = margin_tokens(cfg, 0, w, T)
    gpu, _ = run_gpu_layer(cfg, w, x, resid)
    compare_layer(cfg, w, x, resid, gpu, f"small {kw} T={T}")


@pytest.mark.parametrize("shared", [dict(n_shared=1, d_ff_shared=256, shared_gate=True),
                                    dict(n_shared=2, d_ff_shared=128, shared_gate=False)])
@pytest.mark.parametrize("T", [1, 4])
def test_small_layers_with_shared_experts(shared, T):
    cfg = small_cfg(bits_gate_up=4, bits_down=6, **shared)
    say(f"case small shared {shared} T={T}")
    w = mi.gen_layer_weights(cfg, 1, threads=4)
    x, resid = margin_tokens(cfg, 1, w, T)
    gpu, _ = run_gpu_layer(cfg, w, x, resid)
    compare_layer(cfg, w, x, resid, gpu, f"shared {shared} T={T}")


def test_jittered_bias():
    """Biases not equal to -2^(b-1)*scale: a kernel assuming a fixed zero point fails here."""
    for bits in ((4, 4), (8, 8), (4, 6)):
        cfg = small_cfg(bits_gate_up=bits[0], bits_down=bits[1])
        say(f"case jitter bits={bits}")
        w = mi.gen_layer_weights(cfg, 2, jitter_bias=True, threads=4)
        x, resid = margin_tokens(cfg, 2, w, 2)
        gpu, _ = run_gpu_layer(cfg, w, x, resid)
        compare_layer(cfg, w, x, resid, gpu, f"jitter {bits}")


# --------------------------------------------------------- the workloads
def test_tiny_layer():
    cfg = mi.TINY
    say("case tiny")
    w = mi.gen_layer_weights(cfg, 0, threads=4)
    for t0 in range(4):
        x, resid = margin_tokens(cfg, 0, w, 1 + t0)
        gpu, _ = run_gpu_layer(cfg, w, x[-1:], resid[-1:])
        compare_layer(cfg, w, x[-1:], resid[-1:], gpu, f"tiny token {t0}")


@pytest.mark.parametrize("name,layers,T", [
    ("qwen3_30b_a3b_moe", (0, 47), 2),
    ("qwen1.5_moe_a2.7b", (0,), 2),
    ("dots_llm1_mixed_bit", (0,), 1),
    ("qwen3_30b_a3b_moe_batch32", (0,), 32),
])
def test_full_size_layers(name, layers, T):
    cfg = mi.CONFIGS[name]
    for li in layers:
        say(f"case {name} layer {li} T={T}")
        w = mi.gen_layer_weights(cfg, li)
        x, resid = margin_tokens(cfg, li, w, T)
        if cfg.n_tokens == 1:
            for t in range(T):
                gpu, _ = run_gpu_layer(cfg, w, x[t:t + 1], resid[t:t + 1], graph=True)
                compare_layer(cfg, w, x[t:t + 1], resid[t:t + 1], gpu, f"{name} L{li} t{t}")
        else:
            gpu, _ = run_gpu_layer(cfg, w, x, resid, graph=True)
            compare_layer(cfg, w, x, resid, gpu, f"{name} L{li} T={T}")


@pytest.mark.parametrize("kw", [dict(), dict(bits_gate_up=8, bits_down=8),
                                dict(x_dtype=mi.F16, router_dtype=mi.F16, resid_dtype=mi.F16),
                                dict(d_in=4096, d_ff=1408)],
                         ids=["q4-bf16", "q8", "q4-f16x", "wide"])
def test_many_tokens_per_expert(kw):
    """32 tokens over 4 experts: each expert's token list is cut into several work items."""
    cfg = small_cfg(n_experts=4, top_k=2, **kw)
    say(f"case 32 tokens over 4 experts {kw}")
    w = mi.gen_layer_weights(cfg, 6, threads=8)
    x, resid = margin_tokens(cfg, 6, w, 32)
    gpu, _ = run_gpu_layer(cfg, w, x, resid, graph=True)
    compare_layer(cfg, w, x, resid, gpu, f"32 tokens over 4 experts {kw}")


# ------------------------------------------------------------- edge cases
def test_out_of_range_ids_give_zero_rows():
    from quantized_moe_decode_amd.layer import layer_from_host, tensor_from_encoded
    import quantized_moe_decode_amd as q
    for T in (1, 2):
        cfg = small_cfg(top_k=3)
        say(f"case out-of-range ids T={T}")
        w = mi.gen_layer_weights(cfg, 3, threads=4)
        layer = layer_from_host(cfg, w, DEV, n_tokens=T)
        x, _ = mi.gen_tokens(cfg, 3, T)
        xd = tensor_from_encoded(x, cfg.x_dtype, DEV)
        ids = np.tile(np.array([2, -1, cfg.n_experts], np.int32), (T, 1))
        layer.ids.copy_(torch.from_numpy(ids))
        layer.scores.fill_(1.0)
        layer.act.fill_(7.0)
        layer.partial.fill_(7.0)
        q.moe_decode_expert_ffn(xd, layer.gate, layer.up, layer.down, layer.ids, layer.scores,
                                layer.act, layer.partial, layer.ffn_ws)
        torch.cuda.synchronize()
        act, part = layer.act.cpu().numpy(), layer.partial.cpu().numpy()
        assert np.all(act[:, 1:] == 0) and np.all(part[:, 1:] == 0)
        ref = oracle.expert_ffn(x, cfg.x_dtype, w["gate"], w["up"], w["down"], ids, np.ones((T, 3)))
        for t in range(T):
            assert np.max(np.abs(part[t, 0] - ref["partial"][t, 0])) <= 2e-3 * np.max(np.abs(ref["partial"][t, 0]))


@pytest.mark.parametrize("ids_rows", [
    # an expert repeated inside a token (the ranks then come from the direct count)
    [[5, 5, 2, 9], [2, 5, 5, 5], [9, 1, 1, 0]],
    # distinct per token, shared across tokens, plus out-of-range ids twice in one token
    [[5, 2, -1, 9], [2, 5, 7, 40], [-3, 9, 5, 99]],
    # more than four tokens on one expert (several work items for it)
    [[3, 0, 1, 2], [3, 4, 5, 6], [3, 7, 0, 1], [3, 2, 4, 5], [3, 6, 7, 0], [3, 1, 2, 4]],
], ids=["repeat-in-token", "shared-and-out-of-range", "six-tokens-one-expert"])
def test_multi_token_ids_outside_topk(ids_rows):
    """The multi-token expert FFN with id patterns routing never produces: every
    (token, slot) row matches the oracle's, in its own place."""
    from quantized_moe_decode_amd.layer import layer_from_host, tensor_from_encoded
    import quantized_moe_decode_amd as q
    ids = np.array(ids_rows, np.int32)
    T, K = ids.shape
    cfg = small_cfg(top_k=K, n_experts=10)
    say(f"case multi-token ids {ids.tolist()}")
    w = mi.gen_layer_weights(cfg, 8, threads=4)
    layer = layer_from_host(cfg, w, DEV, n_tokens=T)
    x, _ = mi.gen_tokens(cfg, 8, T)
    xd = tensor_from_encoded(x, cfg.x_dtype, DEV)
    sc = np.random.default_rng([8, T]).uniform(0.1, 1.0, (T, K))
    layer.ids.copy_(torch.from_numpy(ids))
    layer.scores.copy_(torch.from_numpy(sc.astype(np.float32)))
    layer.act.fill_(7.0)
    layer.partial.fill_(7.0)
    q.moe_decode_expert_ffn(xd, layer.gate, layer.up, layer.down, layer.ids, layer.scores,
                            layer.act, layer.partial, layer.ffn_ws)
    torch.cuda.synchronize()
    act, part = layer.act.cpu().numpy(), layer.partial.cpu().numpy()
    ref = oracle.expert_ffn(x, cfg.x_dtype, w["gate"], w["up"], w["down"], ids,
                            sc.astype(np.float32).astype(np.float64))
    for t in range(T):
        for k in range(K):
            if not 0 <= ids[t, k] < cfg.n_experts:
                assert np.all(act[t, k] == 0) and np.all(part[t, k] == 0)
                continue
            ra, rp = ref["act"][t, k], ref["partial"][t, k]
            assert np.max(np.abs(act[t, k] - ra)) <= 2e-3 * np.max(np.abs(ra)), (t, k)
            assert np.max(np.abs(part[t, k] - rp)) <= 2e-3 * np.max(np.abs(rp)), (t, k)


def test_exact_tie_prefers_lower_index():
    """Duplicate router rows give bit-identical fp32 logits; the lower expert id wins."""
    import quantized_moe_decode_amd as q
    say("case router tie")
    E, d_in = 16, 256
    wr = np.zeros((E, d_in), np.float32)
    r = np.random.default_rng([5, 5]).standard_normal(d_in).astype(np.float32)
    wr[11] = wr[4] = r * 0.05
    wr[9] = r * 0.04
    wr[2] = wr[13] = r * 0.03
    x = r.copy()
    xd = torch.from_numpy(x[None]).to(DEV)
    wd = torch.from_numpy(wr).to(DEV)
    ids = torch.zeros(1, 4, dtype=torch.int32, device=DEV)
    sc = torch.zeros(1, 4, device=DEV)
    ws = torch.zeros(q.route_workspace_bytes(1, E), dtype=torch.uint8, device=DEV)
    q.moe_decode_route(xd, wd, 4, True, ids, sc, ws)
    torch.cuda.synchronize()
    assert ids.cpu().numpy().tolist() == [[4, 11, 9, 2]]
    s = sc.cpu().numpy()[0]
    assert s[0] == s[1]
    # the workspace carries the launch epoch from call to call: the same
    # workspace serves the next calls unchanged, and no wait ran out
    for call in range(3):
        ids2 = torch.full_like(ids, -7)
        q.moe_decode_route(xd, wd, 4, True, ids2, sc, ws)
        torch.cuda.synchronize()
        assert ids2.cpu().numpy().tolist() == [[4, 11, 9, 2]], call
    assert q.workspace_status(ws) == q.MOE_OK
    epoch = int(ws[256:260].view(torch.int32).item())
    assert epoch == 4, f"route epoch {epoch} after 4 calls"


def test_many_experts_top32():
    """E = 1024 experts, top-32, 32 tokens: well-separated logits, ids exact."""
    import quantized_moe_decode_amd as q
    say("case E=1024 top-32 T=32")
    E, d_in, T, K = 1024, 64, 32, 32
    rng = np.random.default_rng([6, 6])
    wr = np.zeros((E, d_in), np.float32)
    perm = rng.permutation(E)
    wr[perm, 0] = np.arange(E) * 0.01          # logit of expert perm[i] is 0.01 * i * x0
    x = np.zeros((T, d_in), np.float32)
    x[:, 0] = 1.0 + 0.01 * np.arange(T)
    xd, wd = torch.from_numpy(x).to(DEV), torch.from_numpy(wr).to(DEV)
    ids = torch.zeros(T, K, dtype=torch.int32, device=DEV)
    sc = torch.zeros(T, K, device=DEV)
    ws = torch.zeros(q.route_workspace_bytes(T, E), dtype=torch.uint8, device=DEV)
    q.moe_decode_route(xd, wd, K, True, ids, sc, ws)
    torch.cuda.synchronize()
    ref = oracle.route(x, mi.F32, wr, mi.F32, K, True)
    assert np.array_equal(ids.cpu().numpy(), ref["ids"])
    assert np.max(np.abs(sc.cpu().numpy() - ref["scores"])) <= 1e-5


def test_zero_gate_projection_leaves_residual_exactly():
    cfg = small_cfg(resid_dtype=mi.F32, top_k=2)
    say("case zero gate projection")
    w = mi.gen_layer_weights(cfg, 4, threads=4)
    g = w["gate"]
    zero = mi.encode(np.zeros(g.scales.shape), g.sb_dtype)
    w["gate"] = stack_from_arrays(g.q, zero, zero, g)
    x, resid = mi.gen_tokens(cfg, 4, 2)
    gpu, _ = run_gpu_layer(cfg, w, x, resid)
    assert np.all(gpu["act"] == 0)
    assert np.array_equal(gpu["out"], resid.astype(np.float32))


def test_down_linearity_is_exact():
    """Doubling the down scales and biases doubles every partial bit-exactly on the GPU."""
    cfg = small_cfg(top_k=2, bits_down=6)
    say("case down linearity")
    w = mi.gen_layer_weights(cfg, 5, threads=4)
    x, resid = margin_tokens(cfg, 5, w, 1)
    a, _ = run_gpu_layer(cfg, w, x, resid)
    d = w["down"]
    w2 = dict(w, down=stack_from_arrays(
        d.q, mi.encode(2 * np_decode(d.scales, d.sb_dtype), d.sb_dtype),
        mi.encode(2 * np_decode(d.biases, d.sb_dtype), d.sb_dtype), d))
    b, _ = run_gpu_layer(cfg, w2, x, resid)
    assert np.array_equal(b["partial"], 2 * a["partial"])
    assert np.array_equal(b["act"], a["act"])


def test_repeated_runs_are_bit_identical_and_graph_replays_match():
    cfg = mi.QWEN3
    say("case determinism + graph replays (qwen3 layer 1)")
    w = mi.gen_layer_weights(cfg, 1)
    x, resid = margin_tokens(cfg, 1, w, 1)
    a, layer = run_gpu_layer(cfg, w, x, resid)
    b, _ = run_gpu_layer(cfg, w, x, resid, layer=layer)
    for k in ("ids", "scores", "act", "partial", "out"):
        assert np.array_equal(a[k], b[k]), k
    from quantized_moe_decode_amd.layer import tensor_from_encoded
    xd = tensor_from_encoded(x, cfg.x_dtype, DEV)
    rd = tensor_from_encoded(resid, cfg.resid_dtype, DEV)
    out = torch.zeros(1, cfg.d_in, device=DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        layer.forward(xd, rd, out)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.forward(xd, rd, out)
    for rep in range(4):
        out.fill_(-1.0)
        layer.partial.fill_(3.0)          # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), a["out"]), rep


def test_batch_graph_replays_match_eager():
    """32 tokens (routing, bucketing, the multi-token kernels, tail) captured
    once and replayed four times with eager work on the same buffers between
    the replays: every replay equals the eager result bit for bit."""
    cfg = mi.QWEN3_B32
    say("case graph replays, 32 tokens (qwen3 layer 0)")
    w = mi.gen_layer_weights(cfg, 0)
    x, resid = margin_tokens(cfg, 0, w, 32)
    a, layer = run_gpu_layer(cfg, w, x, resid)
    from quantized_moe_decode_amd.layer import tensor_from_encoded
    xd = tensor_from_encoded(x, cfg.x_dtype, DEV)
    rd = tensor_from_encoded(resid, cfg.resid_dtype, DEV)
    out = torch.zeros(32, cfg.d_in, device=DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        layer.forward(xd, rd, out)
    torch.cuda.current_stream().wait_stream(s)
    assert np.array_equal(out.cpu().numpy(), a["out"])
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.forward(xd, rd, out)
    for rep in range(4):
        out.fill_(-1.0)
        layer.partial.fill_(3.0)          # eager work between replays
        layer.act.fill_(-2.0)
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), a["out"]), rep
