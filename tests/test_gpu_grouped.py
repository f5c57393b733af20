"""The grouped (matrix-core) expert FFN, moe_decode_expert_ffn_grouped, against
the oracle's expert FFN on the same inputs: act and partial of every checked
(token, slot) pair within 2e-3 of the pair's row infinity norm.  Cases: tiny
and ragged shapes (rows not a multiple of the 64-row tiles of a workgroup, an
expert holding 15, 16, 17 or all pairs, so work items end full and part-full),
out-of-range ids (their rows must be zero), fp16 scales, activations past
fp16's range (the per-pair staging factor), the full Qwen3-30B-A3B-shaped
layer at 256 tokens (a sample of the tokens checked), repeated calls bit for
bit, and unsupported formats rejected.  Every case prints its name first."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from gpu_cases import DEV, say, small_cfg
from helpers import rel_err

pytestmark = pytest.mark.gpu
TOL = 2e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_moe_decode_amd  # noqa: F401
    yield


def random_routing(T, K, E, seed, skew=None):
    """ids [T, K] (distinct per token) and scores [T, K]; skew 'one' puts every
    token on experts 0..K-1."""
    rng = np.random.default_rng(seed)
    if skew == "one":
        ids = np.tile(np.arange(K, dtype=np.int32), (T, 1))
    else:
        ids = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    scores = rng.uniform(0.05, 1.0, (T, K)).astype(np.float32)
    return ids, scores


def run_grouped(cfg, w, x, ids, scores):
    import quantized_moe_decode_amd as q
    from quantized_moe_decode_amd.layer import stack_to_device, tensor_from_encoded
    T, K = ids.shape
    g, u, d = (stack_to_device(w[p], DEV) for p in ("gate", "up", "down"))
    xd = tensor_from_encoded(x, cfg.x_dtype, DEV)
    idd = torch.from_numpy(ids).to(DEV)
    scd = torch.from_numpy(scores).to(DEV)
    act = torch.full((T, K, cfg.d_ff), -7.0, device=DEV)
    part = torch.full((T, K, cfg.d_in), -7.0, device=DEV)
    ws = torch.zeros(q.expert_ffn_grouped_workspace_bytes(T, K, cfg.n_experts, cfg.d_ff), device=DEV, dtype=torch.uint8)
    q.moe_decode_expert_ffn_grouped(xd, g, u, d, idd, scd, act, part, ws)
    torch.cuda.synchronize()
    assert q.workspace_status(ws) == q.MOE_OK, "a wait inside the grouped call ran out"
    return act.cpu().numpy(), part.cpu().numpy(), (xd, g, u, d, idd, scd, act, part, ws)


def check(cfg, w, x, ids, scores, label, tokens=None):
    act, part, _ = run_grouped(cfg, w, x, ids, scores)
    tokens = np.arange(ids.shape[0]) if tokens is None else np.asarray(tokens)
    ref = oracle.expert_ffn(x[tokens], cfg.x_dtype, w["gate"], w["up"], w["down"], ids[tokens], scores[tokens])
    worst_a = worst_p = 0.0
    for i, t in enumerate(tokens):
        for k in range(ids.shape[1]):
            worst_a = max(worst_a, rel_err(act[t, k], ref["act"][i, k]))
            worst_p = max(worst_p, rel_err(part[t, k], ref["partial"][i, k]))
    say(f"  {label}: worst relative error act {worst_a:.2e}, partial {worst_p:.2e}")
    assert worst_a <= TOL and worst_p <= TOL, label
    return act, part


SHAPES = [dict(d_in=256, d_ff=192, n_experts=6, top_k=2),
          dict(d_in=1088, d_ff=704, n_experts=9, top_k=4),
          dict(d_in=64, d_ff=64, n_experts=3, top_k=1),
          dict(d_in=512, d_ff=384, n_experts=12, top_k=8, sb_dtype=mi.F16)]


@pytest.mark.parametrize("T", [1, 3, 17, 64])
@pytest.mark.parametrize("kw", SHAPES, ids=["small", "ragged", "smallest", "eight-slots-f16-scales"])
def test_grouped_small(kw, T):
    cfg = small_cfg(**kw)
    say(f"case grouped {kw} T={T}")
    w = mi.gen_layer_weights(cfg, 0, threads=4)
    x, _ = mi.gen_tokens(cfg, 0, T)
    ids, scores = random_routing(T, cfg.top_k, cfg.n_experts, seed=T)
    check(cfg, w, x, ids, scores, f"grouped {kw} T={T}")


@pytest.mark.parametrize("T", [15, 16, 17, 48, 150])
def test_grouped_one_expert_takes_every_token(T):
    """Every token on experts 0..K-1: each expert's list is cut into work items
    of 16, 32 or 64 pairs (by the average pairs per expert), the last one
    part-full or full."""
    cfg = small_cfg(d_in=512, d_ff=384, n_experts=6, top_k=2)
    say(f"case grouped skew T={T}")
    w = mi.gen_layer_weights(cfg, 1, threads=4)
    x, _ = mi.gen_tokens(cfg, 1, T)
    ids, scores = random_routing(T, cfg.top_k, cfg.n_experts, seed=100 + T, skew="one")
    check(cfg, w, x, ids, scores, f"grouped skew T={T}")


def test_grouped_out_of_range_ids_give_zero_rows():
    cfg = small_cfg(d_in=256, d_ff=192, n_experts=6, top_k=3)
    say("case grouped out-of-range ids")
    w = mi.gen_layer_weights(cfg, 2, threads=4)
    T = 20
    x, _ = mi.gen_tokens(cfg, 2, T)
    ids, scores = random_routing(T, cfg.top_k, cfg.n_experts, seed=7)
    ids[::3, 0] = -1
    ids[1::4, 2] = cfg.n_experts
    act, part = check(cfg, w, x, ids, scores, "grouped out-of-range ids")
    bad = (ids < 0) | (ids >= cfg.n_experts)
    assert np.all(act[bad] == 0.0) and np.all(part[bad] == 0.0)


def test_grouped_act_outside_fp16_range():
    """Gate and up scales and biases times 2^8 (exact in bf16): act around 1e5,
    past fp16's largest value, so kernel B's staging factor must fit it."""
    from helpers import np_decode, stack_from_arrays
    cfg = small_cfg(d_in=512, d_ff=384, n_experts=8, top_k=4)
    say("case grouped act range 2^8")
    w = dict(mi.gen_layer_weights(cfg, 3, threads=4))
    for p in ("gate", "up"):
        st = w[p]
        w[p] = stack_from_arrays(st.q, mi.encode(256.0 * np_decode(st.scales, st.sb_dtype), st.sb_dtype),
                                 mi.encode(256.0 * np_decode(st.biases, st.sb_dtype), st.sb_dtype), st)
    T = 24
    x, _ = mi.gen_tokens(cfg, 3, T)
    ids, scores = random_routing(T, cfg.top_k, cfg.n_experts, seed=9)
    act, _ = check(cfg, w, x, ids, scores, "grouped act range")
    assert np.max(np.abs(act)) > 65504.0, "act does not leave fp16's range"


def test_grouped_full_size_256_tokens_and_repeatable():
    """The Qwen3-30B-A3B-shaped layer, 256 tokens x top-8 = 2048 pairs (16 per
    expert on average); 24 tokens checked against the oracle; a second call
    gives the same bits."""
    cfg = mi.QWEN3
    say("case grouped qwen3 T=256")
    w = mi.gen_layer_weights(cfg, 0)
    T = 256
    x, _ = mi.gen_tokens(cfg, 0, T)
    ids, scores = random_routing(T, cfg.top_k, cfg.n_experts, seed=256)
    act, part = check(cfg, w, x, ids, scores, "grouped qwen3 T=256", tokens=np.arange(0, T, 11))
    act2, part2, _ = run_grouped(cfg, w, x, ids, scores)
    assert np.array_equal(act, act2) and np.array_equal(part, part2), "repeated call differs"


def test_grouped_workspace_reused_eager_and_graph_replays():
    """One workspace for many calls: the bucketing launch clears the unit
    counter, the per-item counters and the error word of the one-launch path
    at every call, so eager calls and replays of a captured call (eager work
    between the replays) all give the first call's bits."""
    import quantized_moe_decode_amd as q
    cfg = mi.QWEN3
    say("case grouped workspace reused, eager and graph replays")
    w = mi.gen_layer_weights(cfg, 2)
    T = 64
    x, _ = mi.gen_tokens(cfg, 2, T)
    ids, scores = random_routing(T, cfg.top_k, cfg.n_experts, seed=64)
    act0, part0, args = run_grouped(cfg, w, x, ids, scores)
    xd, g, u, d, idd, scd, act, part, ws = args
    for _ in range(5):
        act.fill_(-7.0)
        part.fill_(-7.0)
        q.moe_decode_expert_ffn_grouped(xd, g, u, d, idd, scd, act, part, ws)
    torch.cuda.synchronize()
    assert q.workspace_status(ws) == q.MOE_OK
    assert np.array_equal(act.cpu().numpy(), act0) and np.array_equal(part.cpu().numpy(), part0)
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        q.moe_decode_expert_ffn_grouped(xd, g, u, d, idd, scd, act, part, ws)   # warm-up on the capture stream
        stream.synchronize()
        with torch.cuda.graph(graph, stream=stream):
            q.moe_decode_expert_ffn_grouped(xd, g, u, d, idd, scd, act, part, ws)
    for rep in range(3):
        act.fill_(-7.0)
        part.fill_(-7.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert q.workspace_status(ws) == q.MOE_OK, f"replay {rep}: a wait ran out"
        assert np.array_equal(act.cpu().numpy(), act0), f"replay {rep}: act differs"
        assert np.array_equal(part.cpu().numpy(), part0), f"replay {rep}: partial differs"


def test_grouped_full_size_1024_tokens():
    """1024 tokens x top-8 on the Qwen3-30B-A3B-shaped layer: 64 pairs per
    expert on average, the 64-pair work items; 16 tokens checked."""
    cfg = mi.QWEN3
    say("case grouped qwen3 T=1024")
    w = mi.gen_layer_weights(cfg, 1)
    T = 1024
    x, _ = mi.gen_tokens(cfg, 1, T)
    ids, scores = random_routing(T, cfg.top_k, cfg.n_experts, seed=1024)
    check(cfg, w, x, ids, scores, "grouped qwen3 T=1024", tokens=np.arange(5, T, 67))


def test_grouped_resident_down_many_items_ragged_row_blocks():
    """512 tokens x top-4 on 9 experts (64 work items of 32 pairs) in the
    one-launch path: each down unit keeps act resident in LDS and takes two
    row blocks; d_in 1088 has 9 row blocks, so the last unit of an item has
    one."""
    cfg = small_cfg(d_in=1088, d_ff=704, n_experts=9, top_k=4)
    say("case grouped resident down, 4 row blocks per workgroup, ragged")
    w = mi.gen_layer_weights(cfg, 5, threads=4)
    T = 512
    x, _ = mi.gen_tokens(cfg, 5, T)
    ids, scores = random_routing(T, cfg.top_k, cfg.n_experts, seed=512)
    check(cfg, w, x, ids, scores, "grouped resident ragged", tokens=np.arange(0, T, 9))


def test_grouped_chunked_down_when_act_does_not_fit():
    """d_ff 1408 with 32-pair items: act (89 KB as fp16) does not fit a
    resident down unit's LDS, so the call takes two launches, gate/up and the
    chunked down kernel."""
    cfg = small_cfg(d_in=256, d_ff=1408, n_experts=4, top_k=2)
    say("case grouped chunked down (d_ff 1408)")
    w = mi.gen_layer_weights(cfg, 6, threads=4)
    T = 64
    x, _ = mi.gen_tokens(cfg, 6, T)
    ids, scores = random_routing(T, cfg.top_k, cfg.n_experts, seed=64)
    check(cfg, w, x, ids, scores, "grouped chunked down")


def test_grouped_rejects_unsupported_formats():
    import quantized_moe_decode_amd as q
    cfg = small_cfg(d_in=256, d_ff=192, n_experts=6, top_k=2, bits_down=8)
    say("case grouped rejects 8-bit down")
    w = mi.gen_layer_weights(cfg, 4, threads=4)
    x, _ = mi.gen_tokens(cfg, 4, 4)
    ids, scores = random_routing(4, 2, 6, seed=1)
    with pytest.raises(q.MoeError) as ei:
        run_grouped(cfg, w, x, ids, scores)
    assert ei.value.status == q.MOE_EUNSUPPORTED


def _layer_case(cfg, seed, T, check_tokens, label, grouped=None):
    """route -> grouped expert FFN (routed and shared) -> tail for T tokens on
    the GPU, checked against the oracle's layer on `check_tokens`."""
    from gpu_cases import compare_layer, margin_tokens, run_gpu_layer
    from quantized_moe_decode_amd.layer import layer_from_host
    w = mi.gen_layer_weights(cfg, seed, threads=8)
    x, resid = margin_tokens(cfg, seed, w, T)
    layer = layer_from_host(cfg, w, DEV, n_tokens=T, grouped=grouped)
    assert layer.grouped
    gpu, _ = run_gpu_layer(cfg, w, x, resid, layer=layer)
    sel = np.asarray(check_tokens)
    sub = {k: (v[sel] if isinstance(v, np.ndarray) and v.shape[:1] == (T,) else v) for k, v in gpu.items()}
    compare_layer(cfg, w, x[sel], resid[sel], sub, label)


@pytest.mark.parametrize("kw,T", [(dict(d_in=512, d_ff=384, n_experts=12, top_k=4), 48),
                                  (dict(n_shared=1, d_ff_shared=256, shared_gate=True), 40),
                                  (dict(d_in=1088, d_ff=704, n_experts=9, top_k=4), 33)],
                         ids=["48-tokens", "shared-40-tokens", "ragged-33-tokens"])
def test_grouped_layer_above_the_decode_limit(kw, T):
    """DecodeLayer with more than 32 tokens takes the grouped path; route and
    tail run at the same token count."""
    cfg = small_cfg(**kw)
    say(f"case grouped layer {kw} T={T}")
    _layer_case(cfg, 5, T, np.arange(T), f"grouped layer T={T}")


@pytest.mark.parametrize("T", [1, 8])
def test_grouped_layer_forced_at_decode_sizes(T):
    cfg = small_cfg(d_in=512, d_ff=384, n_experts=12, top_k=4)
    say(f"case grouped layer forced T={T}")
    _layer_case(cfg, 6, T, np.arange(T), f"grouped forced T={T}", grouped=True)


def test_grouped_layer_qwen3_256_tokens():
    cfg = mi.QWEN3
    say("case grouped layer qwen3 T=256")
    _layer_case(cfg, 0, 256, np.arange(3, 256, 13), "grouped layer qwen3 T=256")
