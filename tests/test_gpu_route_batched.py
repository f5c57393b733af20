"""Routing of many tokens (more than 32, bf16 x, router and gate vector): the
logits as one matrix product on the matrix cores, then one selection
workgroup per token.  Against the oracle: expert ids exact (tokens drawn with
the routing margin, or logits separated by construction), scores and the
shared gate within 1e-5; exact ties to the lower id; the tagged single-launch
routing keeps working on the same workspace afterwards.  Every case prints
its name first."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from gpu_cases import DEV, SCORE_TOL, margin_tokens, say, small_cfg

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_moe_decode_amd  # noqa: F401
    yield


def bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(DEV).to(torch.bfloat16)


def route_gpu(x, wr, K, renorm, wg=None, ws=None):
    import quantized_moe_decode_amd as q
    T, E = x.shape[0], wr.shape[0]
    ids = torch.full((T, K), -7, dtype=torch.int32, device=DEV)
    sc = torch.full((T, K), -7.0, device=DEV)
    gate = torch.full((T,), -7.0, device=DEV) if wg is not None else None
    if ws is None:
        ws = torch.zeros(q.route_workspace_bytes(T, E), dtype=torch.uint8, device=DEV)
    q.moe_decode_route(x, wr, K, renorm, ids, sc, ws, wg, gate)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), sc.cpu().numpy(), None if gate is None else gate.cpu().numpy(), ws


@pytest.mark.parametrize("kw,T", [(dict(n_experts=12, top_k=4), 33), (dict(n_experts=12, top_k=4), 256),
                                  (dict(n_shared=1, d_ff_shared=256, shared_gate=True), 40),
                                  (dict(d_in=1088, n_experts=70, top_k=6, renormalize=False), 100)],
                         ids=["E12-33", "E12-256", "shared-gate-40", "ragged-E70-100"])
def test_batched_route_matches_oracle(kw, T):
    from quantized_moe_decode_amd.layer import tensor_from_encoded
    cfg = small_cfg(**kw)
    say(f"case batched route {kw} T={T}")
    w = mi.gen_layer_weights(cfg, 3, threads=4)
    x, _ = margin_tokens(cfg, 3, w, T)
    xd = tensor_from_encoded(x, cfg.x_dtype, DEV)
    wr = tensor_from_encoded(w["router"], cfg.router_dtype, DEV)
    wg = tensor_from_encoded(w["shared_gate_w"], "bf16", DEV) if cfg.shared_gate else None
    ids, sc, gate, _ = route_gpu(xd, wr, cfg.top_k, cfg.renormalize, wg)
    ref = oracle.route(x, cfg.x_dtype, w["router"], cfg.router_dtype, cfg.top_k, cfg.renormalize,
                       w["shared_gate_w"] if cfg.shared_gate else None)
    assert np.array_equal(ids, ref["ids"])
    assert np.max(np.abs(sc - ref["scores"])) <= SCORE_TOL
    if cfg.shared_gate:
        assert np.max(np.abs(gate - ref["gate"])) <= SCORE_TOL


def test_batched_route_qwen3_shape_1024_tokens():
    from quantized_moe_decode_amd.layer import tensor_from_encoded
    cfg = mi.QWEN3
    say("case batched route qwen3 T=1024")
    w = mi.gen_layer_weights(cfg, 0)
    T = 1024
    x, _ = margin_tokens(cfg, 0, w, T)
    ids, sc, _, _ = route_gpu(tensor_from_encoded(x, cfg.x_dtype, DEV),
                              tensor_from_encoded(w["router"], cfg.router_dtype, DEV), cfg.top_k, True)
    ref = oracle.route(x, cfg.x_dtype, w["router"], cfg.router_dtype, cfg.top_k, True)
    assert np.array_equal(ids, ref["ids"])
    assert np.max(np.abs(sc - ref["scores"])) <= SCORE_TOL


def test_batched_route_ties_top32_and_the_tagged_path_after_it():
    """E = 1024, top-32, 48 tokens, duplicate router rows (bit-identical logits:
    the lower id first); then 8 tokens of the same workspace through the
    tagged single-launch routing, whose words the batched call overwrote."""
    E, d_in, T, K = 1024, 64, 48, 32
    say("case batched route E=1024 top-32 ties T=48, then tagged T=8")
    rng = np.random.default_rng([7, 7])
    wr = np.zeros((E, d_in), np.float32)
    perm = rng.permutation(E)
    i = np.arange(E)
    wr[perm, 0] = (1.0 + (i % 128) / 128.0) * 2.0 ** (i // 128 - 8)   # distinct, increasing, exact in bf16
    wr[perm[-3]] = wr[perm[-1]]                                  # a tie at the top
    x = np.zeros((T, d_in), np.float32)
    x[:, 0] = 1.0 + 0.0078125 * np.arange(T)
    ids, sc, _, ws = route_gpu(bf16(x), bf16(wr), K, True)
    ref = oracle.route(x, mi.F32, wr, mi.F32, K, True)
    assert np.array_equal(ids, ref["ids"])
    lo, hi = sorted((perm[-3], perm[-1]))
    assert all(row[0] == lo and row[1] == hi for row in ids), "tie not broken to the lower id"
    assert np.max(np.abs(sc - ref["scores"])) <= SCORE_TOL
    import quantized_moe_decode_amd as q
    for call in range(2):
        x8 = x[:8] * (1.0 + call)
        ids8, sc8, _, _ = route_gpu(bf16(x8), bf16(wr), K, True, ws=ws[:q.route_workspace_bytes(8, E)])
        ref8 = oracle.route(x8, mi.F32, wr, mi.F32, K, True)
        assert np.array_equal(ids8, ref8["ids"]), call
    assert q.workspace_status(ws) == q.MOE_OK
