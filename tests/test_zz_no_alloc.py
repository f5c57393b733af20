"""moe_decode_expert_ffn_noalloc (the call that takes its workspace from the
library's own device array) against moe_decode_expert_ffn with a caller
workspace, through the C ABI: two calls in a row, the second with a smaller
input, each bit-identical to the workspace call and within the bar of the
oracle.  Every case prints its name before it runs."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from gpu_cases import DEV, say, small_cfg

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_moe_decode_amd  # noqa: F401
    yield


def _run(cfg, T, seed_layer):
    import quantized_moe_decode_amd as q
    from quantized_moe_decode_amd.layer import layer_from_host, tensor_from_encoded
    w = mi.gen_layer_weights(cfg, seed_layer, threads=4)
    layer = layer_from_host(cfg, w, DEV, n_tokens=T)
    x, _ = mi.gen_tokens(cfg, seed_layer, T)
    xd = tensor_from_encoded(x, cfg.x_dtype, DEV)
    rng = np.random.default_rng([seed_layer, T])
    ids = np.stack([rng.choice(cfg.n_experts, cfg.top_k, replace=False) for _ in range(T)]).astype(np.int32)
    sc = rng.uniform(0.1, 1.0, (T, cfg.top_k)).astype(np.float32)
    layer.ids.copy_(torch.from_numpy(ids))
    layer.scores.copy_(torch.from_numpy(sc))
    act_a, part_a = torch.full_like(layer.act, 7.0), torch.full_like(layer.partial, 7.0)
    q.moe_decode_expert_ffn(xd, layer.gate, layer.up, layer.down, layer.ids, layer.scores, act_a, part_a,
                            layer.ffn_ws)
    act_b, part_b = torch.full_like(layer.act, -3.0), torch.full_like(layer.partial, -3.0)
    q.moe_decode_expert_ffn_noalloc(xd, layer.gate, layer.up, layer.down, layer.ids, layer.scores, act_b, part_b)
    torch.cuda.synchronize()
    assert torch.equal(act_a, act_b) and torch.equal(part_a, part_b), "noalloc call differs from the workspace call"
    ref = oracle.expert_ffn(x, cfg.x_dtype, w["gate"], w["up"], w["down"], ids, sc.astype(np.float64))
    pb = part_b.cpu().numpy()
    for t in range(T):
        for k in range(cfg.top_k):
            rp = ref["partial"][t, k]
            assert np.max(np.abs(pb[t, k] - rp)) <= 2e-3 * np.max(np.abs(rp)), (t, k)


def test_noalloc_matches_workspace_call_twice_shrinking():
    import quantized_moe_decode_amd as q
    assert q.expert_ffn_noalloc_max_bytes() >= q.expert_ffn_workspace_bytes(32, 32, 1024)
    big = small_cfg(d_in=512, d_ff=384, n_experts=40, top_k=6)
    say("case noalloc: 32 tokens, 40 experts, top-6")
    _run(big, 32, 11)
    small = small_cfg(d_in=256, d_ff=128, n_experts=6, top_k=2, bits_down=8)
    say("case noalloc: then 3 tokens, 6 experts, top-2 (smaller)")
    _run(small, 3, 12)


def test_noalloc_rejects_out_of_limit_sizes():
    import quantized_moe_decode_amd as q
    cfg = small_cfg()
    say("case noalloc: 33 tokens rejected")
    from quantized_moe_decode_amd.layer import layer_from_host
    w = mi.gen_layer_weights(cfg, 13, threads=4)
    layer = layer_from_host(cfg, w, DEV, n_tokens=33)
    x = torch.zeros(33, cfg.d_in, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(q.MoeError) as e:
        q.moe_decode_expert_ffn_noalloc(x, layer.gate, layer.up, layer.down, layer.ids, layer.scores,
                                        layer.act, layer.partial)
    assert e.value.status == q.MOE_EINVAL
