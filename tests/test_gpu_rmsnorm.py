"""The next layer's RMSNorm folded into the tail, on both paths, against the
oracle (oracle.rmsnorm of the oracle's layer output): the fused layer launch
(moe_decode_layer_rmsnorm) and the three-call tail (moe_decode_tail_rmsnorm),
at small shapes whose tail tiles are ragged and at full size, for 1, 3 and 32
tokens; repeated launches give the same bits.  Every case prints its name
before it runs."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from gpu_cases import DEV, compare_layer, margin_tokens, say, small_cfg
from helpers import rel_err

pytestmark = pytest.mark.gpu
TOL = 2e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_moe_decode_amd  # noqa: F401
    yield


def run_norm(cfg, w, x, resid, fused, eps=None, reps=1, fold=True):
    """The layer with the RMSNorm folded in; returns out, normed, ids, error state."""
    import quantized_moe_decode_amd as q
    from quantized_moe_decode_amd.layer import layer_from_host, tensor_from_encoded
    T = x.shape[0]
    layer = layer_from_host(cfg, w, DEV, n_tokens=T)
    nw = mi.gen_norm_weight(cfg, 0)
    layer.set_next_norm(tensor_from_encoded(nw, mi.BF16, DEV), cfg.norm_eps if eps is None else eps, fold=fold)
    xd = tensor_from_encoded(x, cfg.x_dtype, DEV)
    rd = tensor_from_encoded(resid, cfg.resid_dtype, DEV)
    out = torch.zeros(T, cfg.d_in, device=DEV)
    results = []
    for _ in range(reps):
        layer.normed.fill_(-1.0)
        (layer.forward_fused if fused else layer.forward)(xd, rd, out)
        torch.cuda.synchronize()
        results.append((out.cpu().numpy().copy(), layer.normed.cpu().numpy().copy()))
    err = (layer.fused_error_word() if fused else
           int((fold and q.workspace_status(layer.tail_ws) != q.MOE_OK) or
               q.workspace_status(layer.route_ws) != q.MOE_OK))
    gpu = dict(ids=layer.ids.cpu().numpy(), scores=layer.scores.cpu().numpy(), act=None, partial=None,
               out=results[-1][0], error_word=err)
    if layer.shared_gate is not None:
        gpu["gate"] = layer.shared_gate.cpu().numpy()
    return gpu, results, nw


def check(cfg, w, x, resid, fused, label, eps=None, reps=2, fold=True):
    gpu, results, nw = run_norm(cfg, w, x, resid, fused, eps, reps, fold)
    ref = oracle.layer(cfg, w, x, resid)
    compare_layer(cfg, w, x, resid, gpu, label, ref=ref)
    want = oracle.rmsnorm(ref["out"], nw, mi.BF16, cfg.norm_eps if eps is None else eps)
    e = rel_err(results[-1][1], want)
    say(f"  {label}: normed relative error {e:.2e}")
    assert e <= TOL, f"{label}: normed relative error {e}"
    for o, n in results[1:]:
        assert np.array_equal(o, results[0][0]) and np.array_equal(n, results[0][1]), "runs differ"


@pytest.mark.parametrize("kw", [dict(), dict(d_in=1088, d_ff=704, n_experts=9, top_k=4, bits_down=6),
                                dict(d_in=64, d_ff=64, n_experts=3, top_k=1),
                                dict(n_shared=1, d_ff_shared=256, shared_gate=True),
                                dict(d_in=2048, d_ff=768, n_experts=10, top_k=8)],
                         ids=["base", "ragged-6bit", "smallest", "shared", "eight-slots"])
@pytest.mark.parametrize("fused", [True, False], ids=["fused", "three-call"])
def test_small_layers_with_rmsnorm(kw, fused):
    cfg = small_cfg(**kw)
    say(f"case rmsnorm {'fused' if fused else 'three-call'} {kw}")
    w = mi.gen_layer_weights(cfg, 0, threads=4)
    x, resid = margin_tokens(cfg, 0, w, 1)
    check(cfg, w, x, resid, fused, f"rmsnorm {kw}")


@pytest.mark.parametrize("T", [3, 32])
def test_three_call_tokens_with_rmsnorm(T):
    cfg = small_cfg(d_in=512, d_ff=384, n_experts=12, top_k=4)
    say(f"case rmsnorm three-call T={T}")
    w = mi.gen_layer_weights(cfg, 1, threads=4)
    x, resid = margin_tokens(cfg, 1, w, T)
    check(cfg, w, x, resid, False, f"rmsnorm three-call T={T}")


@pytest.mark.parametrize("name", ["qwen3_30b_a3b_moe", "dots_llm1_mixed_bit", "qwen1.5_moe_a2.7b"])
def test_full_size_with_rmsnorm(name):
    cfg = mi.CONFIGS[name]
    w = mi.gen_layer_weights(cfg, 0)
    x, resid = margin_tokens(cfg, 0, w, 1)
    for fused in (True, False):
        say(f"case rmsnorm {name} {'fused' if fused else 'three-call'}")
        check(cfg, w, x, resid, fused, f"rmsnorm {name} fused={fused}")


def test_rmsnorm_eps_dominates():
    """A large eps (1e4 against a mean square of order 1) shrinks the output by
    1/sqrt(ms + eps): the GPU must add eps inside the root, as the oracle does."""
    cfg = small_cfg()
    say("case rmsnorm eps 1e4")
    w = mi.gen_layer_weights(cfg, 2, threads=4)
    x, resid = margin_tokens(cfg, 2, w, 1)
    for fused in (True, False):
        check(cfg, w, x, resid, fused, f"rmsnorm eps=1e4 fused={fused}", eps=1e4)


@pytest.mark.parametrize("T", [1, 32])
def test_separate_rmsnorm_launch(T):
    """moe_decode_rmsnorm (one workgroup per token) after the layer: the
    separate dispatch the folded forms are measured against."""
    cfg = small_cfg(d_in=1024, d_ff=256, n_experts=8, top_k=2)
    say(f"case separate rmsnorm T={T}")
    w = mi.gen_layer_weights(cfg, 3, threads=4)
    x, resid = margin_tokens(cfg, 3, w, T)
    if T == 1:
        check(cfg, w, x, resid, True, "separate rmsnorm fused layer", fold=False)
    check(cfg, w, x, resid, False, f"separate rmsnorm three-call T={T}", fold=False)
