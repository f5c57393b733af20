"""Activations outside fp16's normal range, through every path that stages act
as fp16 for a packed fp16 dot of the down projection (the fused kernel-B
units, with 4-, 6- and 8-bit codes, and the multi-token kernels, 4-bit),
against the oracle.

The gate and up scales and biases are multiplied by 2^8 (act around 2.6e5,
past fp16's largest finite value 65504) or by 2^-10 (act around 4e-6, where
fp16 has only subnormals); both multiplications are exact in bf16.  Each case
first checks with the oracle that act really is in that range, so the test
cannot pass by missing it.  The residual is zero, so the output is the MoE
term itself: next to a residual of order 1, an fp32 output could not resolve
a MoE term of order 1e-5 to the bar.  Every case prints its name before it
runs.
"""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from gpu_cases import compare_layer, margin_tokens, run_gpu_layer, say, small_cfg
from helpers import np_decode, stack_from_arrays

pytestmark = pytest.mark.gpu

FP16_MAX = 65504.0
FP16_MIN_NORMAL = 2.0 ** -14


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_moe_decode_amd  # noqa: F401
    yield


def scale_gate_up(w, log2f):
    """Gate and up scales and biases times 2^log2f (exact for bf16 scales in range)."""
    out = dict(w)
    for p in ("gate", "up"):
        st = w[p]
        f = 2.0 ** log2f
        out[p] = stack_from_arrays(st.q, mi.encode(f * np_decode(st.scales, st.sb_dtype), st.sb_dtype),
                                   mi.encode(f * np_decode(st.biases, st.sb_dtype), st.sb_dtype), st)
        back = np_decode(out[p].scales, st.sb_dtype) / f
        assert np.array_equal(back, np_decode(st.scales, st.sb_dtype)), "scaling not exact"
    return out


def check_range(cfg, w, x, log2f):
    ref = oracle.layer(cfg, w, x, np.zeros_like(x))
    amax = float(np.max(np.abs(ref["ffn"]["act"])))
    if log2f > 0:
        assert amax > FP16_MAX, f"act max {amax} does not exceed fp16's range"
    else:
        assert amax < FP16_MIN_NORMAL, f"act max {amax} is not below fp16's normal range"
    return amax


@pytest.mark.parametrize("log2f", [8, -10], ids=["large", "tiny"])
@pytest.mark.parametrize("path,T", [("fused", 1), ("three-call", 1), ("three-call", 3), ("three-call", 32)])
def test_act_outside_fp16_range(path, T, log2f):
    cfg = small_cfg(d_in=1024, d_ff=768, n_experts=8, top_k=4)
    say(f"case act range 2^{log2f} {path} T={T}")
    w = scale_gate_up(mi.gen_layer_weights(cfg, 7, threads=4), log2f)
    x, resid = margin_tokens(cfg, 7, w, T)
    resid = np.zeros_like(resid)
    amax = check_range(cfg, w, x, log2f)
    say(f"  oracle act max {amax:.3e}")
    if path == "fused":
        gpu, layer = run_gpu_layer(cfg, w, x, resid, fused=True)
        assert not np.any(layer.fused_ws.cpu().numpy()[:4]), "error word set"
    else:
        gpu, _ = run_gpu_layer(cfg, w, x, resid)
    compare_layer(cfg, w, x, resid, gpu, f"act range 2^{log2f} {path} T={T}")


@pytest.mark.parametrize("log2f", [8, -10], ids=["large", "tiny"])
@pytest.mark.parametrize("bits_down", [6, 8])
def test_act_outside_fp16_range_fused_6_8_bit_down(bits_down, log2f):
    cfg = small_cfg(d_in=1024, d_ff=768, n_experts=8, top_k=4, bits_down=bits_down)
    say(f"case act range 2^{log2f} fused {bits_down}-bit down")
    w = scale_gate_up(mi.gen_layer_weights(cfg, 7, threads=4), log2f)
    x, resid = margin_tokens(cfg, 7, w, 1)
    resid = np.zeros_like(resid)
    amax = check_range(cfg, w, x, log2f)
    say(f"  oracle act max {amax:.3e}")
    gpu, layer = run_gpu_layer(cfg, w, x, resid, fused=True)
    assert not np.any(layer.fused_ws.cpu().numpy()[:4]), "error word set"
    compare_layer(cfg, w, x, resid, gpu, f"act range 2^{log2f} fused {bits_down}-bit down")


def test_act_outside_fp16_range_full_size_fused():
    """The Qwen3-30B-A3B-shaped layer with act past fp16's range, fused launch."""
    cfg = mi.QWEN3
    say("case act range 2^8 qwen3 layer 2 fused")
    w = scale_gate_up(mi.gen_layer_weights(cfg, 2), 8)
    x, resid = margin_tokens(cfg, 2, w, 1)
    resid = np.zeros_like(resid)
    check_range(cfg, w, x, 8)
    gpu, layer = run_gpu_layer(cfg, w, x, resid, graph=True, fused=True)
    compare_layer(cfg, w, x, resid, gpu, "act range 2^8 qwen3 fused")
