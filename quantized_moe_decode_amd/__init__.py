"""Python binding of the MI355X quantized MoE decode library (libmoe_decode.so).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  PyTorch supplies device memory and the stream.  The three calls
mirror the C ABI in ``include/moe_decode.h``:

    moe_decode_route       router logits, softmax, top-k, scores, shared gate
    moe_decode_expert_ffn  kernel A (gate/up + SwiGLU -> act) and kernel B
                           (down * score -> partial) for the selected experts
    moe_decode_tail        out = resid + (sum_k partial_k + shared * gate)

The library must be built (``python quantized_moe_decode_amd/build.py``);
importing this module without it raises ImportError -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import torch  # first: the library then binds to torch's HIP runtime

PKG = os.path.dirname(os.path.abspath(__file__))
# MOE_DECODE_LIB selects another build of the library (the host-sanitizer build in the tests)
LIB_PATH = os.environ.get("MOE_DECODE_LIB") or os.path.join(PKG, "lib", "libmoe_decode.so")

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EHIP, MOE_ETIMEOUT = 0, 1, 2, 3, 4
MOE_WORKSPACE_HEAD_BYTES = 4
MOE_F32, MOE_F16, MOE_BF16 = 0, 1, 2
MOE_MAX_TOKENS, MOE_MAX_GROUPED_TOKENS = 32, 1024     # tokens per call: the decode calls, the grouped call
TORCH_DTYPE_CODE = {torch.float32: MOE_F32, torch.float16: MOE_F16, torch.bfloat16: MOE_BF16}


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)}")
        self.status = status


class CQMat(ctypes.Structure):
    """moe_qmat of the C ABI."""
    _fields_ = [("q", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("biases", ctypes.c_void_p),
                ("n_experts", ctypes.c_int32), ("rows", ctypes.c_int32), ("cols", ctypes.c_int32),
                ("bits", ctypes.c_int32), ("group_size", ctypes.c_int32), ("sb_dtype", ctypes.c_int32)]


class CLayerWeights(ctypes.Structure):
    """moe_layer_weights of the C ABI."""
    _fields_ = [("w_router", ctypes.c_void_p), ("w_router_dtype", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("renormalize", ctypes.c_int32), ("gate", CQMat), ("up", CQMat), ("down", CQMat),
                ("n_shared", ctypes.c_int32), ("shared_gate", CQMat), ("shared_up", CQMat),
                ("shared_down", CQMat), ("w_shared_gate", ctypes.c_void_p)]


class CRMSNorm(ctypes.Structure):
    """moe_rmsnorm of the C ABI."""
    _fields_ = [("weight", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("eps", ctypes.c_float),
                ("normed", ctypes.c_void_p), ("normed_dtype", ctypes.c_int32)]


def _load_library():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python quantized_moe_decode_amd/build.py`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    L.moe_decode_route.argtypes = [vp, i32, i32, i32, vp, i32, i32, i32, i32, vp, i32,
                                   vp, vp, vp, vp, sz, vp]
    L.moe_decode_route.restype = i32
    L.moe_decode_route_workspace_bytes.argtypes = [i32, i32]
    L.moe_decode_route_workspace_bytes.restype = sz
    L.moe_decode_expert_ffn.argtypes = [vp, i32, i32, ctypes.POINTER(CQMat), ctypes.POINTER(CQMat),
                                        ctypes.POINTER(CQMat), vp, vp, i32, vp, vp, vp, sz, vp]
    L.moe_decode_expert_ffn.restype = i32
    L.moe_decode_expert_ffn_workspace_bytes.argtypes = [i32, i32, i32]
    L.moe_decode_expert_ffn_workspace_bytes.restype = sz
    L.moe_decode_expert_ffn_noalloc.argtypes = [vp, i32, i32, ctypes.POINTER(CQMat), ctypes.POINTER(CQMat),
                                                ctypes.POINTER(CQMat), vp, vp, i32, vp, vp, vp]
    L.moe_decode_expert_ffn_noalloc.restype = i32
    L.moe_decode_expert_ffn_noalloc_max_bytes.argtypes = []
    L.moe_decode_expert_ffn_noalloc_max_bytes.restype = sz
    L.moe_decode_expert_ffn_grouped.argtypes = [vp, i32, i32, ctypes.POINTER(CQMat), ctypes.POINTER(CQMat),
                                                ctypes.POINTER(CQMat), vp, vp, i32, vp, vp, vp, sz, vp]
    L.moe_decode_expert_ffn_grouped.restype = i32
    L.moe_decode_expert_ffn_grouped_workspace_bytes.argtypes = [i32, i32, i32, i32]
    L.moe_decode_expert_ffn_grouped_workspace_bytes.restype = sz
    L.moe_decode_gate_up.argtypes = [vp, i32, i32, ctypes.POINTER(CQMat), ctypes.POINTER(CQMat),
                                     vp, i32, vp, vp, sz, vp]
    L.moe_decode_gate_up.restype = i32
    L.moe_decode_down.argtypes = [vp, i32, ctypes.POINTER(CQMat), vp, vp, i32, vp, vp, sz, vp]
    L.moe_decode_down.restype = i32
    L.moe_decode_layer.argtypes = [ctypes.POINTER(CLayerWeights), vp, i32, vp, i32, vp, i32, vp, vp, vp,
                                   vp, sz, vp]
    L.moe_decode_layer.restype = i32
    L.moe_decode_layer_workspace_bytes.argtypes = [ctypes.POINTER(CLayerWeights)]
    L.moe_decode_layer_workspace_bytes.restype = sz
    L.moe_decode_tail.argtypes = [vp, i32, i32, i32, vp, i32, vp, vp, i32, vp, i32, vp]
    L.moe_decode_tail.restype = i32
    L.moe_decode_tail_rmsnorm.argtypes = [vp, i32, i32, i32, vp, i32, vp, vp, i32, vp, i32,
                                          ctypes.POINTER(CRMSNorm), vp, sz, vp]
    L.moe_decode_tail_rmsnorm.restype = i32
    L.moe_decode_tail_rmsnorm_workspace_bytes.argtypes = [i32, i32]
    L.moe_decode_tail_rmsnorm_workspace_bytes.restype = sz
    L.moe_decode_layer_rmsnorm.argtypes = [ctypes.POINTER(CLayerWeights), vp, i32, vp, i32, vp, i32,
                                           ctypes.POINTER(CRMSNorm), vp, vp, vp, vp, sz, vp]
    L.moe_decode_layer_rmsnorm.restype = i32
    L.moe_decode_rmsnorm.argtypes = [vp, i32, i32, i32, ctypes.POINTER(CRMSNorm), vp]
    L.moe_decode_rmsnorm.restype = i32
    L.moe_decode_read_probe.argtypes = [vp, sz, vp, i32, vp]
    L.moe_decode_read_probe.restype = i32
    L.moe_decode_read_probe_blocks.argtypes = [sz]
    L.moe_decode_read_probe_blocks.restype = i32
    L.moe_decode_workspace_status.argtypes = [vp, sz]
    L.moe_decode_workspace_status.restype = i32
    L.moe_decode_status_string.argtypes = [i32]
    L.moe_decode_status_string.restype = ctypes.c_char_p
    L.moe_decode_abi_version.restype = i32
    return L


lib = _load_library()


def status_string(status: int) -> str:
    return lib.moe_decode_status_string(status).decode()


def abi_version() -> int:
    return lib.moe_decode_abi_version()


def _check(status: int, what: str) -> None:
    if status != MOE_OK:
        raise MoeError(status, what)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dt(t: torch.Tensor) -> int:
    try:
        return TORCH_DTYPE_CODE[t.dtype]
    except KeyError:
        raise MoeError(MOE_EUNSUPPORTED, f"dtype {t.dtype}") from None


@dataclasses.dataclass
class QuantStack:
    """A device-resident stack of quantized projection matrices (one per expert).

    q: int32 tensor holding the uint32 words [E, rows, cols*bits/32];
    scales, biases: float16 or bfloat16 tensors [E, rows, cols/64].
    """
    q: torch.Tensor
    scales: torch.Tensor
    biases: torch.Tensor
    rows: int
    cols: int
    bits: int

    @property
    def n_experts(self) -> int:
        return self.q.shape[0]

    def cstruct(self) -> CQMat:
        return CQMat(self.q.data_ptr(), self.scales.data_ptr(), self.biases.data_ptr(),
                     self.n_experts, self.rows, self.cols, self.bits, 64, _dt(self.scales))

    def nbytes(self, experts: int = 1) -> int:
        """Weight bytes of `experts` experts (codes + scales + biases)."""
        per = (self.q[0].numel() * 4 + self.scales[0].numel() * 2 + self.biases[0].numel() * 2)
        return per * experts


def workspace_status(workspace: torch.Tensor) -> int:
    """MOE_OK or MOE_ETIMEOUT for the workspace of moe_decode_route or
    moe_decode_layer (copies its first bytes to the host; synchronises)."""
    head = workspace.view(torch.uint8)[:MOE_WORKSPACE_HEAD_BYTES].cpu().numpy()
    return int(lib.moe_decode_workspace_status(head.ctypes.data_as(ctypes.c_void_p), head.nbytes))


def route_workspace_bytes(n_tokens: int, n_experts: int) -> int:
    return lib.moe_decode_route_workspace_bytes(n_tokens, n_experts)


def expert_ffn_workspace_bytes(n_tokens: int, top_k: int, n_experts: int) -> int:
    return lib.moe_decode_expert_ffn_workspace_bytes(n_tokens, top_k, n_experts)


def moe_decode_route(x: torch.Tensor, w_router: torch.Tensor, top_k: int, renormalize: bool,
                     expert_ids: torch.Tensor, scores: torch.Tensor, workspace: torch.Tensor,
                     w_shared_gate: Optional[torch.Tensor] = None,
                     shared_gate: Optional[torch.Tensor] = None, stream=None) -> None:
    """Routing for x [T, d_in]; writes expert_ids [T, K] int32, scores [T, K] fp32, shared_gate [T]."""
    T, d_in = x.shape
    E = w_router.shape[0]
    st = lib.moe_decode_route(_ptr(x), _dt(x), T, d_in, _ptr(w_router), _dt(w_router), E, top_k,
                              int(bool(renormalize)), _ptr(w_shared_gate),
                              _dt(w_shared_gate) if w_shared_gate is not None else MOE_BF16,
                              _ptr(expert_ids), _ptr(scores), _ptr(shared_gate), _ptr(workspace),
                              workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "moe_decode_route")


def moe_decode_expert_ffn(x: torch.Tensor, gate: QuantStack, up: QuantStack, down: QuantStack,
                          expert_ids: torch.Tensor, scores: Optional[torch.Tensor],
                          act: torch.Tensor, partial: torch.Tensor,
                          workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """Kernel A and kernel B for ids [T, K]; writes act [T, K, d_ff] and partial [T, K, d_in]."""
    T = x.shape[0]
    K = expert_ids.shape[1]
    g, u, d = gate.cstruct(), up.cstruct(), down.cstruct()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.moe_decode_expert_ffn(_ptr(x), _dt(x), T, ctypes.byref(g), ctypes.byref(u),
                                   ctypes.byref(d), _ptr(expert_ids), _ptr(scores), K,
                                   _ptr(act), _ptr(partial), _ptr(workspace), ws_bytes,
                                   _stream(stream))
    _check(st, "moe_decode_expert_ffn")


def expert_ffn_grouped_workspace_bytes(n_tokens: int, top_k: int, n_experts: int, d_ff: int) -> int:
    return int(lib.moe_decode_expert_ffn_grouped_workspace_bytes(n_tokens, top_k, n_experts, d_ff))


def moe_decode_expert_ffn_grouped(x: torch.Tensor, gate: QuantStack, up: QuantStack, down: QuantStack,
                                  expert_ids: torch.Tensor, scores: Optional[torch.Tensor],
                                  act: torch.Tensor, partial: torch.Tensor, workspace: torch.Tensor,
                                  stream=None) -> None:
    """The grouped (matrix-core) expert FFN for many tokens: act [T, K, d_ff], partial [T, K, d_in]."""
    T = x.shape[0]
    K = expert_ids.shape[1]
    g, u, d = gate.cstruct(), up.cstruct(), down.cstruct()
    st = lib.moe_decode_expert_ffn_grouped(_ptr(x), _dt(x), T, ctypes.byref(g), ctypes.byref(u),
                                           ctypes.byref(d), _ptr(expert_ids), _ptr(scores), K,
                                           _ptr(act), _ptr(partial), _ptr(workspace),
                                           workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "moe_decode_expert_ffn_grouped")


def moe_decode_expert_ffn_noalloc(x: torch.Tensor, gate: QuantStack, up: QuantStack, down: QuantStack,
                                  expert_ids: torch.Tensor, scores: Optional[torch.Tensor],
                                  act: torch.Tensor, partial: torch.Tensor, stream=None) -> None:
    """moe_decode_expert_ffn with the library's own device scratch instead of a workspace."""
    T = x.shape[0]
    K = expert_ids.shape[1]
    g, u, d = gate.cstruct(), up.cstruct(), down.cstruct()
    st = lib.moe_decode_expert_ffn_noalloc(_ptr(x), _dt(x), T, ctypes.byref(g), ctypes.byref(u),
                                           ctypes.byref(d), _ptr(expert_ids), _ptr(scores), K,
                                           _ptr(act), _ptr(partial), _stream(stream))
    _check(st, "moe_decode_expert_ffn_noalloc")


def expert_ffn_noalloc_max_bytes() -> int:
    return int(lib.moe_decode_expert_ffn_noalloc_max_bytes())


def moe_decode_gate_up(x: torch.Tensor, gate: QuantStack, up: QuantStack,
                       expert_ids: torch.Tensor, act: torch.Tensor,
                       workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """Kernel A only: act [T, K, d_ff] = silu(W_gate x) * (W_up x) for the selected experts."""
    T = x.shape[0]
    K = expert_ids.shape[1]
    g, u = gate.cstruct(), up.cstruct()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.moe_decode_gate_up(_ptr(x), _dt(x), T, ctypes.byref(g), ctypes.byref(u),
                                _ptr(expert_ids), K, _ptr(act), _ptr(workspace), ws_bytes,
                                _stream(stream))
    _check(st, "moe_decode_gate_up")


def moe_decode_down(act: torch.Tensor, down: QuantStack, expert_ids: torch.Tensor,
                    scores: Optional[torch.Tensor], partial: torch.Tensor,
                    workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """Kernel B only: partial [T, K, d_in] = score * (W_down act) for the selected experts."""
    T, K = expert_ids.shape
    d = down.cstruct()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.moe_decode_down(_ptr(act), T, ctypes.byref(d), _ptr(expert_ids), _ptr(scores), K,
                             _ptr(partial), _ptr(workspace), ws_bytes, _stream(stream))
    _check(st, "moe_decode_down")


def layer_weights(w_router: torch.Tensor, top_k: int, renormalize: bool, gate: QuantStack,
                  up: QuantStack, down: QuantStack, shared=None,
                  w_shared_gate: Optional[torch.Tensor] = None) -> CLayerWeights:
    """The moe_layer_weights struct for a layer (device tensors stay owned by the caller)."""
    E = w_router.shape[0]
    z = CQMat()
    sh = tuple(shared) if shared is not None else None
    return CLayerWeights(w_router.data_ptr(), _dt(w_router), E, top_k, int(bool(renormalize)),
                         gate.cstruct(), up.cstruct(), down.cstruct(),
                         0 if sh is None else sh[0].n_experts,
                         *(z, z, z) if sh is None else tuple(m.cstruct() for m in sh),
                         None if w_shared_gate is None else w_shared_gate.data_ptr())


def layer_workspace_bytes(weights: CLayerWeights) -> int:
    return lib.moe_decode_layer_workspace_bytes(ctypes.byref(weights))


def moe_decode_layer(weights: CLayerWeights, x: torch.Tensor, residual: torch.Tensor,
                     out: torch.Tensor, workspace: torch.Tensor,
                     expert_ids: Optional[torch.Tensor] = None, scores: Optional[torch.Tensor] = None,
                     shared_gate: Optional[torch.Tensor] = None, stream=None) -> None:
    """The fused single-launch layer for one token: out [d_in] (fp32, bf16 or fp16)."""
    st = lib.moe_decode_layer(ctypes.byref(weights), _ptr(x), _dt(x), _ptr(residual), _dt(residual),
                              _ptr(out), _dt(out), _ptr(expert_ids), _ptr(scores), _ptr(shared_gate),
                              _ptr(workspace), workspace.numel() * workspace.element_size(),
                              _stream(stream))
    _check(st, "moe_decode_layer")


def rmsnorm_struct(weight: torch.Tensor, eps: float, normed: torch.Tensor) -> CRMSNorm:
    return CRMSNorm(weight.data_ptr(), _dt(weight), float(eps), normed.data_ptr(), _dt(normed))


def tail_rmsnorm_workspace_bytes(n_tokens: int, d_in: int) -> int:
    return int(lib.moe_decode_tail_rmsnorm_workspace_bytes(n_tokens, d_in))


def moe_decode_tail_rmsnorm(partial: torch.Tensor, residual: torch.Tensor, out: torch.Tensor,
                            norm_weight: torch.Tensor, eps: float, normed: torch.Tensor,
                            workspace: torch.Tensor, shared: Optional[torch.Tensor] = None,
                            shared_gate: Optional[torch.Tensor] = None, stream=None) -> None:
    """moe_decode_tail plus the next layer's RMSNorm of out into normed [T, d_in]."""
    T, K, d_in = partial.shape
    S = 0 if shared is None else shared.shape[1]
    nrm = rmsnorm_struct(norm_weight, eps, normed)
    st = lib.moe_decode_tail_rmsnorm(_ptr(partial), T, K, d_in, _ptr(shared), S, _ptr(shared_gate),
                                     _ptr(residual), _dt(residual), _ptr(out), _dt(out), ctypes.byref(nrm),
                                     _ptr(workspace), workspace.numel() * workspace.element_size(),
                                     _stream(stream))
    _check(st, "moe_decode_tail_rmsnorm")


def moe_decode_layer_rmsnorm(weights: CLayerWeights, x: torch.Tensor, residual: torch.Tensor,
                             out: torch.Tensor, norm_weight: torch.Tensor, eps: float,
                             normed: torch.Tensor, workspace: torch.Tensor,
                             expert_ids: Optional[torch.Tensor] = None, scores: Optional[torch.Tensor] = None,
                             shared_gate: Optional[torch.Tensor] = None, stream=None) -> None:
    """The fused single-launch layer plus the next layer's RMSNorm of out into normed [d_in]."""
    nrm = rmsnorm_struct(norm_weight, eps, normed)
    st = lib.moe_decode_layer_rmsnorm(ctypes.byref(weights), _ptr(x), _dt(x), _ptr(residual), _dt(residual),
                                      _ptr(out), _dt(out), ctypes.byref(nrm), _ptr(expert_ids), _ptr(scores),
                                      _ptr(shared_gate), _ptr(workspace),
                                      workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "moe_decode_layer_rmsnorm")


def moe_decode_rmsnorm(y: torch.Tensor, norm_weight: torch.Tensor, eps: float, normed: torch.Tensor,
                       stream=None) -> None:
    """normed [T, d] = y / sqrt(mean(y^2) + eps) * weight, one workgroup per token."""
    T, d = y.shape
    nrm = rmsnorm_struct(norm_weight, eps, normed)
    _check(lib.moe_decode_rmsnorm(_ptr(y), _dt(y), T, d, ctypes.byref(nrm), _stream(stream)),
           "moe_decode_rmsnorm")


def moe_decode_tail(partial: torch.Tensor, residual: torch.Tensor, out: torch.Tensor,
                    shared: Optional[torch.Tensor] = None,
                    shared_gate: Optional[torch.Tensor] = None, stream=None) -> None:
    """out [T, d_in] = residual + (sum_k partial + sum_s shared * shared_gate)."""
    T, K, d_in = partial.shape
    S = 0 if shared is None else shared.shape[1]
    st = lib.moe_decode_tail(_ptr(partial), T, K, d_in, _ptr(shared), S, _ptr(shared_gate),
                             _ptr(residual), _dt(residual), _ptr(out), _dt(out), _stream(stream))
    _check(st, "moe_decode_tail")


def read_probe_blocks(nbytes: int) -> int:
    """Number of fp32 partial sums moe_decode_read_probe writes for nbytes."""
    return int(lib.moe_decode_read_probe_blocks(nbytes))


def moe_decode_read_probe(data: torch.Tensor, partial_sums: torch.Tensor, stream=None) -> None:
    """Read data (contiguous device tensor) once; one fp32 sum per workgroup into partial_sums."""
    nbytes = data.numel() * data.element_size()
    st = lib.moe_decode_read_probe(_ptr(data), nbytes, _ptr(partial_sums), partial_sums.numel(),
                                   _stream(stream))
    _check(st, "moe_decode_read_probe")


from .layer import DecodeLayer  # noqa: E402  (needs the functions above)

__all__ = ["QuantStack", "DecodeLayer", "moe_decode_route", "moe_decode_expert_ffn",
           "moe_decode_expert_ffn_noalloc", "expert_ffn_noalloc_max_bytes",
           "moe_decode_tail_rmsnorm", "moe_decode_layer_rmsnorm", "tail_rmsnorm_workspace_bytes",
           "moe_decode_rmsnorm",
           "moe_decode_layer", "layer_weights", "layer_workspace_bytes",
           "moe_decode_expert_ffn_grouped", "expert_ffn_grouped_workspace_bytes",
           "moe_decode_gate_up", "moe_decode_down",
           "moe_decode_tail", "route_workspace_bytes", "expert_ffn_workspace_bytes",
           "moe_decode_read_probe", "read_probe_blocks", "workspace_status",
           "MoeError", "status_string", "abi_version", "lib"]
