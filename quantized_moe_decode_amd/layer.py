"""One MoE decode layer on the device: weights, preallocated buffers, and the
route -> expert FFN (routed, then shared) -> tail call sequence.

No arithmetic happens here; every step is a call into libmoe_decode.so on the
caller's stream.  Buffers are allocated once, so `forward` can be captured
into a HIP graph (torch.cuda.CUDAGraph) and replayed.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np
import torch

from . import (MOE_MAX_TOKENS, QuantStack, expert_ffn_grouped_workspace_bytes, expert_ffn_workspace_bytes,
               layer_weights, layer_workspace_bytes, moe_decode_expert_ffn, moe_decode_expert_ffn_grouped,
               moe_decode_layer, moe_decode_layer_rmsnorm, moe_decode_rmsnorm,
               moe_decode_route,
               moe_decode_tail, moe_decode_tail_rmsnorm, route_workspace_bytes,
               tail_rmsnorm_workspace_bytes)

_TORCH_16 = {"f16": torch.float16, "bf16": torch.bfloat16}


def tensor_from_encoded(a: np.ndarray, dtype: str, device) -> torch.Tensor:
    """Device tensor from an encoded host array (float32 values or uint16 bit patterns)."""
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16))
    return t.view(_TORCH_16[dtype]).to(device)


def stack_to_device(stack, device) -> QuantStack:
    """A QuantStack from a host stack with q (uint32), scales/biases (uint16 bits)."""
    q = torch.from_numpy(np.ascontiguousarray(stack.q).view(np.int32)).to(device)
    s = tensor_from_encoded(stack.scales, stack.sb_dtype, device)
    b = tensor_from_encoded(stack.biases, stack.sb_dtype, device)
    return QuantStack(q, s, b, stack.rows, stack.cols, stack.bits)


class DecodeLayer:
    """A quantized MoE layer resident on one GPU, for a fixed number of tokens per step.

    The expert step uses moe_decode_expert_ffn up to MOE_MAX_TOKENS tokens and
    the grouped matrix-core call (moe_decode_expert_ffn_grouped) above that;
    grouped=True or False forces one of them."""

    def __init__(self, router: torch.Tensor, top_k: int, renormalize: bool,
                 gate: QuantStack, up: QuantStack, down: QuantStack,
                 shared: Optional[Sequence[QuantStack]] = None,
                 shared_gate_w: Optional[torch.Tensor] = None, n_tokens: int = 1,
                 grouped: Optional[bool] = None):
        dev = router.device
        self.grouped = n_tokens > MOE_MAX_TOKENS if grouped is None else bool(grouped)

        def ws_bytes(T, K, E, d_ff):
            if self.grouped:
                return expert_ffn_grouped_workspace_bytes(T, K, E, d_ff)
            return expert_ffn_workspace_bytes(T, K, E)
        self.router, self.top_k, self.renormalize = router, top_k, renormalize
        self.gate, self.up, self.down = gate, up, down
        self.shared = tuple(shared) if shared is not None else None
        self.shared_gate_w = shared_gate_w
        self.n_tokens = T = n_tokens
        E, d_in = router.shape
        d_ff = gate.rows
        self.d_in, self.d_ff, self.n_experts = d_in, d_ff, E
        f32 = dict(device=dev, dtype=torch.float32)
        self.ids = torch.zeros(T, top_k, device=dev, dtype=torch.int32)
        self.scores = torch.zeros(T, top_k, **f32)
        self.shared_gate = torch.zeros(T, **f32) if shared_gate_w is not None else None
        self.act = torch.zeros(T, top_k, d_ff, **f32)
        self.partial = torch.zeros(T, top_k, d_in, **f32)
        self.route_ws = torch.zeros(route_workspace_bytes(T, E), device=dev, dtype=torch.uint8)
        nb = ws_bytes(T, top_k, E, d_ff)
        self.ffn_ws = torch.zeros(max(nb, 1), device=dev, dtype=torch.uint8) if nb else None
        if self.shared is not None:
            S = self.shared[0].n_experts
            self.n_shared = S
            self.shared_ids = torch.arange(S, device=dev, dtype=torch.int32).repeat(T, 1).contiguous()
            self.shared_act = torch.zeros(T, S, self.shared[0].rows, **f32)
            self.shared_partial = torch.zeros(T, S, d_in, **f32)
            nb = ws_bytes(T, S, S, self.shared[0].rows)
            self.shared_ws = torch.zeros(max(nb, 1), device=dev, dtype=torch.uint8) if nb else None
        else:
            self.n_shared = 0
        # fused single-launch path (one token per launch)
        self.cweights = layer_weights(router, top_k, renormalize, gate, up, down, self.shared,
                                      shared_gate_w)
        nb = layer_workspace_bytes(self.cweights)
        self.fused_ws = torch.zeros(nb, device=dev, dtype=torch.uint8) if nb else None
        self.norm_w, self.norm_eps, self.normed, self.tail_ws, self.fold_norm = None, 0.0, None, None, True

    def set_next_norm(self, weight: torch.Tensor, eps: float, fold: bool = True,
                      dtype: torch.dtype = torch.float32) -> None:
        """The next layer's RMSNorm (weight [d_in], eps) of this layer's output:
        every forward also writes self.normed [T, d_in] of `dtype` (fp32, bf16
        or fp16), folded into the tail (fold=True) or as a separate
        moe_decode_rmsnorm launch after it."""
        dev = self.router.device
        self.norm_w, self.norm_eps, self.fold_norm = weight, float(eps), fold
        self.normed = torch.zeros(self.n_tokens, self.d_in, device=dev, dtype=dtype)
        self.tail_ws = torch.zeros(tail_rmsnorm_workspace_bytes(self.n_tokens, self.d_in), device=dev,
                                   dtype=torch.uint8)

    def route(self, x: torch.Tensor, stream=None) -> None:
        moe_decode_route(x, self.router, self.top_k, self.renormalize, self.ids, self.scores,
                         self.route_ws, self.shared_gate_w, self.shared_gate, stream)

    def experts(self, x: torch.Tensor, stream=None) -> None:
        ffn = moe_decode_expert_ffn_grouped if self.grouped else moe_decode_expert_ffn
        ffn(x, self.gate, self.up, self.down, self.ids, self.scores, self.act, self.partial, self.ffn_ws, stream)
        if self.shared is not None:
            g, u, d = self.shared
            ffn(x, g, u, d, self.shared_ids, None, self.shared_act, self.shared_partial, self.shared_ws, stream)

    def tail(self, resid: torch.Tensor, out: torch.Tensor, stream=None) -> None:
        shared = self.shared_partial if self.shared is not None else None
        if self.norm_w is not None and self.fold_norm:
            moe_decode_tail_rmsnorm(self.partial, resid, out, self.norm_w, self.norm_eps, self.normed,
                                    self.tail_ws, shared, self.shared_gate, stream)
        else:
            moe_decode_tail(self.partial, resid, out, shared, self.shared_gate, stream)
            if self.norm_w is not None:
                moe_decode_rmsnorm(out.view(-1, self.d_in), self.norm_w, self.norm_eps, self.normed, stream)

    def forward(self, x: torch.Tensor, resid: torch.Tensor, out: torch.Tensor, stream=None) -> None:
        """out [T, d_in] (fp32, bf16 or fp16) = the layer applied to x [T, d_in] with residual resid."""
        self.route(x, stream)
        self.experts(x, stream)
        self.tail(resid, out, stream)

    def forward_fused(self, x: torch.Tensor, resid: torch.Tensor, out: torch.Tensor, stream=None,
                      record: bool = True) -> None:
        """The same layer in one launch (x [1, d_in] or [d_in]); fills ids/scores/gate if record."""
        if self.fused_ws is None:
            raise ValueError("layer not supported by the fused launch")
        rec = (self.ids if record else None, self.scores if record else None,
               self.shared_gate if record else None)
        if self.norm_w is not None and self.fold_norm:
            moe_decode_layer_rmsnorm(self.cweights, x, resid, out, self.norm_w, self.norm_eps, self.normed,
                                     self.fused_ws, *rec, stream=stream)
        else:
            moe_decode_layer(self.cweights, x, resid, out, self.fused_ws, *rec, stream)
            if self.norm_w is not None:
                moe_decode_rmsnorm(out.view(-1, self.d_in), self.norm_w, self.norm_eps, self.normed, stream)

    def fused_error_word(self) -> int:
        """Nonzero if a wait inside a fused launch ever timed out (reads device memory)."""
        return int(self.fused_ws[:4].view(torch.int32).item())

    def expert_bytes_per_step(self) -> int:
        """Bytes of expert weight one step reads when its K selections are distinct (T = 1)."""
        n = (self.gate.nbytes(self.top_k) + self.up.nbytes(self.top_k) + self.down.nbytes(self.top_k))
        if self.shared is not None:
            n += sum(s.nbytes(self.n_shared) for s in self.shared)
        return n


def share_fused_workspace(layers: Sequence[DecodeLayer]) -> Optional[torch.Tensor]:
    """Give every layer the same fused-launch workspace (one zeroed buffer of the
    largest size).  Valid for layers whose launches run in order on one stream,
    as the layers of a decode step do: each launch leaves the workspace ready
    for the next.  A workspace that stays the same buffer stays cache-resident
    from one layer to the next."""
    sizes = [l.fused_ws.numel() for l in layers if l.fused_ws is not None]
    if not sizes:
        return None
    ws = torch.zeros(max(sizes), device=layers[0].router.device, dtype=torch.uint8)
    for l in layers:
        if l.fused_ws is not None:
            l.fused_ws = ws
    return ws


class DecodeStep:
    """One decode step: every layer in order on one stream, each token's step
    captured once into a HIP graph (torch.cuda.CUDAGraph over the library's
    launches) and replayed.

    path "fused": one moe_decode_layer launch per layer (one token per step),
    all layers sharing one fused workspace; path "three-call": route, expert
    FFN (routed, then shared) and tail per layer (any token count).  Inputs
    are given per distinct token (or token batch) r and layer l as device
    tensors xs[r][l], rs[r][l]; layer l writes outs[l] [T, d_in] of
    out_dtype (fp32, bf16 or fp16) and its routing into layers[l].ids /
    .scores.  Layers run back to back: no work of layer l + 1 starts before
    layer l has finished.  repeat > 1 captures the step that many times into
    each token's graph (one replay = repeat steps on the same token), for
    steps so short that the host's graph launches would set the pace.
    """

    def __init__(self, layers: Sequence[DecodeLayer], xs, rs, path: str = "fused",
                 share_workspace: bool = True, out_dtype: torch.dtype = torch.float32, repeat: int = 1):
        if path not in ("fused", "three-call"):
            raise ValueError(path)
        if path == "fused" and any(l.n_tokens != 1 for l in layers):
            raise ValueError("the fused launch takes one token per step")
        self.layers, self.xs, self.rs, self.path = list(layers), xs, rs, path
        self.repeat = max(1, int(repeat))
        dev = layers[0].router.device
        self.outs = [torch.zeros(l.n_tokens, l.d_in, device=dev, dtype=out_dtype) for l in layers]
        self.fused_ws = share_fused_workspace(self.layers) if (path == "fused" and share_workspace) else None
        self.graphs = []

    @property
    def n_distinct(self) -> int:
        return len(self.xs)

    def eager(self, r: int, path: Optional[str] = None) -> None:
        fused = (path or self.path) == "fused"
        for li, lay in enumerate(self.layers):
            if fused:
                lay.forward_fused(self.xs[r][li], self.rs[r][li], self.outs[li])
            else:
                lay.forward(self.xs[r][li], self.rs[r][li], self.outs[li])

    def capture(self, path: Optional[str] = None):
        """One graph per distinct token; returns them (also kept as .graphs when
        path is the step's own)."""
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):           # warm-up launches outside the capture
            for r in range(self.n_distinct):
                self.eager(r, path)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        graphs = []
        for r in range(self.n_distinct):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for _ in range(self.repeat):
                    self.eager(r, path)
            graphs.append(g)
        torch.cuda.synchronize()
        if path is None or path == self.path:
            self.graphs = graphs
        return graphs

    def replay(self, r: int) -> None:
        self.graphs[r].replay()

    def error_words(self) -> int:
        """Nonzero if a wait inside any launch of the step ever timed out: the
        fused workspaces' error words, or the route workspaces' (reads device
        memory)."""
        from . import MOE_OK, workspace_status
        if self.path == "fused":
            return max((l.fused_error_word() for l in self.layers), default=0)
        return int(any(workspace_status(l.route_ws) != MOE_OK for l in self.layers))


def layer_from_host(cfg, weights: dict, device, n_tokens: Optional[int] = None,
                    grouped: Optional[bool] = None) -> DecodeLayer:
    """Build a DecodeLayer from host weights in the generator's layout."""
    router = tensor_from_encoded(weights["router"], cfg.router_dtype, device)
    gate, up, down = (stack_to_device(weights[p], device) for p in ("gate", "up", "down"))
    shared = None
    if cfg.n_shared:
        shared = [stack_to_device(weights[p], device)
                  for p in ("shared_gate_proj", "shared_up", "shared_down")]
    wg = None
    if cfg.shared_gate:
        wg = tensor_from_encoded(weights["shared_gate_w"], "bf16", device)
    return DecodeLayer(router, cfg.top_k, cfg.renormalize, gate, up, down, shared, wg,
                       n_tokens if n_tokens is not None else cfg.n_tokens, grouped)
