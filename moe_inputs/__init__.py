"""Seeded synthetic inputs for the quantized MoE decode layer.

This module is shared by the CPU oracle's tests and by the GPU path's tests and
benchmark.  It holds random draws and dtype encodings only -- none of the
layer's arithmetic (no dot products, no softmax, no unpacking).

Formats (from the problem statement and the pages' "affine" 4/6/8-bit weights,
mlxcel PR #276, "Scope / flags" and "Next"):

* A quantized projection stack of ``n_experts`` matrices, each ``rows x cols``
  (output x contraction), stores unsigned ``bits``-bit codes packed LSB-first
  into little-endian uint32 words, row-major: ``q[e, r, :]`` holds the
  ``cols * bits / 32`` words of row ``r``.  Element ``j`` of a row occupies
  bits ``[bits*j, bits*j + bits)`` of the row's bit stream; for 6-bit codes an
  element may straddle two words (16 codes per 3 words).
* ``scales[e, r, g]`` and ``biases[e, r, g]`` (fp16 or bf16 bit patterns in
  uint16) belong to the group ``g`` of 64 consecutive elements of row ``r``.
  The weight is ``scale * q + bias``.

Because every code value is drawn i.i.d. uniform over ``[0, 2**bits)`` and a
row of ``64*G`` codes fills its words exactly, the packed words of such a row
are themselves i.i.d. uniform 32-bit words.  The generator therefore draws the
words directly; no packing routine is needed here.

Value distributions (the tiny configuration states its own; the others extend
it so that the weight range is the same for every bit width):
  q ~ U{0 .. 2^b - 1};  scale ~ U(0.005, 0.02) * 2^(4-b), rounded to the
  scale dtype;  bias = -2^(b-1) * scale (exact: a power-of-two multiple of the
  rounded scale).  An optional jitter multiplies the bias by 1 + U(-0.25, 0.25)
  so that a kernel hard-coding the zero point cannot pass.
  x, resid ~ N(0, 1);  router and shared-gate weights ~ N(0, 1/d_in).

Seeds: every tensor is drawn from
``np.random.default_rng([2026, cfg_id, layer, tensor_id, expert])`` and every
token from ``[2026, cfg_id, layer, 1000 + token, attempt]``, so any expert of
any layer can be regenerated on its own.
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Optional, Sequence

import numpy as np

SEED_ROOT = 2026
GROUP = 64

# dtype names used throughout (matching the C-ABI enum values in moe_decode.h)
F32, F16, BF16 = "f32", "f16", "bf16"
DTYPE_CODE = {F32: 0, F16: 1, BF16: 2}

# projection slots: tensor ids are 10 * slot + {0: codes, 1: scales, 2: bias jitter}
PROJ_SLOT = {"gate": 0, "up": 1, "down": 2, "shared_gate_proj": 3,
             "shared_up": 4, "shared_down": 5}
TID_ROUTER = 100
TID_SHARED_GATE_W = 101
TID_NORM_W = 102


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    """One MoE decode-layer workload (shapes, formats and counts)."""
    name: str
    cfg_id: int            # seed component for tokens
    weight_cfg_id: int     # seed component for weights (the batch-32 case reuses the Qwen3 weights)
    d_in: int
    d_ff: int
    n_experts: int
    top_k: int
    renormalize: bool
    bits_gate_up: int
    bits_down: int
    sb_dtype: str          # scale/bias dtype
    x_dtype: str
    router_dtype: str
    resid_dtype: str
    n_shared: int = 0
    d_ff_shared: int = 0
    shared_gate: bool = False   # sigmoid(x . w_g) scalar gate on the shared sum
    n_tokens: int = 1
    n_layers: int = 1
    norm_eps: float = 1e-6          # the next layer's RMSNorm, when folded into the tail

    def proj_shape(self, proj: str):
        """(n_experts, rows, cols, bits) of a projection stack."""
        shared = proj.startswith("shared")
        ne = self.n_shared if shared else self.n_experts
        dff = self.d_ff_shared if shared else self.d_ff
        if proj in ("gate", "up", "shared_gate_proj", "shared_up"):
            return ne, dff, self.d_in, self.bits_gate_up
        if proj in ("down", "shared_down"):
            return ne, self.d_in, dff, self.bits_down
        raise KeyError(proj)


def qmat_bytes(rows: int, cols: int, bits: int) -> int:
    """Bytes of one expert matrix: packed codes + one 2-byte scale and bias per group."""
    return rows * cols * bits // 8 + rows * (cols // GROUP) * 4


def expert_bytes(cfg: LayerConfig, shared: bool = False) -> int:
    """Weight bytes of one expert (gate + up + down)."""
    dff = cfg.d_ff_shared if shared else cfg.d_ff
    return (2 * qmat_bytes(dff, cfg.d_in, cfg.bits_gate_up)
            + qmat_bytes(cfg.d_in, dff, cfg.bits_down))


# The five workloads.  Names say what they are; sizes follow the pages' models.
TINY = LayerConfig("tiny_e8_top2", 0, 0, d_in=256, d_ff=128, n_experts=8, top_k=2,
                   renormalize=True, bits_gate_up=4, bits_down=4, sb_dtype=F16,
                   x_dtype=F32, router_dtype=F32, resid_dtype=F32)
QWEN3 = LayerConfig("qwen3_30b_a3b_moe", 1, 1, d_in=2048, d_ff=768, n_experts=128,
                    top_k=8, renormalize=True, bits_gate_up=4, bits_down=4,
                    sb_dtype=BF16, x_dtype=BF16, router_dtype=BF16, resid_dtype=BF16,
                    n_layers=48)
QWEN15 = LayerConfig("qwen1.5_moe_a2.7b", 2, 2, d_in=2048, d_ff=1408, n_experts=60,
                     top_k=4, renormalize=False, bits_gate_up=8, bits_down=8,
                     sb_dtype=BF16, x_dtype=BF16, router_dtype=BF16, resid_dtype=BF16,
                     n_shared=1, d_ff_shared=5632, shared_gate=True, n_layers=24)
DOTS = LayerConfig("dots_llm1_mixed_bit", 3, 3, d_in=4096, d_ff=1408, n_experts=128,
                   top_k=6, renormalize=True, bits_gate_up=4, bits_down=6,
                   sb_dtype=BF16, x_dtype=BF16, router_dtype=BF16, resid_dtype=BF16,
                   n_shared=2, d_ff_shared=1408, shared_gate=False, n_layers=12)
QWEN3_B32 = dataclasses.replace(QWEN3, name="qwen3_30b_a3b_moe_batch32", cfg_id=4,
                                weight_cfg_id=1, n_tokens=32)
# 256 tokens per step (a prefill chunk) on the same weights: the grouped expert FFN
QWEN3_P256 = dataclasses.replace(QWEN3, name="qwen3_30b_a3b_moe_prefill256", cfg_id=5,
                                 weight_cfg_id=1, n_tokens=256)

CONFIGS: Dict[str, LayerConfig] = {c.name: c for c in (TINY, QWEN3, QWEN15, DOTS, QWEN3_B32, QWEN3_P256)}


def rng_for(*key: int) -> np.random.Generator:
    return np.random.default_rng([SEED_ROOT, *key])


# ----------------------------------------------------------------- encodings
def to_bf16_bits(a) -> np.ndarray:
    """Round to bfloat16 (round-to-nearest-even from float32) and return the uint16 bits."""
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def to_f16_bits(a) -> np.ndarray:
    """Round to IEEE binary16 (numpy's round-to-nearest-even) and return the uint16 bits."""
    return np.asarray(a, dtype=np.float64).astype(np.float16).view(np.uint16)


def encode(a, dtype: str) -> np.ndarray:
    """Encode values in `dtype`: float32 array for f32, uint16 bit patterns otherwise."""
    if dtype == F32:
        return np.asarray(a, dtype=np.float32)
    if dtype == BF16:
        return to_bf16_bits(a)
    if dtype == F16:
        return to_f16_bits(a)
    raise ValueError(dtype)


def scale_bits_to_float(bits16: np.ndarray, dtype: str) -> np.ndarray:
    """Decode uint16 scale bit patterns (used only to build the exact bias)."""
    if dtype == BF16:
        return (bits16.astype(np.uint32) << 16).view(np.float32)
    return bits16.view(np.float16).astype(np.float32)


# -------------------------------------------------------------- weight stacks
def gen_expert_proj(cfg: LayerConfig, layer: int, proj: str, expert: int,
                    jitter_bias: bool = False):
    """One expert's packed codes, scales and biases for projection `proj`.

    Returns (q uint32 [rows, cols*bits/32], scales uint16 [rows, cols/64],
    biases uint16 [rows, cols/64]).
    """
    _, rows, cols, bits = cfg.proj_shape(proj)
    slot = PROJ_SLOT[proj]
    wc = cfg.weight_cfg_id
    words = rows * cols * bits // 32
    q = rng_for(wc, layer, 10 * slot, expert).integers(
        0, 1 << 32, size=words, dtype=np.uint32).reshape(rows, cols * bits // 32)
    g = cols // GROUP
    r = rng_for(wc, layer, 10 * slot + 1, expert)
    s = r.uniform(0.005, 0.02, size=(rows, g)) * 2.0 ** (4 - bits)
    s_bits = encode(s, cfg.sb_dtype)
    s_val = scale_bits_to_float(s_bits, cfg.sb_dtype).astype(np.float64)
    b = -(2.0 ** (bits - 1)) * s_val
    if jitter_bias:
        j = rng_for(wc, layer, 10 * slot + 2, expert).uniform(-0.25, 0.25, size=(rows, g))
        b = b * (1.0 + j)
    b_bits = encode(b, cfg.sb_dtype)
    return q, s_bits, b_bits


@dataclasses.dataclass
class QStack:
    """A host-side quantized projection stack (all experts)."""
    q: np.ndarray        # uint32 [E, rows, words_per_row]
    scales: np.ndarray   # uint16 [E, rows, groups]
    biases: np.ndarray   # uint16 [E, rows, groups]
    rows: int
    cols: int
    bits: int
    sb_dtype: str

    @property
    def n_experts(self) -> int:
        return self.q.shape[0]


def gen_proj_stack(cfg: LayerConfig, layer: int, proj: str,
                   experts: Optional[Sequence[int]] = None,
                   jitter_bias: bool = False, threads: int = 8) -> QStack:
    """A projection stack for the listed experts (default: all), in list order."""
    ne, rows, cols, bits = cfg.proj_shape(proj)
    experts = list(range(ne)) if experts is None else list(experts)
    wpr = cols * bits // 32
    g = cols // GROUP
    q = np.empty((len(experts), rows, wpr), np.uint32)
    s = np.empty((len(experts), rows, g), np.uint16)
    b = np.empty((len(experts), rows, g), np.uint16)

    def one(i):
        q[i], s[i], b[i] = gen_expert_proj(cfg, layer, proj, experts[i], jitter_bias)

    if threads > 1 and len(experts) > 1:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(one, range(len(experts))))
    else:
        for i in range(len(experts)):
            one(i)
    return QStack(q, s, b, rows, cols, bits, cfg.sb_dtype)


def gen_router(cfg: LayerConfig, layer: int) -> np.ndarray:
    """Router weight Wr [n_experts, d_in] in the router dtype (f32 array or bf16 bits)."""
    w = rng_for(cfg.weight_cfg_id, layer, TID_ROUTER, 0).normal(
        0.0, 1.0 / np.sqrt(cfg.d_in), size=(cfg.n_experts, cfg.d_in))
    return encode(w, cfg.router_dtype)


def gen_shared_gate_w(cfg: LayerConfig, layer: int) -> np.ndarray:
    """Shared-expert gate vector w_g [d_in] (bf16 bits)."""
    w = rng_for(cfg.weight_cfg_id, layer, TID_SHARED_GATE_W, 0).normal(
        0.0, 1.0 / np.sqrt(cfg.d_in), size=cfg.d_in)
    return encode(w, BF16)


def gen_norm_weight(cfg: LayerConfig, layer: int) -> np.ndarray:
    """The next layer's RMSNorm weight [d_in] (bf16 bits), U(0.5, 1.5)."""
    w = rng_for(cfg.weight_cfg_id, layer, TID_NORM_W, 0).uniform(0.5, 1.5, size=cfg.d_in)
    return encode(w, BF16)


def gen_token(cfg: LayerConfig, layer: int, token: int, attempt: int = 0):
    """One token's (x [d_in], resid [d_in]) in their dtypes, for a given draw attempt."""
    r = rng_for(cfg.cfg_id, layer, 1000 + token, attempt)
    x = r.standard_normal(cfg.d_in)
    resid = r.standard_normal(cfg.d_in)
    return encode(x, cfg.x_dtype), encode(resid, cfg.resid_dtype)


def gen_tokens(cfg: LayerConfig, layer: int, n_tokens: int, attempts: Optional[Sequence[int]] = None):
    """Stacked (x [T, d_in], resid [T, d_in]) for tokens 0..T-1."""
    attempts = [0] * n_tokens if attempts is None else list(attempts)
    xs, rs = zip(*(gen_token(cfg, layer, t, attempts[t]) for t in range(n_tokens)))
    return np.stack(xs), np.stack(rs)


def gen_layer_weights_for(cfg: LayerConfig, layer: int, experts: Sequence[int],
                          threads: int = 8) -> dict:
    """A layer's weights with the routed stacks holding only the listed experts
    (stack entry i is expert experts[i]); router and shared tensors complete."""
    out = {p: gen_proj_stack(cfg, layer, p, experts=experts, threads=threads)
           for p in ("gate", "up", "down")}
    out["router"] = gen_router(cfg, layer)
    if cfg.n_shared:
        for p in ("shared_gate_proj", "shared_up", "shared_down"):
            out[p] = gen_proj_stack(cfg, layer, p, threads=threads)
    out["shared_gate_w"] = gen_shared_gate_w(cfg, layer) if cfg.shared_gate else None
    return out


def gen_layer_weights(cfg: LayerConfig, layer: int, jitter_bias: bool = False,
                      threads: int = 8) -> dict:
    """Every weight tensor of one layer: routed stacks, router, and shared stacks if any."""
    out = {p: gen_proj_stack(cfg, layer, p, jitter_bias=jitter_bias, threads=threads)
           for p in ("gate", "up", "down")}
    out["router"] = gen_router(cfg, layer)
    if cfg.n_shared:
        for p in ("shared_gate_proj", "shared_up", "shared_down"):
            out[p] = gen_proj_stack(cfg, layer, p, jitter_bias=jitter_bias, threads=threads)
    out["shared_gate_w"] = gen_shared_gate_w(cfg, layer) if cfg.shared_gate else None
    return out
