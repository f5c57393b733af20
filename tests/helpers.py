"""Test-side tools that are independent of both the oracle and the HIP path.

* a big-integer packer/unpacker written from the format definition
  (element j of a row occupies bits [b*j, b*j + b) of the row's little-endian
  bit stream), used to pin the oracle's unpacking;
* a numpy bit-matrix unpacker (``np.unpackbits``) and numpy dtype decoders,
  used to build dense dequantised matrices for library-routine special cases;
* margin-controlled token selection: a token draw is accepted when every gap
  between consecutive logits among its top K+1 (computed by the oracle, fp64)
  is at least 1e-3, so the selected set and its order are fixed.
"""
from __future__ import annotations

import numpy as np

import moe_inputs as mi

MARGIN = 1e-3


# ------------------------------------------------------------ big-int codec
def bigint_pack(codes: np.ndarray, bits: int) -> np.ndarray:
    """codes [rows, cols] -> uint32 words [rows, cols*bits/32] (LSB-first)."""
    codes = np.asarray(codes, dtype=np.int64)
    rows, cols = codes.shape
    assert (cols * bits) % 32 == 0
    nwords = cols * bits // 32
    out = np.empty((rows, nwords), np.uint32)
    for r in range(rows):
        acc = 0
        for j in range(cols):
            c = int(codes[r, j])
            assert 0 <= c < (1 << bits)
            acc |= c << (bits * j)
        raw = acc.to_bytes(nwords * 4, "little")
        out[r] = np.frombuffer(raw, dtype="<u4")
    return out


def bigint_unpack(words: np.ndarray, bits: int, cols: int) -> np.ndarray:
    words = np.atleast_2d(np.asarray(words, dtype=np.uint32))
    out = np.empty((words.shape[0], cols), np.int64)
    for r in range(words.shape[0]):
        acc = int.from_bytes(words[r].astype("<u4").tobytes(), "little")
        for j in range(cols):
            out[r, j] = (acc >> (bits * j)) & ((1 << bits) - 1)
    return out


# ------------------------------------------------------- numpy bit unpacker
def np_unpack(words: np.ndarray, bits: int, cols: int) -> np.ndarray:
    """Vectorised unpack via the little-endian bit matrix: [..., words] -> [..., cols]."""
    w = np.ascontiguousarray(words, dtype="<u4")
    lead = w.shape[:-1]
    by = w.view(np.uint8).reshape(*lead, -1)
    bitm = np.unpackbits(by, axis=-1, bitorder="little")[..., : cols * bits]
    bitm = bitm.reshape(*lead, cols, bits).astype(np.int64)
    return (bitm << np.arange(bits, dtype=np.int64)).sum(-1)


def np_decode(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of encoded arrays using numpy's own conversions."""
    a = np.asarray(a)
    if dtype == mi.F32:
        return a.astype(np.float32).astype(np.float64)
    if dtype == mi.F16:
        return a.astype(np.uint16).view(np.float16).astype(np.float64)
    if dtype == mi.BF16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def dense(stack: mi.QStack, experts=None) -> np.ndarray:
    """Dense float64 weights [E, rows, cols] = scale * q + bias per group of 64."""
    q = stack.q if experts is None else stack.q[list(experts)]
    s = stack.scales if experts is None else stack.scales[list(experts)]
    b = stack.biases if experts is None else stack.biases[list(experts)]
    codes = np_unpack(q, stack.bits, stack.cols).astype(np.float64)
    sv = np.repeat(np_decode(s, stack.sb_dtype), mi.GROUP, axis=-1)
    bv = np.repeat(np_decode(b, stack.sb_dtype), mi.GROUP, axis=-1)
    return sv * codes + bv


def make_stack(codes, scales, biases, bits: int, sb_dtype: str) -> mi.QStack:
    """A QStack from explicit codes [E, rows, cols] and float scales/biases [E, rows, cols/64]."""
    codes = np.asarray(codes)
    E, rows, cols = codes.shape
    q = np.stack([bigint_pack(codes[e], bits) for e in range(E)])
    s = mi.encode(np.asarray(scales, np.float64), sb_dtype).reshape(E, rows, cols // 64)
    b = mi.encode(np.asarray(biases, np.float64), sb_dtype).reshape(E, rows, cols // 64)
    return mi.QStack(q, s, b, rows, cols, bits, sb_dtype)


def stack_from_arrays(q, s, b, like: mi.QStack) -> mi.QStack:
    return mi.QStack(np.ascontiguousarray(q), np.ascontiguousarray(s), np.ascontiguousarray(b),
                     like.rows, like.cols, like.bits, like.sb_dtype)


# ---------------------------------------------------------- routing margin
def margin_ok(logits_row: np.ndarray, top_k: int, margin: float = MARGIN) -> bool:
    """Every consecutive gap among the top K+1 logits is >= margin (fixes set and order)."""
    s = np.sort(np.asarray(logits_row, np.float64))[::-1]
    n = min(top_k + 1, s.size)
    return bool(np.all(np.diff(s[:n]) <= -margin))


def pick_tokens(cfg: mi.LayerConfig, layer: int, n_tokens: int, router, wg=None,
                max_attempts: int = 64):
    """Per-token draw attempts whose routing has the margin; returns (x, resid, attempts)."""
    import oracle
    attempts = []
    for t in range(n_tokens):
        for a in range(max_attempts):
            x, _ = mi.gen_token(cfg, layer, t, a)
            r = oracle.route(x, cfg.x_dtype, router, cfg.router_dtype, cfg.top_k,
                             cfg.renormalize)
            if margin_ok(r["logits"][0], cfg.top_k):
                attempts.append(a)
                break
        else:
            raise RuntimeError(f"no margin-satisfying draw for token {t}")
    x, resid = mi.gen_tokens(cfg, layer, n_tokens, attempts)
    return x, resid, attempts


def oracle_layer_selected(cfg, layer_idx, x, resid):
    """The oracle's layer result generating only the selected experts (oracle.layer_selected)."""
    import oracle
    return oracle.layer_selected(cfg, layer_idx, x, resid)


def rel_err(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    if scale == 0.0:
        return float(np.max(np.abs(got - ref))) if got.size else 0.0
    return float(np.max(np.abs(got - ref)) / scale)
