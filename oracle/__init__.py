"""ctypes front end of the plain CPU oracle (``moe_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the smoke check in
``__graft_entry__`` and by the benchmark's CPU-baseline leg -- never by the
product path.  It shares no code with the HIP library; both sides see the
same inputs only through the seeded generator in ``moe_inputs``.

All results are float64.  Inputs are the generator's host arrays: float32
arrays for f32 tensors, uint16 bit patterns for f16/bf16 tensors, uint32
packed codes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "moe_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")
DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2}


SAN_LIB = os.path.join(HERE, "liboracle_san.so")
SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]


def build(force: bool = True, sanitize: bool = False) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math).  sanitize=True
    builds liboracle_san.so with AddressSanitizer and UndefinedBehaviorSanitizer
    (any finding aborts); load it with MOE_ORACLE_LIB set to its path and gcc's
    libasan preloaded."""
    out = SAN_LIB if sanitize else LIB
    if force or not os.path.exists(out):
        tmp = out + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-Wall", "-Wextra", "-fno-fast-math", *(SANITIZE_FLAGS if sanitize else []),
                               "-o", tmp, SRC, "-lm"])
        os.replace(tmp, out)
    return out


class _QMat(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("biases", ctypes.c_void_p), ("n_experts", ctypes.c_int32),
                ("rows", ctypes.c_int32), ("cols", ctypes.c_int32),
                ("bits", ctypes.c_int32), ("sb_dtype", ctypes.c_int32)]


_lib = None


def _load(path: str):
    L = ctypes.CDLL(path)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    L.oracle_route.argtypes = [vp, i32, i32, i32, vp, i32, i32, i32, i32, vp, i32,
                               vp, vp, vp, vp, vp]
    L.oracle_route.restype = i32
    L.oracle_expert_ffn.argtypes = [vp, i32, i32, i32, i32, ctypes.POINTER(_QMat),
                                    ctypes.POINTER(_QMat), ctypes.POINTER(_QMat),
                                    vp, vp, i32, vp, vp]
    L.oracle_expert_ffn.restype = i32
    L.oracle_tail.argtypes = [vp, i32, i32, i32, vp, i32, vp, vp, i32, vp]
    L.oracle_tail.restype = i32
    L.oracle_rmsnorm.argtypes = [vp, i32, i32, vp, i32, ctypes.c_double, vp]
    L.oracle_rmsnorm.restype = i32
    L.oracle_round_to_dtype.argtypes = [vp, ctypes.c_size_t, i32]
    L.oracle_round_to_dtype.restype = i32
    L.oracle_unpack_row.argtypes = [vp, i32, i64, vp]
    L.oracle_unpack_row.restype = None
    L.oracle_dequant_row.argtypes = [ctypes.POINTER(_QMat), i64, i64, vp]
    L.oracle_dequant_row.restype = None
    L.oracle_decode_value.argtypes = [vp, i32, i64]
    L.oracle_decode_value.restype = ctypes.c_double
    L.oracle_num_threads.restype = i32
    L.oracle_set_num_threads.argtypes = [i32]
    return L


def lib():
    global _lib
    if _lib is None:
        path = os.environ.get("MOE_ORACLE_LIB", LIB)
        if path == LIB and not os.path.exists(LIB):
            build()
        _lib = _load(path)
    return _lib


def use_library(path: Optional[str]):
    """Swap the loaded oracle library (None restores the default); returns the previous handle.

    Used only by the mutation tests, which compile deliberately broken copies
    of the oracle source and check that the pins reject them.
    """
    global _lib
    old = _lib
    _lib = _load(path if path is not None else LIB)
    return old


def restore_library(handle) -> None:
    global _lib
    _lib = handle


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype=None):
    a = np.ascontiguousarray(a if dtype is None else np.asarray(a, dtype=dtype))
    return a


def _qmat(stack) -> _QMat:
    q, s, b = _c(stack.q, np.uint32), _c(stack.scales, np.uint16), _c(stack.biases, np.uint16)
    m = _QMat(q.ctypes.data, s.ctypes.data, b.ctypes.data, q.shape[0], stack.rows,
              stack.cols, stack.bits, DTYPE_CODE[stack.sb_dtype])
    m._keep = (q, s, b)  # keep the buffers alive with the struct
    return m


def num_threads() -> int:
    return lib().oracle_num_threads()


def set_num_threads(n: int) -> None:
    lib().oracle_set_num_threads(n)


def unpack_row(words: np.ndarray, bits: int, cols: int) -> np.ndarray:
    w = _c(words, np.uint32)
    out = np.empty(cols, np.uint32)
    lib().oracle_unpack_row(_p(w), bits, cols, _p(out))
    return out


def dequant_row(stack, expert: int, row: int) -> np.ndarray:
    m = _qmat(stack)
    out = np.empty(stack.cols, np.float64)
    lib().oracle_dequant_row(ctypes.byref(m), expert, row, _p(out))
    return out


def decode(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of an encoded array (element by element through the oracle)."""
    a = _c(a)
    flat = a.reshape(-1)
    out = np.array([lib().oracle_decode_value(_p(flat), DTYPE_CODE[dtype], i)
                    for i in range(flat.size)], np.float64)
    return out.reshape(a.shape)


def route(x, x_dtype, w_router, wr_dtype, top_k, renormalize, w_shared_gate=None,
          wg_dtype="bf16"):
    """Router logits, softmax, top-k ids and scores (and the shared gate) per token."""
    x = _c(x)
    if x.ndim == 1:
        x = x[None]
    T, d_in = x.shape
    wr = _c(w_router)
    E = wr.shape[0]
    logits = np.empty((T, E)); probs = np.empty((T, E))
    ids = np.empty((T, top_k), np.int32); scores = np.empty((T, top_k))
    gate = np.empty(T) if w_shared_gate is not None else None
    wg = None if w_shared_gate is None else _c(w_shared_gate)
    rc = lib().oracle_route(_p(x), DTYPE_CODE[x_dtype], T, d_in, _p(wr), DTYPE_CODE[wr_dtype],
                            E, top_k, int(bool(renormalize)), _p(wg), DTYPE_CODE[wg_dtype],
                            _p(logits), _p(probs), _p(ids), _p(scores), _p(gate))
    if rc != 0:
        raise ValueError("oracle_route: invalid sizes")
    return dict(logits=logits, probs=probs, ids=ids, scores=scores, gate=gate)


def expert_ffn(x, x_dtype, gate, up, down, ids, scores=None):
    """act [T, K, d_ff] and partial [T, K, d_in] for the given ids/scores."""
    x = _c(x)
    if x.ndim == 1:
        x = x[None]
    T, d_in = x.shape
    ids = _c(ids, np.int32).reshape(T, -1)
    K = ids.shape[1]
    d_ff = gate.rows
    sc = None if scores is None else _c(scores, np.float64).reshape(T, K)
    act = np.empty((T, K, d_ff)); partial = np.empty((T, K, d_in))
    g, u, d = _qmat(gate), _qmat(up), _qmat(down)
    rc = lib().oracle_expert_ffn(_p(x), DTYPE_CODE[x_dtype], T, d_in, d_ff, ctypes.byref(g),
                                 ctypes.byref(u), ctypes.byref(d), _p(ids), _p(sc), K,
                                 _p(act), _p(partial))
    if rc != 0:
        raise ValueError("oracle_expert_ffn: inconsistent shapes")
    return dict(act=act, partial=partial)


def tail(partial, resid, resid_dtype, shared=None, gate=None):
    """out [T, d_in] = resid + (sum_k partial + sum_s shared * gate)."""
    partial = _c(partial, np.float64)
    T, K, d_in = partial.shape
    resid = _c(resid).reshape(T, d_in)
    S = 0
    sh = None
    if shared is not None:
        sh = _c(shared, np.float64).reshape(T, -1, d_in)
        S = sh.shape[1]
    gt = None if gate is None else _c(gate, np.float64).reshape(T)
    out = np.empty((T, d_in))
    rc = lib().oracle_tail(_p(partial), T, K, d_in, _p(sh), S, _p(gt), _p(resid),
                           DTYPE_CODE[resid_dtype], _p(out))
    if rc != 0:
        raise ValueError("oracle_tail: invalid sizes")
    return out


def rmsnorm(y, weight, w_dtype, eps):
    """The next layer's RMSNorm of the layer output y [T, d] (float64):
    y / sqrt(mean(y^2) + eps) * weight, per token; weight [d] encoded in w_dtype."""
    y = _c(y, np.float64)
    if y.ndim == 1:
        y = y[None]
    T, d = y.shape
    w = _c(weight)
    out = np.empty((T, d))
    rc = lib().oracle_rmsnorm(_p(y), T, d, _p(w), DTYPE_CODE[w_dtype], float(eps), _p(out))
    if rc != 0:
        raise ValueError("oracle_rmsnorm: invalid sizes")
    return out


def round_to(values, dtype):
    """values (float64) rounded to the nearest value of dtype ("f32" leaves them
    as they are; "bf16", "f16": ties to even, overflow to infinity), as float64."""
    v = np.array(values, dtype=np.float64, copy=True, order="C")
    rc = lib().oracle_round_to_dtype(_p(v), v.size, DTYPE_CODE[dtype])
    if rc != 0:
        raise ValueError(f"oracle_round_to_dtype: dtype {dtype}")
    return v


def layer(cfg, weights: dict, x, resid, ids=None, scores=None):
    """The whole layer for the tokens in x: route -> routed experts -> shared -> tail.

    `weights` is what ``moe_inputs.gen_layer_weights`` returns.  When `ids`
    and `scores` are given they replace the routing result (used to feed
    identical routing to both sides).
    """
    r = route(x, cfg.x_dtype, weights["router"], cfg.router_dtype, cfg.top_k,
              cfg.renormalize, weights.get("shared_gate_w"))
    use_ids = r["ids"] if ids is None else ids
    use_scores = r["scores"] if scores is None else scores
    f = expert_ffn(x, cfg.x_dtype, weights["gate"], weights["up"], weights["down"],
                   use_ids, use_scores)
    shared = None
    sf = None
    if cfg.n_shared:
        T = f["act"].shape[0]
        sids = np.tile(np.arange(cfg.n_shared, dtype=np.int32), (T, 1))
        sf = expert_ffn(x, cfg.x_dtype, weights["shared_gate_proj"], weights["shared_up"],
                        weights["shared_down"], sids, None)
        shared = sf["partial"]
    gate = r["gate"] if cfg.shared_gate else None
    out = tail(f["partial"], resid, cfg.resid_dtype, shared, gate)
    return dict(route=r, ffn=f, shared=sf, out=out)


def selected_weights(cfg, layer_idx, x):
    """The weights layer() needs for the tokens in x on layer `layer_idx` of a
    seeded workload, generating (with the shared input generator) only the
    experts this oracle's routing selects, so that the routed stacks of a
    full-size layer need not be on the host: returns (weights, ids, scores)
    where the routed stacks' entry i is expert sel[i] and ids are positions
    in that list, for layer(..., ids=ids, scores=scores)."""
    import moe_inputs as mi
    r = route(x, cfg.x_dtype, mi.gen_router(cfg, layer_idx), cfg.router_dtype, cfg.top_k,
              cfg.renormalize)
    sel = sorted(set(int(e) for e in r["ids"].reshape(-1)))
    w = mi.gen_layer_weights_for(cfg, layer_idx, sel)
    pos = {e: i for i, e in enumerate(sel)}
    sub_ids = np.vectorize(pos.get)(r["ids"]).astype(np.int32)
    return w, sub_ids, r["scores"]


def layer_selected(cfg, layer_idx, x, resid):
    """layer() for layer `layer_idx` of a seeded workload on the selected experts
    only (selected_weights); the route result keeps the true expert ids."""
    w, sub_ids, scores = selected_weights(cfg, layer_idx, x)
    return layer(cfg, w, x, resid, ids=sub_ids, scores=scores)
