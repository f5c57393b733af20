"""CPU tests of the C ABI: the library loads, exports every declared symbol, and
rejects invalid arguments on the host before anything is enqueued.

Every call here carries at least one flaw that host validation catches, so no
kernel is ever launched (the pointers are placeholders and are never read).
"""
import ctypes
import os
import re

import pytest

import quantized_moe_decode_amd as qmd
from quantized_moe_decode_amd import (CQMat, MOE_BF16, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_F16,
                                      MOE_F32, MOE_OK, lib)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_decode.h")

P = 0x10000          # placeholder "device" address, 16-byte aligned, never dereferenced
MIS = 0x10008        # misaligned placeholder


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_decode_\w+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("moe_decode_route", "moe_decode_expert_ffn", "moe_decode_tail",
              "moe_decode_gate_up", "moe_decode_down"):
        assert n in names


@pytest.mark.parametrize("name", declared_functions())
def test_library_exports_declared_symbol(name):
    assert hasattr(lib, name), name


def test_abi_version_and_status_strings():
    assert qmd.abi_version() == 4
    for code in (0, 1, 2, 3, 4):
        assert qmd.status_string(code).startswith("MOE_")
    assert "unknown" in qmd.status_string(99)


def test_workspace_status_reads_the_error_word():
    """moe_decode_workspace_status interprets a host copy of a workspace's head:
    a zero error word is MOE_OK, any nonzero one MOE_ETIMEOUT; too short or null
    heads are rejected."""
    f = lib.moe_decode_workspace_status
    for word, want in ((0, MOE_OK), (1, qmd.MOE_ETIMEOUT), (0x80000000, qmd.MOE_ETIMEOUT)):
        head = (ctypes.c_uint32 * 4)(word, 0, 0, 0)
        assert f(ctypes.cast(head, ctypes.c_void_p), 16) == want
        assert f(ctypes.cast(head, ctypes.c_void_p), qmd.MOE_WORKSPACE_HEAD_BYTES) == want
    head = (ctypes.c_uint32 * 1)(0)
    assert f(ctypes.cast(head, ctypes.c_void_p), qmd.MOE_WORKSPACE_HEAD_BYTES - 1) == MOE_EINVAL
    assert f(None, 16) == MOE_EINVAL


def test_workspace_sizes():
    assert qmd.route_workspace_bytes(1, 128) >= (128 + 1) * 8          # one tagged 64-bit word per logit
    assert qmd.route_workspace_bytes(32, 1024) >= 32 * 1025 * 8
    assert qmd.route_workspace_bytes(0, 8) == 0
    assert qmd.expert_ffn_workspace_bytes(1, 8, 128) == 0
    mw = min(32 * 8, 128) + 1
    assert qmd.expert_ffn_workspace_bytes(32, 8, 128) >= (1 + mw + mw + 1 + 256) * 4


def _route(**kw):
    a = dict(x=P, x_dt=MOE_BF16, T=1, d_in=2048, wr=P, wr_dt=MOE_BF16, E=128, K=8, renorm=1,
             wg=None, wg_dt=MOE_BF16, ids=P, scores=P, gate=None, ws=P, ws_bytes=1 << 20)
    a.update(kw)
    return lib.moe_decode_route(a["x"], a["x_dt"], a["T"], a["d_in"], a["wr"], a["wr_dt"], a["E"],
                                a["K"], a["renorm"], a["wg"], a["wg_dt"], a["ids"], a["scores"],
                                a["gate"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(x=None), MOE_EINVAL),
    (dict(ids=None), MOE_EINVAL),
    (dict(ws=None), MOE_EINVAL),
    (dict(T=0), MOE_EINVAL),
    (dict(T=1025), MOE_EINVAL),
    (dict(K=0), MOE_EINVAL),
    (dict(K=33), MOE_EINVAL),
    (dict(E=4, K=5), MOE_EINVAL),
    (dict(E=1025), MOE_EINVAL),
    (dict(d_in=100), MOE_EINVAL),
    (dict(d_in=8192 + 64), MOE_EINVAL),
    (dict(wg=P), MOE_EINVAL),              # shared-gate vector without an output
    (dict(gate=P), MOE_EINVAL),            # output without a shared-gate vector
    (dict(x=MIS), MOE_EINVAL),
    (dict(ws_bytes=16), MOE_EINVAL),
    (dict(x_dt=7), MOE_EUNSUPPORTED),
    (dict(wr_dt=-1), MOE_EUNSUPPORTED),
])
def test_route_rejects(kw, want):
    assert _route(**kw) == want


def _qm(**kw):
    a = dict(q=P, s=P, b=P, E=128, rows=768, cols=2048, bits=4, gs=64, dt=MOE_BF16)
    a.update(kw)
    return CQMat(a["q"], a["s"], a["b"], a["E"], a["rows"], a["cols"], a["bits"], a["gs"], a["dt"])


def _ffn(gate=None, up=None, down=None, **kw):
    a = dict(x=P, x_dt=MOE_BF16, T=1, ids=P, scores=P, K=8, act=P, partial=P, ws=None, ws_bytes=0)
    a.update(kw)
    g = gate or _qm()
    u = up or _qm()
    d = down or _qm(rows=2048, cols=768)
    return lib.moe_decode_expert_ffn(a["x"], a["x_dt"], a["T"], ctypes.byref(g), ctypes.byref(u),
                                     ctypes.byref(d), a["ids"], a["scores"], a["K"], a["act"],
                                     a["partial"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("case,want", [
    (dict(x=None), MOE_EINVAL),
    (dict(act=None), MOE_EINVAL),
    (dict(T=0), MOE_EINVAL),
    (dict(T=2), MOE_EINVAL),                                   # several tokens need a workspace
    (dict(K=0), MOE_EINVAL),
    (dict(K=40), MOE_EINVAL),
    (dict(x=MIS), MOE_EINVAL),
    (dict(x_dt=5), MOE_EUNSUPPORTED),
    (dict(gate=_qm(bits=5)), MOE_EUNSUPPORTED),
    (dict(gate=_qm(bits=2)), MOE_EUNSUPPORTED),
    (dict(down=_qm(rows=2048, cols=768, gs=32)), MOE_EUNSUPPORTED),
    (dict(down=_qm(rows=2048, cols=768, dt=MOE_F32)), MOE_EUNSUPPORTED),
    (dict(up=_qm(bits=8)), MOE_EUNSUPPORTED),                  # gate and up must share bits
    (dict(up=_qm(dt=MOE_F16)), MOE_EUNSUPPORTED),              # one scale dtype per call
    (dict(up=_qm(rows=512)), MOE_EINVAL),
    (dict(down=_qm(rows=2048, cols=512)), MOE_EINVAL),
    (dict(down=_qm(rows=1024, cols=768)), MOE_EINVAL),
    (dict(down=_qm(rows=2048, cols=768, E=64)), MOE_EINVAL),
    (dict(gate=_qm(cols=2000), up=_qm(cols=2000)), MOE_EINVAL),
    (dict(gate=_qm(q=MIS)), MOE_EINVAL),
    (dict(gate=_qm(q=None)), MOE_EINVAL),
    (dict(gate=_qm(E=0)), MOE_EINVAL),
    (dict(gate=_qm(rows=16384), up=_qm(rows=16384)), MOE_EINVAL),
])
def test_expert_ffn_rejects(case, want):
    assert _ffn(**case) == want


def _grouped(gate=None, up=None, down=None, **kw):
    a = dict(x=P, x_dt=MOE_BF16, T=256, ids=P, scores=P, K=8, act=P, partial=P, ws=P, ws_bytes=1 << 20)
    a.update(kw)
    g, u = gate or _qm(), up or _qm()
    d = down or _qm(rows=2048, cols=768)
    return lib.moe_decode_expert_ffn_grouped(a["x"], a["x_dt"], a["T"], ctypes.byref(g), ctypes.byref(u),
                                             ctypes.byref(d), a["ids"], a["scores"], a["K"], a["act"],
                                             a["partial"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("case,want", [
    (dict(x=None), MOE_EINVAL),
    (dict(ids=None), MOE_EINVAL),
    (dict(partial=None), MOE_EINVAL),
    (dict(ws=None), MOE_EINVAL),
    (dict(T=0), MOE_EINVAL),
    (dict(T=1025), MOE_EINVAL),
    (dict(K=0), MOE_EINVAL),
    (dict(K=33), MOE_EINVAL),
    (dict(x=MIS), MOE_EINVAL),
    (dict(act=P + 4), MOE_EINVAL),
    (dict(ws=P + 8), MOE_EINVAL),
    (dict(ws_bytes=64), MOE_EINVAL),
    (dict(x_dt=MOE_F16), MOE_EUNSUPPORTED),                    # bf16 x only
    (dict(down=_qm(rows=2048, cols=768, bits=6)), MOE_EUNSUPPORTED),
    (dict(gate=_qm(bits=8), up=_qm(bits=8)), MOE_EUNSUPPORTED),
    (dict(down=_qm(rows=2048, cols=768, dt=MOE_F16)), MOE_EUNSUPPORTED),   # one scale dtype per call
    (dict(up=_qm(rows=512)), MOE_EINVAL),
    (dict(down=_qm(rows=1024, cols=768)), MOE_EINVAL),
    (dict(down=_qm(rows=2048, cols=768, E=64)), MOE_EINVAL),
    (dict(gate=_qm(E=2000), up=_qm(E=2000), down=_qm(rows=2048, cols=768, E=2000)), MOE_EINVAL),
])
def test_expert_ffn_grouped_rejects(case, want):
    assert _grouped(**case) == want


def test_token_limits_match_the_header():
    h = open(HEADER).read()
    for name in ("MOE_MAX_TOKENS", "MOE_MAX_GROUPED_TOKENS"):
        assert int(re.search(rf"#define {name} (\d+)", h).group(1)) == getattr(qmd, name)


def test_grouped_workspace_bytes():
    """The head (error word, work-item count, unit counter, one spare word),
    the work lists (expert, first pair and pair count per work item, at most
    ceil(pairs / 16) + n_experts + 1 items), one counter per work item and the
    pair list, int32; then the fp16 copy of act and one fp32 factor per pair
    and block of 128 act values, each 256-byte aligned."""
    f = qmd.expert_ffn_grouped_workspace_bytes
    for T, K, E, F in [(1, 1, 1, 64), (256, 8, 128, 768), (1024, 32, 1024, 8192), (17, 3, 9, 704)]:
        mw = (T * K + 15) // 16 + E + 1
        need = (4 + 4 * mw + T * K) * 4 + T * K * F * 2 + T * K * ((F + 127) // 128) * 4
        assert need <= f(T, K, E, F) <= need + 3 * 256 and f(T, K, E, F) % 256 == 0
    assert f(0, 8, 128, 768) == 0 and f(4, 0, 128, 768) == 0 and f(4, 8, 0, 768) == 0 and f(4, 8, 8, 0) == 0


def _gate_up(gate=None, up=None, **kw):
    a = dict(x=P, x_dt=MOE_BF16, T=1, ids=P, K=8, act=P, ws=None, ws_bytes=0)
    a.update(kw)
    g, u = gate or _qm(), up or _qm()
    return lib.moe_decode_gate_up(a["x"], a["x_dt"], a["T"], ctypes.byref(g), ctypes.byref(u),
                                  a["ids"], a["K"], a["act"], a["ws"], a["ws_bytes"], None)


def _down(down=None, **kw):
    a = dict(act=P, T=1, ids=P, scores=P, K=8, partial=P, ws=None, ws_bytes=0)
    a.update(kw)
    d = down or _qm(rows=2048, cols=768)
    return lib.moe_decode_down(a["act"], a["T"], ctypes.byref(d), a["ids"], a["scores"], a["K"],
                               a["partial"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("case,want", [
    (dict(x=None), MOE_EINVAL),
    (dict(ids=None), MOE_EINVAL),
    (dict(act=None), MOE_EINVAL),
    (dict(act=MIS), MOE_EINVAL),
    (dict(T=40), MOE_EINVAL),
    (dict(T=3), MOE_EINVAL),
    (dict(x_dt=9), MOE_EUNSUPPORTED),
    (dict(up=_qm(bits=6)), MOE_EUNSUPPORTED),
    (dict(up=_qm(rows=64)), MOE_EINVAL),
    (dict(gate=_qm(gs=128)), MOE_EUNSUPPORTED),
])
def test_gate_up_rejects(case, want):
    assert _gate_up(**case) == want


@pytest.mark.parametrize("case,want", [
    (dict(act=None), MOE_EINVAL),
    (dict(partial=None), MOE_EINVAL),
    (dict(ids=None), MOE_EINVAL),
    (dict(K=0), MOE_EINVAL),
    (dict(T=2, ws=P, ws_bytes=8), MOE_EINVAL),
    (dict(down=_qm(rows=2048, cols=768, bits=7)), MOE_EUNSUPPORTED),
    (dict(down=_qm(rows=2048, cols=768, q=MIS)), MOE_EINVAL),
])
def test_down_rejects(case, want):
    assert _down(**case) == want


def _lw(**kw):
    a = dict(wr=P, wr_dt=MOE_BF16, E=128, K=8, renorm=1, gate=_qm(), up=_qm(),
             down=_qm(rows=2048, cols=768), S=0, sg=qmd.CQMat(), su=qmd.CQMat(), sd=qmd.CQMat(),
             wg=None)
    a.update(kw)
    return qmd.CLayerWeights(a["wr"], a["wr_dt"], a["E"], a["K"], a["renorm"], a["gate"], a["up"],
                             a["down"], a["S"], a["sg"], a["su"], a["sd"], a["wg"])


def _layer(w=None, **kw):
    a = dict(x=P, x_dt=MOE_BF16, resid=P, rdt=MOE_BF16, out=P, odt=MOE_F32, ws=P, ws_bytes=1 << 30)
    a.update(kw)
    w = w or _lw()
    return lib.moe_decode_layer(ctypes.byref(w), a["x"], a["x_dt"], a["resid"], a["rdt"], a["out"], a["odt"],
                                None, None, None, a["ws"], a["ws_bytes"], None)


def test_layer_workspace_bytes():
    n = qmd.layer_workspace_bytes(_lw())
    assert n >= (8 * 768 + 8 * 2048 + 129) * 4
    assert qmd.layer_workspace_bytes(_lw(K=0)) == 0
    shared = dict(S=1, sg=_qm(E=1, rows=5632), su=_qm(E=1, rows=5632), sd=_qm(E=1, rows=2048, cols=5632))
    assert qmd.layer_workspace_bytes(_lw(**shared)) > n


@pytest.mark.parametrize("case,want", [
    (dict(x=None), MOE_EINVAL),
    (dict(out=None), MOE_EINVAL),
    (dict(ws=None), MOE_EINVAL),
    (dict(ws_bytes=64), MOE_EINVAL),
    (dict(x=MIS), MOE_EINVAL),
    (dict(x_dt=6), MOE_EUNSUPPORTED),
    (dict(x_dt=MOE_F32), MOE_EUNSUPPORTED),                   # router dtype must match x
    (dict(odt=3), MOE_EUNSUPPORTED),
    (dict(out=P + 2), MOE_EINVAL),                            # fp32 out not 4-byte aligned
    (dict(out=P + 1, odt=MOE_BF16), MOE_EINVAL),              # bf16 out not 2-byte aligned
    (dict(w=_lw(wr=None)), MOE_EINVAL),
    (dict(w=_lw(K=0)), MOE_EINVAL),
    (dict(w=_lw(K=33)), MOE_EINVAL),
    (dict(w=_lw(E=64)), MOE_EINVAL),                          # n_experts must match the stacks
    (dict(w=_lw(up=_qm(bits=8))), MOE_EUNSUPPORTED),
    (dict(w=_lw(down=_qm(rows=2048, cols=768, dt=MOE_F16))), MOE_EUNSUPPORTED),
    (dict(w=_lw(wg=P)), MOE_EINVAL),                          # shared gate without shared experts
    (dict(w=_lw(S=9)), MOE_EINVAL),
    (dict(w=_lw(S=1, sg=_qm(E=1, rows=512), su=_qm(E=1, rows=512), sd=_qm(E=1, rows=2048, cols=768))),
     MOE_EINVAL),                                             # shared d_ff inconsistent
    (dict(w=_lw(S=1, sg=_qm(E=1, bits=8), su=_qm(E=1, bits=8), sd=_qm(E=1, rows=2048, cols=768))),
     MOE_EUNSUPPORTED),                                       # shared bits differ from routed
    (dict(w=_lw(S=2, sg=_qm(E=1), su=_qm(E=1), sd=_qm(E=1, rows=2048, cols=768))), MOE_EINVAL),
])
def test_layer_rejects(case, want):
    assert _layer(**case) == want


def _tail(**kw):
    a = dict(partial=P, T=1, K=8, D=2048, shared=None, S=0, gate=None, resid=P, rdt=MOE_BF16, out=P,
             odt=MOE_F32)
    a.update(kw)
    return lib.moe_decode_tail(a["partial"], a["T"], a["K"], a["D"], a["shared"], a["S"], a["gate"],
                               a["resid"], a["rdt"], a["out"], a["odt"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(partial=None), MOE_EINVAL),
    (dict(out=None), MOE_EINVAL),
    (dict(T=0), MOE_EINVAL),
    (dict(T=1025), MOE_EINVAL),
    (dict(K=0), MOE_EINVAL),
    (dict(D=96), MOE_EINVAL),
    (dict(S=1), MOE_EINVAL),             # shared count without the buffer
    (dict(shared=P), MOE_EINVAL),        # buffer without a count
    (dict(S=-1, shared=P), MOE_EINVAL),
    (dict(rdt=3), MOE_EUNSUPPORTED),
    (dict(odt=-1), MOE_EUNSUPPORTED),
    (dict(out=P + 2), MOE_EINVAL),
    (dict(out=P + 1, odt=MOE_F16), MOE_EINVAL),
])
def test_tail_rejects(kw, want):
    assert _tail(**kw) == want


def _norm(**kw):
    a = dict(weight=P, dt=MOE_BF16, eps=1e-6, normed=P, ndt=MOE_F32)
    a.update(kw)
    return qmd.CRMSNorm(a["weight"], a["dt"], a["eps"], a["normed"], a["ndt"])


@pytest.mark.parametrize("kw,want", [
    (dict(weight=None), MOE_EINVAL),
    (dict(normed=None), MOE_EINVAL),
    (dict(dt=7), MOE_EUNSUPPORTED),
    (dict(ndt=7), MOE_EUNSUPPORTED),
    (dict(eps=-1.0), MOE_EINVAL),
    (dict(eps=float("nan")), MOE_EINVAL),
    (dict(eps=float("inf")), MOE_EINVAL),
    (dict(weight=P + 1), MOE_EINVAL),                    # bf16 weight not 2-byte aligned
    (dict(normed=P + 2), MOE_EINVAL),                    # fp32 normed not 4-byte aligned
    (dict(normed=P + 1, ndt=MOE_BF16), MOE_EINVAL),
])
def test_rmsnorm_descriptor_rejected_by_every_entry_point(kw, want):
    """The same checks of the RMSNorm descriptor in the separate call, the
    folded three-call tail and the folded fused layer."""
    n = _norm(**kw)
    assert lib.moe_decode_rmsnorm(P, MOE_F32, 1, 2048, ctypes.byref(n), None) == want
    assert lib.moe_decode_tail_rmsnorm(P, 1, 8, 2048, None, 0, None, P, MOE_BF16, P, MOE_F32,
                                       ctypes.byref(n), P, 1 << 20, None) == want
    w = _lw()
    assert lib.moe_decode_layer_rmsnorm(ctypes.byref(w), P, MOE_BF16, P, MOE_BF16, P, MOE_F32,
                                        ctypes.byref(n), None, None, None, P, 1 << 30, None) == want


@pytest.mark.parametrize("kw,want", [
    (dict(y=None), MOE_EINVAL),
    (dict(ydt=9), MOE_EUNSUPPORTED),
    (dict(y=P + 1, ydt=MOE_BF16), MOE_EINVAL),
    (dict(T=0), MOE_EINVAL),
    (dict(T=1025), MOE_EINVAL),
    (dict(d=0), MOE_EINVAL),
])
def test_rmsnorm_rejects(kw, want):
    a = dict(y=P, ydt=MOE_F32, T=1, d=2048)
    a.update(kw)
    n = _norm()
    assert lib.moe_decode_rmsnorm(a["y"], a["ydt"], a["T"], a["d"], ctypes.byref(n), None) == want


@pytest.mark.parametrize("data,nbytes,out,n,want", [
    (None, 4096, P, 64, MOE_EINVAL),
    (P, 4096, None, 64, MOE_EINVAL),
    (P, 0, P, 64, MOE_EINVAL),
    (P, 4100, P, 64, MOE_EINVAL),           # not a multiple of 16 bytes
    (P + 8, 4096, P, 64, MOE_EINVAL),       # not 16-byte aligned
    (P, 1 << 30, P, 1, MOE_EINVAL),         # too few partial sums for the grid
])
def test_read_probe_rejects(data, nbytes, out, n, want):
    assert lib.moe_decode_read_probe(data, nbytes, out, n, None) == want


def test_read_probe_blocks():
    assert lib.moe_decode_read_probe_blocks(0) == 0
    assert lib.moe_decode_read_probe_blocks(16) == 1
    assert 1 <= lib.moe_decode_read_probe_blocks(1 << 30) <= 4096


def test_binding_raises_on_error():
    """The Python layer turns a status into MoeError (host-side rejection, no launch)."""
    import torch
    x = torch.zeros(1, 100, dtype=torch.bfloat16)          # d_in not a multiple of 64
    with pytest.raises(qmd.MoeError) as ei:
        qmd.moe_decode_route(x, torch.zeros(8, 100, dtype=torch.bfloat16), 2, True,
                             torch.zeros(1, 2, dtype=torch.int32), torch.zeros(1, 2),
                             torch.zeros(4096, dtype=torch.uint8), stream=_FakeStream())
    assert ei.value.status == MOE_EINVAL
    assert MOE_OK == 0


class _FakeStream:
    cuda_stream = 0


def test_noalloc_rejects_invalid_calls_on_the_host():
    """moe_decode_expert_ffn_noalloc validates like moe_decode_expert_ffn, before
    it looks up its device array: these calls never reach the device."""
    f = lib.moe_decode_expert_ffn_noalloc
    g = _qm(rows=768, cols=2048)
    d = _qm(rows=2048, cols=768)
    args = lambda T, gate=g: (P, MOE_BF16, T, ctypes.byref(gate) if gate is not None else None,
                              ctypes.byref(g), ctypes.byref(d), P, P, 8, P, P, None)
    assert f(*args(2, gate=None)) == MOE_EINVAL          # null stack
    assert f(*args(33)) == MOE_EINVAL                   # more tokens than the limit
    assert f(*args(0)) == MOE_EINVAL
    assert qmd.expert_ffn_noalloc_max_bytes() == qmd.expert_ffn_workspace_bytes(32, 32, 1024)
