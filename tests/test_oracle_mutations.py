"""CPU tests: deliberately broken copies of the oracle must each fail at least one pin.

Each mutation is a plausible mistake (a dropped term, a wrong sign, a wrong
or transposed index, a swapped operand).  The copy is compiled to a temporary
library, swapped in, and the pins are run until one rejects it.  This shows
that the pins constrain every step of the oracle, not only its happy path.
All mutated indices stay inside the arrays they read.
"""
import os
import subprocess

import pytest

import oracle
import oracle_pins

MUTATIONS = [
    ("drop the bias", "return s * (double)code_at(row, m->bits, j) + b;",
     "return s * (double)code_at(row, m->bits, j);"),
    ("bias sign", "return s * (double)code_at(row, m->bits, j) + b;",
     "return s * (double)code_at(row, m->bits, j) - b;"),
    ("neighbouring scale group", "groups + j / 64);", "groups + (j / 64 + 1) % groups);"),
    ("scale row ignored", "size_t gi = (size_t)((e * m->rows + r) * groups",
     "size_t gi = (size_t)((e * m->rows) * groups"),
    ("no 6-bit straddle", "if (sh + (uint64_t)bits > 32)", "if (0)"),
    ("swapped neighbouring codes", "uint64_t bit = (uint64_t)bits * (uint64_t)j;",
     "uint64_t bit = (uint64_t)bits * (uint64_t)(j ^ 1);"),
    ("sigmoid sign", "return 1.0 / (1.0 + exp(-z));", "return 1.0 / (1.0 + exp(z));"),
    ("swiglu operands swapped", "a[r] = g * sigmoid(g) * u;", "a[r] = u * sigmoid(u) * g;"),
    ("gate used for up", "double u = qrow_dot(up, e, r, xv);", "double u = qrow_dot(gp, e, r, xv);"),
    ("score dropped", "o[i] = s * qrow_dot(dp, e, i, a);", "o[i] = qrow_dot(dp, e, i, a);"),
    ("renormalisation dropped", "sc[k] = renormalize ? p[id[k]] / sel : p[id[k]];",
     "sc[k] = p[id[k]];"),
    ("softmax not normalised", "p[e] /= z;", "p[e] /= 1.0;"),
    ("tie goes to the higher index", "if (best < 0 || l[e] > l[best])",
     "if (best < 0 || l[e] >= l[best])"),
    ("ascending top-k", "if (best < 0 || l[e] > l[best])", "if (best < 0 || l[e] < l[best])"),
    ("router operand transposed", "load_val(wr, wr_dt, (size_t)e * d_in + j)",
     "load_val(wr, wr_dt, (size_t)j * n_experts + e)"),
    ("shared gate without sigmoid", "gate[t] = sigmoid(acc);", "gate[t] = acc;"),
    ("every token reads token 0", "xv[j] = load_val(x, x_dt, (size_t)t * d_in + j);",
     "xv[j] = load_val(x, x_dt, (size_t)j);"),
    ("gate scales the routed sum", "(routed + sh * gv)", "(routed * gv + sh)"),
    ("residual dropped", "load_val(resid, resid_dt, (size_t)t * d_in + i) + (routed + sh * gv)",
     "(routed + sh * gv)"),
    ("only the last shared expert", "sh += shared[", "sh = shared["),
    ("only the last slot", "routed += partial[", "routed = partial["),
    ("fp16 exponent off by one", "expo - 25", "expo - 24"),
    ("bf16 decode shifted", "uint32_t u = (uint32_t)b << 16;", "uint32_t u = (uint32_t)b << 15;"),
    ("rmsnorm sum instead of mean", "double ms = ss / (double)d;", "double ms = ss;"),
    ("rmsnorm eps outside the root", "double inv = 1.0 / sqrt(ms + eps);", "double inv = 1.0 / (sqrt(ms) + eps);"),
    ("rmsnorm weight dropped", "yt[i] * inv * load_val(weight, w_dt, (size_t)i);", "yt[i] * inv;"),
    ("rmsnorm weight reversed", "load_val(weight, w_dt, (size_t)i);", "load_val(weight, w_dt, (size_t)(d - 1 - i));"),
    ("rounding truncates", "double r = rint(x / q) * q;", "double r = trunc(x / q) * q;"),
    ("rounding ties away from zero", "double r = rint(x / q) * q;", "double r = round(x / q) * q;"),
    ("rounding one significand bit short", "const double q = ldexp(1.0, e - p + 1);",
     "const double q = ldexp(1.0, e - p + 2);"),
    ("rounding without subnormals", "        if (e < emin)\n            e = emin;\n", ""),
    ("rounding never overflows", "            r = copysign(INFINITY, x);", "            r = copysign(vmax, x);"),
    ("bf16 rounded as binary16", "p = 8; emin = -126; emax = 127;", "p = 11; emin = -14; emax = 15;"),
    ("rmsnorm first token's mean for all", "const double *yt = y + (size_t)t * d;\n        double ss = 0.0;\n        for (int i = 0; i < d; ++i)\n            ss += yt[i] * yt[i];",
     "const double *yt = y + (size_t)t * d;\n        double ss = 0.0;\n        for (int i = 0; i < d; ++i)\n            ss += y[i] * y[i];"),
]


@pytest.mark.parametrize("desc,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutant_is_rejected(desc, old, new, tmp_path):
    src = open(oracle.SRC).read()
    assert src.count(old) == 1, f"mutation anchor not unique: {old!r}"
    mutated = src.replace(old, new)
    c = tmp_path / "mutant.c"
    so = tmp_path / "libmutant.so"
    c.write_text(mutated)
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                           "-o", str(so), str(c), "-lm"])
    prev = oracle.use_library(str(so))
    caught = None
    try:
        for pin in oracle_pins.ALL_PINS:
            try:
                pin()
            except Exception as exc:  # AssertionError, or a ValueError from a shape check
                caught = (pin.__name__, type(exc).__name__)
                break
    finally:
        oracle.restore_library(prev)
    assert caught is not None, f"no pin rejects the mutant: {desc}"
