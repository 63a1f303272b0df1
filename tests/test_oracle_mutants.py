"""Plant plausible mistakes in a copy of the oracle's C source and check that
each one fails at least one pin (CPU only; the copies are built in a temporary
directory and never replace the real oracle).

This is what makes the pins worth trusting: a dropped term, a wrong operand,
a transposed index or a wrong layout in the recurrence must not survive them.
"""
import ctypes
import os
import subprocess
import types

import pytest

import oracle
import test_oracle_pins as pins

_SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "eq2-undecayed-state": ("pred += St[i * Dv + j] * k[i];", "pred += S[i * Dv + j] * k[i];"),
    "eq4-reads-pre-write-state": ("acc += S[i * Dv + j] * q[i];", "acc += St[i * Dv + j] * q[i];"),
    "eq2-error-sign": ("e[j] = v[j] - pred;", "e[j] = pred - v[j];"),
    "eq3-dropped-beta": ("beta * k[i] * e[j]", "k[i] * e[j]"),
    "eq3-query-instead-of-key": ("beta * k[i] * e[j]", "beta * q[i] * e[j]"),
    "eq1-dropped-decay": ("St[i * Dv + j] = alpha * S[i * Dv + j];", "St[i * Dv + j] = S[i * Dv + j];"),
    "eq4-transposed-state": ("acc += S[i * Dv + j] * q[i];", "acc += S[j * Dk + i] * q[i];"),
    "eq2-transposed-state": ("pred += St[i * Dv + j] * k[i];", "pred += St[j * Dk + i] * k[i];"),
    "wrong-token-layout": ("const int64_t row = (b * T + t) * H + h;", "const int64_t row = (b * H + h) * T + t;"),
    "shared-initial-state": ("memcpy(S, S0 + bh * Dk * Dv,", "memcpy(S, S0,"),
    "decay-squared": ("St[i * Dv + j] = alpha * S[i * Dv + j];", "St[i * Dv + j] = alpha * alpha * S[i * Dv + j];"),
}

PIN_TESTS = [getattr(pins, n) for n in dir(pins) if n.startswith("test_") and n != "test_threads_do_not_change_result"]


def _mutant_module(tmp_path, name, old, new):
    src = open(_SRC).read()
    assert src.count(old) >= 1, f"mutation anchor for {name} not found"
    path = tmp_path / f"{name}.c"
    path.write_text(src.replace(old, new, 1))
    so = tmp_path / f"{name}.so"
    subprocess.run(["gcc", "-O1", "-std=c99", "-fopenmp", "-fPIC", "-shared", str(path), "-o", str(so), "-lm"],
                   check=True)
    core = oracle._configure(ctypes.CDLL(str(so)))
    ns = types.SimpleNamespace(
        gdn_recurrence=lambda *a, **kw: oracle.gdn_recurrence(*a, _core=core, **kw),
        gdn_decode_step=lambda *a, **kw: oracle.gdn_decode_step(*a, _core=core, **kw),
        gdn_recurrence_bwd=lambda *a, **kw: oracle.gdn_recurrence_bwd(*a, _core=core, **kw),
    )
    return ns


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    mod = _mutant_module(tmp_path, name, old, new)
    caught = []
    for fn in PIN_TESTS:
        try:
            if "C" in fn.__code__.co_varnames[:fn.__code__.co_argcount]:
                fn(mod, 4, "R")
            else:
                fn(mod)
        except (AssertionError, ValueError):
            caught.append(fn.__name__)
    assert caught, f"mutant {name} passed every pin"


# Mistakes planted in the reverse mode; each must fail a pin of
# test_oracle_bwd_pins (finite differences, closed form, invariants).
BWD_MUTANTS = {
    "bwd-dq-pre-write-state": ("acc += S[i * Dv + j] * dyt[j];", "acc += St[i * Dv + j] * dyt[j];"),
    "bwd-dbeta-without-dS": ("db += kt[i] * dS[i * Dv + j] * e[j];", "db += kt[i] * e[j];"),
    "bwd-undecayed-adjoint": ("for (int64_t i = 0; i < SS; ++i) dS[i] *= a;", "(void)a;"),
    "bwd-dk-sign": ("dk[row * Dk + i] -= acc;", "dk[row * Dk + i] += acc;"),
    "bwd-dalpha-current-state": ("da += Sp[i] * dS[i];", "da += S[i] * dS[i];"),
    "bwd-readout-term-dropped": ("dS[i * Dv + j] += qt[i] * dyt[j];", "dS[i * Dv + j] += 0.0 * qt[i] * dyt[j];"),
    "bwd-de-without-beta": ("de[j] = bt * acc;", "de[j] = acc;"),
    "bwd-first-checkpoint-only": ("memcpy(S, ck + s * SS,", "memcpy(S, ck,"),
    "bwd-write-term-not-removed": ("dS[i * Dv + j] -= kt[i] * de[j];", "dS[i * Dv + j] -= 0.0 * kt[i] * de[j];"),
}


@pytest.mark.parametrize("name", sorted(BWD_MUTANTS))
def test_bwd_mutant_is_caught(tmp_path, name):
    import test_oracle_bwd_pins as bpins
    old, new = BWD_MUTANTS[name]
    core = _mutant_module(tmp_path, name, old, new)
    caught = []
    for n in dir(bpins):
        if not n.startswith("test_"):
            continue
        fn = getattr(bpins, n)
        try:
            if "shape" in fn.__code__.co_varnames[:fn.__code__.co_argcount]:
                fn(core, (1, 70, 1, 3, 2, 16))
            else:
                fn(core)
        except (AssertionError, ValueError):
            caught.append(n)
    assert caught, f"mutant {name} passed every pin"
