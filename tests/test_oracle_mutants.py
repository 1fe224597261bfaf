"""The pins must catch plausible mistakes in the oracle.

Each case plants one mistake in a copy of the oracle's C source (on the CPU,
in a temporary directory), builds it, swaps it in for the real library and
runs every pin of ``test_oracle.py``.  At least one pin has to fail for every
mutant; a mutant that passes all pins would mean the pins cannot tell that
mistake from the method.
"""
import ctypes
import inspect
import os
import subprocess

import pytest

import oracle
import test_oracle

SRC = os.path.join(os.path.dirname(oracle.__file__), "kda_oracle.c")


def _swap_write_and_readout(src):
    """Readout from the pre-write state: move the readout block before the write."""
    w0 = src.index("        /* write: S = S~ + e k^T */")
    r0 = src.index("        /* readout: o = S q */")
    r1 = src.index("    }\n}\n", r0)
    write_blk, read_blk = src[w0:r0], src[r0:r1]
    return src[:w0] + read_blk + write_blk + src[r1:]


MUTANTS = {
    "decay_sign": ("alpha[c] = exp(la[c]);", "alpha[c] = exp(-la[c]);"),
    "no_decay": ("S[i * dk + c] *= alpha[c];", "S[i * dk + c] *= 1.0;"),
    "decay_rows_not_columns": ("S[i * dk + c] *= alpha[c];", "S[i * dk + c] *= alpha[i % dk];"),
    "error_sign": ("beta * (v[i] - vhat[i])", "beta * (v[i] + vhat[i])"),
    "error_without_beta": (": beta * (v[i] - vhat[i]);", ": (v[i] - vhat[i]);"),
    "predict_with_q": ("acc += S[i * dk + c] * k[c];\n            vhat[i] = acc;",
                       "acc += S[i * dk + c] * q[c];\n            vhat[i] = acc;"),
    "write_with_q": ("S[i * dk + c] += err[i] * k[c];", "S[i * dk + c] += err[i] * q[c];"),
    "readout_with_k": ("acc += S[i * dk + c] * q[c];\n            o[i] = acc;",
                       "acc += S[i * dk + c] * k[c];\n            o[i] = acc;"),
    "readout_before_write": None,
    "token_stride": ("hv.tok_stride_k = H * dk;\n        hv.tok_stride_v = H * dv;\n        hv.tok_stride_b = H;\n        head_recurrence(&hv, dk, dv, write_mode, S, work);\n        if (S_final) memcpy(S_final + bh",
                     "hv.tok_stride_k = dk;\n        hv.tok_stride_v = H * dv;\n        hv.tok_stride_b = H;\n        head_recurrence(&hv, dk, dv, write_mode, S, work);\n        if (S_final) memcpy(S_final + bh"),
    "beta_head_index": ("hv.beta = beta + b * T * H + h;", "hv.beta = beta + b * T * H;"),
    "state_transposed_on_load": ("if (S0) memcpy(S, S0 + bh * dv * dk, sizeof(double) * (size_t)(dv * dk));\n        else memset(S, 0, sizeof(double) * (size_t)(dv * dk));\n        head_view hv;\n        hv.q = q + (b",
                                 "if (S0) { for (long i_ = 0; i_ < dv; ++i_) for (long c_ = 0; c_ < dk; ++c_) S[c_ * dv + i_] = S0[bh * dv * dk + i_ * dk + c_]; }\n        else memset(S, 0, sizeof(double) * (size_t)(dv * dk));\n        head_view hv;\n        hv.q = q + (b"),
}

PINS = [f for name, f in inspect.getmembers(test_oracle, inspect.isfunction)
        if name.startswith("test_pin_")]


def _pin_calls(fn):
    """All parameterisations of a pin as zero-argument callables."""
    params = getattr(fn, "pytestmark", [])
    grids = [m for m in params if m.name == "parametrize"]
    calls = [{}]
    for m in grids:
        names = [n.strip() for n in m.args[0].split(",")]
        new = []
        for base in calls:
            for vals in m.args[1]:
                vals = vals if len(names) > 1 else (vals,)
                d = dict(base)
                d.update(zip(names, vals))
                new.append(d)
        calls = new
    return [lambda fn=fn, kw=kw: fn(**kw) for kw in calls]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_every_planted_mistake_fails_a_pin(name, tmp_path):
    src = open(SRC).read()
    if MUTANTS[name] is None:
        mutated = _swap_write_and_readout(src)
    else:
        old, new = MUTANTS[name]
        assert src.count(old) == 1, f"mutation anchor for {name} not unique"
        mutated = src.replace(old, new)
    assert mutated != src
    c_path = tmp_path / "mutant.c"
    so_path = tmp_path / "libmutant.so"
    c_path.write_text(mutated)
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-o",
                    str(so_path), str(c_path), "-lm"], check=True)
    saved = oracle._lib
    oracle._lib = oracle._bind(ctypes.CDLL(str(so_path)))
    caught = []
    try:
        for pin in PINS:
            for call in _pin_calls(pin):
                try:
                    call()
                except (AssertionError, RuntimeError, ValueError, FloatingPointError):
                    caught.append(pin.__name__)
                    break
    finally:
        oracle._lib = saved
    assert caught, f"mutant {name} passed every pin"
