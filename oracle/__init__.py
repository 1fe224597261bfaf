"""Float64 CPU oracle for the Kimi Delta Attention forward pass.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``, the smoke check in
``__graft_entry__.py`` and the ``cpu_baseline`` leg of ``bench.py`` may import
this package.  The GPU library and its Python binding never import it, and the
two share no code: the oracle is a plain C translation of the recurrence
(``kda_oracle.c``) plus a numpy chunked schedule (``chunked.py``) used only as
a second, independently written check of the first.

What the oracle computes is stated in ``kda_oracle.c``'s header: the KDA
recurrence of the "KDA derivation summary" page (sect. 3 and 5), state
d_v x d_k, readout from the post-write state, no query scale.

Arrays are numpy float64, token-major and contiguous:
q, k, log_alpha [B, T, H, dk]; v, out [B, T, H, dv]; beta [B, T, H];
states [B, H, dv, dk].
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "libkda_oracle.so")
# KDA_ORACLE_LIBRARY names a prebuilt copy to load instead (for instance one
# built with the address and undefined-behaviour sanitizers); it is not rebuilt.
_LIB_OVERRIDE = os.environ.get("KDA_ORACLE_LIBRARY")

WRITE_DELTA = 0
WRITE_ADD = 1

_lib = None


def build(force: bool = False) -> str:
    """Compile kda_oracle.c into libkda_oracle.so with gcc (-O2, OpenMP).

    Generic x86-64 code (no -march=native) so the library built here also runs
    on another host's CPU.
    """
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _bind(lib):
    """Declare the C signatures on a loaded oracle library."""
    dp = ctypes.POINTER(ctypes.c_double)
    lib.kda_oracle_forward.argtypes = [dp] * 8 + [ctypes.c_long] * 5 + [ctypes.c_int]
    lib.kda_oracle_forward.restype = ctypes.c_int
    lib.kda_oracle_forward_varlen.argtypes = (
        [dp] * 8 + [ctypes.POINTER(ctypes.c_int)] + [ctypes.c_long] * 5 + [ctypes.c_int])
    lib.kda_oracle_forward_varlen.restype = ctypes.c_int
    lib.kda_oracle_max_threads.argtypes = []
    lib.kda_oracle_max_threads.restype = ctypes.c_int
    lib.kda_oracle_set_threads.argtypes = [ctypes.c_int]
    lib.kda_oracle_set_threads.restype = None
    return lib


def _load():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            _lib = _bind(ctypes.CDLL(_LIB_OVERRIDE))
        else:
            build()
            _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def build_native(out_dir: str) -> str:
    """Compile kda_oracle.c for the CPU it runs on (-O3 -march=native, OpenMP)
    into out_dir and return the library's path.  Used for the timed CPU
    baseline on the host that runs the GPU; the same source as build()."""
    os.makedirs(out_dir, exist_ok=True)
    path = os.path.join(out_dir, "libkda_oracle_native.so")
    cmd = ["gcc", "-O3", "-march=native", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-Wall", "-Wextra", "-o", path, _SRC, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True)
    return path


def use_library(path: str) -> None:
    """Load the oracle from another build of kda_oracle.c (build_native)."""
    global _lib
    _lib = _bind(ctypes.CDLL(path))


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    if a is None:
        return ctypes.POINTER(ctypes.c_double)()
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _mode(write: str) -> int:
    if write == "delta":
        return WRITE_DELTA
    if write == "add":
        return WRITE_ADD
    raise ValueError(f"write must be 'delta' or 'add', got {write!r}")


def prepare(q_raw, k_raw, g=None, gate: str = "channel"):
    """Raw inputs to the recurrence's inputs, in float64.

    q and k are divided by their L2 norm over the key channels (the "Kimi K3
    notes 1: KDA" page, sect. 4: q and k pass a feature map and an L2
    normalisation before the recurrence); a zero row stays zero.  The gate is
    log_alpha = -softplus(g) = -log(1 + e^g), the parameterisation the library
    reads for the pages' alpha in (0, 1] (elementwise, per channel, or one
    value per token and head broadcast to every channel; "none" gives 0).
    Returns (q, k, log_alpha [.., H, dk]).
    """
    q = _f64(q_raw)
    k = _f64(k_raw)

    def unit(x):
        n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
        return np.divide(x, n, out=np.zeros_like(x), where=n > 0)

    if gate == "none":
        la = np.zeros_like(k)
    else:
        gg = _f64(g)
        la = -np.logaddexp(0.0, gg)            # -log(e^0 + e^g)
        if gate == "scalar":
            la = np.broadcast_to(la[..., None], k.shape).copy()
        elif gate != "channel":
            raise ValueError(f"gate must be 'channel', 'scalar' or 'none', got {gate!r}")
    return unit(q), unit(k), la


def forward(q, k, v, log_alpha, beta, S0=None, write: str = "delta"):
    """Token-by-token recurrence for a dense batch.

    Returns ``(out [B,T,H,dv], S_final [B,H,dv,dk])`` in float64.  ``S0=None``
    is the zero state.
    """
    q, k, v, la, be = (_f64(x) for x in (q, k, v, log_alpha, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or la.shape != q.shape or v.shape != (B, T, H, dv) or be.shape != (B, T, H):
        raise ValueError("inconsistent input shapes")
    s0 = None if S0 is None else _f64(S0)
    if s0 is not None and s0.shape != (B, H, dv, dk):
        raise ValueError("S0 must be [B, H, dv, dk]")
    out = np.empty((B, T, H, dv), dtype=np.float64)
    sf = np.empty((B, H, dv, dk), dtype=np.float64)
    rc = _load().kda_oracle_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(la), _ptr(be), _ptr(s0),
                                    _ptr(out), _ptr(sf), B, T, H, dk, dv, _mode(write))
    if rc != 0:
        raise RuntimeError(f"kda_oracle_forward failed with code {rc}")
    return out, sf


def forward_varlen(q, k, v, log_alpha, beta, cu_seqlens, S0=None, write: str = "delta"):
    """Recurrence over N packed sequences of a [1, T_total, H, d] stream.

    ``cu_seqlens`` holds N+1 non-decreasing offsets starting at 0.  Returns
    ``(out [1,T_total,H,dv], S_final [N,H,dv,dk])``.
    """
    q, k, v, la, be = (_f64(x) for x in (q, k, v, log_alpha, beta))
    _, T_total, H, dk = q.shape
    dv = v.shape[-1]
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    N = cu.shape[0] - 1
    s0 = None if S0 is None else _f64(S0)
    if s0 is not None and s0.shape != (N, H, dv, dk):
        raise ValueError("S0 must be [N, H, dv, dk]")
    out = np.empty((1, T_total, H, dv), dtype=np.float64)
    sf = np.empty((N, H, dv, dk), dtype=np.float64)
    rc = _load().kda_oracle_forward_varlen(
        _ptr(q), _ptr(k), _ptr(v), _ptr(la), _ptr(be), _ptr(s0), _ptr(out), _ptr(sf),
        cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int)), N, T_total, H, dk, dv, _mode(write))
    if rc != 0:
        raise RuntimeError(f"kda_oracle_forward_varlen failed with code {rc}")
    return out, sf


def max_threads() -> int:
    """OpenMP threads the oracle's parallel regions use."""
    return int(_load().kda_oracle_max_threads())


def set_threads(n: int) -> None:
    _load().kda_oracle_set_threads(int(n))
