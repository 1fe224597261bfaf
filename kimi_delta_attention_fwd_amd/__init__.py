"""Python binding for libkda, the MI355X (gfx950) Kimi Delta Attention forward.

The functions named ``kda_*`` mirror the C ABI of ``include/libkda.h`` one to
one: they only marshal arguments (tensor -> device pointer, stream -> handle)
and turn a non-OK status into :class:`KdaError`.  Every step of the
computation runs in the HIP kernels of ``libkda.so``; there is no fallback.
If the library has not been built, importing this package still works but the
first call raises, naming the build command.

Convenience wrappers (``chunk_fwd``, ``chunk_fwd_varlen``, ``recurrent_step``)
infer sizes from tensor shapes and allocate outputs with torch; torch is used
here for device memory and streams only.

Layouts (token-major, last index fastest): q, k, log_alpha [B, T, H, dk];
v, out [B, T, H, dv]; beta [B, T, H]; states [B, H, dv, dk] (fp32).
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "KdaError", "library_path", "load",
    "kda_chunk_fwd", "kda_chunk_fwd_f32", "kda_chunk_fwd_varlen", "kda_chunk_fwd_varlen_f32",
    "kda_chunk_fwd_segmented", "kda_chunk_fwd_segmented_f32", "kda_chunk_fwd_varlen_segmented",
    "kda_chunk_fwd_varlen_segmented_f32", "kda_chunk_segmented_workspace_bytes", "kda_chunk_auto_segments",
    "kda_chunk_fwd_segmented_noalloc", "NOALLOC_SCRATCH_BYTES",
    "kda_chunk_fwd_ex", "kda_chunk_fwd_ex_f32", "kda_chunk_fwd_varlen_ex", "kda_chunk_fwd_varlen_ex_f32",
    "kda_recurrent_fwd_ex", "kda_recurrent_fwd_ex_f32", "variant",
    "kda_recurrent_step", "kda_recurrent_step_f32", "kda_recurrent_fwd", "kda_recurrent_fwd_f32",
    "kda_check_cu_seqlens_host", "kda_stream_copy",
    "kda_status_string", "kda_last_error", "kda_version",
    "chunk_fwd", "chunk_fwd_varlen", "recurrent_step", "recurrent_fwd",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
# KDA_LIBRARY names another build of the library to load (for instance one
# whose host code carries the address and undefined-behaviour sanitizers).
_LIB_PATH = os.environ.get("KDA_LIBRARY") or os.path.join(_PKG, "libkda.so")
_lib = None

STATUS = {0: "KDA_OK", 1: "KDA_ERR_NULL_POINTER", 2: "KDA_ERR_BAD_SHAPE", 3: "KDA_ERR_UNSUPPORTED",
          4: "KDA_ERR_MISALIGNED", 5: "KDA_ERR_HIP", 6: "KDA_ERR_ALIASING"}


class KdaError(RuntimeError):
    """A libkda call returned a status other than KDA_OK."""

    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn}: {STATUS.get(status, status)}: {message}")
        self.status = status
        self.message = message


def library_path() -> str:
    return _LIB_PATH


def load():
    """Load libkda.so (once) and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"{_LIB_PATH} is not built; run `python -m kimi_delta_attention_fwd_amd.build` "
            "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I = ctypes.c_void_p, ctypes.c_int
    chunk = [P] * 8 + [I] * 6 + [P]
    varlen = [P] * 9 + [I] * 6 + [P]
    step = [P] * 7 + [I] * 4 + [P]
    multi = [P] * 7 + [I] * 5 + [P]
    multi_ex = [P] * 7 + [I] * 6 + [P]
    chunk_ex = [P] * 8 + [I] * 8 + [P, ctypes.c_size_t, P]
    varlen_ex = [P] * 9 + [I] * 8 + [P, ctypes.c_size_t, P]
    Z = ctypes.c_size_t
    chunk_seg = [P] * 8 + [I] * 7 + [P, Z, P]
    varlen_seg = [P] * 9 + [I] * 7 + [P, Z, P]
    for name, args in (("kda_chunk_fwd", chunk), ("kda_chunk_fwd_f32", chunk),
                       ("kda_chunk_fwd_varlen", varlen), ("kda_chunk_fwd_varlen_f32", varlen),
                       ("kda_chunk_fwd_segmented", chunk_seg), ("kda_chunk_fwd_segmented_f32", chunk_seg),
                       ("kda_chunk_fwd_varlen_segmented", varlen_seg),
                       ("kda_chunk_fwd_varlen_segmented_f32", varlen_seg),
                       ("kda_recurrent_step", step), ("kda_recurrent_step_f32", step),
                       ("kda_recurrent_fwd", multi), ("kda_recurrent_fwd_f32", multi),
                       ("kda_recurrent_fwd_ex", multi_ex), ("kda_recurrent_fwd_ex_f32", multi_ex),
                       ("kda_chunk_fwd_ex", chunk_ex), ("kda_chunk_fwd_ex_f32", chunk_ex),
                       ("kda_chunk_fwd_varlen_ex", varlen_ex), ("kda_chunk_fwd_varlen_ex_f32", varlen_ex)):
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = I
    lib.kda_chunk_fwd_segmented_noalloc.argtypes = [P] * 8 + [I] * 7 + [P]
    lib.kda_chunk_fwd_segmented_noalloc.restype = I
    lib.kda_chunk_segmented_workspace_bytes.argtypes = [I] * 5
    lib.kda_chunk_segmented_workspace_bytes.restype = Z
    lib.kda_chunk_auto_segments.argtypes = [I] * 7
    lib.kda_chunk_auto_segments.restype = I
    lib.kda_chunk_segmented_workspace_bytes_ex.argtypes = [I] * 8
    lib.kda_chunk_segmented_workspace_bytes_ex.restype = Z
    lib.kda_chunk_auto_segments_ex.argtypes = [I] * 8
    lib.kda_chunk_auto_segments_ex.restype = I
    lib.kda_chunk_auto_schedule.argtypes = [I] * 7
    lib.kda_chunk_auto_schedule.restype = I
    lib.kda_stream_copy.argtypes = [P, P, Z, P]
    lib.kda_stream_copy.restype = I
    lib.kda_check_cu_seqlens_host.argtypes = [P, I, I]
    lib.kda_check_cu_seqlens_host.restype = I
    lib.kda_status_string.argtypes = [I]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_last_error.argtypes = []
    lib.kda_last_error.restype = ctypes.c_char_p
    lib.kda_version.argtypes = []
    lib.kda_version.restype = I
    _lib = lib
    return lib


def _ptr(x):
    """Device pointer of a tensor (or an int address, or None -> NULL)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn: str, status: int):
    if status != 0:
        raise KdaError(fn, status, load().kda_last_error().decode())


# --- the C ABI, one to one -------------------------------------------------------------------
def kda_chunk_fwd(q, k, v, log_alpha, beta, S0, out, S_final, B, T, H, dk, dv, C, stream=None):
    _check("kda_chunk_fwd", load().kda_chunk_fwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S0), _ptr(out), _ptr(S_final),
        B, T, H, dk, dv, C, _stream(stream)))


def kda_chunk_fwd_f32(q, k, v, log_alpha, beta, S0, out, S_final, B, T, H, dk, dv, C, stream=None):
    _check("kda_chunk_fwd_f32", load().kda_chunk_fwd_f32(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S0), _ptr(out), _ptr(S_final),
        B, T, H, dk, dv, C, _stream(stream)))


def kda_chunk_fwd_varlen(q, k, v, log_alpha, beta, S0, out, S_final, cu_seqlens, N, T_total, H, dk, dv, C,
                         stream=None):
    _check("kda_chunk_fwd_varlen", load().kda_chunk_fwd_varlen(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S0), _ptr(out), _ptr(S_final),
        _ptr(cu_seqlens), N, T_total, H, dk, dv, C, _stream(stream)))


def kda_chunk_fwd_varlen_f32(q, k, v, log_alpha, beta, S0, out, S_final, cu_seqlens, N, T_total, H, dk, dv,
                             C, stream=None):
    _check("kda_chunk_fwd_varlen_f32", load().kda_chunk_fwd_varlen_f32(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S0), _ptr(out), _ptr(S_final),
        _ptr(cu_seqlens), N, T_total, H, dk, dv, C, _stream(stream)))


def kda_chunk_fwd_segmented(q, k, v, log_alpha, beta, S0, out, S_final, B, T, H, dk, dv, C, nseg, workspace,
                            workspace_bytes, stream=None):
    _check("kda_chunk_fwd_segmented", load().kda_chunk_fwd_segmented(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S0), _ptr(out), _ptr(S_final),
        B, T, H, dk, dv, C, nseg, _ptr(workspace), workspace_bytes, _stream(stream)))


def kda_chunk_fwd_segmented_f32(q, k, v, log_alpha, beta, S0, out, S_final, B, T, H, dk, dv, C, nseg,
                                workspace, workspace_bytes, stream=None):
    _check("kda_chunk_fwd_segmented_f32", load().kda_chunk_fwd_segmented_f32(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S0), _ptr(out), _ptr(S_final),
        B, T, H, dk, dv, C, nseg, _ptr(workspace), workspace_bytes, _stream(stream)))


def kda_chunk_fwd_varlen_segmented(q, k, v, log_alpha, beta, S0, out, S_final, cu_seqlens, N, T_total, H, dk,
                                   dv, C, nseg, workspace, workspace_bytes, stream=None):
    _check("kda_chunk_fwd_varlen_segmented", load().kda_chunk_fwd_varlen_segmented(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S0), _ptr(out), _ptr(S_final),
        _ptr(cu_seqlens), N, T_total, H, dk, dv, C, nseg, _ptr(workspace), workspace_bytes, _stream(stream)))


def kda_chunk_fwd_varlen_segmented_f32(q, k, v, log_alpha, beta, S0, out, S_final, cu_seqlens, N, T_total, H,
                                       dk, dv, C, nseg, workspace, workspace_bytes, stream=None):
    _check("kda_chunk_fwd_varlen_segmented_f32", load().kda_chunk_fwd_varlen_segmented_f32(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S0), _ptr(out), _ptr(S_final),
        _ptr(cu_seqlens), N, T_total, H, dk, dv, C, nseg, _ptr(workspace), workspace_bytes, _stream(stream)))


def kda_chunk_fwd_segmented_noalloc(q, k, v, log_alpha, beta, S0, out, S_final, B, T, H, dk, dv, C, nseg,
                                    stream=None):
    """kda_chunk_fwd_segmented with the library's static scratch array instead
    of a workspace (no device allocation; calls overlapping on one GPU race)."""
    _check("kda_chunk_fwd_segmented_noalloc", load().kda_chunk_fwd_segmented_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S0), _ptr(out), _ptr(S_final),
        B, T, H, dk, dv, C, nseg, _stream(stream)))


NOALLOC_SCRATCH_BYTES = 64 << 20


def kda_chunk_segmented_workspace_bytes(nseq, H, dk, dv, nseg) -> int:
    return load().kda_chunk_segmented_workspace_bytes(nseq, H, dk, dv, nseg)


def kda_chunk_auto_segments(B, T, H, dk, dv, C, fp32_inputs) -> int:
    return load().kda_chunk_auto_segments(B, T, H, dk, dv, C, 1 if fp32_inputs else 0)


def kda_chunk_segmented_workspace_bytes_ex(nseq, T_total, H, dk, dv, nseg, variant, fp32_inputs) -> int:
    return load().kda_chunk_segmented_workspace_bytes_ex(nseq, T_total, H, dk, dv, nseg, variant,
                                                         1 if fp32_inputs else 0)


def kda_chunk_auto_segments_ex(B, T, H, dk, dv, C, fp32_inputs, variant) -> int:
    return load().kda_chunk_auto_segments_ex(B, T, H, dk, dv, C, 1 if fp32_inputs else 0, variant)


def kda_chunk_auto_schedule(B, T, H, dk, dv, C, fp32_inputs) -> int:
    return load().kda_chunk_auto_schedule(B, T, H, dk, dv, C, 1 if fp32_inputs else 0)


def kda_recurrent_step(q, k, v, log_alpha, beta, S, out, N, H, dk, dv, stream=None):
    _check("kda_recurrent_step", load().kda_recurrent_step(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S), _ptr(out), N, H, dk, dv,
        _stream(stream)))


def kda_recurrent_step_f32(q, k, v, log_alpha, beta, S, out, N, H, dk, dv, stream=None):
    _check("kda_recurrent_step_f32", load().kda_recurrent_step_f32(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S), _ptr(out), N, H, dk, dv,
        _stream(stream)))


def kda_recurrent_fwd(q, k, v, log_alpha, beta, S, out, N, T, H, dk, dv, stream=None):
    _check("kda_recurrent_fwd", load().kda_recurrent_fwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S), _ptr(out), N, T, H, dk, dv,
        _stream(stream)))


def kda_recurrent_fwd_f32(q, k, v, log_alpha, beta, S, out, N, T, H, dk, dv, stream=None):
    _check("kda_recurrent_fwd_f32", load().kda_recurrent_fwd_f32(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S), _ptr(out), N, T, H, dk, dv,
        _stream(stream)))


GATES = {"channel": 0, "scalar": 1, "none": 2}
WRITES = {"delta": 0, "add": 4}
SCHED_MAP_OUTPUTS = 16
SCHEDULES = ("two-pass", "one-pass")


def variant(gate="channel", write="delta", raw=False, schedule="two-pass") -> int:
    """Variant selector of the *_ex entry points: gate "channel" (KDA, GLA),
    "scalar" (one decay per token and head) or "none"; write "delta" or "add";
    raw=True for un-normalised q, k and gate pre-activations g (fused prep);
    schedule "one-pass" for the segmented schedule without a second pass
    (KDA_SCHED_MAP_OUTPUTS; chunk entry points only)."""
    if schedule not in SCHEDULES:
        raise ValueError(f"schedule must be one of {SCHEDULES}, got {schedule!r}")
    return GATES[gate] | WRITES[write] | (8 if raw else 0) | (SCHED_MAP_OUTPUTS if schedule == "one-pass" else 0)


def kda_chunk_fwd_ex(q, k, v, log_alpha, beta, S0, out, S_final, B, T, H, dk, dv, C, variant, nseg=1,
                     workspace=None, workspace_bytes=0, stream=None):
    _check("kda_chunk_fwd_ex", load().kda_chunk_fwd_ex(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S0), _ptr(out), _ptr(S_final),
        B, T, H, dk, dv, C, variant, nseg, _ptr(workspace), workspace_bytes, _stream(stream)))


def kda_chunk_fwd_ex_f32(q, k, v, log_alpha, beta, S0, out, S_final, B, T, H, dk, dv, C, variant, nseg=1,
                         workspace=None, workspace_bytes=0, stream=None):
    _check("kda_chunk_fwd_ex_f32", load().kda_chunk_fwd_ex_f32(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S0), _ptr(out), _ptr(S_final),
        B, T, H, dk, dv, C, variant, nseg, _ptr(workspace), workspace_bytes, _stream(stream)))


def kda_chunk_fwd_varlen_ex(q, k, v, log_alpha, beta, S0, out, S_final, cu_seqlens, N, T_total, H, dk, dv, C,
                            variant, nseg=1, workspace=None, workspace_bytes=0, stream=None):
    _check("kda_chunk_fwd_varlen_ex", load().kda_chunk_fwd_varlen_ex(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S0), _ptr(out), _ptr(S_final),
        _ptr(cu_seqlens), N, T_total, H, dk, dv, C, variant, nseg, _ptr(workspace), workspace_bytes,
        _stream(stream)))


def kda_chunk_fwd_varlen_ex_f32(q, k, v, log_alpha, beta, S0, out, S_final, cu_seqlens, N, T_total, H, dk, dv,
                                C, variant, nseg=1, workspace=None, workspace_bytes=0, stream=None):
    _check("kda_chunk_fwd_varlen_ex_f32", load().kda_chunk_fwd_varlen_ex_f32(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S0), _ptr(out), _ptr(S_final),
        _ptr(cu_seqlens), N, T_total, H, dk, dv, C, variant, nseg, _ptr(workspace), workspace_bytes,
        _stream(stream)))


def kda_recurrent_fwd_ex(q, k, v, log_alpha, beta, S, out, N, T, H, dk, dv, variant, stream=None):
    _check("kda_recurrent_fwd_ex", load().kda_recurrent_fwd_ex(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S), _ptr(out), N, T, H, dk, dv, variant,
        _stream(stream)))


def kda_recurrent_fwd_ex_f32(q, k, v, log_alpha, beta, S, out, N, T, H, dk, dv, variant, stream=None):
    _check("kda_recurrent_fwd_ex_f32", load().kda_recurrent_fwd_ex_f32(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S), _ptr(out), N, T, H, dk, dv, variant,
        _stream(stream)))


def kda_stream_copy(src, dst, nbytes, stream=None):
    """Bandwidth reference: copy nbytes from src to dst with the decode kernels'
    16-byte nontemporal access pattern."""
    _check("kda_stream_copy", load().kda_stream_copy(_ptr(src), _ptr(dst), nbytes, _stream(stream)))


def kda_check_cu_seqlens_host(cu_seqlens_host, N, T_total) -> int:
    """Check a host (CPU) int32 cu_seqlens; returns the status code."""
    return load().kda_check_cu_seqlens_host(_ptr(cu_seqlens_host), N, T_total)


def kda_status_string(status: int) -> str:
    return load().kda_status_string(status).decode()


def kda_last_error() -> str:
    return load().kda_last_error().decode()


def kda_version() -> int:
    return load().kda_version()


# --- convenience wrappers: sizes from shapes, outputs allocated with torch ---------------------
def _mode(q):
    import torch
    if not isinstance(q, torch.Tensor):
        raise TypeError(f"q must be a torch.Tensor, got {type(q).__name__}")
    if q.dtype == torch.bfloat16:
        return False
    if q.dtype == torch.float32:
        return True
    raise TypeError(f"q, k, v must be bfloat16 or float32, got {q.dtype}")


def _validate(q, named, shapes, dtypes):
    """Checks the convenience wrappers make before any C call (the C ABI sees
    only pointers): every tensor is a torch tensor of the expected shape and
    dtype, contiguous (the kernels assume the dense token-major layout), and on
    the same GPU as q.  Raises TypeError or ValueError; does no arithmetic."""
    import torch
    for name, t in named.items():
        if t is None:
            continue
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
        if name in dtypes and t.dtype != dtypes[name]:
            raise TypeError(f"{name} must be {dtypes[name]}, got {t.dtype}")
        if name in shapes and tuple(t.shape) != tuple(shapes[name]):
            raise ValueError(f"{name} must have shape {tuple(shapes[name])}, got {tuple(t.shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous (got strides {t.stride()}); call .contiguous() first")
    for name, t in named.items():
        if t is None:
            continue
        if t.device.type != "cuda":
            raise TypeError(f"{name} must be on a GPU (device 'cuda'), got {t.device}")
        if t.device != q.device:
            raise ValueError(f"{name} is on {t.device}, q on {q.device}: all tensors must be on one GPU")


def _gate_spec(gate, raw, q, lead_shape, dk):
    """Expected shape and dtype of the gate argument: fp32 log_alpha, or with
    raw=True the pre-activations g in q's dtype; [.., dk] per channel, [..]
    scalar, None for gate="none"."""
    import torch
    if gate not in GATES:
        raise ValueError(f"gate must be one of {sorted(GATES)}, got {gate!r}")
    dtype = q.dtype if raw else torch.float32
    shape = tuple(lead_shape) + ((dk,) if gate == "channel" else ())
    return shape, dtype


def _workspace(nseq, H, dk, dv, nseg, device, T_total=0, var=0, f32=False):
    import torch
    nbytes = kda_chunk_segmented_workspace_bytes_ex(nseq, T_total, H, dk, dv, nseg, var, f32)
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device), nbytes


def _schedule(schedule, nseq, T, H, dk, dv, C, f32):
    """The schedule's variant bit: "auto" asks the library's run-time models."""
    if schedule == "auto":
        return kda_chunk_auto_schedule(nseq, T, H, dk, dv, C, f32)
    if schedule not in SCHEDULES:
        raise ValueError(f"schedule must be 'auto' or one of {SCHEDULES}, got {schedule!r}")
    return SCHED_MAP_OUTPUTS if schedule == "one-pass" else 0


def chunk_fwd(q, k, v, log_alpha, beta, S0=None, C=64, output_final_state=True, stream=None, segments="auto",
              gate="channel", write="delta", raw=False, schedule="auto"):
    """Chunk prefill of a dense batch.  Returns ``(out, S_final or None)``.

    ``segments``: 1 for the single pass, n > 1 for the segment-parallel
    schedule with n segments per sequence, "auto" for the library's choice.
    ``schedule`` (segments > 1): "two-pass", "one-pass" (no second pass, a
    larger workspace) or "auto": with segments="auto" the library's run-time
    models pick the schedule and its segment count, else "two-pass".
    ``gate`` / ``write`` / ``raw`` select a variant (see :func:`variant`); with
    gate="scalar" log_alpha is [B, T, H], with gate="none" it may be None;
    with raw=True it holds the pre-activations g in q's dtype.
    """
    import torch
    f32 = _mode(q)
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError(f"q and v must be [B, T, H, d], got {tuple(q.shape)} and {tuple(v.shape)}")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if write not in WRITES:
        raise ValueError(f"write must be one of {sorted(WRITES)}, got {write!r}")
    g_shape, g_dtype = _gate_spec(gate, raw, q, (B, T, H), dk)
    if gate != "none" and log_alpha is None:
        raise ValueError(f"log_alpha is required with gate={gate!r}")
    _validate(q, dict(q=q, k=k, v=v, log_alpha=log_alpha if gate != "none" else None, beta=beta, S0=S0),
              dict(k=(B, T, H, dk), v=(B, T, H, dv), log_alpha=g_shape, beta=(B, T, H), S0=(B, H, dv, dk)),
              dict(k=q.dtype, v=q.dtype, log_alpha=g_dtype, beta=torch.float32, S0=torch.float32))
    out = torch.empty((B, T, H, dv), dtype=q.dtype, device=q.device)
    sf = torch.empty((B, H, dv, dk), dtype=torch.float32, device=q.device) if output_final_state else None
    if segments == "auto":
        sched = _schedule(schedule, B, T, H, dk, dv, C, f32)
        nseg = kda_chunk_auto_segments_ex(B, T, H, dk, dv, C, f32, sched)
    else:
        sched = _schedule("two-pass" if schedule == "auto" else schedule, B, T, H, dk, dv, C, f32)
        nseg = int(segments)
    var = variant(gate, write, raw) | (sched if nseg > 1 else 0)
    if var != 0:
        ws, nbytes = _workspace(B, H, dk, dv, nseg, q.device, B * T, var, f32) if nseg > 1 else (None, 0)
        fn = kda_chunk_fwd_ex_f32 if f32 else kda_chunk_fwd_ex
        fn(q, k, v, log_alpha, beta, S0, out, sf, B, T, H, dk, dv, C, var, nseg, ws, nbytes, stream)
    elif nseg == 1:
        fn = kda_chunk_fwd_f32 if f32 else kda_chunk_fwd
        fn(q, k, v, log_alpha, beta, S0, out, sf, B, T, H, dk, dv, C, stream)
    else:
        ws, nbytes = _workspace(B, H, dk, dv, nseg, q.device)
        fn = kda_chunk_fwd_segmented_f32 if f32 else kda_chunk_fwd_segmented
        fn(q, k, v, log_alpha, beta, S0, out, sf, B, T, H, dk, dv, C, nseg, ws, nbytes, stream)
    return out, sf


def chunk_fwd_varlen(q, k, v, log_alpha, beta, cu_seqlens, S0=None, C=64, output_final_state=True, stream=None,
                     segments=1, schedule="two-pass"):
    """Chunk prefill of N packed sequences ([1, T_total, H, d] tensors, device cu_seqlens [N+1]).

    ``segments`` > 1 cuts every sequence into that many segments run in
    parallel, with ``schedule`` "two-pass" or "one-pass"; "auto" splits only
    the sequences much longer than the rest, on the device (the one-pass
    schedule with nseg = 0).
    """
    import torch
    f32 = _mode(q)
    if q.dim() != 4 or q.shape[0] != 1 or v.dim() != 4:
        raise ValueError(f"q and v must be packed [1, T_total, H, d], got {tuple(q.shape)} and {tuple(v.shape)}")
    _, T_total, H, dk = q.shape
    dv = v.shape[-1]
    if not isinstance(cu_seqlens, torch.Tensor) or cu_seqlens.dim() != 1 or cu_seqlens.shape[0] < 1:
        raise ValueError("cu_seqlens must be a 1-d int32 tensor of N + 1 offsets")
    N = cu_seqlens.shape[0] - 1
    _validate(q, dict(q=q, k=k, v=v, log_alpha=log_alpha, beta=beta, S0=S0, cu_seqlens=cu_seqlens),
              dict(k=(1, T_total, H, dk), v=(1, T_total, H, dv), log_alpha=(1, T_total, H, dk), beta=(1, T_total, H),
                   S0=(N, H, dv, dk)),
              dict(k=q.dtype, v=q.dtype, log_alpha=torch.float32, beta=torch.float32, S0=torch.float32,
                   cu_seqlens=torch.int32))
    out = torch.empty((1, T_total, H, dv), dtype=q.dtype, device=q.device)
    sf = torch.empty((N, H, dv, dk), dtype=torch.float32, device=q.device) if output_final_state else None
    if segments == "auto":
        nseg, sched = 0, SCHED_MAP_OUTPUTS
    else:
        nseg = int(segments)
        sched = _schedule(schedule, 1, 1, H, dk, dv, C, f32)
    if nseg == 1 or N == 0:
        fn = kda_chunk_fwd_varlen_f32 if f32 else kda_chunk_fwd_varlen
        fn(q, k, v, log_alpha, beta, S0, out, sf, cu_seqlens, N, T_total, H, dk, dv, C, stream)
    elif sched:
        ws, nbytes = _workspace(N, H, dk, dv, nseg, q.device, T_total, sched, f32)
        fn = kda_chunk_fwd_varlen_ex_f32 if f32 else kda_chunk_fwd_varlen_ex
        fn(q, k, v, log_alpha, beta, S0, out, sf, cu_seqlens, N, T_total, H, dk, dv, C, sched, nseg, ws, nbytes,
           stream)
    else:
        ws, nbytes = _workspace(N, H, dk, dv, nseg, q.device)
        fn = kda_chunk_fwd_varlen_segmented_f32 if f32 else kda_chunk_fwd_varlen_segmented
        fn(q, k, v, log_alpha, beta, S0, out, sf, cu_seqlens, N, T_total, H, dk, dv, C, nseg, ws, nbytes, stream)
    return out, sf


def recurrent_step(q, k, v, log_alpha, beta, S, out=None, stream=None):
    """One decode step on [N, H, d] tensors; S [N, H, dv, dk] fp32 is updated in place."""
    import torch
    f32 = _mode(q)
    if q.dim() != 3 or v.dim() != 3:
        raise ValueError(f"q and v must be [N, H, d], got {tuple(q.shape)} and {tuple(v.shape)}")
    N, H, dk = q.shape
    dv = v.shape[-1]
    _validate(q, dict(q=q, k=k, v=v, log_alpha=log_alpha, beta=beta, S=S, out=out),
              dict(k=(N, H, dk), v=(N, H, dv), log_alpha=(N, H, dk), beta=(N, H), S=(N, H, dv, dk), out=(N, H, dv)),
              dict(k=q.dtype, v=q.dtype, log_alpha=torch.float32, beta=torch.float32, S=torch.float32,
                   out=q.dtype))
    if S is None:
        raise ValueError("S (the state, updated in place) is required")
    if out is None:
        out = torch.empty((N, H, dv), dtype=q.dtype, device=q.device)
    fn = kda_recurrent_step_f32 if f32 else kda_recurrent_step
    fn(q, k, v, log_alpha, beta, S, out, N, H, dk, dv, stream)
    return out


def recurrent_fwd(q, k, v, log_alpha, beta, S, out=None, stream=None, gate="channel", write="delta", raw=False):
    """T decode tokens per sequence on [N, T, H, d] tensors in one launch; S
    [N, H, dv, dk] fp32 is updated in place.  Returns out [N, T, H, dv].

    The result has the bits of T single steps.  From about T = 16 on,
    ``chunk_fwd(q, k, v, log_alpha, beta, S0=S, C=16 or 32)`` on the same
    tensors is faster (same result up to rounding)."""
    import torch
    f32 = _mode(q)
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError(f"q and v must be [N, T, H, d], got {tuple(q.shape)} and {tuple(v.shape)}")
    N, T, H, dk = q.shape
    dv = v.shape[-1]
    if write not in WRITES:
        raise ValueError(f"write must be one of {sorted(WRITES)}, got {write!r}")
    g_shape, g_dtype = _gate_spec(gate, raw, q, (N, T, H), dk)
    if gate != "none" and log_alpha is None:
        raise ValueError(f"log_alpha is required with gate={gate!r}")
    _validate(q, dict(q=q, k=k, v=v, log_alpha=log_alpha if gate != "none" else None, beta=beta, S=S, out=out),
              dict(k=(N, T, H, dk), v=(N, T, H, dv), log_alpha=g_shape, beta=(N, T, H), S=(N, H, dv, dk),
                   out=(N, T, H, dv)),
              dict(k=q.dtype, v=q.dtype, log_alpha=g_dtype, beta=torch.float32, S=torch.float32, out=q.dtype))
    if S is None:
        raise ValueError("S (the state, updated in place) is required")
    if out is None:
        out = torch.empty((N, T, H, dv), dtype=q.dtype, device=q.device)
    var = variant(gate, write, raw)
    if var != 0:
        fn = kda_recurrent_fwd_ex_f32 if f32 else kda_recurrent_fwd_ex
        fn(q, k, v, log_alpha, beta, S, out, N, T, H, dk, dv, var, stream)
    else:
        fn = kda_recurrent_fwd_f32 if f32 else kda_recurrent_fwd
        fn(q, k, v, log_alpha, beta, S, out, N, T, H, dk, dv, stream)
    return out
