"""C ABI of libkda on the CPU: the library loads, exports every function the
public header declares, and rejects invalid calls with the documented status
codes before any HIP call (no GPU needed).  No test here launches a kernel.

The pointers below are fake device addresses: validation only looks at their
values (NULL, alignment, overlap), never dereferences them.
"""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libkda.h")

kda = pytest.importorskip("kimi_delta_attention_fwd_amd")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kda.library_path()):
        import __graft_entry__
        __graft_entry__.build()
    return kda.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("kda_chunk_fwd", "kda_chunk_fwd_f32", "kda_chunk_fwd_varlen", "kda_chunk_fwd_varlen_f32",
              "kda_recurrent_step", "kda_recurrent_step_f32", "kda_status_string", "kda_last_error"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in libkda.h but not exported"


def test_status_strings_and_version(lib):
    for code, name in kda.STATUS.items():
        assert kda.kda_status_string(code) == name
    assert kda.kda_status_string(99) == "KDA_ERR_UNKNOWN"
    assert kda.kda_version() >= 100


A = 0x7F0000000000  # fake, 256-byte aligned "device" base address
MB = 1 << 20


def chunk(lib, f32=False, q=A, k=A + 64 * MB, v=A + 128 * MB, la=A + 192 * MB, beta=A + 256 * MB, S0=None,
          out=A + 320 * MB, Sf=A + 384 * MB, B=2, T=100, H=4, dk=64, dv=64, C=64):
    fn = lib.kda_chunk_fwd_f32 if f32 else lib.kda_chunk_fwd
    return fn(q, k, v, la, beta, S0, out, Sf, B, T, H, dk, dv, C, None)


def varlen(lib, cu=A + 448 * MB, N=3, T_total=100, **kw):
    args = dict(q=A, k=A + 64 * MB, v=A + 128 * MB, la=A + 192 * MB, beta=A + 256 * MB, S0=None,
                out=A + 320 * MB, Sf=A + 384 * MB, H=4, dk=64, dv=64, C=64)
    args.update(kw)
    return lib.kda_chunk_fwd_varlen(args["q"], args["k"], args["v"], args["la"], args["beta"], args["S0"],
                                    args["out"], args["Sf"], cu, N, T_total, args["H"], args["dk"],
                                    args["dv"], args["C"], None)


def step(lib, q=A, k=A + MB, v=A + 2 * MB, la=A + 3 * MB, beta=A + 4 * MB, S=A + 8 * MB, out=A + 64 * MB,
         N=4, H=2, dk=128, dv=128):
    return lib.kda_recurrent_step(q, k, v, la, beta, S, out, N, H, dk, dv, None)


def test_chunk_rejects_bad_shapes(lib):
    assert chunk(lib, B=-1) == 2
    assert chunk(lib, T=-5) == 2
    assert chunk(lib, H=0) == 2
    assert "H must be" in kda.kda_last_error()


@pytest.mark.parametrize("dk,dv,C", [(8, 64, 64), (64, 96, 64), (256, 64, 64), (64, 64, 48), (64, 64, 128),
                                     (64, 64, 8)])
def test_chunk_rejects_unsupported_sizes(lib, dk, dv, C):
    assert chunk(lib, dk=dk, dv=dv, C=C) == 3


def test_chunk_fp32_mode_accepts_every_chunk_length(lib):
    # fp32 operands at dk = 128, C = 64 do not fit the LDS: the library runs
    # 32-token chunks instead, so validation accepts the request (B = 0: no launch)
    for C in (16, 32, 64):
        assert chunk(lib, f32=True, dk=128, dv=128, C=C, B=0) == 0, kda.kda_last_error()


def test_chunk_rejects_null_pointers(lib):
    assert chunk(lib, q=None) == 1
    assert chunk(lib, beta=None) == 1
    assert chunk(lib, out=None) == 1


def test_chunk_rejects_misaligned_pointers(lib):
    assert chunk(lib, q=A + 2) == 4
    assert chunk(lib, la=A + 192 * MB + 4) == 4
    assert chunk(lib, S0=A + 500 * MB + 8) == 4
    assert chunk(lib, beta=A + 256 * MB + 2) == 4


def test_chunk_rejects_aliasing(lib):
    assert chunk(lib, out=A + 16) == 6                      # out inside q
    assert chunk(lib, Sf=A + 64 * MB) == 6                  # S_final on k
    S0 = A + 500 * MB
    assert chunk(lib, S0=S0, Sf=S0 + 256) == 6              # partial overlap of S0 / S_final
    assert "identical" in kda.kda_last_error()


def test_chunk_zero_work_calls_succeed_without_a_gpu(lib):
    # no sequences: nothing to launch
    assert chunk(lib, B=0) == 0
    # no tokens and no final state requested: nothing to launch
    assert chunk(lib, T=0, Sf=None, q=None, k=None, v=None, la=None, beta=None, out=None) == 0
    assert kda.kda_last_error() == ""


def test_varlen_validation(lib):
    assert varlen(lib, cu=None) == 1
    assert varlen(lib, cu=A + 448 * MB + 2) == 4
    assert varlen(lib, N=-1) == 2
    assert varlen(lib, N=0, T_total=0, q=None, k=None, v=None, la=None, beta=None, out=None) == 0


def test_check_cu_seqlens_host(lib):
    good = np.array([0, 5, 5, 12], dtype=np.int32)
    assert kda.kda_check_cu_seqlens_host(good.ctypes.data, 3, 12) == 0
    assert kda.kda_check_cu_seqlens_host(good.ctypes.data, 3, 13) == 2
    bad = np.array([0, 5, 4, 12], dtype=np.int32)
    assert kda.kda_check_cu_seqlens_host(bad.ctypes.data, 3, 12) == 2
    assert "decreases" in kda.kda_last_error()
    start = np.array([1, 5], dtype=np.int32)
    assert kda.kda_check_cu_seqlens_host(start.ctypes.data, 1, 5) == 2
    assert kda.kda_check_cu_seqlens_host(None, 1, 5) == 1


def test_step_validation(lib):
    assert step(lib, N=-1) == 2
    assert step(lib, H=0) == 2
    assert step(lib, dk=48) == 3
    assert step(lib, S=None) == 1
    assert step(lib, S=A + 8 * MB + 4) == 4
    assert step(lib, out=A + 8 * MB) == 6                   # out inside S
    assert step(lib, N=0) == 0


def test_binding_raises_kda_error(lib):
    with pytest.raises(kda.KdaError) as ei:
        kda.kda_chunk_fwd(A, A + 64 * MB, A + 128 * MB, A + 192 * MB, A + 256 * MB, None, A + 320 * MB, None,
                          1, 10, 1, 64, 64, 24, stream=0)
    assert ei.value.status == 3


def test_chunk_allows_in_place_state_continuation(lib):
    # S_final == S0 is allowed; validation passes and only the launch is left.  B = 0 keeps
    # the call launch-free on a machine without a GPU.
    S0 = A + 500 * MB
    assert chunk(lib, S0=S0, Sf=S0, B=0) == 0


# ---------------------------------------------------------------- segment-parallel schedule
WS = A + 1024 * MB   # fake workspace address, 256-byte aligned, clear of every other buffer


def seg(lib, nseg=4, ws=WS, wsb=None, f32=False, B=1, T=4096, H=2, dk=64, dv=64, C=64, **kw):
    args = dict(q=A, k=A + 64 * MB, v=A + 128 * MB, la=A + 192 * MB, beta=A + 256 * MB, S0=None,
                out=A + 320 * MB, Sf=A + 384 * MB)
    args.update(kw)
    if wsb is None:
        wsb = lib.kda_chunk_segmented_workspace_bytes(B, H, dk, dv, nseg)
    fn = lib.kda_chunk_fwd_segmented_f32 if f32 else lib.kda_chunk_fwd_segmented
    return fn(args["q"], args["k"], args["v"], args["la"], args["beta"], args["S0"], args["out"], args["Sf"],
              B, T, H, dk, dv, C, nseg, ws, wsb, None)


def test_segmented_workspace_bytes_formula(lib):
    f = lib.kda_chunk_segmented_workspace_bytes
    assert f(1, 16, 128, 128, 1) == 0
    nh, dk, dv, s = 16, 128, 128, 8
    maps = nh * (s - 1) * (dv + dk) * dk * 4
    maps = (maps + 255) // 256 * 256
    assert f(1, nh, dk, dv, s) == maps + nh * s * dv * dk * 4
    # B and H enter only through their product
    assert f(2, 3, 32, 16, 5) == f(6, 1, 32, 16, 5) == f(3, 2, 32, 16, 5)
    assert f(1, 1, 48, 64, 2) == 0 and f(1, 1, 64, 64, 0) == 0 and f(1, 1, 64, 64, 2000) == 0


def test_auto_segments_model(lib):
    # the mid workload already fills 256 compute units: one pass
    assert kda.kda_chunk_auto_segments(4, 8192, 32, 128, 128, 64, False) == 1
    # the long workload (16 heads, 1024 chunks each) is split into 9 segments,
    # the measured best with a lead segment (1.40 ms against 1.55 for 8 and
    # 1.94 for 10: at 9 the second pass is exactly 256 workgroups); the small
    # bf16 workload (8 heads, 16 chunks) also into 9, within 2 us of the best
    # measured (44-46 us against 63 for one pass)
    assert kda.kda_chunk_auto_segments(1, 65536, 16, 128, 128, 64, False) == 9
    assert kda.kda_chunk_auto_segments(2, 1024, 4, 64, 64, 64, False) == 9
    # more long-sequence shapes, each pick the measured best over 1..20
    # segments on one MI355X (ms): B1 T32768 H16 d128 -> 9 (0.74), B2 T32768
    # H16 -> 5 (1.19), B1 T65536 H32 -> 5 (2.34), B1 T16384 H16 -> 9 (0.41),
    # B1 T131072 H8 -> 16 (1.67; 17 takes 2.02: its map launch needs a third
    # round of workgroups), B1 T65536 H16 d64 -> 16 (0.68)
    for (B, T, H, d), want in (((1, 32768, 16, 128), 9), ((2, 32768, 16, 128), 5), ((1, 65536, 32, 128), 5),
                               ((1, 16384, 16, 128), 9), ((1, 131072, 8, 128), 16), ((1, 65536, 16, 64), 16)):
        assert kda.kda_chunk_auto_segments(B, T, H, d, d, 64, False) == want, (B, T, H, d)
    # never more segments than chunks, never below 1
    assert kda.kda_chunk_auto_segments(1, 100, 1, 64, 64, 64, False) <= 2
    assert kda.kda_chunk_auto_segments(0, 0, 1, 64, 64, 64, True) == 1
    assert kda.kda_chunk_auto_segments(1, 64, 1, 48, 64, 64, False) == 1


def test_auto_schedule_model(lib):
    """The one-pass schedule's model picks the measured best segment count on
    every shape timed on one MI355X (ms: B1 T65536 H16 d128 one-pass 7/8/9 =
    1.33/1.11/1.43; B1 T65536 H16 d64 0.58/0.52/0.76; B2 T32768 H16 d128
    4 -> 0.97 against 1.14 and 1.04 for 3 and 5; B1 T131072 H8 d128 8 -> 1.24;
    fp32 B1 T65536 H16 d128 8 -> 3.69), and kda_chunk_auto_schedule picks it
    over the two-pass schedule where it measured faster, except B2 T32768 H16,
    where the two models come within 1% (measured 0.97 against 1.04 ms)."""
    one = 16
    for (B, T, H, d, f32), nseg, sched in (((1, 65536, 16, 128, False), 8, one), ((1, 65536, 16, 64, False), 8, one),
                                           ((2, 32768, 16, 128, False), 4, 0), ((1, 131072, 8, 128, False), 8, one),
                                           ((1, 65536, 16, 128, True), 8, one), ((2, 1024, 4, 64, False), 8, one)):
        assert kda.kda_chunk_auto_segments_ex(B, T, H, d, d, 64, f32, one) == nseg, (B, T, H, d, f32)
        assert kda.kda_chunk_auto_schedule(B, T, H, d, d, 64, f32) == sched, (B, T, H, d, f32)
    # without the schedule bit: the two-pass model
    assert kda.kda_chunk_auto_segments_ex(1, 65536, 16, 128, 128, 64, False, 0) == 9
    # the mid workload fills the GPU in one pass: no segmented schedule
    assert kda.kda_chunk_auto_schedule(4, 8192, 32, 128, 128, 64, False) == 0


def test_segmented_validation(lib):
    assert seg(lib, nseg=0) == 2
    assert seg(lib, nseg=1025) == 2
    assert seg(lib, ws=None) == 1
    assert "workspace" in kda.kda_last_error()
    assert seg(lib, ws=WS + 16) == 4
    assert seg(lib, wsb=1024) == 2
    assert "needed" in kda.kda_last_error()
    assert seg(lib, ws=A + 320 * MB) == 6                  # workspace on top of out
    assert "workspace overlaps out" in kda.kda_last_error()
    assert seg(lib, ws=A) == 6                             # workspace on top of q
    # one segment needs no workspace; the usual checks still apply
    assert seg(lib, nseg=1, ws=None, B=0) == 0
    assert seg(lib, nseg=1, q=A + 2) == 4
    assert seg(lib, f32=True, dk=128, dv=128, C=64, B=0) == 0   # runs as 32-token chunks (no launch here)


def test_segmented_varlen_validation(lib):
    fn = lib.kda_chunk_fwd_varlen_segmented
    wsb = lib.kda_chunk_segmented_workspace_bytes(3, 4, 64, 64, 3)
    args = [A, A + 64 * MB, A + 128 * MB, A + 192 * MB, A + 256 * MB, None, A + 320 * MB, A + 384 * MB,
            A + 448 * MB, 3, 100, 4, 64, 64, 64]
    assert fn(*args, 3, None, wsb, None) == 1
    assert fn(*args, 3, WS, wsb - 4, None) == 2
    assert fn(*args, -1, WS, wsb, None) == 2


def test_recurrent_fwd_validation(lib):
    def multi(q=A, k=A + MB, v=A + 2 * MB, la=A + 3 * MB, beta=A + 4 * MB, S=A + 8 * MB, out=A + 64 * MB,
              N=4, T=3, H=2, dk=128, dv=128):
        return lib.kda_recurrent_fwd(q, k, v, la, beta, S, out, N, T, H, dk, dv, None)
    assert multi(T=-1) == 2
    assert multi(T=0, q=None, k=None, v=None, la=None, beta=None, S=None, out=None) == 0
    assert multi(N=0) == 0
    assert multi(q=None) == 1
    assert multi(S=A + 8 * MB + 4) == 4
    assert multi(dk=96) == 3
    # out must not overlap q, which holds N*T*H*dk elements (3 tokens, so 3x a step's)
    assert multi(out=A + 4 * 2 * 128 * 2 * 2 - 16) == 6
    assert lib.kda_recurrent_fwd_f32(A, A + MB, A + 2 * MB, A + 3 * MB, A + 4 * MB, A + 8 * MB, A + 64 * MB,
                                     4, 2, 2, 16, 256, None) == 3


def test_variant_validation(lib):
    P = A
    def ex(variant, la=A + 192 * MB, nseg=1, ws=None, wsb=0):
        return lib.kda_chunk_fwd_ex(A, A + 64 * MB, A + 128 * MB, la, A + 256 * MB, None, A + 320 * MB,
                                    A + 384 * MB, 2, 100, 4, 64, 64, 64, variant, nseg, ws, wsb, None)
    assert ex(3) == 2 and ex(32) == 2 and ex(-1) == 2 and ex(8 | 3) == 2 and ex(16 | 3) == 2
    assert "variant" in kda.kda_last_error()
    # the schedule without a second pass: its own, larger workspace is checked
    assert ex(16, nseg=2) == 1 and "workspace" in kda.kda_last_error()
    need = kda.kda_chunk_segmented_workspace_bytes_ex(2, 200, 4, 64, 64, 2, 16, False)
    assert ex(16, nseg=2, ws=A + 512 * MB, wsb=need - 1) == 2 and "workspace" in kda.kda_last_error()
    assert ex(0, la=None) == 1                  # the per-channel gate needs log_alpha
    assert ex(1, la=None) == 1                  # so does the scalar gate
    assert ex(1, la=A + 192 * MB + 4) != 4      # 4-byte alignment is enough for one gate per token
    assert ex(0, la=A + 192 * MB + 4) == 4
    assert ex(2 | 4, la=A + 192 * MB + 2, nseg=0) == 2   # log_alpha not read with no gate; nseg still checked
    assert kda.variant("scalar", "add") == 5 and kda.variant() == 0 and kda.variant("none") == 2
    def rex(variant, la=A + 3 * MB):
        return lib.kda_recurrent_fwd_ex(A, A + MB, A + 2 * MB, la, A + 4 * MB, A + 8 * MB, A + 64 * MB,
                                        4, 0, 2, 128, 128, variant, None)
    assert rex(3) == 2 and rex(2, la=None) == 0
    assert rex(16) == 2                         # no schedule bit for the decode entry points


def test_one_pass_workspace_bytes(lib):
    """Workspace of the schedule without a second pass: a map per segment
    (nseg of them, (dv + dk) dk fp32 each), the incoming states, each rounded
    up to 256 bytes, then T_total H dk values of the input type; the two-pass
    schedule's size without the schedule bit; 0 for one segment or bad sizes."""
    def r256(x):
        return (x + 255) // 256 * 256
    for nseq, T, H, dk, dv, nseg, f32 in ((1, 65536, 16, 128, 128, 8, False), (3, 1001, 2, 64, 32, 5, True),
                                          (2, 7, 1, 16, 128, 2, False)):
        es = 4 if f32 else 2
        want = (r256(4 * nseq * H * nseg * (dv + dk) * dk) + r256(4 * nseq * H * nseg * dv * dk)
                + T * H * dk * es)
        assert kda.kda_chunk_segmented_workspace_bytes_ex(nseq, T, H, dk, dv, nseg, 16, f32) == want
        assert kda.kda_chunk_segmented_workspace_bytes_ex(nseq, T, H, dk, dv, nseg, 0, f32) == \
            kda.kda_chunk_segmented_workspace_bytes(nseq, H, dk, dv, nseg)
    # nseg = 0 (packed sequences split on the device): two segments and the plan, one int per sequence
    assert kda.kda_chunk_segmented_workspace_bytes_ex(5, 1000, 2, 64, 64, 0, 16, False) == \
        kda.kda_chunk_segmented_workspace_bytes_ex(5, 1000, 2, 64, 64, 2, 16, False) + 4 * 5
    assert kda.kda_chunk_segmented_workspace_bytes_ex(5, 1000, 2, 64, 64, 0, 0, False) == 0
    assert kda.kda_chunk_segmented_workspace_bytes_ex(1, 100, 2, 64, 64, 1, 16, False) == 0
    assert kda.kda_chunk_segmented_workspace_bytes_ex(1, 100, 2, 48, 64, 4, 16, False) == 0
    assert kda.kda_chunk_segmented_workspace_bytes_ex(1, 100, 2, 64, 64, 4, 32, False) == 0
    assert kda.variant(schedule="one-pass") == 16 and kda.variant("none", "add", schedule="one-pass") == 22


def test_raw_input_variant_validation(lib):
    def ex(variant, la=A + 192 * MB, B=2, out=A + 320 * MB, nseg=2):
        # nseg = 2 without a workspace: a call whose other arguments pass stops
        # at the workspace check (status 1, "workspace"), before any launch
        return lib.kda_chunk_fwd_ex(A, A + 64 * MB, A + 128 * MB, la, A + 256 * MB, None, out, A + 384 * MB,
                                    B, 100, 4, 64, 64, 64, variant, nseg, None, 0, None)
    assert ex(8 | 1, la=A + 192 * MB + 2) == 1 and "workspace" in kda.kda_last_error()   # 2-byte aligned g
    assert ex(1, la=A + 192 * MB + 2) == 4        # one fp32 log_alpha per token needs 4-byte alignment
    assert ex(8, la=None) == 1 and "log_alpha" in kda.kda_last_error()
    # bf16 g [B, T, H, dk] occupies 2 bytes per element: out right after it does not overlap
    g_bytes = 2 * 100 * 4 * 64 * 2
    assert ex(8, out=A + 192 * MB + g_bytes) == 1 and "workspace" in kda.kda_last_error()
    assert ex(8, out=A + 192 * MB + g_bytes - 16) == 6


def test_stream_copy_validation(lib):
    # every check runs before the launch, so none of these touches a GPU
    assert lib.kda_stream_copy(A, A + 64 * MB, 0, None) == 0
    assert lib.kda_stream_copy(None, A, 16, None) == 1 and lib.kda_stream_copy(A, None, 16, None) == 1
    assert lib.kda_stream_copy(A, A + 64 * MB, 24, None) == 2
    assert "multiple of 16" in kda.kda_last_error()
    assert lib.kda_stream_copy(A + 8, A + 64 * MB, 32, None) == 4
    assert lib.kda_stream_copy(A, A + 64 * MB + 4, 32, None) == 4
    assert lib.kda_stream_copy(A, A + 16, 32, None) == 6      # the ranges overlap
    assert lib.kda_stream_copy(A + 16, A, 32, None) == 6


def test_noalloc_rejects_requests_beyond_its_scratch_before_any_hip_call(lib):
    # B=4 H=32 d=128 in 16 segments needs about 96 MiB of scratch, more than the static 64 MiB
    lib.kda_chunk_fwd_segmented_noalloc.argtypes = [ctypes.c_void_p] * 8 + [ctypes.c_int] * 7 + [ctypes.c_void_p]
    st = lib.kda_chunk_fwd_segmented_noalloc(A, A + 64 * MB, A + 128 * MB, A + 192 * MB, A + 256 * MB, None,
                                             A + 320 * MB, A + 384 * MB, 4, 100, 32, 128, 128, 64, 16, None)
    assert st == 3
    assert "scratch" in kda.kda_last_error()
    # and the usual argument checks come first
    st = lib.kda_chunk_fwd_segmented_noalloc(None, A + 64 * MB, A + 128 * MB, A + 192 * MB, A + 256 * MB, None,
                                             A + 320 * MB, A + 384 * MB, 1, 100, 2, 64, 64, 64, 3, None)
    assert st == 1
