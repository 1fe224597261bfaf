"""The allocation-free segmented prefill (kda_chunk_fwd_segmented_noalloc)
through the C ABI, against the workspace entry point kda_chunk_fwd_segmented
with the same segment count: the same kernels on the same inputs, so outputs
and final states must agree bit for bit.  Two calls in a row share the
library's one scratch array, the second on a smaller problem (fewer heads, a
smaller d_k, fewer segments), so stale contents of the first call must not
leak into the second.  Both results are also held to the float64 oracle on a
few heads.  A request larger than the scratch array is rejected before any
launch.
"""
import os

import numpy as np
import pytest
import torch

import kda_synth
import oracle

kda = pytest.importorskip("kimi_delta_attention_fwd_amd")

pytestmark = pytest.mark.gpu
f64 = kda_synth.to_f64


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    if not os.path.exists(kda.library_path()):
        import __graft_entry__
        __graft_entry__.build()
    kda.load()
    return torch.device("cuda:0")


def rel(gpu, ref):
    return float(np.max(np.abs(gpu - ref)) / max(np.max(np.abs(ref)), 1e-30))


def run_both(p, C, nseg):
    B, T, H, dk = p.q.shape
    dv = p.v.shape[-1]
    outs = []
    for noalloc in (False, True):
        out = torch.full((B, T, H, dv), float("nan"), dtype=p.q.dtype, device=p.q.device)
        sf = torch.full((B, H, dv, dk), float("nan"), dtype=torch.float32, device=p.q.device)
        if noalloc:
            kda.kda_chunk_fwd_segmented_noalloc(p.q, p.k, p.v, p.log_alpha, p.beta, p.S0, out, sf, B, T, H, dk,
                                                dv, C, nseg)
        else:
            nbytes = kda.kda_chunk_segmented_workspace_bytes(B, H, dk, dv, nseg)
            ws = torch.empty(nbytes, dtype=torch.uint8, device=p.q.device)
            kda.kda_chunk_fwd_segmented(p.q, p.k, p.v, p.log_alpha, p.beta, p.S0, out, sf, B, T, H, dk, dv, C,
                                        nseg, ws, nbytes)
        torch.cuda.synchronize()
        outs.append((out, sf))
    return outs


def check(p, C, nseg, name):
    (o_ws, s_ws), (o_na, s_na) = run_both(p, C, nseg)
    print(f"case {name}: noalloc vs workspace, nseg={nseg}", flush=True)
    assert torch.equal(o_na, o_ws), f"{name}: outputs differ from the workspace entry point"
    assert torch.equal(s_na, s_ws), f"{name}: final states differ from the workspace entry point"
    B, T, H, dk = p.q.shape
    pairs = [(0, 0), (B - 1, H - 1)]
    for b, h in pairs:
        sl = lambda t: None if t is None else t[b:b + 1, :, h:h + 1]
        S0 = None if p.S0 is None else p.S0[b:b + 1, h:h + 1]
        o_ref, s_ref = oracle.forward(f64(sl(p.q)), f64(sl(p.k)), f64(sl(p.v)), f64(sl(p.log_alpha)),
                                      f64(p.beta[b:b + 1, :, h:h + 1]), S0=f64(S0))
        e_o = rel(f64(o_na[b:b + 1, :, h:h + 1]), o_ref)
        e_s = rel(f64(s_na[b:b + 1, h:h + 1]), s_ref)
        print(f"  (b={b}, h={h}): out rel err {e_o:.3e}, S_final rel err {e_s:.3e}", flush=True)
        assert e_o < 2e-2 and e_s < 2e-2


def test_noalloc_matches_workspace_entry_two_calls(dev):
    # first call: 8 heads of d = 128 over 6 segments, then a smaller one
    p1 = kda_synth.prefill(2, 2000, 4, 128, 128, s0_sigma=0.1, seed=71, device=dev)
    check(p1, 64, 6, "first B2 T2000 H4 d128 C64")
    p2 = kda_synth.prefill(1, 700, 2, 64, 64, s0_sigma=0.1, seed=72, device=dev)
    check(p2, 32, 3, "second B1 T700 H2 d64 C32")


def test_noalloc_rejects_requests_beyond_the_scratch_array(dev):
    B, T, H, dk, dv, C, nseg = 4, 64, 32, 128, 128, 64, 16
    need = kda.kda_chunk_segmented_workspace_bytes(B, H, dk, dv, nseg)
    assert need > kda.NOALLOC_SCRATCH_BYTES
    p = kda_synth.prefill(B, T, H, dk, dv, seed=73, device=dev)
    out = torch.empty((B, T, H, dv), dtype=p.q.dtype, device=dev)
    with pytest.raises(kda.KdaError) as ei:
        kda.kda_chunk_fwd_segmented_noalloc(p.q, p.k, p.v, p.log_alpha, p.beta, None, out, None, B, T, H, dk, dv,
                                            C, nseg)
    assert ei.value.status == 3 and "scratch" in ei.value.message
