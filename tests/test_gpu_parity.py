"""GPU parity: libkda (through its C ABI) against the float64 oracle.

Every test feeds the HIP path and the oracle the very same seeded inputs (the
oracle gets an exact float64 copy of the bf16 / fp32 tensors the GPU reads)
and compares element by element with the normwise relative error
    max_i |gpu_i - ref_i| / max_i |ref_i|
computed separately for the outputs and the final states.  Bars: 2e-2 for bf16
inputs (fp32 accumulation), 1e-4 for fp32 inputs.

Reduced shapes span several chunks and 16-row tiles with a ragged tail; the
full-size workloads (the same launch configurations bench.py times) are checked
on sampled heads, which the oracle recomputes from their whole token history.
"""
import os

import numpy as np
import pytest
import torch

import kda_synth
import oracle

kda = pytest.importorskip("kimi_delta_attention_fwd_amd")

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f32": 1e-4}
f64 = kda_synth.to_f64


def note(msg):
    print(msg, flush=True)


def rel(gpu, ref):
    return float(np.max(np.abs(gpu - ref)) / max(np.max(np.abs(ref)), 1e-30))


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    if not os.path.exists(kda.library_path()):
        import __graft_entry__
        __graft_entry__.build()
    kda.load()
    return torch.device("cuda:0")


def gpu_chunk(p, C, final=True, segments=1):
    out, sf = kda.chunk_fwd(p.q, p.k, p.v, p.log_alpha, p.beta, S0=p.S0, C=C, output_final_state=final,
                            segments=segments)
    torch.cuda.synchronize()
    return out, sf


def oracle_dense(p):
    return oracle.forward(f64(p.q), f64(p.k), f64(p.v), f64(p.log_alpha), f64(p.beta), S0=f64(p.S0))


def sampled(p, pairs):
    """(b, h) pairs of a dense batch, packed as an oracle batch of single heads."""
    def pick(t):
        if t is None:
            return None
        return torch.stack([t[b, :, h] for b, h in pairs]).unsqueeze(2)
    S0 = None if p.S0 is None else torch.stack([p.S0[b, h] for b, h in pairs]).unsqueeze(1)
    return oracle.forward(f64(pick(p.q)), f64(pick(p.k)), f64(pick(p.v)), f64(pick(p.log_alpha)),
                          f64(torch.stack([p.beta[b, :, h] for b, h in pairs]).unsqueeze(2)), S0=f64(S0))


def _ratio(num, den):
    """num / den elementwise, 0 where both are 0 (a slice that is exactly zero
    in the reference and in the result)."""
    return np.where(num == 0, 0.0, num / np.maximum(den, 1e-300))


def worst_per_head(gpu, ref, axes):
    """Largest normwise relative error over the (sequence, head) slices of a
    4-d array, each slice normalised by its own max |ref|."""
    d, a = np.abs(gpu - ref), np.abs(ref)
    return float(np.max(_ratio(d.max(axis=axes), a.max(axis=axes))))


def worst_per_chunk(gpu, ref, width=64):
    """Same for the width-token windows of every (sequence, head) of an output
    laid out [B, T, H, dv], each window normalised by its own max |ref|."""
    B, T, H, V = gpu.shape
    nc = -(-T // width)
    pad = ((0, 0), (0, nc * width - T), (0, 0), (0, 0))
    d = np.pad(np.abs(gpu - ref), pad).reshape(B, nc, width, H, V)
    a = np.pad(np.abs(ref), pad).reshape(B, nc, width, H, V)
    return float(np.max(_ratio(d.max(axis=(2, 4)), a.max(axis=(2, 4)))))


WORST = {}   # name -> (per-head out, per-chunk out, per-head state): the worst cases seen


def assert_close_device(name, out, sf, o_ref, s_ref, tol, width=64):
    """assert_close's metrics for two device results too large to copy to the
    host as float64 (out [B, T, H, dv] with T a multiple of width, states
    [B, H, dv, dk]); computed in fp32 on the GPU, exact for bf16 values."""
    def metrics(x, y, head_axes):
        d, a = (x.float() - y.float()).abs(), y.float().abs()
        e = (d.amax() / a.amax().clamp_min(1e-30)).item()
        ratio = lambda num, den: torch.where(num == 0, torch.zeros_like(num), num / den.clamp_min(1e-30))
        h = ratio(d.amax(dim=head_axes), a.amax(dim=head_axes)).amax().item()
        return d, a, e, h
    assert torch.isfinite(out).all() and torch.isfinite(sf).all()
    d, a, e_o, h_o = metrics(out, o_ref, (1, 3))
    B, T, H, V = out.shape
    dc, ac = d.view(B, T // width, width, H, V).amax(dim=(2, 4)), a.view(B, T // width, width, H, V).amax(dim=(2, 4))
    c_o = torch.where(dc == 0, torch.zeros_like(dc), dc / ac.clamp_min(1e-30)).amax().item()
    del d, a, dc, ac
    _, _, e_s, h_s = metrics(sf, s_ref, (2, 3))
    WORST[name] = (h_o, c_o, h_s)
    note(f"  {name}: out rel err {e_o:.3e} (worst head {h_o:.3e}, worst {width}-token chunk {c_o:.3e}), "
         f"S_final rel err {e_s:.3e} (worst head {h_s:.3e}) (bar {tol:g})")
    for what, v in (("output", e_o), ("state", e_s), ("output of one (sequence, head)", h_o),
                    ("output of one chunk", c_o), ("state of one (sequence, head)", h_s)):
        assert v < tol, f"{name}: {what} error {v}"


def assert_close(name, out, sf, o_ref, s_ref, tol):
    """Normwise relative error of the whole output and final state, and also the
    worst (sequence, head) slice and the worst 64-token window of each
    (sequence, head), each normalised by its own max |ref|: an error confined to
    one head or one chunk of small outputs cannot hide under the tensor's
    largest values."""
    assert np.all(np.isfinite(out)) and (sf is None or np.all(np.isfinite(sf)))
    e_o = rel(out, o_ref)
    e_s = rel(sf, s_ref) if s_ref is not None else 0.0
    h_o = worst_per_head(out, o_ref, (1, 3)) if out.ndim == 4 else e_o
    c_o = worst_per_chunk(out, o_ref) if out.ndim == 4 else e_o
    h_s = worst_per_head(sf, s_ref, (2, 3)) if (s_ref is not None and sf.ndim == 4) else e_s
    WORST[name] = (h_o, c_o, h_s)
    note(f"  {name}: out rel err {e_o:.3e} (worst head {h_o:.3e}, worst 64-token chunk {c_o:.3e}), "
         f"S_final rel err {e_s:.3e} (worst head {h_s:.3e}) (bar {tol:g})")
    assert e_o < tol, f"{name}: output error {e_o}"
    assert e_s < tol, f"{name}: state error {e_s}"
    assert h_o < tol, f"{name}: output error {h_o} in one (sequence, head)"
    assert c_o < tol, f"{name}: output error {c_o} in one 64-token chunk of one (sequence, head)"
    assert h_s < tol, f"{name}: state error {h_s} in one (sequence, head)"


# ---------------------------------------------------------------- small full-oracle cases
def test_tiny_fp32_workload(dev):
    w = kda_synth.WORKLOADS["tiny"]
    note("case tiny: B1 H1 T64 d16 fp32 C16")
    p = kda_synth.workload("tiny", device=dev)
    out, sf = gpu_chunk(p, w["C"])
    o_ref, s_ref = oracle_dense(p)
    assert_close("tiny", f64(out), f64(sf), o_ref, s_ref, TOL["f32"])


def test_small_bf16_workload(dev):
    w = kda_synth.WORKLOADS["small"]
    note("case small: B2 H4 T1024 d64 bf16 C64, S0 ~ N(0, 0.1)")
    p = kda_synth.workload("small", device=dev)
    out, sf = gpu_chunk(p, w["C"])
    o_ref, s_ref = oracle_dense(p)
    assert_close("small", f64(out), f64(sf), o_ref, s_ref, TOL["bf16"])


SHAPES = [
    # B, T, H, dk, dv, C, dtype
    (2, 200, 3, 128, 128, 64, "bf16"),   # ragged tail, 6 heads (no XCD remap)
    (1, 333, 8, 128, 128, 64, "bf16"),   # 8 heads (XCD remap on), 5 full chunks + 13 tokens
    (2, 100, 2, 64, 32, 32, "bf16"),
    (1, 77, 2, 32, 64, 16, "bf16"),
    (2, 50, 2, 16, 16, 16, "bf16"),
    (1, 130, 2, 64, 128, 64, "bf16"),   # dk != dv
    (1, 70, 1, 128, 16, 32, "bf16"),
    (1, 100, 2, 64, 64, 64, "f32"),
    (2, 90, 2, 128, 128, 32, "f32"),
    (1, 70, 3, 32, 16, 16, "f32"),
    (1, 129, 2, 16, 64, 64, "f32"),
]


@pytest.mark.parametrize("with_s0", [False, True])
@pytest.mark.parametrize("B,T,H,dk,dv,C,dtype", SHAPES)
def test_chunk_shapes(dev, B, T, H, dk, dv, C, dtype, with_s0):
    note(f"case chunk B{B} T{T} H{H} dk{dk} dv{dv} C{C} {dtype} S0={with_s0}")
    p = kda_synth.prefill(B, T, H, dk, dv, dtype=dtype, s0_sigma=0.1 if with_s0 else None,
                          seed=1000 + T + dk + dv + C, device=dev)
    out, sf = gpu_chunk(p, C)
    o_ref, s_ref = oracle_dense(p)
    assert_close("chunk", f64(out), f64(sf), o_ref, s_ref, TOL[dtype])


def test_chunk_matches_across_chunk_sizes(dev):
    """The chunk length is a schedule choice only: C = 16, 32, 64 agree."""
    note("case chunk-size invariance B1 T300 H2 d64 bf16")
    p = kda_synth.prefill(1, 300, 2, 64, 64, dtype="bf16", s0_sigma=0.1, seed=77, device=dev)
    o_ref, s_ref = oracle_dense(p)
    for C in (16, 32, 64):
        out, sf = gpu_chunk(p, C)
        assert_close(f"C={C}", f64(out), f64(sf), o_ref, s_ref, TOL["bf16"])


def test_chunk_edge_cases(dev):
    note("case edge: T=0 copies S0, T=1, in-place S_final == S0, no S_final")
    p = kda_synth.prefill(2, 0, 3, 64, 64, dtype="bf16", s0_sigma=0.1, seed=5, device=dev)
    out, sf = gpu_chunk(p, 64)
    assert out.shape[1] == 0 and torch.equal(sf, p.S0)
    p = kda_synth.prefill(2, 0, 3, 64, 64, dtype="bf16", s0_sigma=None, seed=5, device=dev)
    _, sf = gpu_chunk(p, 64)
    assert torch.count_nonzero(sf) == 0
    p = kda_synth.prefill(2, 1, 3, 64, 64, dtype="bf16", s0_sigma=0.1, seed=6, device=dev)
    out, sf = gpu_chunk(p, 64)
    o_ref, s_ref = oracle_dense(p)
    assert_close("T=1", f64(out), f64(sf), o_ref, s_ref, TOL["bf16"])
    # in place: S_final is the S0 buffer
    p = kda_synth.prefill(1, 150, 2, 128, 128, dtype="bf16", s0_sigma=0.1, seed=8, device=dev)
    o_ref, s_ref = oracle_dense(p)
    S = p.S0.clone()
    out = torch.empty_like(p.v)
    kda.kda_chunk_fwd(p.q, p.k, p.v, p.log_alpha, p.beta, S, out, S, 1, 150, 2, 128, 128, 64)
    torch.cuda.synchronize()
    assert_close("in-place", f64(out), f64(S), o_ref, s_ref, TOL["bf16"])
    out2, none = gpu_chunk(p, 64, final=False)
    assert none is None and torch.equal(out2, out)


SWEEP = [(dtype, dk, dv, C, H) for dtype in ("bf16", "f32")
         for dk, dv in ((16, 16), (32, 64), (64, 64), (128, 128), (64, 32))
         for C in (16, 32, 64) for H in (2, 8)]


@pytest.mark.parametrize("dtype,dk,dv,C,H", SWEEP)
def test_chunk_config_sweep(dev, dtype, dk, dv, C, H):
    """The single-pass kernel over input type x (dk, dv) x C x head count on a
    ragged T = 130 (8 heads group a head's value blocks on one XCD, 2 do
    not).  fp32 at dk = 128 with C = 64 runs as 32-token chunks (its 64-token
    operands do not fit the LDS); it is held to the same bar."""
    note(f"case sweep {dtype} dk{dk} dv{dv} C{C} H{H} T130")
    p = kda_synth.prefill(1, 130, H, dk, dv, dtype=dtype, s0_sigma=0.1, seed=5, device=dev)
    out, sf = kda.chunk_fwd(p.q, p.k, p.v, p.log_alpha, p.beta, S0=p.S0, C=C, segments=1)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle_dense(p)
    assert_close(f"sweep {dtype} dk{dk} dv{dv} C{C} H{H}", f64(out), f64(sf), o_ref, s_ref, TOL[dtype])


def test_chunk_fp32_dk128_c64_all_schedules(dev):
    """fp32 inputs at dk = 128 with C = 64 (run as 32-token chunks) through the
    single pass, the segmented schedule and packed sequences, against the
    oracle at the fp32 bar, and bit for bit against an explicit C = 32 call."""
    note("case fp32 dk128 C64: B2 T300 H2 dk128 dv128, single pass / 3 segments / varlen")
    p = kda_synth.prefill(2, 300, 2, 128, 128, dtype="f32", s0_sigma=0.1, seed=6, device=dev)
    o_ref, s_ref = oracle_dense(p)
    for segments in (1, 3):
        out, sf = gpu_chunk(p, 64, segments=segments)
        assert_close(f"fp32 dk128 C64 segments={segments}", f64(out), f64(sf), o_ref, s_ref, TOL["f32"])
        o32, s32 = gpu_chunk(p, 32, segments=segments)
        assert torch.equal(out, o32) and torch.equal(sf, s32)
    lengths = [130, 0, 77, 200]
    pv = kda_synth.prefill_varlen(lengths, 2, 128, 64, dtype="f32", s0_sigma=0.1, seed=7, device=dev)
    out, sf = kda.chunk_fwd_varlen(pv.q, pv.k, pv.v, pv.log_alpha, pv.beta, pv.cu_seqlens, S0=pv.S0, C=64)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.forward_varlen(f64(pv.q), f64(pv.k), f64(pv.v), f64(pv.log_alpha), f64(pv.beta),
                                         np.array(pv.cu_host), S0=f64(pv.S0))
    assert_close("fp32 dk128 C64 varlen", f64(out), f64(sf), o_ref, s_ref, TOL["f32"])


def test_chunk_decay_at_precondition_edge(dev):
    """log_alpha = -4.9 in every channel: 78 nats of decay per 16-token block,
    just inside the kernel's documented range."""
    note("case strong decay: log_alpha = -4.9, B1 T200 H2 d128 bf16")
    p = kda_synth.prefill(1, 200, 2, 128, 128, dtype="bf16", s0_sigma=0.1, seed=9, device=dev)
    p.log_alpha.fill_(-4.9)
    out, sf = gpu_chunk(p, 64)
    o_ref, s_ref = oracle_dense(p)
    assert_close("log_alpha=-4.9", f64(out), f64(sf), o_ref, s_ref, TOL["bf16"])
    note("case mixed decay: half the channels at -4.5, the rest ~ -softplus(N(-4,1.5))")
    p = kda_synth.prefill(1, 200, 2, 128, 128, dtype="bf16", s0_sigma=0.1, seed=10, device=dev)
    p.log_alpha[..., ::2] = -4.5
    out, sf = gpu_chunk(p, 64)
    o_ref, s_ref = oracle_dense(p)
    assert_close("mixed decay", f64(out), f64(sf), o_ref, s_ref, TOL["bf16"])


def test_chunk_repeated_key_full_writes(dev):
    """Every token of a head writes with the same unit key, beta = 1 and no
    decay: I + A is all ones below the diagonal, the hardest case for the
    triangular solve (its inverse has entries of +-1 while the powers of A
    grow like binomial coefficients)."""
    for dtype, tol in (("bf16", TOL["bf16"]), ("f32", TOL["f32"])):
        note(f"case repeated key: B1 T200 H2 d64 {dtype}, beta = 1, log_alpha = 0")
        p = kda_synth.prefill(1, 200, 2, 64, 64, dtype=dtype, s0_sigma=0.1, seed=21, device=dev)
        p.k.copy_(p.k[:, :1].expand_as(p.k))
        p.beta.fill_(1.0)
        p.log_alpha.zero_()
        out, sf = gpu_chunk(p, 64 if dtype == "bf16" else 32)
        o_ref, s_ref = oracle_dense(p)
        assert_close(f"repeated key {dtype}", f64(out), f64(sf), o_ref, s_ref, tol)


def test_chunk_mixes_fast_and_sub_block_paths(dev):
    """Strong decay only in some chunks: those take the sub-block path, the
    others the fast path, inside one sequence (and in fp32 mode)."""
    for dtype, tol in (("bf16", TOL["bf16"]), ("f32", TOL["f32"])):
        note(f"case mixed paths: B2 T300 H2 d64 {dtype}, tokens 70..100 and 250..260 at log_alpha = -3.5")
        p = kda_synth.prefill(2, 300, 2, 64, 64, dtype=dtype, s0_sigma=0.1, seed=14, device=dev)
        p.log_alpha[:, 70:100] = -3.5
        p.log_alpha[1, 250:260, 1, :32] = -3.5
        out, sf = gpu_chunk(p, 64 if dtype == "bf16" else 32)
        o_ref, s_ref = oracle_dense(p)
        assert_close(f"mixed paths {dtype}", f64(out), f64(sf), o_ref, s_ref, tol)


@pytest.mark.parametrize("dtype,dk,C", [("bf16", 64, 64), ("f32", 64, 32), ("bf16", 32, 32), ("bf16", 16, 64),
                                        ("bf16", 128, 64)])
def test_chunk_some_operand_waves_on_block_references(dev, dtype, dk, C):
    """Strong decay in the key channels of the first operand wave only (a
    quarter of them): in those chunks the other operand waves keep chunk-start
    references (w = 1) while one wave takes block references."""
    q4 = dk // 4
    note(f"case partial block references: B1 T600 H2 dk{dk} dv64 {dtype} C{C}, channels 0..{q4 - 1} of head 1 "
         "at -4.5")
    p = kda_synth.prefill(1, 600, 2, dk, 64, dtype=dtype, s0_sigma=0.1, seed=41, device=dev)
    p.log_alpha[:, 70:100] = -3.5
    p.log_alpha[:, 400:430, 1, :q4] = -4.5
    out, sf = gpu_chunk(p, C)
    o_ref, s_ref = oracle_dense(p)
    assert_close(f"partial block references {dtype}", f64(out), f64(sf), o_ref, s_ref, TOL[dtype])


# ---------------------------------------------------------------- strong and complete forgetting
# The per-channel gate lets a key channel be kept while another is cleared
# ("KDA derivation summary", sect. 5; alpha in (0, 1] with no lower bound in
# "Kimi K3 notes 1: KDA", sect. 4).  These cases decay some channels by far
# more than the fp32 range inside one 16-token block: runs at log_alpha = -30
# and -40 per token, and hard clears at -1e4 (alpha = 0 in fp32 and in float64).
DEEP = [("bf16", 128, 128, 64), ("bf16", 64, 64, 32), ("bf16", 32, 64, 16), ("bf16", 16, 32, 64),
        ("f32", 64, 64, 64), ("f32", 128, 64, 32), ("f32", 32, 32, 16)]


def deep_gates(la, kind):
    """Deep decay written into log_alpha [B, T, H, dk] in place."""
    B, T, H, dk = la.shape
    if kind == "run30":      # a quarter of the channels of head 0, then every channel of the last head
        la[:, 40:100, 0, : max(dk // 4, 4)] = -30.0
        la[:, 150:170, H - 1] = -30.0
    elif kind == "clear":    # a quarter of the channels cleared every 37 tokens, one token clears everything
        la[:, ::37, :, ::4] = -1e4
        la[:, 101, :, :] = -1e4
    elif kind == "all40":    # every channel at -40 for a long run (every block too deep to factor)
        la[:, 60:200] = -40.0
    else:
        raise ValueError(kind)


@pytest.mark.parametrize("kind", ["run30", "clear", "all40"])
@pytest.mark.parametrize("dtype,dk,dv,C", DEEP)
def test_chunk_deep_decay(dev, dtype, dk, dv, C, kind):
    B, T, H = 2, 260, 2
    note(f"case deep decay {kind}: B{B} T{T} H{H} dk{dk} dv{dv} {dtype} C{C}")
    p = kda_synth.prefill(B, T, H, dk, dv, dtype=dtype, s0_sigma=0.1, seed=131, device=dev)
    deep_gates(p.log_alpha, kind)
    out, sf = gpu_chunk(p, C)
    o_ref, s_ref = oracle_dense(p)
    assert_close(f"deep {kind} {dtype} dk{dk} C{C}", f64(out), f64(sf), o_ref, s_ref, TOL[dtype])


@pytest.mark.parametrize("bv", ["16", "32"])
def test_chunk_deep_decay_narrow_value_blocks(dev, bv, monkeypatch):
    """One or two state waves: the hard-block corrections of a chunk are shared
    by fewer waves (one wave takes every block at BV = 16)."""
    monkeypatch.setenv("KDA_CHUNK_BV", bv)
    for dtype, dk, C in (("bf16", 128, 64), ("f32", 64, 64)):
        note(f"case deep decay BV={bv}: B1 T260 H2 dk{dk} dv64 {dtype} C{C}")
        p = kda_synth.prefill(1, 260, 2, dk, 64, dtype=dtype, s0_sigma=0.1, seed=133, device=dev)
        deep_gates(p.log_alpha, "clear")
        deep_gates(p.log_alpha, "run30")
        out, sf = gpu_chunk(p, C)
        o_ref, s_ref = oracle_dense(p)
        assert_close(f"deep BV={bv} {dtype}", f64(out), f64(sf), o_ref, s_ref, TOL[dtype])


def test_segmented_and_varlen_deep_decay(dev):
    """Deep decay through the segment maps (the augmented state), the lead
    segment and the second pass, and through packed sequences."""
    for dtype, dk, C in (("bf16", 128, 64), ("f32", 64, 32)):
        for nseg in (3, 5):
            note(f"case segmented deep decay: B1 T600 H2 dk{dk} {dtype} C{C}, {nseg} segments")
            p = kda_synth.prefill(1, 600, 2, dk, 64, dtype=dtype, s0_sigma=0.1, seed=135, device=dev)
            deep_gates(p.log_alpha, "clear")
            p.log_alpha[:, 300:420, 1, : dk // 4] = -30.0
            out, sf = gpu_chunk(p, C, segments=nseg)
            o_ref, s_ref = oracle_dense(p)
            assert_close(f"segmented deep {dtype} nseg={nseg}", f64(out), f64(sf), o_ref, s_ref, TOL[dtype])
        lengths = [130, 0, 77, 300]
        note(f"case varlen deep decay: lengths {lengths} H2 dk{dk} {dtype} C{C}")
        p = kda_synth.prefill_varlen(lengths, 2, dk, 64, dtype=dtype, s0_sigma=0.1, seed=137, device=dev)
        deep_gates(p.log_alpha, "clear")
        deep_gates(p.log_alpha, "all40")
        for segments in (1, 3):
            out, sf = kda.chunk_fwd_varlen(p.q, p.k, p.v, p.log_alpha, p.beta, p.cu_seqlens, S0=p.S0, C=C,
                                           segments=segments)
            torch.cuda.synchronize()
            o_ref, s_ref = oracle.forward_varlen(f64(p.q), f64(p.k), f64(p.v), f64(p.log_alpha), f64(p.beta),
                                                 np.array(p.cu_host), S0=f64(p.S0))
            assert_close(f"varlen deep {dtype} segments={segments}", f64(out), f64(sf), o_ref, s_ref, TOL[dtype])


@pytest.mark.parametrize("gate,write", [("channel", "add"), ("scalar", "delta")])
def test_chunk_variants_deep_decay(dev, gate, write):
    """The additive write (GLA: only P needs the correction) and the scalar gate
    (every channel of a token clears together)."""
    for dtype, C in (("bf16", 64), ("f32", 32)):
        note(f"case variant deep decay gate={gate} write={write} B2 T260 H2 d64 {dtype} C{C}")
        p = kda_synth.prefill(2, 260, 2, 64, 64, dtype=dtype, s0_sigma=0.1, seed=139, device=dev)
        deep_gates(p.log_alpha, "clear")
        deep_gates(p.log_alpha, "run30")
        if gate == "scalar":
            p.log_alpha[..., 1:] = p.log_alpha[..., :1]
        la, la_full = variant_inputs(p, gate)
        o_ref, s_ref = oracle_variant(p, la_full, write)
        for segments in (1, 3):
            out, sf = kda.chunk_fwd(p.q, p.k, p.v, la, p.beta, S0=p.S0, C=C, segments=segments, gate=gate,
                                    write=write)
            torch.cuda.synchronize()
            assert_close(f"deep {gate}/{write} {dtype} segments={segments}", f64(out), f64(sf), o_ref, s_ref,
                         TOL[dtype])


def test_chunk_raw_inputs_deep_gates(dev):
    """Raw gate pre-activations g = 40 (log_alpha = -40) and g = 1e4 (a clear):
    the softplus inside the kernel, then the deep-decay path."""
    for dtype, dk, C in (("bf16", 128, 64), ("f32", 64, 32)):
        B, T, H, dv = 2, 260, 2, 64
        p = kda_synth.prefill_raw(B, T, H, dk, dv, dtype=dtype, s0_sigma=0.1, seed=141, device=dev)
        p.log_alpha[:, 40:120, :, : dk // 4] = 40.0
        p.log_alpha[:, 150:160, 1] = 40.0
        p.log_alpha[:, ::29, :, 1::4] = 1e4
        for gate in ("channel", "scalar"):
            note(f"case raw deep gates {gate}: B{B} T{T} H{H} dk{dk} {dtype} C{C}")
            o_ref, s_ref = oracle_raw(p, gate)
            for segments in (1, 3):
                out, sf = kda.chunk_fwd(p.q, p.k, p.v, raw_gate_arg(p, gate), p.beta, S0=p.S0, C=C,
                                        segments=segments, gate=gate, raw=True)
                torch.cuda.synchronize()
                assert_close(f"raw deep {gate} {dtype} segments={segments}", f64(out), f64(sf), o_ref, s_ref,
                             TOL[dtype])


def test_decode_equals_chunk_prefill_deep_decay(dev):
    """The two schedules of the one recurrence on a stream with deep decay and
    hard clears: decode steps, the multi-token decode and one chunk prefill
    agree with each other and with the oracle."""
    N, H, dk, dv, steps = 8, 4, 128, 128, 150
    note(f"case decode vs chunk prefill, deep decay: N{N} H{H} d128 bf16, {steps} tokens")
    d = kda_synth.decode(N, H, dk, dv, steps, seed=143, device=dev, step_block=50)
    tm = lambda t: t.transpose(0, 1).contiguous()
    la = tm(d.log_alpha)                   # [N, T, H, dk]
    deep_gates(la, "clear")
    la[:, 60:90, 0] = -30.0
    la[:, 100:140, 2, :32] = -40.0
    d.log_alpha.copy_(la.transpose(0, 1))
    S = d.S0.clone()
    outs = [kda.recurrent_step(d.q[t], d.k[t], d.v[t], d.log_alpha[t], d.beta[t], S) for t in range(steps)]
    dec = torch.stack(outs, dim=1)
    S_multi = d.S0.clone()
    multi = kda.recurrent_fwd(tm(d.q), tm(d.k), tm(d.v), la, tm(d.beta), S_multi)
    pre, sf = kda.chunk_fwd(tm(d.q), tm(d.k), tm(d.v), la, tm(d.beta), S0=d.S0, C=64, segments=1)
    torch.cuda.synchronize()
    assert torch.equal(multi, dec) and torch.equal(S_multi, S), "multi-token decode differs from single steps"
    e_o, e_s = rel(f64(dec), f64(pre)), rel(f64(S), f64(sf))
    note(f"  decode vs prefill: out rel diff {e_o:.3e}, state rel diff {e_s:.3e}")
    assert e_o < TOL["bf16"] and e_s < TOL["bf16"]
    o_ref, s_ref = oracle.forward(f64(tm(d.q)), f64(tm(d.k)), f64(tm(d.v)), f64(la), f64(tm(d.beta)),
                                  S0=f64(d.S0))
    assert_close("decode deep", f64(dec), f64(S), o_ref, s_ref, TOL["bf16"])
    assert_close("prefill deep", f64(pre), f64(sf), o_ref, s_ref, TOL["bf16"])


def test_chunk_guard_bands_untouched(dev):
    """Outputs written through interior pointers of larger buffers: the bands
    around out and S_final keep their sentinel values (no out-of-bounds stores)."""
    note("case guard bands B2 T150 H3 d64 bf16")
    B, T, H, dk, dv = 2, 150, 3, 64, 64
    p = kda_synth.prefill(B, T, H, dk, dv, dtype="bf16", s0_sigma=0.1, seed=12, device=dev)
    pad = 4096
    n_out, n_s = B * T * H * dv, B * H * dv * dk
    big_out = torch.full((n_out + 2 * pad,), 7.0, dtype=torch.bfloat16, device=dev)
    big_s = torch.full((n_s + 2 * pad,), -3.0, dtype=torch.float32, device=dev)
    out = big_out[pad:pad + n_out].view(B, T, H, dv)
    sf = big_s[pad:pad + n_s].view(B, H, dv, dk)
    kda.kda_chunk_fwd(p.q, p.k, p.v, p.log_alpha, p.beta, p.S0, out, sf, B, T, H, dk, dv, 64)
    torch.cuda.synchronize()
    assert torch.all(big_out[:pad] == 7.0) and torch.all(big_out[pad + n_out:] == 7.0)
    assert torch.all(big_s[:pad] == -3.0) and torch.all(big_s[pad + n_s:] == -3.0)
    o_ref, s_ref = oracle_dense(p)
    assert_close("guarded", f64(out), f64(sf), o_ref, s_ref, TOL["bf16"])


def test_chunk_is_deterministic(dev):
    note("case determinism B2 T500 H8 d128 bf16 (two runs, bitwise)")
    p = kda_synth.prefill(2, 500, 8, 128, 128, dtype="bf16", s0_sigma=0.1, seed=13, device=dev)
    o1, s1 = gpu_chunk(p, 64)
    o2, s2 = gpu_chunk(p, 64)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


# ---------------------------------------------------------------- segment-parallel schedule
SEG_SHAPES = [
    # B, T, H, dk, dv, C, dtype, segments, with_s0
    (1, 1000, 2, 64, 64, 64, "bf16", 2, True),
    (1, 1000, 2, 64, 64, 64, "bf16", 3, False),
    (2, 700, 2, 128, 128, 64, "bf16", 5, True),    # 11 chunks: segments of 3, 3, 3, 2 and 0 chunks
    (1, 1000, 1, 64, 64, 64, "bf16", 23, True),    # more segments than chunks: empty segments
    (1, 333, 2, 32, 64, 32, "f32", 4, True),
    (1, 300, 3, 128, 16, 64, "bf16", 3, True),     # dv < dk
    (1, 300, 2, 16, 128, 32, "bf16", 3, True),     # dk < dv: 16-row value blocks
    (2, 260, 2, 64, 32, 16, "f32", 6, True),
    (1, 520, 8, 128, 128, 64, "bf16", 4, True),    # 8 heads: XCD-aware workgroup mapping
]


@pytest.mark.parametrize("B,T,H,dk,dv,C,dtype,nseg,with_s0", SEG_SHAPES)
def test_segmented_matches_oracle(dev, B, T, H, dk, dv, C, dtype, nseg, with_s0):
    """The segment-parallel schedule (map launch with the lead segment,
    composition, second pass) against the oracle, and against the single pass
    on the same inputs."""
    note(f"case segmented B{B} T{T} H{H} dk{dk} dv{dv} C{C} {dtype} segments={nseg} S0={with_s0}")
    p = kda_synth.prefill(B, T, H, dk, dv, dtype=dtype, s0_sigma=0.1 if with_s0 else None,
                          seed=2000 + T + dk + dv + nseg, device=dev)
    out, sf = gpu_chunk(p, C, segments=nseg)
    o_ref, s_ref = oracle_dense(p)
    assert_close("segmented", f64(out), f64(sf), o_ref, s_ref, TOL[dtype])
    o1, s1 = gpu_chunk(p, C, segments=1)
    assert_close("segmented vs single pass", f64(out), f64(sf), f64(o1), f64(s1), TOL[dtype])


def test_segmented_strong_and_mixed_decay(dev):
    """Segments that take the sub-block decay path, and a decay strong enough
    that the segment maps are nearly zero."""
    for dtype, tol, C in (("bf16", TOL["bf16"], 64), ("f32", TOL["f32"], 32)):
        note(f"case segmented mixed paths: B1 T600 H2 d64 {dtype}, 4 segments")
        p = kda_synth.prefill(1, 600, 2, 64, 64, dtype=dtype, s0_sigma=0.1, seed=41, device=dev)
        p.log_alpha[:, 70:100] = -3.5
        p.log_alpha[:, 400:430, 1, :32] = -4.5
        out, sf = gpu_chunk(p, C, segments=4)
        o_ref, s_ref = oracle_dense(p)
        assert_close(f"segmented mixed {dtype}", f64(out), f64(sf), o_ref, s_ref, tol)


def test_segmented_in_place_and_no_final_state(dev):
    note("case segmented in place: S_final == S0, and S_final not requested")
    B, T, H, dk, dv, C, nseg = 1, 800, 2, 128, 128, 64, 3
    p = kda_synth.prefill(B, T, H, dk, dv, dtype="bf16", s0_sigma=0.1, seed=43, device=dev)
    o_ref, s_ref = oracle_dense(p)
    nbytes = kda.kda_chunk_segmented_workspace_bytes(B, H, dk, dv, nseg)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    S = p.S0.clone()
    out = torch.empty_like(p.v)
    kda.kda_chunk_fwd_segmented(p.q, p.k, p.v, p.log_alpha, p.beta, S, out, S, B, T, H, dk, dv, C, nseg, ws,
                                nbytes)
    torch.cuda.synchronize()
    assert_close("segmented in-place", f64(out), f64(S), o_ref, s_ref, TOL["bf16"])
    out2 = torch.empty_like(p.v)
    kda.kda_chunk_fwd_segmented(p.q, p.k, p.v, p.log_alpha, p.beta, p.S0, out2, None, B, T, H, dk, dv, C, nseg,
                                ws, nbytes)
    torch.cuda.synchronize()
    assert torch.equal(out2, out)


def test_segmented_varlen(dev):
    lengths = [300, 64, 1, 0, 517, 129]
    for dtype in ("bf16", "f32"):
        note(f"case segmented varlen lengths {lengths} H2 d64 {dtype} C32, 3 segments per sequence")
        p = kda_synth.prefill_varlen(lengths, 2, 64, 64, dtype=dtype, s0_sigma=0.1, seed=45, device=dev)
        out, sf = kda.chunk_fwd_varlen(p.q, p.k, p.v, p.log_alpha, p.beta, p.cu_seqlens, S0=p.S0, C=32,
                                       segments=3)
        torch.cuda.synchronize()
        o_ref, s_ref = oracle.forward_varlen(f64(p.q), f64(p.k), f64(p.v), f64(p.log_alpha), f64(p.beta),
                                             np.array(p.cu_host), S0=f64(p.S0))
        assert_close(f"segmented varlen {dtype}", f64(out), f64(sf), o_ref, s_ref, TOL[dtype])


@pytest.mark.parametrize("lead", ["0", "10", "25", "60"])
def test_segmented_lead_ratios(dev, lead, monkeypatch):
    """KDA_SEG_LEAD sets segment 0's length relative to the others (0: equal
    segments, segment 0 mapped like the rest): dense and packed inputs, with
    sequences short enough that segment 0 is empty."""
    monkeypatch.setenv("KDA_SEG_LEAD", lead)
    note(f"case segment lead {lead}: B1 T1000 H2 d64 bf16 C64, 5 segments; varlen, 4 segments")
    p = kda_synth.prefill(1, 1000, 2, 64, 64, dtype="bf16", s0_sigma=0.1, seed=47, device=dev)
    o_ref, s_ref = oracle_dense(p)
    out, sf = gpu_chunk(p, 64, segments=5)
    assert_close(f"lead {lead} dense", f64(out), f64(sf), o_ref, s_ref, TOL["bf16"])
    lengths = [700, 5, 0, 130, 64]
    p = kda_synth.prefill_varlen(lengths, 2, 128, 64, dtype="bf16", s0_sigma=0.1, seed=48, device=dev)
    out, sf = kda.chunk_fwd_varlen(p.q, p.k, p.v, p.log_alpha, p.beta, p.cu_seqlens, S0=p.S0, C=32, segments=4)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.forward_varlen(f64(p.q), f64(p.k), f64(p.v), f64(p.log_alpha), f64(p.beta),
                                         np.array(p.cu_host), S0=f64(p.S0))
    assert_close(f"lead {lead} varlen", f64(out), f64(sf), o_ref, s_ref, TOL["bf16"])


def test_segmented_is_deterministic(dev):
    note("case segmented determinism B1 T900 H2 d128 bf16, 4 segments (two runs, bitwise)")
    p = kda_synth.prefill(1, 900, 2, 128, 128, dtype="bf16", s0_sigma=0.1, seed=47, device=dev)
    o1, s1 = gpu_chunk(p, 64, segments=4)
    o2, s2 = gpu_chunk(p, 64, segments=4)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


# ---------------------------------------------------------------- segmented schedule without a second pass
@pytest.mark.parametrize("B,T,H,dk,dv,C,dtype,nseg,with_s0", SEG_SHAPES)
def test_one_pass_matches_oracle(dev, B, T, H, dk, dv, C, dtype, nseg, with_s0):
    """The schedule without a second pass (map launch with every later
    segment's outputs from a zero state, composition through S_final, output
    epilogue) against the oracle, and against the two-pass schedule."""
    note(f"case one-pass B{B} T{T} H{H} dk{dk} dv{dv} C{C} {dtype} segments={nseg} S0={with_s0}")
    p = kda_synth.prefill(B, T, H, dk, dv, dtype=dtype, s0_sigma=0.1 if with_s0 else None,
                          seed=2000 + T + dk + dv + nseg, device=dev)
    out, sf = kda.chunk_fwd(p.q, p.k, p.v, p.log_alpha, p.beta, S0=p.S0, C=C, segments=nseg, schedule="one-pass")
    torch.cuda.synchronize()
    o_ref, s_ref = oracle_dense(p)
    assert_close("one-pass", f64(out), f64(sf), o_ref, s_ref, TOL[dtype])
    o2, s2 = gpu_chunk(p, C, segments=nseg)
    assert_close("one-pass vs two-pass", f64(out), f64(sf), f64(o2), f64(s2), TOL[dtype])


def test_one_pass_varlen_variants_and_deep_decay(dev):
    """Packed sequences (empty and one-token ones included), every variant,
    raw inputs and deep decay through the schedule without a second pass."""
    lengths = [300, 64, 1, 0, 517, 129]
    for dtype in ("bf16", "f32"):
        note(f"case one-pass varlen lengths {lengths} H2 d64 {dtype} C32, 3 segments per sequence")
        p = kda_synth.prefill_varlen(lengths, 2, 64, 64, dtype=dtype, s0_sigma=0.1, seed=45, device=dev)
        out, sf = kda.chunk_fwd_varlen(p.q, p.k, p.v, p.log_alpha, p.beta, p.cu_seqlens, S0=p.S0, C=32,
                                       segments=3, schedule="one-pass")
        torch.cuda.synchronize()
        o_ref, s_ref = oracle.forward_varlen(f64(p.q), f64(p.k), f64(p.v), f64(p.log_alpha), f64(p.beta),
                                             np.array(p.cu_host), S0=f64(p.S0))
        assert_close(f"one-pass varlen {dtype}", f64(out), f64(sf), o_ref, s_ref, TOL[dtype])
    for gate, write in VARIANTS:
        for dtype, C in (("bf16", 64), ("f32", 32)):
            note(f"case one-pass variant {gate}/{write}: B1 T700 H2 d64 {dtype} C{C}, 4 segments")
            p = kda_synth.prefill(1, 700, 2, 64, 64, dtype=dtype, s0_sigma=0.1, seed=61, device=dev)
            la, la_full = variant_inputs(p, gate)
            o_ref, s_ref = oracle.forward(f64(p.q), f64(p.k), f64(p.v), f64(la_full), f64(p.beta), S0=f64(p.S0),
                                          write=write)
            out, sf = kda.chunk_fwd(p.q, p.k, p.v, la, p.beta, S0=p.S0, C=C, segments=4, gate=gate, write=write,
                                    schedule="one-pass")
            torch.cuda.synchronize()
            assert_close(f"one-pass {gate}/{write} {dtype}", f64(out), f64(sf), o_ref, s_ref, TOL[dtype])
    for gate in ("channel", "scalar"):
        note(f"case one-pass raw inputs gate={gate}: B1 T600 H2 d128 bf16 C64, 3 segments")
        p = kda_synth.prefill_raw(1, 600, 2, 128, 128, dtype="bf16", s0_sigma=0.1, seed=63, device=dev)
        o_ref, s_ref = oracle_raw(p, gate, "delta")
        out, sf = kda.chunk_fwd(p.q, p.k, p.v, raw_gate_arg(p, gate), p.beta, S0=p.S0, C=64, segments=3,
                                gate=gate, raw=True, schedule="one-pass")
        torch.cuda.synchronize()
        assert_close(f"one-pass raw {gate}", f64(out), f64(sf), o_ref, s_ref, TOL["bf16"])
    for dtype, dk, C in (("bf16", 128, 64), ("f32", 64, 32)):
        note(f"case one-pass deep decay: B1 T600 H2 dk{dk} {dtype} C{C}, 5 segments")
        p = kda_synth.prefill(1, 600, 2, dk, 64, dtype=dtype, s0_sigma=0.1, seed=135, device=dev)
        deep_gates(p.log_alpha, "clear")
        p.log_alpha[:, 300:420, 1, : dk // 4] = -30.0
        out, sf = kda.chunk_fwd(p.q, p.k, p.v, p.log_alpha, p.beta, S0=p.S0, C=C, segments=5, schedule="one-pass")
        torch.cuda.synchronize()
        o_ref, s_ref = oracle_dense(p)
        assert_close(f"one-pass deep {dtype}", f64(out), f64(sf), o_ref, s_ref, TOL[dtype])


@pytest.mark.parametrize("lengths", [[700, 64, 130, 0, 90, 1], [200, 200, 200], [1000, 990, 30]])
def test_one_pass_varlen_device_split(dev, lengths):
    """Packed sequences with segments="auto": the one-pass schedule whose
    split is planned on the device (here the 700-token sequence is split and
    the others run whole; with equal or two equally long sequences nothing is
    split and every map is the identity)."""
    for dtype, C in (("bf16", 32), ("f32", 32)):
        note(f"case one-pass device split: lengths {lengths} H2 d64 {dtype} C{C}")
        p = kda_synth.prefill_varlen(lengths, 2, 64, 64, dtype=dtype, s0_sigma=0.1, seed=71, device=dev)
        out, sf = kda.chunk_fwd_varlen(p.q, p.k, p.v, p.log_alpha, p.beta, p.cu_seqlens, S0=p.S0, C=C,
                                       segments="auto")
        torch.cuda.synchronize()
        o_ref, s_ref = oracle.forward_varlen(f64(p.q), f64(p.k), f64(p.v), f64(p.log_alpha), f64(p.beta),
                                             np.array(p.cu_host), S0=f64(p.S0))
        assert_close(f"one-pass device split {dtype}", f64(out), f64(sf), o_ref, s_ref, TOL[dtype])


def test_one_pass_varlen_device_split_many_sequences(dev):
    """The plan of the device-side split made by one workgroup over more
    sequences than it has threads (reductions across threads): 600 short
    sequences and two long ones, one of which is split."""
    rng = np.random.default_rng(81)
    lengths = [int(x) for x in rng.integers(0, 40, size=600)]
    lengths[123] = 2000
    lengths[480] = 700
    note(f"case one-pass device split, {len(lengths)} sequences (two long: 2000 and 700 tokens) H1 d32 bf16 C32")
    p = kda_synth.prefill_varlen(lengths, 1, 32, 32, dtype="bf16", s0_sigma=0.1, seed=82, device=dev)
    out, sf = kda.chunk_fwd_varlen(p.q, p.k, p.v, p.log_alpha, p.beta, p.cu_seqlens, S0=p.S0, C=32, segments="auto")
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.forward_varlen(f64(p.q), f64(p.k), f64(p.v), f64(p.log_alpha), f64(p.beta),
                                         np.array(p.cu_host), S0=f64(p.S0))
    assert_close("one-pass device split, many sequences", f64(out), f64(sf), o_ref, s_ref, TOL["bf16"])


def test_one_pass_in_place_no_final_state_and_determinism(dev):
    note("case one-pass in place: S_final == S0, S_final not requested, two runs bitwise")
    B, T, H, dk, dv, C, nseg = 1, 800, 2, 128, 128, 64, 3
    p = kda_synth.prefill(B, T, H, dk, dv, dtype="bf16", s0_sigma=0.1, seed=43, device=dev)
    o_ref, s_ref = oracle_dense(p)
    var = kda.variant(schedule="one-pass")
    nbytes = kda.kda_chunk_segmented_workspace_bytes_ex(B, B * T, H, dk, dv, nseg, var, False)
    assert nbytes > kda.kda_chunk_segmented_workspace_bytes(B, H, dk, dv, nseg)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    S = p.S0.clone()
    out = torch.empty_like(p.v)
    kda.kda_chunk_fwd_ex(p.q, p.k, p.v, p.log_alpha, p.beta, S, out, S, B, T, H, dk, dv, C, var, nseg, ws, nbytes)
    torch.cuda.synchronize()
    assert_close("one-pass in-place", f64(out), f64(S), o_ref, s_ref, TOL["bf16"])
    out2 = torch.empty_like(p.v)
    kda.kda_chunk_fwd_ex(p.q, p.k, p.v, p.log_alpha, p.beta, p.S0, out2, None, B, T, H, dk, dv, C, var, nseg, ws,
                         nbytes)
    torch.cuda.synchronize()
    assert torch.equal(out2, out)
    with pytest.raises(kda.KdaError):   # one byte short of the workspace it needs
        kda.kda_chunk_fwd_ex(p.q, p.k, p.v, p.log_alpha, p.beta, p.S0, out2, None, B, T, H, dk, dv, C, var, nseg,
                             ws, nbytes - 1)


# ---------------------------------------------------------------- variants (gate, write)
VARIANTS = [("scalar", "delta"), ("none", "delta"), ("channel", "add"), ("scalar", "add"), ("none", "add")]


def variant_inputs(p, gate):
    """The log_alpha argument of a variant and the per-channel log_alpha the
    oracle sees for it (a scalar gate broadcast to every key channel, or 0)."""
    if gate == "channel":
        return p.log_alpha, p.log_alpha
    if gate == "scalar":
        la = p.log_alpha[..., 0].contiguous()
        return la, la.unsqueeze(-1).expand_as(p.log_alpha).contiguous()
    return None, torch.zeros_like(p.log_alpha)


def oracle_variant(p, la_full, write, S0=None):
    return oracle.forward(f64(p.q), f64(p.k), f64(p.v), f64(la_full), f64(p.beta),
                          S0=f64(p.S0 if S0 is None else S0), write=write)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("gate,write", VARIANTS)
def test_chunk_variants(dev, gate, write, dtype):
    B, T, H, dk, dv = 2, 200, 2, 64, 64
    C = 64 if dtype == "bf16" else 32
    note(f"case chunk variant gate={gate} write={write} B{B} T{T} H{H} d{dk} {dtype} C{C}")
    p = kda_synth.prefill(B, T, H, dk, dv, dtype=dtype, s0_sigma=0.1, seed=81, device=dev)
    la, la_full = variant_inputs(p, gate)
    o_ref, s_ref = oracle_variant(p, la_full, write)
    for segments in (1, 3):
        out, sf = kda.chunk_fwd(p.q, p.k, p.v, la, p.beta, S0=p.S0, C=C, segments=segments, gate=gate, write=write)
        torch.cuda.synchronize()
        assert_close(f"{gate}/{write} segments={segments}", f64(out), f64(sf), o_ref, s_ref, TOL[dtype])


def test_chunk_variant_varlen_and_wide_heads(dev):
    lengths = [130, 0, 77, 200]
    for gate, write in (("scalar", "delta"), ("channel", "add")):
        note(f"case varlen variant gate={gate} write={write} lengths {lengths} H2 dk128 dv128 bf16")
        p = kda_synth.prefill_varlen(lengths, 2, 128, 128, dtype="bf16", s0_sigma=0.1, seed=83, device=dev)
        la, la_full = variant_inputs(p, gate)
        T_total, N = sum(lengths), len(lengths)
        out = torch.empty_like(p.v)
        sf = torch.empty((N, 2, 128, 128), dtype=torch.float32, device=dev)
        kda.kda_chunk_fwd_varlen_ex(p.q, p.k, p.v, la, p.beta, p.S0, out, sf, p.cu_seqlens, N, T_total, 2, 128,
                                    128, 64, kda.variant(gate, write))
        torch.cuda.synchronize()
        o_ref, s_ref = oracle.forward_varlen(f64(p.q), f64(p.k), f64(p.v), f64(la_full), f64(p.beta),
                                             np.array(p.cu_host), S0=f64(p.S0), write=write)
        assert_close(f"varlen {gate}/{write}", f64(out), f64(sf), o_ref, s_ref, TOL["bf16"])


@pytest.mark.parametrize("gate,write", VARIANTS)
def test_decode_variants(dev, gate, write):
    for dtype, T in (("bf16", 5), ("f32", 5), ("bf16", 19), ("f32", 19)):   # 19: two token tiles
        N, H, dk, dv = 3, 2, 128, 64
        note(f"case decode variant gate={gate} write={write} N{N} T{T} H{H} dk{dk} dv{dv} {dtype}")
        p = kda_synth.prefill(N, T, H, dk, dv, dtype=dtype, s0_sigma=0.1, seed=85, device=dev)
        la, la_full = variant_inputs(p, gate)
        o_ref, s_ref = oracle_variant(p, la_full, write)
        S = p.S0.clone()
        out = kda.recurrent_fwd(p.q, p.k, p.v, la, p.beta, S, gate=gate, write=write)
        torch.cuda.synchronize()
        assert_close(f"decode {gate}/{write} T={T}", f64(out), f64(S), o_ref, s_ref, TOL[dtype])
        if T > 5:
            continue
        # one token per launch through the same entry point (the step kernel)
        S = p.S0.clone()
        outs = [kda.recurrent_fwd(p.q[:, t:t + 1].contiguous(), p.k[:, t:t + 1].contiguous(),
                                  p.v[:, t:t + 1].contiguous(),
                                  None if la is None else la[:, t:t + 1].contiguous(),
                                  p.beta[:, t:t + 1].contiguous(), S, gate=gate, write=write) for t in range(T)]
        torch.cuda.synchronize()
        assert_close(f"decode {gate}/{write} T=1 x{T}", f64(torch.cat(outs, dim=1)), f64(S), o_ref, s_ref,
                     TOL[dtype])


# ---------------------------------------------------------------- fused input preparation
def oracle_raw(p, gate, write="delta", varlen=False):
    """The oracle on the raw inputs: q, k normalised and log_alpha = -softplus(g)
    by oracle.prepare (float64), then the recurrence."""
    g = None if gate == "none" else (p.log_alpha[..., 0] if gate == "scalar" else p.log_alpha)
    qn, kn, la = oracle.prepare(f64(p.q), f64(p.k), None if g is None else f64(g), gate=gate)
    if varlen:
        return oracle.forward_varlen(qn, kn, f64(p.v), la, f64(p.beta), np.array(p.cu_host), S0=f64(p.S0),
                                     write=write)
    return oracle.forward(qn, kn, f64(p.v), la, f64(p.beta), S0=f64(p.S0), write=write)


def raw_gate_arg(p, gate):
    if gate == "channel":
        return p.log_alpha
    if gate == "scalar":
        return p.log_alpha[..., 0].contiguous()
    return None


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("gate,write", [("channel", "delta"), ("scalar", "delta"), ("none", "delta"),
                                        ("channel", "add")])
def test_chunk_raw_inputs(dev, gate, write, dtype):
    """q, k un-normalised (different scales per token) and gate pre-activations:
    normalisation and softplus inside the kernel, both schedules."""
    B, T, H, dk, dv = 2, 230, 2, 128 if dtype == "bf16" else 64, 64
    C = 64 if dtype == "bf16" else 32
    note(f"case raw inputs gate={gate} write={write} B{B} T{T} H{H} dk{dk} dv{dv} {dtype} C{C}")
    p = kda_synth.prefill_raw(B, T, H, dk, dv, dtype=dtype, s0_sigma=0.1, q_sigma=2.0, k_sigma=0.5, seed=91,
                              device=dev)
    # a spread of key and query norms across tokens
    scale = torch.exp(torch.linspace(-2.0, 2.0, T, device=dev)).view(1, T, 1, 1)
    p.k = (p.k.float() * scale).to(p.k.dtype)
    p.q = (p.q.float() * scale.flip(1)).to(p.q.dtype)
    o_ref, s_ref = oracle_raw(p, gate, write)
    for segments in (1, 3):
        out, sf = kda.chunk_fwd(p.q, p.k, p.v, raw_gate_arg(p, gate), p.beta, S0=p.S0, C=C, segments=segments,
                                gate=gate, write=write, raw=True)
        torch.cuda.synchronize()
        assert_close(f"raw {gate}/{write} segments={segments}", f64(out), f64(sf), o_ref, s_ref, TOL[dtype])


NARROW = [(1, 200, 2, 128, 128, 64, "bf16"), (2, 150, 2, 64, 64, 32, "f32"), (1, 130, 3, 128, 64, 16, "bf16")]


@pytest.mark.parametrize("bv", ["16", "32"])
def test_chunk_narrow_value_blocks(dev, bv, monkeypatch):
    """The library takes the widest value block that fits, so the one- and
    two-state-wave kernels serve dv = 16 and 32 by default; KDA_CHUNK_BV selects
    them for wider heads too.  Single pass, segmented and raw inputs against
    the oracle."""
    monkeypatch.setenv("KDA_CHUNK_BV", bv)
    for B, T, H, dk, dv, C, dtype in NARROW:
        note(f"case value block {bv}: B{B} T{T} H{H} dk{dk} dv{dv} C{C} {dtype}")
        p = kda_synth.prefill(B, T, H, dk, dv, dtype=dtype, s0_sigma=0.1, seed=31 + T, device=dev)
        o_ref, s_ref = oracle_dense(p)
        for segments in (1, 3):
            out, sf = gpu_chunk(p, C, segments=segments)
            assert_close(f"BV={bv} segments={segments}", f64(out), f64(sf), o_ref, s_ref, TOL[dtype])
    p = kda_synth.prefill_raw(1, 170, 2, 128, 128, dtype="bf16", s0_sigma=0.1, q_sigma=2.0, k_sigma=0.5, seed=33,
                              device=dev)
    o_ref, s_ref = oracle_raw(p, "channel", "delta")
    out, sf = kda.chunk_fwd(p.q, p.k, p.v, raw_gate_arg(p, "channel"), p.beta, S0=p.S0, C=64, segments=1,
                            gate="channel", write="delta", raw=True)
    torch.cuda.synchronize()
    assert_close(f"BV={bv} raw", f64(out), f64(sf), o_ref, s_ref, TOL["bf16"])


@pytest.mark.parametrize("dtype,dk,C", [("bf16", 128, 64), ("bf16", 64, 64), ("f32", 64, 32)])
def test_chunk_raw_inputs_strong_and_mixed_decay(dev, dtype, dk, C):
    """Raw gates where some chunks decay by more than 80 nats in some key
    channels (g = 2: about 2.1 nats per token, 34 per 16-token block): waves
    whose channels all stay within 80 nats over the chunk take the products
    path, the others the log-domain path with block references, inside one
    sequence; per-channel and scalar gates."""
    B, T, H, dv = 2, 300, 2, 64
    note(f"case raw inputs, strong and mixed decay: B{B} T{T} H{H} dk{dk} dv{dv} {dtype} C{C}")
    p = kda_synth.prefill_raw(B, T, H, dk, dv, dtype=dtype, s0_sigma=0.1, seed=97, device=dev)
    p.log_alpha[:, 70:140, :, : dk // 4] = 2.0      # a quarter of the key channels (one operand wave's)
    p.log_alpha[1, 200:260, 1] = 1.5                 # every channel of one head
    for gate in ("channel", "scalar"):
        o_ref, s_ref = oracle_raw(p, gate)
        out, sf = kda.chunk_fwd(p.q, p.k, p.v, raw_gate_arg(p, gate), p.beta, S0=p.S0, C=C, segments=1,
                                gate=gate, raw=True)
        torch.cuda.synchronize()
        assert_close(f"raw strong/mixed {gate}", f64(out), f64(sf), o_ref, s_ref, TOL[dtype])


def test_chunk_raw_inputs_varlen_and_zero_rows(dev):
    lengths = [150, 1, 0, 97]
    note(f"case raw inputs varlen lengths {lengths} H2 d128 bf16, zero q and k rows")
    p = kda_synth.prefill_raw(1, sum(lengths), 2, 128, 128, dtype="bf16", seed=93, device=dev)
    cu = [0]
    for n in lengths:
        cu.append(cu[-1] + n)
    p.cu_host = cu
    p.cu_seqlens = torch.tensor(cu, dtype=torch.int32, device=dev)
    p.S0 = torch.randn((len(lengths), 2, 128, 128), device=dev) * 0.1
    p.k[0, 5, 1] = 0     # a zero key writes nothing
    p.q[0, 9, 0] = 0     # a zero query reads nothing
    out = torch.empty_like(p.v)
    sf = torch.empty_like(p.S0)
    kda.kda_chunk_fwd_varlen_ex(p.q, p.k, p.v, p.log_alpha, p.beta, p.S0, out, sf, p.cu_seqlens, len(lengths),
                                sum(lengths), 2, 128, 128, 64, kda.variant(raw=True))
    torch.cuda.synchronize()
    o_ref, s_ref = oracle_raw(p, "channel", varlen=True)
    assert torch.isfinite(out.float()).all()
    assert_close("raw varlen", f64(out), f64(sf), o_ref, s_ref, TOL["bf16"])


@pytest.mark.parametrize("gate", ["channel", "scalar", "none"])
def test_decode_raw_inputs(dev, gate):
    for dtype in ("bf16", "f32"):
        N, T, H, dk, dv = 4, 21, 2, 64, 128   # two token tiles; 8 heads, 2 workgroups each
        note(f"case decode raw inputs gate={gate} N{N} T{T} H{H} dk{dk} dv{dv} {dtype}")
        p = kda_synth.prefill_raw(N, T, H, dk, dv, dtype=dtype, s0_sigma=0.1, q_sigma=3.0, k_sigma=0.3, seed=95,
                                  device=dev)
        o_ref, s_ref = oracle_raw(p, gate)
        S = p.S0.clone()
        out = kda.recurrent_fwd(p.q, p.k, p.v, raw_gate_arg(p, gate), p.beta, S, gate=gate, raw=True)
        torch.cuda.synchronize()
        assert_close(f"decode raw {gate}", f64(out), f64(S), o_ref, s_ref, TOL[dtype])


# ---------------------------------------------------------------- packed variable length
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_varlen_small(dev, dtype):
    lengths = [5, 0, 64, 130, 1, 77]
    note(f"case varlen lengths {lengths} H3 d64 {dtype} C32")
    p = kda_synth.prefill_varlen(lengths, 3, 64, 64, dtype=dtype, s0_sigma=0.1, seed=21, device=dev)
    out, sf = kda.chunk_fwd_varlen(p.q, p.k, p.v, p.log_alpha, p.beta, p.cu_seqlens, S0=p.S0, C=32)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.forward_varlen(f64(p.q), f64(p.k), f64(p.v), f64(p.log_alpha), f64(p.beta),
                                         np.array(p.cu_host), S0=f64(p.S0))
    assert_close("varlen", f64(out), f64(sf), o_ref, s_ref, TOL[dtype])


def test_varlen_equals_dense_per_sequence(dev):
    """A packed stream gives each sequence exactly what a dense call on that
    sequence alone gives (same kernel, same chunk grid)."""
    lengths = [100, 64, 37]
    note(f"case varlen vs dense lengths {lengths} H2 d128 bf16")
    p = kda_synth.prefill_varlen(lengths, 2, 128, 128, dtype="bf16", s0_sigma=0.1, seed=22, device=dev)
    out, sf = kda.chunk_fwd_varlen(p.q, p.k, p.v, p.log_alpha, p.beta, p.cu_seqlens, S0=p.S0, C=64)
    for n, L in enumerate(lengths):
        a, b = p.cu_host[n], p.cu_host[n + 1]
        o_n, s_n = kda.chunk_fwd(p.q[:, a:b].contiguous(), p.k[:, a:b].contiguous(), p.v[:, a:b].contiguous(),
                                 p.log_alpha[:, a:b].contiguous(), p.beta[:, a:b].contiguous(),
                                 S0=p.S0[n:n + 1].contiguous(), C=64, segments=1)
        torch.cuda.synchronize()
        assert torch.equal(out[:, a:b], o_n) and torch.equal(sf[n:n + 1], s_n)


def test_varlen_malformed_offsets_stay_in_bounds(dev):
    """cu_seqlens that break the precondition (negative, decreasing, past
    T_total): the kernel clamps each sequence to [0, T_total] with end >= start.
    Inputs sit between NaN bands and out between sentinel bands; the bands are
    neither read (states stay finite) nor written, and every output row and state
    that one clamped sequence alone owns matches the oracle on that sequence."""
    T_total, H, dk, dv, pad = 100, 2, 64, 64, 256
    cu = [-3, 0, 40, 30, T_total + 50]   # clamped: [0, 0), [0, 40), [40, 40), [30, 100)
    note(f"case varlen malformed offsets {cu} T_total {T_total} H{H} d64 bf16")
    p = kda_synth.prefill_varlen([T_total], H, dk, dv, dtype="bf16", s0_sigma=None, seed=24, device=dev)
    g = torch.Generator(device=dev).manual_seed(25)
    S0 = torch.randn((4, H, dv, dk), generator=g, device=dev) * 0.1

    def banded(t, fill):
        big = torch.full((1, T_total + 2 * pad) + tuple(t.shape[2:]), fill, dtype=t.dtype, device=dev)
        big[:, pad:pad + T_total] = t
        return big, big[:, pad:pad + T_total]

    ins = [banded(t, float("nan")) for t in (p.q, p.k, p.v, p.log_alpha, p.beta)]
    big_out, out = banded(torch.empty_like(p.v), 9.0)
    big_out[:, pad:pad + T_total] = 9.0
    sf = torch.empty_like(S0)
    cu_dev = torch.tensor(cu, dtype=torch.int32, device=dev)
    kda.kda_chunk_fwd_varlen(*(view for _, view in ins), S0, out, sf, cu_dev, 4, T_total, H, dk, dv, 64)
    torch.cuda.synchronize()
    assert torch.all(big_out[:, :pad] == 9.0) and torch.all(big_out[:, pad + T_total:] == 9.0)
    assert torch.all(torch.isfinite(sf))
    assert torch.equal(sf[0], S0[0]) and torch.equal(sf[2], S0[2])   # empty after clamping
    for n, (a, b), own in ((1, (0, 40), (0, 30)), (3, (30, 100), (40, 100))):
        o_ref, s_ref = oracle.forward(f64(p.q[:, a:b]), f64(p.k[:, a:b]), f64(p.v[:, a:b]),
                                      f64(p.log_alpha[:, a:b]), f64(p.beta[:, a:b]), S0=f64(S0[n:n + 1]))
        lo, hi = own[0] - a, own[1] - a
        assert_close(f"clamped sequence {n}", f64(out[:, own[0]:own[1]]), f64(sf[n:n + 1]),
                     o_ref[:, lo:hi], s_ref, TOL["bf16"])


@pytest.mark.parametrize("segments", [1, "auto"])
def test_varlen_workload_sampled(dev, segments):
    """The varlen workload in one pass, and with the device-side split of its
    longest sequence (what bench.py times), on one sampled head per sequence."""
    w = kda_synth.WORKLOADS["varlen"]
    note(f"case varlen workload: 8 sequences U[2048,16384] x H16 d128 bf16 C64 (sampled heads), segments={segments}")
    p = kda_synth.workload("varlen", device=dev)
    out, sf = kda.chunk_fwd_varlen(p.q, p.k, p.v, p.log_alpha, p.beta, p.cu_seqlens, S0=p.S0, C=w["C"],
                                   segments=segments)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all() and torch.isfinite(sf).all()
    errs_o, errs_s = [], []
    for n in range(len(p.cu_host) - 1):
        a, b = p.cu_host[n], p.cu_host[n + 1]
        h = (5 * n + 3) % w["H"]
        sl = lambda t: t[:, a:b, h:h + 1]
        o_ref, s_ref = oracle.forward(f64(sl(p.q)), f64(sl(p.k)), f64(sl(p.v)), f64(sl(p.log_alpha)),
                                      f64(p.beta[:, a:b, h:h + 1]), S0=f64(p.S0[n:n + 1, h:h + 1]))
        errs_o.append(rel(f64(out[:, a:b, h:h + 1]), o_ref))
        errs_s.append(rel(f64(sf[n:n + 1, h:h + 1]), s_ref))
    note(f"  varlen sampled: worst out rel err {max(errs_o):.3e}, worst S rel err {max(errs_s):.3e}")
    assert max(errs_o) < TOL["bf16"] and max(errs_s) < TOL["bf16"]


# ---------------------------------------------------------------- full-size prefill workloads
def test_mid_workload_sampled(dev):
    w = kda_synth.WORKLOADS["mid"]
    note("case mid workload: B4 H32 T8192 d128 bf16 C64 (8 sampled heads)")
    p = kda_synth.workload("mid", device=dev)
    out, sf = gpu_chunk(p, w["C"])
    assert torch.isfinite(out.float()).all() and torch.isfinite(sf).all()
    pairs = [(0, 0), (0, 31), (1, 7), (1, 16), (2, 3), (2, 25), (3, 12), (3, 30)]
    o_ref, s_ref = sampled(p, pairs)
    o_gpu = np.stack([f64(out[b, :, h]) for b, h in pairs])[:, :, None]
    s_gpu = np.stack([f64(sf[b, h]) for b, h in pairs])[:, None]
    assert_close("mid sampled", o_gpu, s_gpu, o_ref, s_ref, TOL["bf16"])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prep_workload_sampled(dev, dtype):
    """The fused input preparation at the sizes the bench times it on: the mid
    sizes with raw q, k and gate pre-activations in the input type (bf16, and
    fp32 with the same recipe; one launch of the raw-input kernel), sampled
    heads against the oracle on the raw inputs."""
    w = kda_synth.WORKLOADS["mid"]
    B, T, H, dk, dv, C = w["B"], w["T"], w["H"], w["dk"], w["dv"], w["C"]
    note(f"case fused preparation at mid sizes: B4 H32 T8192 d128, raw q, k, {dtype} g (4 sampled heads)")
    p = kda_synth.prefill_raw(B, T, H, dk, dv, dtype=dtype, g_mu=w["g_mu"], g_sigma=w["g_sigma"],
                              seed=kda_synth.SEEDS["mid"], device=dev)
    out = torch.empty((B, T, H, dv), dtype=kda_synth.DTYPES[dtype], device=dev)
    sf = torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev)
    chunk_ex = kda.kda_chunk_fwd_ex if dtype == "bf16" else kda.kda_chunk_fwd_ex_f32
    chunk_ex(p.q, p.k, p.v, p.log_alpha, p.beta, None, out, sf, B, T, H, dk, dv, C,
                         kda.variant(raw=True), 1, None, 0)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all() and torch.isfinite(sf).all()
    pairs = [(0, 2), (1, 29), (2, 14), (3, 31)]
    pick = lambda t: torch.stack([t[b, :, h] for b, h in pairs]).unsqueeze(2)
    qn, kn, la = oracle.prepare(f64(pick(p.q)), f64(pick(p.k)), f64(pick(p.log_alpha)), gate="channel")
    o_ref, s_ref = oracle.forward(qn, kn, f64(pick(p.v)), la, f64(torch.stack([p.beta[b, :, h] for b, h in pairs]).unsqueeze(2)))
    o_gpu = np.stack([f64(out[b, :, h]) for b, h in pairs])[:, :, None]
    s_gpu = np.stack([f64(sf[b, h]) for b, h in pairs])[:, None]
    assert_close(f"prep sampled {dtype}", o_gpu, s_gpu, o_ref, s_ref, TOL[dtype])


@pytest.mark.parametrize("segments", [1, 4])
def test_scalar_gate_workload_sampled(dev, segments):
    """The general variant kernel at the mid sizes, with one decay per token
    and head (the scalar gate): the single pass, and the one-pass segmented
    schedule with 4 segments (the variant map pass, its outputs and the
    epilogue), sampled heads against the oracle with the gate broadcast over
    the key channels."""
    w = kda_synth.WORKLOADS["mid"]
    B, T, H, dk, dv, C = w["B"], w["T"], w["H"], w["dk"], w["dv"], w["C"]
    note(f"case scalar gate at mid sizes: B4 H32 T8192 d128, {segments} segment(s) (4 sampled heads)")
    p = kda_synth.workload("mid", device=dev)
    la = p.log_alpha[..., 0].contiguous()   # [B, T, H]
    out = torch.empty((B, T, H, dv), dtype=torch.bfloat16, device=dev)
    sf = torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev)
    var = kda.variant(gate="scalar", schedule="one-pass" if segments > 1 else "two-pass")
    ws, wsb = None, 0
    if segments > 1:
        wsb = kda.kda_chunk_segmented_workspace_bytes_ex(B, B * T, H, dk, dv, segments, var, False)
        assert wsb > 0
        ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    kda.kda_chunk_fwd_ex(p.q, p.k, p.v, la, p.beta, None, out, sf, B, T, H, dk, dv, C, var, segments, ws, wsb)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all() and torch.isfinite(sf).all()
    pairs = [(0, 5), (1, 17), (2, 30), (3, 8)]
    ref = kda_synth.Prefill(p.q, p.k, p.v, la[..., None].expand(B, T, H, dk), p.beta, None)
    o_ref, s_ref = sampled(ref, pairs)
    o_gpu = np.stack([f64(out[b, :, h]) for b, h in pairs])[:, :, None]
    s_gpu = np.stack([f64(sf[b, h]) for b, h in pairs])[:, None]
    assert_close(f"scalar gate sampled, {segments} segment(s)", o_gpu, s_gpu, o_ref, s_ref, TOL["bf16"])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_multi_workload_sampled(dev, dtype):
    """The multi-token launch the bench times: the decode workload's sizes
    (256 sequences x 32 heads, d = 128) with 4 tokens per launch, in bf16 and
    fp32 inputs, sampled heads against the oracle."""
    w = kda_synth.WORKLOADS["decode"]
    N, H, dk, dv, T = w["N"], w["H"], w["dk"], w["dv"], 4
    note(f"case multi-token decode at decode sizes: N256 H32 d128 {dtype}, T4 (12 sampled heads)")
    p = kda_synth.prefill(N, T, H, dk, dv, dtype=dtype, g_mu=w["g_mu"], g_sigma=w["g_sigma"],
                          beta=w["beta"], s0_sigma=w["s0_sigma"], seed=kda_synth.SEEDS["decode"], device=dev)
    S = p.S0.clone()
    out = kda.recurrent_fwd(p.q, p.k, p.v, p.log_alpha, p.beta, S)
    torch.cuda.synchronize()
    pairs = [(n, h) for n, h in zip(range(5, 256, 21), range(1, 32, 3))]
    o_ref, s_ref = sampled(p, pairs)
    o_gpu = np.stack([f64(out[n, :, h]) for n, h in pairs])[:, :, None]
    s_gpu = np.stack([f64(S[n, h]) for n, h in pairs])[:, None]
    assert_close(f"multi-token decode sampled {dtype}", o_gpu, s_gpu, o_ref, s_ref, TOL[dtype])


def test_long_workload_sampled(dev):
    """Both schedules of the long workload: the segment-parallel one with the
    library's segment count (what bench.py times) and the single pass."""
    w = kda_synth.WORKLOADS["long"]
    p = kda_synth.workload("long", device=dev)
    pairs = [(0, 0), (0, 9), (0, 15)]
    o_ref, s_ref = sampled(p, pairs)
    for segments, schedule in (("auto", "auto"), ("auto", "two-pass"), (1, "auto")):
        note(f"case long workload: B1 H16 T65536 d128 bf16 C64, S0 in (3 sampled heads), segments={segments} "
             f"schedule={schedule}")
        out, sf = kda.chunk_fwd(p.q, p.k, p.v, p.log_alpha, p.beta, S0=p.S0, C=w["C"], segments=segments,
                                schedule=schedule)
        torch.cuda.synchronize()
        assert torch.isfinite(out.float()).all() and torch.isfinite(sf).all()
        o_gpu = np.stack([f64(out[b, :, h]) for b, h in pairs])[:, :, None]
        s_gpu = np.stack([f64(sf[b, h]) for b, h in pairs])[:, None]
        assert_close(f"long sampled ({segments}, {schedule})", o_gpu, s_gpu, o_ref, s_ref, TOL["bf16"])
        del out, sf


def test_workloads_fp32_inputs_sampled(dev):
    """The fp32-input mode at the full prefill sizes: the mid, long and varlen
    workloads with the same recipe in fp32 (dk = 128 with C = 64 runs as
    32-token chunks), each schedule the library picks, sampled heads against
    the oracle at the fp32 bar."""
    w = kda_synth.WORKLOADS["mid"]
    note("case mid workload in fp32: B4 H32 T8192 d128 C64 (4 sampled heads)")
    p = kda_synth.workload("mid", device=dev, dtype="f32")
    out, sf = gpu_chunk(p, w["C"])
    pairs = [(0, 5), (1, 30), (2, 17), (3, 0)]
    o_ref, s_ref = sampled(p, pairs)
    o_gpu = np.stack([f64(out[b, :, h]) for b, h in pairs])[:, :, None]
    s_gpu = np.stack([f64(sf[b, h]) for b, h in pairs])[:, None]
    assert_close("mid fp32 sampled", o_gpu, s_gpu, o_ref, s_ref, TOL["f32"])
    del p, out, sf

    w = kda_synth.WORKLOADS["long"]
    note("case long workload in fp32: B1 H16 T65536 d128 C64, S0 in (2 sampled heads), segments=auto")
    p = kda_synth.workload("long", device=dev, dtype="f32")
    out, sf = gpu_chunk(p, w["C"], segments="auto")
    pairs = [(0, 4), (0, 13)]
    o_ref, s_ref = sampled(p, pairs)
    o_gpu = np.stack([f64(out[b, :, h]) for b, h in pairs])[:, :, None]
    s_gpu = np.stack([f64(sf[b, h]) for b, h in pairs])[:, None]
    assert_close("long fp32 sampled", o_gpu, s_gpu, o_ref, s_ref, TOL["f32"])
    del p, out, sf

    w = kda_synth.WORKLOADS["varlen"]
    note("case varlen workload in fp32: 8 sequences U[2048,16384] x H16 d128 C64 (one head per sequence)")
    p = kda_synth.workload("varlen", device=dev, dtype="f32")
    out, sf = kda.chunk_fwd_varlen(p.q, p.k, p.v, p.log_alpha, p.beta, p.cu_seqlens, S0=p.S0, C=w["C"])
    torch.cuda.synchronize()
    for n in range(len(p.cu_host) - 1):
        a, b = p.cu_host[n], p.cu_host[n + 1]
        h = (3 * n + 1) % w["H"]
        sl = lambda t: t[:, a:b, h:h + 1]
        o_ref, s_ref = oracle.forward(f64(sl(p.q)), f64(sl(p.k)), f64(sl(p.v)), f64(sl(p.log_alpha)),
                                      f64(p.beta[:, a:b, h:h + 1]), S0=f64(p.S0[n:n + 1, h:h + 1]))
        assert_close(f"varlen fp32 sequence {n} ({b - a} tokens) head {h}", f64(sl(out)),
                     f64(sf[n:n + 1, h:h + 1]), o_ref, s_ref, TOL["f32"])


# ---------------------------------------------------------------- decode step
@pytest.mark.parametrize("N,H,dk,dv,dtype", [(3, 2, 64, 32, "bf16"), (2, 3, 128, 128, "bf16"),
                                             (4, 1, 16, 128, "f32"), (2, 2, 32, 64, "f32"),
                                             (5, 2, 128, 16, "f32"),
                                             # head counts that are multiples of 8, several
                                             # workgroups per head: the XCD-grouped mapping
                                             (4, 2, 64, 128, "f32"), (2, 4, 128, 64, "bf16")])
def test_decode_steps(dev, N, H, dk, dv, dtype):
    steps = 40
    note(f"case decode N{N} H{H} dk{dk} dv{dv} {dtype} x{steps} steps")
    d = kda_synth.decode(N, H, dk, dv, steps, dtype=dtype, seed=31 + dk + dv, device=dev, step_block=8)
    S = d.S0.clone()
    outs = []
    for t in range(steps):
        outs.append(kda.recurrent_step(d.q[t], d.k[t], d.v[t], d.log_alpha[t], d.beta[t], S))
    torch.cuda.synchronize()
    out = torch.stack(outs, dim=1)   # [N, steps, H, dv]
    o_ref, s_ref = oracle.forward(f64(d.q.transpose(0, 1)), f64(d.k.transpose(0, 1)), f64(d.v.transpose(0, 1)),
                                  f64(d.log_alpha.transpose(0, 1)), f64(d.beta.transpose(0, 1)), S0=f64(d.S0))
    assert_close("decode", f64(out), f64(S), o_ref, s_ref, TOL[dtype])


DECODE_SWEEP = [(dtype, dk, dv, T, N) for dtype in ("bf16", "f32")
                for dk, dv in ((16, 16), (32, 64), (64, 128), (128, 128), (128, 32))
                for T in (1, 3, 17) for N in (3, 4)]


@pytest.mark.parametrize("dtype,dk,dv,T,N", DECODE_SWEEP)
def test_decode_config_sweep(dev, dtype, dk, dv, T, N):
    """Both decode kernels over input type x (dk, dv) x T (1: the step kernel;
    17: two token tiles of the multi-token kernel) x head count (N x 2 = 6 or
    8 heads: a head's workgroups grouped on one XCD for 8)."""
    H = 2
    note(f"case decode sweep {dtype} dk{dk} dv{dv} T{T} N{N} H{H}")
    p = kda_synth.prefill(N, T, H, dk, dv, dtype=dtype, s0_sigma=0.1, seed=7 + T, device=dev)
    S = p.S0.clone()
    out = kda.recurrent_fwd(p.q, p.k, p.v, p.log_alpha, p.beta, S)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle_dense(p)
    assert_close(f"decode sweep {dtype} dk{dk} dv{dv} T{T} N{N}", f64(out), f64(S), o_ref, s_ref, TOL[dtype])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_workload_sampled(dev, dtype):
    """The decode workload at full size (256 sequences x 32 heads, d = 128, 1024
    one-token steps), in its bf16 inputs and in fp32 with the same recipe: 16 sampled heads against the oracle at every step, and
    the whole stream against the other schedule of the same recurrence, one
    chunk prefill (C = 64, as the mid prefill) of the 1024 tokens laid out
    [N, T, H, d] from the same initial states: every output and every final
    state, plus the prefill's sampled heads against the oracle."""
    w = kda_synth.WORKLOADS["decode"]
    N, H, dk, dv, steps = w["N"], w["H"], w["dk"], w["dv"], w["steps"]
    note(f"case decode workload: 256 seq x H32 d128 {dtype}, 1024 steps (16 sampled heads, every step)")
    d = kda_synth.decode(N, H, dk, dv, steps, dtype=dtype, device=dev)
    S = d.S0.clone()
    heads = [(n, h) for n, h in zip(range(3, 256, 16), range(0, 32, 2))]
    out_all = torch.empty((steps, N, H, dv), dtype=kda_synth.DTYPES[dtype], device=dev)
    ni = torch.tensor([n for n, _ in heads], device=dev)
    hi = torch.tensor([h for _, h in heads], device=dev)
    for t in range(steps):
        kda.recurrent_step(d.q[t], d.k[t], d.v[t], d.log_alpha[t], d.beta[t], S, out=out_all[t])
    torch.cuda.synchronize()
    assert torch.isfinite(S).all()
    out_s = out_all[:, ni, hi].transpose(0, 1)                         # [n, steps, dv]
    pick = lambda t: t[:, ni, hi].transpose(0, 1).unsqueeze(2)      # [n, steps, 1, d]
    o_ref, s_ref = oracle.forward(f64(pick(d.q)), f64(pick(d.k)), f64(pick(d.v)), f64(pick(d.log_alpha)),
                                  f64(d.beta[:, ni, hi].transpose(0, 1).unsqueeze(2)),
                                  S0=f64(d.S0[ni, hi].unsqueeze(1)))
    s_ref = s_ref.reshape(len(heads), 1, dv, dk)
    assert_close(f"decode sampled {dtype}", f64(out_s)[:, :, None], f64(S[ni, hi]).reshape(len(heads), 1, dv, dk),
                 o_ref, s_ref, TOL[dtype])

    note(f"case decode workload vs chunk prefill of the same stream: N256 T1024 H32 d128 {dtype} C64")
    tm = lambda t: t.transpose(0, 1).contiguous()                   # [steps, N, ...] -> [N, steps, ...]
    pre, sf = kda.chunk_fwd(tm(d.q), tm(d.k), tm(d.v), tm(d.log_alpha), tm(d.beta), S0=d.S0, C=64, segments=1)
    torch.cuda.synchronize()
    dec = tm(out_all)                                                 # [N, steps, H, dv]
    del d
    # the whole stream: both schedules, every output and state
    assert_close_device(f"decode vs prefill (all heads) {dtype}", pre, sf, dec, S, TOL[dtype])
    assert_close(f"prefill sampled {dtype}", f64(pre[ni, :, hi])[:, :, None], f64(sf[ni, hi]).reshape(len(heads), 1, dv, dk),
                 o_ref, s_ref, TOL[dtype])


def test_decode_equals_chunk_prefill_on_same_stream(dev):
    """Both schedules of the one recurrence on the same token stream: decode
    steps and one chunk prefill agree with each other and with the oracle."""
    N, H, dk, dv, steps = 16, 4, 128, 128, 200
    note(f"case decode vs chunk prefill: N{N} H{H} d128 bf16, {steps} tokens")
    d = kda_synth.decode(N, H, dk, dv, steps, seed=41, device=dev, step_block=50)
    S = d.S0.clone()
    outs = [kda.recurrent_step(d.q[t], d.k[t], d.v[t], d.log_alpha[t], d.beta[t], S) for t in range(steps)]
    dec = torch.stack(outs, dim=1)
    tm = lambda t: t.transpose(0, 1).contiguous()
    pre, sf = kda.chunk_fwd(tm(d.q), tm(d.k), tm(d.v), tm(d.log_alpha), tm(d.beta), S0=d.S0, C=64, segments=1)
    torch.cuda.synchronize()
    e_o = rel(f64(dec), f64(pre))
    e_s = rel(f64(S), f64(sf))
    note(f"  decode vs prefill: out rel diff {e_o:.3e}, state rel diff {e_s:.3e}")
    assert e_o < TOL["bf16"] and e_s < TOL["bf16"]
    o_ref, s_ref = oracle.forward(f64(tm(d.q)), f64(tm(d.k)), f64(tm(d.v)), f64(tm(d.log_alpha)),
                                  f64(tm(d.beta)), S0=f64(d.S0))
    assert_close("decode", f64(dec), f64(S), o_ref, s_ref, TOL["bf16"])
    assert_close("prefill", f64(pre), f64(sf), o_ref, s_ref, TOL["bf16"])


# ---------------------------------------------------------------- multi-token decode
@pytest.mark.parametrize("N,T,H,dk,dv,dtype", [(3, 2, 2, 64, 32, "bf16"), (2, 5, 3, 128, 128, "bf16"),
                                               (4, 16, 1, 16, 128, "f32"), (2, 7, 2, 32, 64, "f32"),
                                               (5, 3, 2, 128, 16, "bf16"), (1, 64, 2, 128, 128, "bf16"),
                                               # head counts that are multiples of 8 (a head's
                                               # workgroups grouped on one XCD), one and two token tiles
                                               (4, 5, 2, 128, 128, "bf16"), (2, 3, 4, 64, 128, "f32"),
                                               (2, 20, 4, 128, 128, "bf16"),
                                               # longer streams: five token tiles with a ragged tail
                                               (2, 67, 4, 128, 128, "bf16"), (3, 45, 2, 64, 128, "f32")])
def test_recurrent_fwd_matches_oracle(dev, N, T, H, dk, dv, dtype):
    note(f"case multi-token decode N{N} T{T} H{H} dk{dk} dv{dv} {dtype}")
    p = kda_synth.prefill(N, T, H, dk, dv, dtype=dtype, s0_sigma=0.1, seed=61 + T + dk + dv, device=dev)
    S = p.S0.clone()
    out = kda.recurrent_fwd(p.q, p.k, p.v, p.log_alpha, p.beta, S)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle_dense(p)
    assert_close("recurrent_fwd", f64(out), f64(S), o_ref, s_ref, TOL[dtype])


def test_recurrent_fwd_equals_single_steps(dev):
    """T tokens in one launch give bit for bit what T single-step launches give."""
    for dtype, (N, T, H, dk, dv) in (("bf16", (3, 6, 2, 128, 64)), ("f32", (3, 6, 2, 128, 64)),
                                     ("bf16", (4, 19, 2, 128, 128)), ("f32", (2, 17, 4, 64, 128))):
        note(f"case multi-token vs single steps N{N} T{T} H{H} dk{dk} dv{dv} {dtype} (bitwise)")
        p = kda_synth.prefill(N, T, H, dk, dv, dtype=dtype, s0_sigma=0.1, seed=67, device=dev)
        S1 = p.S0.clone()
        out1 = kda.recurrent_fwd(p.q, p.k, p.v, p.log_alpha, p.beta, S1)
        S2 = p.S0.clone()
        outs = [kda.recurrent_step(p.q[:, t].contiguous(), p.k[:, t].contiguous(), p.v[:, t].contiguous(),
                                   p.log_alpha[:, t].contiguous(), p.beta[:, t].contiguous(), S2)
                for t in range(T)]
        torch.cuda.synchronize()
        assert torch.equal(out1, torch.stack(outs, dim=1)) and torch.equal(S1, S2)


def test_recurrent_fwd_edge_cases(dev):
    note("case multi-token decode edges: T = 0 leaves S alone, T = 1, guard bands around out and S")
    p = kda_synth.prefill(2, 0, 2, 64, 64, dtype="bf16", s0_sigma=0.1, seed=71, device=dev)
    S = p.S0.clone()
    kda.recurrent_fwd(p.q, p.k, p.v, p.log_alpha, p.beta, S)
    torch.cuda.synchronize()
    assert torch.equal(S, p.S0)
    N, T, H, dk, dv = 2, 9, 3, 64, 64
    p = kda_synth.prefill(N, T, H, dk, dv, dtype="bf16", s0_sigma=0.1, seed=73, device=dev)
    pad = 2048
    n_out, n_s = N * T * H * dv, N * H * dv * dk
    big_out = torch.full((n_out + 2 * pad,), 7.0, dtype=torch.bfloat16, device=dev)
    big_s = torch.full((n_s + 2 * pad,), -3.0, dtype=torch.float32, device=dev)
    out = big_out[pad:pad + n_out].view(N, T, H, dv)
    S = big_s[pad:pad + n_s].view(N, H, dv, dk)
    S.copy_(p.S0)
    kda.kda_recurrent_fwd(p.q, p.k, p.v, p.log_alpha, p.beta, S, out, N, T, H, dk, dv)
    torch.cuda.synchronize()
    assert torch.all(big_out[:pad] == 7.0) and torch.all(big_out[pad + n_out:] == 7.0)
    assert torch.all(big_s[:pad] == -3.0) and torch.all(big_s[pad + n_s:] == -3.0)
    o_ref, s_ref = oracle_dense(p)
    assert_close("recurrent_fwd guarded", f64(out), f64(S), o_ref, s_ref, TOL["bf16"])


def test_decode_is_deterministic(dev):
    note("case decode determinism N8 H4 d128")
    d = kda_synth.decode(8, 4, 128, 128, 3, seed=51, device=dev, step_block=3)
    S1, S2 = d.S0.clone(), d.S0.clone()
    o1 = [kda.recurrent_step(d.q[t], d.k[t], d.v[t], d.log_alpha[t], d.beta[t], S1) for t in range(3)]
    o2 = [kda.recurrent_step(d.q[t], d.k[t], d.v[t], d.log_alpha[t], d.beta[t], S2) for t in range(3)]
    torch.cuda.synchronize()
    assert torch.equal(S1, S2) and all(torch.equal(a, b) for a, b in zip(o1, o2))


@pytest.mark.parametrize("n16", [1, 256 * 1000 + 37])
def test_stream_copy_is_exact(dev, n16):
    # the bandwidth reference copies bit for bit, a partial last workgroup included,
    # and the guard bands around dst
    note(f"case stream copy {n16} x 16 B")
    g = torch.Generator(device=dev).manual_seed(61)
    src = torch.randn(4 * n16, generator=g, device=dev)
    pad = 64
    big = torch.full((4 * n16 + 2 * pad,), 5.0, device=dev)
    dst = big[pad:pad + 4 * n16]
    kda.kda_stream_copy(src, dst, 16 * n16)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    assert torch.all(big[:pad] == 5.0) and torch.all(big[pad + 4 * n16:] == 5.0)


def test_graph_capture_replays_match_eager(dev):
    """Decode steps, a multi-token launch and chunk prefills (single pass, the
    two segmented schedules, whose three launches share a workspace, and the
    device-side split of packed sequences) captured in one HIP graph: every
    replay gives the eager result bit for bit, with eager work and
    synchronisation between the replays."""
    note("case HIP graph: 3 decode steps, multi T4, chunk single pass + 3 segments two- and one-pass + varlen split")
    bf = torch.bfloat16
    N, H, dk, dv = 8, 4, 128, 128
    d = kda_synth.decode(N, H, dk, dv, 3, seed=71, device=dev)
    pm = kda_synth.prefill(N, 4, H, dk, dv, dtype="bf16", s0_sigma=0.1, seed=72, device=dev)
    pc = kda_synth.prefill(1, 300, 2, 64, 64, dtype="bf16", s0_sigma=0.1, seed=73, device=dev)
    S_dec, S_multi = torch.empty_like(d.S0), torch.empty_like(pm.S0)
    outs = [torch.empty((N, H, dv), dtype=bf, device=dev) for _ in range(3)]
    out_m = torch.empty((N, 4, H, dv), dtype=bf, device=dev)
    out_c = [torch.empty_like(pc.v) for _ in range(3)]
    sf_c = [torch.empty_like(pc.S0) for _ in range(3)]
    nseg = 3
    ws_bytes = kda.kda_chunk_segmented_workspace_bytes(1, 2, 64, 64, nseg)
    ws = torch.empty(ws_bytes // 4 + 64, dtype=torch.float32, device=dev)
    one = kda.variant(schedule="one-pass")
    ws1_bytes = kda.kda_chunk_segmented_workspace_bytes_ex(1, 300, 2, 64, 64, nseg, one, False)
    ws1 = torch.empty(ws1_bytes // 4 + 64, dtype=torch.float32, device=dev)
    pv = kda_synth.prefill_varlen([500, 40, 90], 2, 64, 64, dtype="bf16", s0_sigma=0.1, seed=74, device=dev)
    Tv, Nv = pv.cu_host[-1], len(pv.cu_host) - 1
    out_v, sf_v = torch.empty_like(pv.v), torch.empty_like(pv.S0)
    wsv_bytes = kda.kda_chunk_segmented_workspace_bytes_ex(Nv, Tv, 2, 64, 64, 0, one, False)
    wsv = torch.empty(wsv_bytes // 4 + 64, dtype=torch.float32, device=dev)

    def work():   # on the current stream (the capture stream inside the graph context)
        for t in range(3):
            kda.kda_recurrent_step(d.q[t], d.k[t], d.v[t], d.log_alpha[t], d.beta[t], S_dec, outs[t], N, H, dk, dv)
        kda.kda_recurrent_fwd(pm.q, pm.k, pm.v, pm.log_alpha, pm.beta, S_multi, out_m, N, 4, H, dk, dv)
        kda.kda_chunk_fwd(pc.q, pc.k, pc.v, pc.log_alpha, pc.beta, pc.S0, out_c[0], sf_c[0], 1, 300, 2, 64, 64, 64)
        kda.kda_chunk_fwd_segmented(pc.q, pc.k, pc.v, pc.log_alpha, pc.beta, pc.S0, out_c[1], sf_c[1],
                                    1, 300, 2, 64, 64, 64, nseg, ws, ws_bytes)
        kda.kda_chunk_fwd_ex(pc.q, pc.k, pc.v, pc.log_alpha, pc.beta, pc.S0, out_c[2], sf_c[2],
                             1, 300, 2, 64, 64, 64, one, nseg, ws1, ws1_bytes)
        kda.kda_chunk_fwd_varlen_ex(pv.q, pv.k, pv.v, pv.log_alpha, pv.beta, pv.S0, out_v, sf_v, pv.cu_seqlens, Nv,
                                    Tv, 2, 64, 64, 32, one, 0, wsv, wsv_bytes)

    results = lambda: [S_dec, S_multi, out_m] + outs + out_c + sf_c + [out_v, sf_v]
    S_dec.copy_(d.S0)
    S_multi.copy_(pm.S0)
    work()
    torch.cuda.synchronize()
    ref = [x.clone() for x in results()]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    for replay in range(3):
        S_dec.copy_(d.S0)   # eager work between the replays
        S_multi.copy_(pm.S0)
        for x in [out_m] + outs + out_c + sf_c + [out_v, sf_v]:
            x.fill_(float("nan"))
        for w in (ws, ws1, wsv):
            w.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(results(), ref)):
            assert torch.equal(a, b), f"replay {replay}: result {i} differs from the eager run"
