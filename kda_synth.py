"""Seeded synthetic inputs for the KDA forward pass.

This module only draws random numbers and prepares inputs the way a caller
would (L2-normalised q and k, gates through sigmoid / softplus); it holds none
of the method's arithmetic and is shared by the GPU tests, the oracle checks
and bench.py.  Both sides receive the very same tensors: the oracle gets a
float64 copy of what the GPU reads (bf16 values upcast exactly).

Workloads (sizes and distributions as described for the method's benchmark
configurations; N(mu, s) is read as mean mu, standard deviation s):

  tiny    B=1  H=1  T=64    dk=dv=16,  fp32 q/k/v, C=16; beta ~ U(0,1);
          log_alpha = -softplus(g), g ~ N(-3, 1); zero initial state.
  small   B=2  H=4  T=1024  dk=dv=64,  bf16 q/k/v, C=64; beta ~ U(0,1);
          g ~ N(-3, 1); initial state ~ N(0, 0.1).
  mid     B=4  H=32 T=8192  dk=dv=128, bf16, C=64; beta = sigmoid(N(0,1));
          g ~ N(-4, 1.5); no initial state (zero), final state written.
  long    B=1  H=16 T=65536 dk=dv=128, bf16, C=64; as mid, initial state
          ~ N(0, 0.1) in, final state out.
  varlen  8 sequences, lengths uniform integers in [2048, 16384], H=16,
          dk=dv=128 packed into one [1, T_total, H, d] stream; as long, one
          initial state per sequence.
  decode  256 sequences x H=32, dk=dv=128, state ~ N(0, 0.1) fp32, 1024
          one-token steps with bf16 q/k/v; beta and g as mid.

In every workload q, k ~ N(0, 1) are L2-normalised per token in fp32 (no
epsilon) before rounding to the input type; v ~ N(0, 1); all draws are i.i.d.
per (batch, token, head, channel).
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

WORKLOADS = {
    "tiny": dict(B=1, H=1, T=64, dk=16, dv=16, C=16, dtype="f32", g_mu=-3.0, g_sigma=1.0,
                 beta="uniform", s0_sigma=None),
    "small": dict(B=2, H=4, T=1024, dk=64, dv=64, C=64, dtype="bf16", g_mu=-3.0, g_sigma=1.0,
                  beta="uniform", s0_sigma=0.1),
    "mid": dict(B=4, H=32, T=8192, dk=128, dv=128, C=64, dtype="bf16", g_mu=-4.0, g_sigma=1.5,
                beta="sigmoid", s0_sigma=None),
    "long": dict(B=1, H=16, T=65536, dk=128, dv=128, C=64, dtype="bf16", g_mu=-4.0, g_sigma=1.5,
                 beta="sigmoid", s0_sigma=0.1),
    "varlen": dict(N=8, len_lo=2048, len_hi=16384, H=16, dk=128, dv=128, C=64, dtype="bf16", g_mu=-4.0,
                   g_sigma=1.5, beta="sigmoid", s0_sigma=0.1),
    "decode": dict(N=256, H=32, dk=128, dv=128, steps=1024, dtype="bf16", g_mu=-4.0, g_sigma=1.5,
                   beta="sigmoid", s0_sigma=0.1),
}

SEEDS = {"tiny": 0, "small": 1, "mid": 2, "long": 3, "varlen": 3, "decode": 4}

DTYPES = {"bf16": torch.bfloat16, "f32": torch.float32}


@dataclass
class Prefill:
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    log_alpha: torch.Tensor
    beta: torch.Tensor
    S0: torch.Tensor | None
    cu_seqlens: torch.Tensor | None = None    # device int32 [N+1] (packed layout)
    cu_host: list | None = None


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _unit_rows(shape, g, device, dtype):
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    x = x / x.norm(dim=-1, keepdim=True)
    return x.to(dtype)


def _gates(shape_tok, dk, g, device, g_mu, g_sigma, beta_kind):
    if beta_kind == "uniform":
        beta = torch.rand(shape_tok, generator=g, device=device, dtype=torch.float32)
    elif beta_kind == "sigmoid":
        beta = torch.sigmoid(torch.randn(shape_tok, generator=g, device=device, dtype=torch.float32))
    else:
        raise ValueError(beta_kind)
    pre = torch.randn(shape_tok + (dk,), generator=g, device=device, dtype=torch.float32) * g_sigma + g_mu
    log_alpha = -torch.nn.functional.softplus(pre)
    return log_alpha, beta


def prefill(B, T, H, dk, dv, *, dtype="bf16", g_mu=-4.0, g_sigma=1.5, beta="sigmoid", s0_sigma=None,
            seed=0, device="cuda") -> Prefill:
    """Dense [B, T, H, d] inputs."""
    g = _gen(seed, device)
    dt = DTYPES[dtype]
    q = _unit_rows((B, T, H, dk), g, device, dt)
    k = _unit_rows((B, T, H, dk), g, device, dt)
    v = torch.randn((B, T, H, dv), generator=g, device=device, dtype=torch.float32).to(dt)
    log_alpha, be = _gates((B, T, H), dk, g, device, g_mu, g_sigma, beta)
    S0 = None
    if s0_sigma is not None:
        S0 = torch.randn((B, H, dv, dk), generator=g, device=device, dtype=torch.float32) * s0_sigma
    return Prefill(q, k, v, log_alpha, be, S0)


def prefill_raw(B, T, H, dk, dv, *, dtype="bf16", g_mu=-4.0, g_sigma=1.5, q_sigma=1.0, k_sigma=1.0,
                beta="sigmoid", s0_sigma=None, seed=0, device="cuda") -> Prefill:
    """Dense inputs as they come out of the projections, for the fused input
    preparation: q ~ N(0, q_sigma), k ~ N(0, k_sigma) NOT normalised, and the
    gate pre-activations g ~ N(g_mu, g_sigma) in the input type in place of
    log_alpha (the `log_alpha` field holds g)."""
    g = _gen(seed, device)
    dt = DTYPES[dtype]
    q = (torch.randn((B, T, H, dk), generator=g, device=device, dtype=torch.float32) * q_sigma).to(dt)
    k = (torch.randn((B, T, H, dk), generator=g, device=device, dtype=torch.float32) * k_sigma).to(dt)
    v = torch.randn((B, T, H, dv), generator=g, device=device, dtype=torch.float32).to(dt)
    if beta == "sigmoid":
        be = torch.sigmoid(torch.randn((B, T, H), generator=g, device=device, dtype=torch.float32))
    else:
        be = torch.rand((B, T, H), generator=g, device=device, dtype=torch.float32)
    pre = (torch.randn((B, T, H, dk), generator=g, device=device, dtype=torch.float32) * g_sigma + g_mu).to(dt)
    S0 = None
    if s0_sigma is not None:
        S0 = torch.randn((B, H, dv, dk), generator=g, device=device, dtype=torch.float32) * s0_sigma
    return Prefill(q, k, v, pre, be, S0)


def prefill_varlen(lengths, H, dk, dv, *, dtype="bf16", g_mu=-4.0, g_sigma=1.5, beta="sigmoid", s0_sigma=0.1,
                   seed=0, device="cuda") -> Prefill:
    """Packed [1, T_total, H, d] inputs for the given sequence lengths."""
    lengths = [int(x) for x in lengths]
    T_total = sum(lengths)
    p = prefill(1, T_total, H, dk, dv, dtype=dtype, g_mu=g_mu, g_sigma=g_sigma, beta=beta, s0_sigma=None,
                seed=seed, device=device)
    cu = [0]
    for n in lengths:
        cu.append(cu[-1] + n)
    p.cu_host = cu
    p.cu_seqlens = torch.tensor(cu, dtype=torch.int32, device=device)
    if s0_sigma is not None:
        g = _gen(seed + 7919, device)
        p.S0 = torch.randn((len(lengths), H, dv, dk), generator=g, device=device, dtype=torch.float32) * s0_sigma
    return p


def varlen_lengths(n=8, lo=2048, hi=16384, seed=3):
    """Sequence lengths, uniform integers in [lo, hi] (CPU generator, so every
    device draws the same lengths)."""
    g = torch.Generator()
    g.manual_seed(seed * 1000 + 17)
    return [int(x) for x in torch.randint(lo, hi + 1, (n,), generator=g)]


def workload(name: str, device="cuda", seed=None, dtype=None) -> Prefill:
    """A named prefill workload; `dtype` overrides its input type (the same
    recipe and shapes in fp32, say)."""
    w = WORKLOADS[name]
    seed = SEEDS[name] if seed is None else seed
    dt = w["dtype"] if dtype is None else dtype
    if name == "varlen":
        lengths = varlen_lengths(w["N"], w["len_lo"], w["len_hi"], seed=seed)
        return prefill_varlen(lengths, w["H"], w["dk"], w["dv"], dtype=dt, g_mu=w["g_mu"],
                              g_sigma=w["g_sigma"], beta=w["beta"], s0_sigma=w["s0_sigma"], seed=seed,
                              device=device)
    return prefill(w["B"], w["T"], w["H"], w["dk"], w["dv"], dtype=dt, g_mu=w["g_mu"],
                   g_sigma=w["g_sigma"], beta=w["beta"], s0_sigma=w["s0_sigma"], seed=seed, device=device)


@dataclass
class DecodeInputs:
    q: torch.Tensor          # [steps, N, H, dk]
    k: torch.Tensor
    v: torch.Tensor          # [steps, N, H, dv]
    log_alpha: torch.Tensor  # [steps, N, H, dk] fp32
    beta: torch.Tensor       # [steps, N, H] fp32
    S0: torch.Tensor         # [N, H, dv, dk] fp32


def decode(N, H, dk, dv, steps, *, dtype="bf16", g_mu=-4.0, g_sigma=1.5, beta="sigmoid", s0_sigma=0.1,
           seed=4, device="cuda", step_block=64) -> DecodeInputs:
    """Pre-generated decode token stream.  Generated in blocks of steps to
    bound temporary memory; deterministic for a given (seed, step_block)."""
    dt = DTYPES[dtype]
    q = torch.empty((steps, N, H, dk), dtype=dt, device=device)
    k = torch.empty_like(q)
    v = torch.empty((steps, N, H, dv), dtype=dt, device=device)
    la = torch.empty((steps, N, H, dk), dtype=torch.float32, device=device)
    be = torch.empty((steps, N, H), dtype=torch.float32, device=device)
    for s0 in range(0, steps, step_block):
        s1 = min(steps, s0 + step_block)
        p = prefill(s1 - s0, 1, N * H, dk, dv, dtype=dtype, g_mu=g_mu, g_sigma=g_sigma, beta=beta,
                    s0_sigma=None, seed=seed * 100003 + s0, device=device)
        q[s0:s1] = p.q.view(s1 - s0, N, H, dk)
        k[s0:s1] = p.k.view(s1 - s0, N, H, dk)
        v[s0:s1] = p.v.view(s1 - s0, N, H, dv)
        la[s0:s1] = p.log_alpha.view(s1 - s0, N, H, dk)
        be[s0:s1] = p.beta.view(s1 - s0, N, H)
    g = _gen(seed, device)
    S0 = torch.randn((N, H, dv, dk), generator=g, device=device, dtype=torch.float32) * s0_sigma
    return DecodeInputs(q, k, v, la, be, S0)


def to_f64(t):
    """Exact float64 numpy copy (bf16 and fp32 values upcast without rounding)."""
    if t is None:
        return None
    return t.detach().to("cpu").to(torch.float64).numpy()
