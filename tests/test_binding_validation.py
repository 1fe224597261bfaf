"""The Python binding's convenience wrappers check their tensors before any C
call: shapes against q, dtypes, contiguity, and that everything lives on one
GPU.  A wrong tensor raises TypeError or ValueError instead of reaching the
kernels as a bad pointer.  These run on the CPU: the checks come before the
library is loaded, and CPU tensors are themselves one of the rejected cases.
"""
import pytest
import torch

kda = pytest.importorskip("kimi_delta_attention_fwd_amd")


def chunk_inputs(B=2, T=10, H=3, dk=16, dv=8, dtype=torch.bfloat16, gate="channel", raw=False):
    q = torch.zeros((B, T, H, dk), dtype=dtype)
    k = torch.zeros_like(q)
    v = torch.zeros((B, T, H, dv), dtype=dtype)
    gdt = dtype if raw else torch.float32
    la = torch.zeros((B, T, H, dk) if gate == "channel" else (B, T, H), dtype=gdt)
    beta = torch.zeros((B, T, H), dtype=torch.float32)
    S0 = torch.zeros((B, H, dv, dk), dtype=torch.float32)
    return dict(q=q, k=k, v=v, log_alpha=la, beta=beta, S0=S0)


def call_chunk(a, **kw):
    return kda.chunk_fwd(a["q"], a["k"], a["v"], a["log_alpha"], a["beta"], S0=a["S0"], **kw)


def test_cpu_tensors_are_rejected():
    with pytest.raises(TypeError, match="on a GPU"):
        call_chunk(chunk_inputs())


@pytest.mark.parametrize("name,shape", [("k", (2, 10, 3, 8)), ("v", (2, 9, 3, 8)), ("log_alpha", (2, 10, 3)),
                                        ("beta", (2, 10, 1)), ("S0", (2, 3, 16, 8))])
def test_shape_mismatch(name, shape):
    a = chunk_inputs()
    a[name] = torch.zeros(shape, dtype=a[name].dtype)
    with pytest.raises(ValueError, match=name):
        call_chunk(a)


def test_dtype_mismatch():
    a = chunk_inputs()
    a["log_alpha"] = a["log_alpha"].to(torch.bfloat16)       # a bf16 gate without raw=True
    with pytest.raises(TypeError, match="log_alpha"):
        call_chunk(a)
    a = chunk_inputs()
    a["k"] = a["k"].float()
    with pytest.raises(TypeError, match="k must be"):
        call_chunk(a)
    with pytest.raises(TypeError, match="bfloat16 or float32"):
        call_chunk(chunk_inputs(dtype=torch.float16))


def test_raw_gate_takes_q_dtype_and_scalar_gate_its_shape():
    a = chunk_inputs(raw=True)
    with pytest.raises(TypeError, match="on a GPU"):          # shapes and dtypes pass, the device does not
        call_chunk(a, raw=True)
    a = chunk_inputs(gate="scalar")
    with pytest.raises(TypeError, match="on a GPU"):
        call_chunk(a, gate="scalar")
    with pytest.raises(ValueError, match="log_alpha"):
        call_chunk(chunk_inputs(), gate="scalar")             # a per-channel gate passed as scalar


def test_non_contiguous_views_are_rejected():
    a = chunk_inputs(B=2, T=3, H=2, dk=16)
    a["q"] = torch.zeros((2, 2, 3, 16), dtype=torch.bfloat16).transpose(1, 2)   # [B, H, T, d] viewed as [B, T, H, d]
    with pytest.raises(ValueError, match="contiguous"):
        call_chunk(a)


def test_varlen_and_decode_wrappers_check_too():
    a = chunk_inputs(B=1, T=10, H=2)
    cu = torch.tensor([0, 4, 10], dtype=torch.int64)
    with pytest.raises(TypeError, match="cu_seqlens"):
        kda.chunk_fwd_varlen(a["q"], a["k"], a["v"], a["log_alpha"], a["beta"], cu, S0=None)
    q = torch.zeros((4, 2, 16), dtype=torch.bfloat16)
    S = torch.zeros((4, 2, 8, 16), dtype=torch.float32)
    la = torch.zeros((4, 2, 16), dtype=torch.float32)
    with pytest.raises(ValueError, match="beta must have shape"):
        kda.recurrent_step(q, q, torch.zeros((4, 2, 8), dtype=torch.bfloat16), la, torch.zeros((4, 3)), S)
    with pytest.raises(ValueError, match="S must have shape"):
        kda.recurrent_step(q, q, torch.zeros((4, 2, 8), dtype=torch.bfloat16), la, torch.zeros((4, 2)),
                           torch.zeros((4, 2, 16, 8)))
    qm = torch.zeros((4, 3, 2, 16), dtype=torch.bfloat16)
    with pytest.raises(TypeError, match="on a GPU"):
        kda.recurrent_fwd(qm, qm, torch.zeros((4, 3, 2, 8), dtype=torch.bfloat16), torch.zeros((4, 3, 2, 16)),
                          torch.zeros((4, 3, 2)), S)
