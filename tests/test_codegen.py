"""Checks on the gfx950 machine code of the built library (no GPU needed).

A vector memory store of more than 8 bytes reads its data registers after it
issues; a vector ALU instruction that writes those registers must come at
least one cycle later.  The compiler inserts that wait for every such store
except a buffer store whose scalar offset is a register, and there the
overwrite has been seen to replace part of the stored data (one column group
of an output block, only under some timings).  The kernels therefore never
give a wide buffer store a register scalar offset; these tests disassemble
the device code objects of libkda.so and check both that rule and the
property it protects.

The kernels of the measured paths are also held to their register budget:
the code-object metadata of each must show no spilled vector registers and
no scratch memory, and the chunk kernels must fit a compute unit's 160 KiB
of LDS.
"""
import os
import re
import shutil
import subprocess
import tempfile

import pytest
import yaml

PKG = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "kimi_delta_attention_fwd_amd")
LIB = os.path.join(PKG, "libkda.so")
OBJDUMP = "/opt/rocm/llvm/bin/llvm-objdump"
READELF = "/opt/rocm/llvm/bin/llvm-readelf"

WIDE_STORE = re.compile(r"^(buffer|global|flat)_store_dwordx(3|4)\s+(?:v\[\d+:\d+\],\s*)?v\[(\d+):(\d+)\]")
BUF_STORE = re.compile(r"^buffer_store_dwordx(3|4)\s+v\[\d+:\d+\],\s*\S+,\s*s\[\d+:\d+\],\s*(\S+)")
VALU_DST = re.compile(r"^v_\S+\s+(?:v(\d+)\b|v\[(\d+):(\d+)\])")


@pytest.fixture(scope="module")
def disassembly():
    if not os.path.exists(LIB):
        pytest.skip("libkda.so is not built")
    if not os.path.exists(OBJDUMP):
        pytest.skip("llvm-objdump not found")
    with tempfile.TemporaryDirectory() as d:
        lib = os.path.join(d, "libkda.so")
        shutil.copy(LIB, lib)
        # --offloading writes each bundled code object next to its input
        subprocess.run([OBJDUMP, "--offloading", lib], cwd=d, check=True, capture_output=True)
        objs = sorted(f for f in os.listdir(d) if f.endswith("gfx950"))
        assert objs, "no gfx950 code object in libkda.so"
        lines = []
        for f in objs:
            out = subprocess.run([OBJDUMP, "-d", "--mcpu=gfx950", os.path.join(d, f)],
                                 check=True, capture_output=True, text=True).stdout
            lines += [l.split("//")[0].strip() for l in out.splitlines()]
    return [l for l in lines if l]


def test_wide_buffer_stores_take_constant_scalar_offset(disassembly):
    offenders = []
    for l in disassembly:
        m = BUF_STORE.match(l)
        if m and m.group(2).startswith("s"):
            offenders.append(l)
    assert not offenders, f"{len(offenders)} wide buffer stores with a register scalar offset, e.g. {offenders[0]}"


def test_wide_store_data_not_overwritten_at_once(disassembly):
    n_stores = 0
    bad = []
    for i, l in enumerate(disassembly):
        m = WIDE_STORE.match(l)
        if not m:
            continue
        n_stores += 1
        lo, hi = int(m.group(3)), int(m.group(4))
        nxt = next((x for x in disassembly[i + 1:i + 4] if not x.endswith(">:") and not x.startswith(".")), "")
        d = VALU_DST.match(nxt)
        if d:
            a = int(d.group(1) or d.group(2))
            b = int(d.group(1) or d.group(3))
            if not (b < lo or a > hi):
                bad.append(f"{l}  ->  {nxt}")
    assert n_stores > 0
    assert not bad, f"{len(bad)} wide stores whose data is overwritten by the next instruction, e.g. {bad[0]}"


@pytest.fixture(scope="module")
def kernel_metadata():
    """name -> the code-object metadata of every gfx950 kernel in libkda.so."""
    if not os.path.exists(LIB):
        pytest.skip("libkda.so is not built")
    if not (os.path.exists(OBJDUMP) and os.path.exists(READELF)):
        pytest.skip("llvm-objdump or llvm-readelf not found")
    kernels = {}
    with tempfile.TemporaryDirectory() as d:
        lib = os.path.join(d, "libkda.so")
        shutil.copy(LIB, lib)
        subprocess.run([OBJDUMP, "--offloading", lib], cwd=d, check=True, capture_output=True)
        for f in sorted(f for f in os.listdir(d) if f.endswith("gfx950")):
            notes = subprocess.run([READELF, "--notes", os.path.join(d, f)], check=True, capture_output=True,
                                   text=True).stdout
            doc = notes[notes.index("---"):notes.rindex("...")]
            for k in yaml.safe_load(doc)["amdhsa.kernels"]:
                kernels[k[".name"]] = k
    assert kernels, "no kernel metadata in libkda.so"
    return kernels


# Instantiations on the measured paths, by the start of their mangled names:
# chunk_fwd_kernel<In, DK, BV, C, MAP, VAR> (bf16, d_k = 128, BV = 64, C = 64:
# the plain single pass, the variant and raw-input single passes, the plain
# map pass; fp32 at d_k = 64), the composition and output epilogue of the
# segmented schedules, and the decode kernels.
HOT = [
    "_ZN3kda16chunk_fwd_kernelIDF16bLi128ELi64ELi64ELb0ELi0E",
    "_ZN3kda16chunk_fwd_kernelIDF16bLi128ELi64ELi64ELb0ELi1E",
    "_ZN3kda16chunk_fwd_kernelIDF16bLi128ELi64ELi64ELb0ELi2E",
    "_ZN3kda16chunk_fwd_kernelIDF16bLi128ELi64ELi64ELb1ELi0E",
    "_ZN3kda16chunk_fwd_kernelIfLi64ELi64ELi64ELb0ELi0E",
    "_ZN3kda18seg_compose_kernelILi128E",
    "_ZN3kda14seg_out_kernelIDF16bLi128E",
    "_ZN3kda18decode_step_kernel",
    "_ZN3kda19decode_multi_kernel",
]


def test_measured_kernels_spill_no_vector_registers(kernel_metadata):
    bad = []
    for prefix in HOT:
        found = [k for n, k in kernel_metadata.items() if n.startswith(prefix)]
        assert found, f"no kernel named {prefix}..."
        for k in found:
            if k[".vgpr_spill_count"] != 0 or k[".private_segment_fixed_size"] != 0:
                bad.append(f"{k['.name']}: {k['.vgpr_spill_count']} spilled VGPRs, "
                           f"{k['.private_segment_fixed_size']} B of scratch")
    assert not bad, "\n".join(bad)


def test_chunk_kernels_fit_the_register_file_and_lds(kernel_metadata):
    chunk = [k for n, k in kernel_metadata.items() if n.startswith("_ZN3kda16chunk_fwd_kernel")]
    assert len(chunk) >= 8
    for k in chunk:
        assert k[".group_segment_fixed_size"] <= 160 * 1024, k[".name"]
        # every wave of a workgroup resident at once: 512 registers per SIMD lane
        # shared by the workgroup's waves on that SIMD
        waves_per_simd = -(-k[".max_flat_workgroup_size"] // (64 * 4))
        assert k[".vgpr_count"] + k[".agpr_count"] <= 512 // waves_per_simd, k[".name"]
