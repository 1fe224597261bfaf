"""Build libkda.so (gfx950) in-tree with hipcc.

Translation units:
  csrc/kda_chunk_inst.hip  x 8   chunk prefill kernels, one per (input type, dk)
  csrc/kda_decode.hip            decode-step kernels
  csrc/kda_noalloc.hip           allocation-free segmented entry point (static scratch)
  csrc/kda_api.cpp               C ABI: validation and dispatch (host only)

Objects go to <repo>/_build/, the library to kimi_delta_attention_fwd_amd/libkda.so.
Run ``python -m kimi_delta_attention_fwd_amd.build`` or call ``build()``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libkda.so")

ARCH = "gfx950"
# Packed fp32 VALU instructions are disabled in all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# Extra flags of the chunk kernels.  LLVM's default scheduling strategy: on the
# current kernels the memory-clause strategy (which once ran them 1.2-1.5%
# faster) is 0.6-1.6% slower on every prefill workload, with the same results
# bit for bit; max-ILP and iterative-minreg are slower still.
CHUNK_FLAGS = []
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Wall", "-Wno-unused-function"]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: install ROCm or set HIPCC")


def _run(cmd):
    proc = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the device-only target feature; drop that line.
    err = "\n".join(l for l in proc.stderr.splitlines() if "packed-fp32-ops" not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"command failed ({proc.returncode}): {' '.join(cmd)}\n{err}")
    return err


def build(jobs: int | None = None, verbose: bool = False) -> str:
    """Compile every HIP translation unit for gfx950 and link libkda.so."""
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    units = []
    for f32 in (0, 1):
        for dk in (16, 32, 64, 128):
            obj = os.path.join(BUILD, f"kda_chunk_{'f32' if f32 else 'bf16'}_{dk}.o")
            units.append([hipcc, *COMMON, *DEVICE_FLAGS, *CHUNK_FLAGS, f"-DKDA_INST_F32={f32}", f"-DKDA_INST_DK={dk}",
                          "-c", os.path.join(CSRC, "kda_chunk_inst.hip"), "-o", obj])
    units.append([hipcc, *COMMON, *DEVICE_FLAGS, "-c", os.path.join(CSRC, "kda_decode.hip"),
                  "-o", os.path.join(BUILD, "kda_decode.o")])
    units.append([hipcc, *COMMON, *DEVICE_FLAGS, "-c", os.path.join(CSRC, "kda_noalloc.hip"),
                  "-o", os.path.join(BUILD, "kda_noalloc.o")])
    units.append([hipcc, *COMMON, "-c", os.path.join(CSRC, "kda_api.cpp"),
                  "-o", os.path.join(BUILD, "kda_api.o")])
    jobs = jobs or min(8, os.cpu_count() or 4)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        for msg in ex.map(_run, units):
            if verbose and msg.strip():
                print(msg)
    objs = [u[u.index("-o") + 1] for u in units]
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
