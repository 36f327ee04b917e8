"""Builds libbitmap_spmm.so (and the streaming-read probe libbsp_probe.so)
in this directory with hipcc for gfx950.

    python -m bit_unstructured_sparse_amd.build

One shared library holds the host encoders (encode.cpp, encode_union.cpp,
encode_cbc.cpp) and every HIP kernel
(spmm.hip with its kernels_*.hip includes). The probe (probe_read.hip) is a
measurement aid the benchmark loads; the SpMM library does not contain it.
Packed-fp32 VALU forms are switched off for the device pass; hipcc's host
pass warns that it does not know that feature, which is harmless.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libbitmap_spmm.so")
PROBE_LIB = os.path.join(HERE, "libbsp_probe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = [os.path.join(CSRC, "spmm.hip"), os.path.join(CSRC, "encode.cpp"), os.path.join(CSRC, "encode_union.cpp"),
           os.path.join(CSRC, "encode_cbc.cpp")]
PROBE_SOURCES = [os.path.join(CSRC, "probe_read.hip")]


def command(out: str, sources=SOURCES):
    return [HIPCC, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC,
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function",
            *sources, "-o", out, "-lpthread"]


def _compile(out: str, sources, verbose: bool) -> str:
    tmp = out + f".tmp{os.getpid()}"
    cmd = command(tmp, sources)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if noise not in ln]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    _compile(PROBE_LIB, PROBE_SOURCES, verbose)
    return _compile(LIB, SOURCES, verbose)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
