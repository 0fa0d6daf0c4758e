"""Build libmla_decode.so (the decode path) and libmla_peaks.so (the
attainable-peak microbenchmarks) for gfx950, in-tree, with hipcc.

    python -m sparse_mla_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libmla_decode.so")
SOURCES = [os.path.join(HERE, "csrc", "mla_kernels.hip"), os.path.join(HERE, "csrc", "mla_api.cpp")]
PEAKS_LIB = os.path.join(HERE, "libmla_peaks.so")
PEAKS_SOURCES = [os.path.join(HERE, "csrc", "mla_peaks.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # no packed fp32 (v_pk_*_f32) in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # The LDS-DMA asm writes M0, which the compiler otherwise leaves unused in
    # these kernels (checked in the generated code); silence the reserved-
    # register clobber warning that this triggers.
    "-Wno-inline-asm",
    "-I" + os.path.join(ROOT, "include"),
    "-I" + os.path.join(HERE, "csrc"),
]


def build(verbose: bool = False) -> str:
    _compile(SOURCES, LIB, verbose)
    _compile(PEAKS_SOURCES, PEAKS_LIB, verbose)
    return LIB


def _compile(sources, lib: str, verbose: bool) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC] + FLAGS + sources + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature.
    err = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, lib)


if __name__ == "__main__":
    print(build(verbose=True))
