"""Build the projector's HIP library in-tree: cryo_em_fourier_amd/libtp.so,
and the peak probes that bench.py measures roofline denominators with:
cryo_em_fourier_amd/libtp_peaks.so (not part of the projector's path).

    python -m cryo_em_fourier_amd.build

hipcc cross-compiles for gfx950 without a GPU.  Packed fp32 VALU ops are
disabled (ordinary fp32 code only), hardware float atomics are enabled.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libtp.so")
SOURCES = ["tp_api.hip", "tp_kernels.hip", "tp_adjoint.hip", "tp_rotate.hip"]
PEAKS_LIB = os.path.join(HERE, "libtp_peaks.so")
PEAKS_SOURCES = ["peaks.hip"]
ARCH = os.environ.get("TP_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-shared",
        "-munsafe-fp-atomics",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall",
        "-Wno-unused-function",
    ]


def _compile(sources: list[str], out: str, verbose: bool) -> str:
    srcs = [os.path.join(CSRC, s) for s in sources]
    tmp = out + ".tmp"
    cmd = [hipcc(), *flags(), *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed ({r.returncode})")
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    """Compile both libraries; returns the projector library's path."""
    _compile(PEAKS_SOURCES, PEAKS_LIB, verbose)
    return _compile(SOURCES, LIB, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
