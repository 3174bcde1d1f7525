"""Build step of the FLARE++ mixer library: compiles the HIP sources for gfx950 into
``rank_latent_routing_amd/libflarepp.so`` with hipcc, and the roofline microbenchmarks into
``rank_latent_routing_amd/libflarepp_microbench.so`` (a library of their own, used only by the
benchmark script).

Usage: ``python -m rank_latent_routing_amd.build``.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libflarepp.so")
SOURCES = [os.path.join(PKG, "csrc", n) for n in ("kernels.hip", "backward.hip", "project.hip", "flarepp.cpp")]
MB_LIB = os.path.join(PKG, "libflarepp_microbench.so")
MB_SOURCES = [os.path.join(PKG, "csrc", "microbench.hip")]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-std=c++17",
    # Packed fp32 VALU instructions are kept out of the generated code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _compile(sources, lib, verbose):
    hipcc = os.environ.get("HIPCC", "hipcc")
    tmp = lib + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(PKG, "csrc")]
    for src in sources:
        cmd += ["-x", "hip", src]
    cmd += ["-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False) -> str:
    """Compile the library and the microbenchmarks (always, even when built copies exist) and return
    the library's path."""
    _compile(MB_SOURCES, MB_LIB, verbose)
    return _compile(SOURCES, LIB, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
