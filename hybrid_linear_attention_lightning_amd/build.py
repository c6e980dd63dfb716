"""Build the HIP library liblightning_la.so for gfx950 (MI355X), in-tree.

    python -m hybrid_linear_attention_lightning_amd.build

Compiles every source under csrc/ with hipcc for --offload-arch=gfx950 and
links one shared library with the C ABI declared in include/lightning_la.h.
hipcc cross-compiles, so no GPU is needed to build.  LA_EXTRA_FLAGS (an
environment variable) appends hipcc flags, e.g. to build a copy with other
definitions for comparison.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "liblightning_la.so")
OBJDIR = os.path.join(PKG, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-command-line-argument",
    # packed fp32 instructions stay off: plain float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core results in ordinary VGPRs: the prefill kernel scales and
    # packs its accumulators on the vector ALU, and accumulators placed in
    # AGPRs cost a copy in and out for each such access (measured ~4% faster)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I", INCLUDE,
] + os.environ.get("LA_EXTRA_FLAGS", "").split()


def sources():
    return sorted(
        os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp"))
    )


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-x", "hip", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed on %s" % src)
    return obj


def build(verbose: bool = True) -> str:
    """Compile all HIP sources and link liblightning_la.so; always rebuilds."""
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build()
