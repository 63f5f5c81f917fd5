"""Build libpkv.so (the HIP kernels + C ABI) in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpkv.so")
SOURCES = ["pkv_abi.cpp", "pkv_attn_generic.hip", "pkv_attn_mfma.hip", "pkv_attn_dma.hip", "pkv_attn_m32.hip",
           "pkv_attn_mla.hip", "pkv_append.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed-fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics", "-Wno-unused-result",
    # the ring loads name M0 in their clobber list on purpose (see pkv_ring.h)
    "-Wno-inline-asm",
    "-I", os.path.join(HERE, "..", "include"),
]


def build(verbose: bool = False) -> str:
    """Compile every source into libpkv.so (always recompiles)."""
    srcs = []
    for s in SOURCES:
        path = os.path.join(CSRC, s)
        srcs += (["-x", "hip", path] if s.endswith(".hip") else ["-x", "hip", path])
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [HIPCC] + FLAGS + srcs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    errs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{errs}")
    if verbose and errs.strip():
        print(errs)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
