"""Build libattn_sink.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Usage: python -m attention_learnable_sinks_amd.build
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libattn_sink.so")
SOURCES = ["api.cpp", "layout.cpp", "fwd.hip", "bwd.hip", "decode.hip", "merge.hip"]
ARCH = "gfx950"

# -packed-fp32-ops: keep the compiler from forming packed fp32 VALU instructions.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-munsafe-fp-atomics",
    "-mllvm", "-amdgpu-mfma-vgpr-form",  # MFMA accumulators in VGPRs: no accvgpr moves around the softmax
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    cc = hipcc()
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".", "_") + ".o")
        _run([cc, *HIP_FLAGS, "-I", os.path.join(ROOT, "include"), "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    # A kernel template whose host-side instantiation failed leaves its launch stub
    # undefined; catch that here rather than at load time.
    nm = shutil.which("nm")
    if nm:
        und = subprocess.run([nm, "-D", "--undefined-only", tmp], capture_output=True, text=True).stdout
        missing = [l.split()[-1] for l in und.splitlines() if "attn_sink" in l]
        if missing:
            os.remove(tmp)
            raise RuntimeError(f"undefined library symbols after linking: {missing}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
