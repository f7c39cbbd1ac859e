"""Build libgdr.so (HIP, gfx950) in-tree with hipcc.

    python -m chunkwise_gated_delta_cumsum_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libgdr.so")
SOURCES = [os.path.join(CSRC, "gdr_api.hip")]
DEPS = SOURCES + [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hpp")] + [
    os.path.join(INCLUDE, "gdr.h")]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def flags():
    return ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
            # packed fp32 VALU ops stay off (see the numerics notes in gdr.h)
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # MFMA accumulators in ordinary VGPRs: the state and the products
            # are also touched by VALU code, which cannot read AGPRs directly
            "-mllvm", "-amdgpu-mfma-vgpr-form",
            "-Wno-unused-result", "-I", INCLUDE, "-I", CSRC]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc()] + flags() + ["-o", tmp] + SOURCES
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines()
                    if "packed-fp32-ops" not in l and l.strip())
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{out}")
    if verbose and out:
        print(out)
    os.replace(tmp, LIB)
    return LIB


def is_stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(d) > t for d in DEPS)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
