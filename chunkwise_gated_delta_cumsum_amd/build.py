"""Build libgdr.so (HIP, gfx950) in-tree with hipcc.

    python -m chunkwise_gated_delta_cumsum_amd.build

The host logic (gdr_api.hip) and the kernel launchers (one translation unit
per kernel family) compile in parallel to objects under _build/, which are
then linked into the shared library.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libgdr.so")
SOURCES = [os.path.join(CSRC, f) for f in (
    "gdr_api.hip", "gdr_launch_prep.hip", "gdr_launch_prep128.hip", "gdr_launch_scan_f16.hip",
    "gdr_launch_scan_lin.hip", "gdr_launch_scan_f32.hip", "gdr_launch_scan128_f16.hip",
    "gdr_launch_scan128_f32.hip", "gdr_launch_prep32.hip", "gdr_launch_scan32_f16.hip",
    "gdr_launch_scan32_f32.hip", "gdr_launch_decode.hip", "gdr_launch_check.hip",
    "gdr_launch_prep_h16.hip", "gdr_launch_prep128_h16.hip", "gdr_launch_prep32_h16.hip",
    "gdr_launch_scan_h16.hip", "gdr_launch_scan_lin_h16.hip", "gdr_launch_scan128_h16.hip",
    "gdr_launch_scan32_h16.hip")]
OBJDIR = os.path.join(ROOT, "_build")
DEPS = SOURCES + [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hpp")] + [
    os.path.join(INCLUDE, "gdr.h")]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def flags():
    return ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
            # packed fp32 VALU ops stay off (see the numerics notes in gdr.h)
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # MFMA accumulators in ordinary VGPRs: the state and the products
            # are also touched by VALU code, which cannot read AGPRs directly
            "-mllvm", "-amdgpu-mfma-vgpr-form",
            "-Wno-unused-result", "-I", INCLUDE, "-I", CSRC]


def _run(cmd):
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines()
                    if "packed-fp32-ops" not in l and l.strip())
    return res.returncode, out


def build(verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    tag = "%d" % os.getpid()
    objs = [os.path.join(OBJDIR, os.path.basename(src)[:-4] + "." + tag + ".o") for src in SOURCES]
    cmds = [[hipcc()] + flags() + ["-c", "-o", obj, src] for src, obj in zip(SOURCES, objs)]
    if verbose:
        for cmd in cmds:
            print(" ".join(cmd), flush=True)
    with ThreadPoolExecutor(max_workers=min(len(cmds), max(1, os.cpu_count() or 1))) as ex:
        results = list(ex.map(_run, cmds))
    for cmd, (rc, out) in zip(cmds, results):
        if rc != 0:
            raise RuntimeError(f"hipcc failed ({rc}) for {cmd[-1]}:\n{out}")
        if verbose and out:
            print(out)
    tmp = LIB + ".tmp" + tag
    link = [hipcc(), "--offload-arch=gfx950", "-fPIC", "-shared", "-o", tmp] + objs
    if verbose:
        print(" ".join(link), flush=True)
    rc, out = _run(link)
    for obj in objs:
        if os.path.exists(obj):
            os.remove(obj)
    if rc != 0:
        raise RuntimeError(f"hipcc link failed ({rc}):\n{out}")
    os.replace(tmp, LIB)
    return LIB


def is_stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(d) > t for d in DEPS)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
