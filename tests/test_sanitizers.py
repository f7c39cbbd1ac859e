"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two builds, each loaded into a child Python process that preloads its
sanitizer runtime (a report ends the child with a non-zero status):

* The C ABI's host logic: csrc/gdr_api.hip with host-side
  -fsanitize=address,undefined (the device side is untouched), linked with
  stubs in place of the kernel launchers (tests/sanitize/launch_stubs.hip):
  on the CPU nothing is launched.  The child runs all of
  tests/test_abi_host.py against it: every validation path, the workspace,
  segment and slab queries, the no-alloc size check and the binding's
  argument checks.
* The oracle: oracle/gdr_oracle.c built by gcc with
  -fsanitize=address,undefined.  The child runs the recurrence on small
  problems (both rules, grouped heads, per-channel decay, an initial state,
  ragged lengths) and must reproduce the normal build bit for bit.
"""
import glob
import os
import shutil
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "chunkwise_gated_delta_cumsum_amd", "csrc")
HERE = os.path.dirname(os.path.abspath(__file__))


def _clang_asan_runtime():
    pats = ["/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so",
            "/opt/rocm/llvm/lib/clang/*/lib/x86_64-unknown-linux-gnu/libclang_rt.asan.so"]
    for pat in pats:
        found = sorted(glob.glob(pat))
        if found:
            return found[-1]
    return None


def _gcc_runtime(name):
    try:
        path = subprocess.check_output(["gcc", f"-print-file-name={name}"], text=True).strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _run_child(cmd, env_extra, timeout=600):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["PYTHONPATH"] = ROOT + os.pathsep + env.get("PYTHONPATH", "")
    res = subprocess.run(cmd, cwd=ROOT, env=env, stdout=subprocess.PIPE,
                         stderr=subprocess.STDOUT, text=True, timeout=timeout)
    out = res.stdout
    assert res.returncode == 0, out[-6000:]
    for marker in ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer"):
        assert marker not in out, out[-6000:]
    return out


def test_abi_host_logic_under_sanitizers(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    runtime = _clang_asan_runtime()
    if not os.path.exists(hipcc) or runtime is None:
        pytest.skip("hipcc or the clang sanitizer runtime is not available")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer"]
    common = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC"] + san + inc
    api_o, stub_o = str(tmp_path / "api.o"), str(tmp_path / "stubs.o")
    lib = str(tmp_path / "libgdr_sanitized.so")
    procs = [subprocess.Popen([hipcc] + common + ["-c", "-o", api_o,
                                                  os.path.join(CSRC, "gdr_api.hip")]),
             subprocess.Popen([hipcc, "--cuda-host-only"] + common + [
                 "-c", "-o", stub_o, os.path.join(HERE, "sanitize", "launch_stubs.hip")])]
    assert all(p.wait() == 0 for p in procs)
    subprocess.check_call([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC"] + san[:4] +
                          ["-shared-libsan", "-o", lib, api_o, stub_o])
    out = _run_child([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                      os.path.join(HERE, "test_abi_host.py")],
                     {"LD_PRELOAD": runtime, "GDR_TEST_LIBRARY": lib})
    assert " passed" in out and "failed" not in out, out[-3000:]


def test_oracle_under_sanitizers(tmp_path):
    import oracle
    from chunkwise_gated_delta_cumsum_amd.inputs import Workload, make_inputs
    asan, ubsan = _gcc_runtime("libasan.so"), _gcc_runtime("libubsan.so")
    if shutil.which("gcc") is None or asan is None or ubsan is None:
        pytest.skip("gcc or its sanitizer runtimes are not available")
    lib = str(tmp_path / "libgdr_oracle_sanitized.so")
    subprocess.check_call(["gcc", "-O1", "-g", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                           "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
                           "-o", lib, os.path.join(ROOT, "oracle", "gdr_oracle.c"), "-lm"])
    cases = {
        "scalar_gqa_s0": (Workload("s1", B=2, T=37, H=2, HV=4, K=8, V=8, g_mu=3.0,
                                   s0_std=0.1, seed=3), "delta"),
        "perch_ragged": (Workload("s2", B=1, T=29, H=2, HV=2, K=16, V=8, per_channel=True,
                                  g_mu=4.0, seed=4), "delta"),
        "linear_gqa": (Workload("s3", B=2, T=21, H=1, HV=3, K=8, V=16, g_mu=3.0,
                                s0_std=0.1, seed=5), "linear"),
        "perch_linear_s0": (Workload("s4", B=1, T=13, H=2, HV=4, K=8, V=8, per_channel=True,
                                     g_mu=4.0, s0_std=0.1, seed=6), "linear"),
    }
    ref = {}
    for name, (w, rule) in cases.items():
        inp = make_inputs(w)
        o, s = oracle.recurrence(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.scale, inp.s0,
                                 rule=rule)
        for f, x in (("q", inp.q), ("k", inp.k), ("v", inp.v), ("g", inp.g),
                     ("beta", inp.beta), ("o", o), ("s", s)):
            ref[f"{name}_{f}"] = np.asarray(x, dtype=np.float64)
        if inp.s0 is not None:
            ref[f"{name}_s0"] = np.asarray(inp.s0, dtype=np.float64)
        ref[f"{name}_scale"] = np.float64(inp.scale)
        ref[f"{name}_rule"] = np.array(rule)
    npz = str(tmp_path / "ref.npz")
    np.savez(npz, **ref)
    out = _run_child([sys.executable, os.path.join(HERE, "sanitize", "oracle_child.py"),
                      lib, npz],
                     {"LD_PRELOAD": asan + " " + ubsan, "OMP_NUM_THREADS": "2"})
    assert "4 problems equal" in out, out[-3000:]
