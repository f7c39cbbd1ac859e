"""bench.py end to end on the GPU (one short run in a child process): the
JSON line's contract and the parity of its timed output against the oracle."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                         stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True,
                         timeout=100, cwd=ROOT)
    assert res.returncode == 0, res.stderr[-2000:]
    lines = [l for l in res.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, res.stdout[-2000:]
    return json.loads(lines[0])


def test_bench_line_tiny_fp32():
    rec = run_bench("--config", "0", "--steps", "3", "--warmup", "2", "--cpu-budget", "0.5")
    assert rec["config"]["workload"] == "tiny_fp32_T256_H2_D64"
    assert rec["n_gpus"] == 1 and rec["steps"] == 3 and rec["warmup"] == 2
    assert rec["value"] > 0 and rec["unit"] == "tokens/s" and rec["higher_is_better"]
    assert rec["dtype"] == "fp32" and rec["data"] == "synthetic"
    assert rec["fwd_entry_point_matches"]
    rf = rec["roofline"]
    assert rf["bound"] == "hbm" and rf["peak"] == 8000.0
    assert rf["frac"] == pytest.approx(rf["achieved"] / rf["peak"])
    cb = rec["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["cores"] >= 1
    par = cb["parity"]
    print(par, flush=True)
    assert par["pass"] and par["err_o"] <= 1e-3 and par["err_state"] <= 1e-3


@pytest.mark.parametrize("flags,tol", [(("--rule", "linear"), 1e-3), (("--chunk", "128"), 1e-3),
                                       (("--chunk", "32"), 1e-3), (("--dtype", "fp16"), 2e-2),
                                       (("--config", "1", "--dtype", "fp16"), 2e-2)],
                         ids=["linear", "c128", "c32", "fp16", "4096-fp16"])
def test_bench_line_options(flags, tol):
    """The launch-path options of the bench, each checked against the oracle
    in the same run (the 4096-token workload's prefix sample for the last)."""
    args = ("--config", "0") if "--config" not in flags else ()
    rec = run_bench(*args, *flags, "--steps", "3", "--warmup", "2", "--cpu-budget", "0.5")
    par = rec["cpu_baseline"]["parity"]
    print(flags, rec["config"]["workload"], par, flush=True)
    assert rec["fwd_entry_point_matches"] and par["pass"] and par["tol"] == tol
    assert par["err_o"] <= tol and (par["err_state"] is None or par["err_state"] <= tol)


def test_bench_line_decode():
    rec = run_bench("--workload", "decode_kda_bf16_B32_H16_D128", "--steps", "3", "--warmup", "2",
                    "--cpu-budget", "0.5")
    assert rec["config"]["T"] == 1 and rec["value"] > 0
    par = rec["cpu_baseline"]["parity"]
    print(par, flush=True)
    assert par["pass"] and par["err_o"] <= 2e-2 and par["err_state"] <= 2e-2
