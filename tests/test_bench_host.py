"""Host logic of bench.py (no GPU): the byte and flop models its roofline
figures rest on, the parity report of its cpu_baseline leg, and the refusal
of more than one GPU.

The byte model is pinned to per-token figures derived by hand from the
definition of the compulsory bytes (every input read once, q and k once per
q/k head, o written once in fp32, the initial and final states): per token
and value head, q and k (2 K bytes each at 16 bits, shared by the G value
heads of a group), v (2 V), g (4, or 4 K per channel), beta (4), o (4 V),
plus the K V fp32 state read and written once per head, spread over the T
tokens.  The flop model is pinned to the per-token MAC count of the chunk
algorithm written out term by term at K = V = 128, C = 64, G = 1: the two
decayed Grams' lower triangles (63/2 + 65/2) K = 8,192, the UT forward
substitution 63/2 (K + V) = 8,064, W S, q S and K^T r 3 K V = 49,152, and
A_qk r 65/2 V = 4,160: 69,568 MAC.
"""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
import oracle  # noqa: E402
from chunkwise_gated_delta_cumsum_amd.inputs import WORKLOADS, make_inputs  # noqa: E402


def per_token_head(w):
    G = w.HV // w.H
    qk = 2 * 2 * w.K / G
    g = 4 * (w.K if w.per_channel else 1)
    state = (2 if w.s0_std > 0 else 1) * w.K * w.V * 4 / w.T
    return qk + 2 * w.V + g + 4 + 4 * w.V + state


@pytest.mark.parametrize("i,bytes_per_tok_head", [(1, 1304), (2, 1804), (3, 1040), (4, 1289)])
def test_compulsory_bytes(i, bytes_per_tok_head):
    w = WORKLOADS[i]
    tm = bench.traffic_model(w)
    assert round(per_token_head(w)) == bytes_per_tok_head
    assert tm["compulsory"] == pytest.approx(per_token_head(w) * w.B * w.T * w.HV, rel=1e-12)
    # the two stages' compulsory bytes: q and k are read by both
    qk = 2 * w.B * w.T * w.H * w.K * 2
    assert tm["stage"]["chunk_prep"] + tm["stage"]["state_scan"] == tm["compulsory"] + qk
    # the design moves at least the compulsory bytes of each stage
    for s in ("chunk_prep", "state_scan"):
        assert tm["design"][s] > tm["stage"][s]


def test_algorithmic_flops():
    w = WORKLOADS[1]
    per_tok_head = bench.algorithmic_flops(w) / (w.B * w.T * w.HV)
    assert per_tok_head == 2 * (8192 + 8064 + 49152 + 4160) == 2 * 69568
    # the Gram terms are shared by the G value heads of a group
    w3 = WORKLOADS[3]
    assert bench.algorithmic_flops(w3) / (w3.B * w3.T * w3.HV) == 2 * (8192 / 2 + 8064 + 49152
                                                                       + 4160)
    # the totals of the four large workloads, as rounded where the workloads
    # are tabulated (a dropped term moves a total by 3% or more)
    for i, gf in ((1, 6.84), (2, 73.0), (3, 134.1), (4, 109.4)):
        assert bench.algorithmic_flops(WORKLOADS[i]) / 1e9 == pytest.approx(gf, rel=2e-3)


def test_cpu_baseline_parity_report():
    inp = make_inputs(WORKLOADS[0])
    w = inp.w
    ro, rs = oracle.recurrence(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.scale, inp.s0)
    seen = []

    def exact(Ts):
        seen.append(Ts)
        return ro[:, :Ts].astype(np.float32), (rs.astype(np.float32) if Ts == w.T else None)

    rec = bench.cpu_baseline(inp, 0.2, gpu_out=exact)
    par = rec["parity"]
    assert seen and par["pass"] and par["tol"] == bench.PARITY_TOL["fp32"]
    assert par["err_o"] < 1e-6
    assert (par["err_state"] is None) == (seen[0] != w.T)
    assert rec["kind"] == "oracle" and rec["cores"] >= 1

    def off(Ts):
        o = ro[:, :Ts].copy()
        o[0, Ts - 1, 1, 3] += 0.05 * np.sqrt((o ** 2).mean())
        return o, None

    par = bench.cpu_baseline(inp, 0.2, gpu_out=off)["parity"]
    assert not par["pass"] and par["err_o"] == pytest.approx(0.05, rel=1e-3)


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=60)
    assert res.returncode == 2
    assert "one GPU" in res.stderr and res.stdout == ""
