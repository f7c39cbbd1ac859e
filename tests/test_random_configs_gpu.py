"""Parity on seeded random configurations across the supported space.

The hand-written cases cover each option on its own and in the pairs the
workloads use; this module draws 72 configurations at random from every
combination the C ABI accepts: chunk length (32, 64, 128), K and V (64,
128), grouped heads (G = 1, 2, 4), one decay per value head or per key
channel with slow or fast decays, bf16 or fp32 inputs (draws 48-71 may
also take fp16), the delta or the linear rule, in-kernel q/k normalisation,
forced scan segments and slab widths, an initial state, and ragged lengths
(any T up to 5 chunks past a multiple).  Each runs gdr_chunk_fwd against the
fp64 oracle recurrence with the bounds of the other parity tests (1e-3 for
fp32 inputs, 2e-2 for bf16 and fp16, on o and the final state).  The draws are seeded, so every run checks the
same configurations; their parameters are printed with the errors.
"""
import numpy as np
import pytest

import oracle
from chunkwise_gated_delta_cumsum_amd.inputs import Workload, make_inputs
from helpers import TOL, rel_err, run_gpu

pytestmark = pytest.mark.gpu

N_CONFIGS = 72
N_BEFORE_FP16 = 48


def draw(i):
    rng = np.random.default_rng(1000 + i)
    C = int(rng.choice([32, 64, 128]))
    K = int(rng.choice([64, 128]))
    V = int(rng.choice([64, 128]))
    H = int(rng.choice([1, 2]))
    G = int(rng.choice([1, 2, 4]))
    B = int(rng.choice([1, 2]))
    T = int(rng.integers(1, 5 * C + 40))
    per_channel = bool(rng.random() < 0.4)
    dtype = "fp32" if rng.random() < 0.25 else "bf16"
    if i >= N_BEFORE_FP16 and dtype == "bf16" and rng.random() < 0.6:
        dtype = "fp16"
    rule = "linear" if rng.random() < 0.25 else "delta"
    l2norm = bool(rng.random() < 0.25)
    mu = float(rng.choice([1.0, 3.0, 5.0]))
    s0 = 0.1 if rng.random() < 0.5 else 0.0
    segments = int(rng.choice([0, 0, 1, 2, 3, 5]))
    # slab: automatic, or (64- and 32-row chunks) a forced width
    slab = 0 if C == 128 else int(rng.choice([0, 32, 64]))
    w = Workload(f"rand{i}", B=B, T=T, H=H, HV=H * G, K=K, V=V, chunk=C,
                 per_channel=per_channel, dtype=dtype, g_mu=mu, s0_std=s0, seed=2000 + i,
                 normalize_qk=not l2norm)
    return w, dict(rule=rule, qk_l2norm=l2norm, segments=segments, slab=slab)


CASES = [draw(i) for i in range(N_CONFIGS)]


@pytest.mark.parametrize("w,kw", CASES, ids=[c[0].name for c in CASES])
def test_random_config(gpu_lib, w, kw):
    inp = make_inputs(w)
    o, s = run_gpu(gpu_lib, inp, **kw)
    q, k = inp.q, inp.k
    if kw["qk_l2norm"]:
        q, k = oracle.l2norm_rows(q), oracle.l2norm_rows(k)
    ro, rs = oracle.recurrence(q, k, inp.v, inp.g, inp.beta, inp.scale, inp.s0, rule=kw["rule"])
    eo, es = rel_err(o, ro), rel_err(s, rs)
    print(f"{w.name}: B={w.B} T={w.T} H={w.H} HV={w.HV} K={w.K} V={w.V} C={w.chunk} "
          f"pc={w.per_channel} {w.dtype} mu={w.g_mu} s0={w.s0_std} {kw}: "
          f"err_o={eo:.2e} err_S={es:.2e}", flush=True)
    assert np.isfinite(o).all() and np.isfinite(s).all()
    assert eo <= TOL[w.dtype] and es <= TOL[w.dtype], (eo, es)
