"""GPU parity with 32- and 128-row chunks (gdr_problem.chunk = 32 or 128; the
64-row default is covered by test_gpu_parity.py).  The chunk length is a free
parameter of the method: the "Chunkwise parallel algorithms" page names 64 or
128, and the scalar-g kernel page takes chunk_size as an argument.  The
result is the same recurrence for any chunk length, so the reference is the
fp64 oracle recurrence as for 64-row chunks; bounds 1e-3 for fp32 inputs and
2e-2 for bf16 inputs on o and the final state.  The stage test checks the
C x C A_kk, A_qk and M^-1 against the oracle's chunk form at the same C.
"""
import numpy as np
import pytest

import oracle
from chunkwise_gated_delta_cumsum_amd.inputs import WORKLOADS, Workload, make_inputs
from helpers import TOL, rel_err, rel_err_rows, run_gpu, to_device

pytestmark = pytest.mark.gpu

CHUNKS = [32, 128]


@pytest.fixture(params=CHUNKS, ids=[f"C{c}" for c in CHUNKS])
def C(request):
    return request.param


def oracle_full(inp, rule="delta"):
    return oracle.recurrence(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.scale, inp.s0, rule=rule)


def check(o, s, ro, rs, dtype, label):
    eo, es = rel_err(o, ro), rel_err(s, rs)
    print(f"{label}: err_o={eo:.3e} err_S={es:.3e} (tol {TOL[dtype]})", flush=True)
    assert np.isfinite(o).all() and np.isfinite(s).all()
    assert eo <= TOL[dtype] and es <= TOL[dtype], (eo, es)


def small(C, per_channel=False, dtype="bf16", T=300, H=2, HV=2, K=128, V=128, s0=0.1, seed=17,
          mu=3.0):
    return Workload(f"edge{C}", B=2, T=T, H=H, HV=HV, K=K, V=V, chunk=C,
                    per_channel=per_channel, dtype=dtype, g_mu=mu, s0_std=s0, seed=seed)


# ------------------------------------------- the five workloads, reduced -----
SMALL = [(0, {}), (1, dict(T=1000)), (2, dict(B=2, T=700)), (3, dict(T=777)), (4, dict(T=2000))]


@pytest.mark.parametrize("idx,kw", SMALL, ids=[WORKLOADS[i].name for i, _ in SMALL])
def test_end_to_end_small(gpu_lib, C, idx, kw):
    w = WORKLOADS[idx].with_(chunk=C, **kw)
    inp = make_inputs(w)
    o, s = run_gpu(gpu_lib, inp)
    check(o, s, *oracle_full(inp), w.dtype, f"C={C} {w.name}")


# ------------------------------------------- full size, every scan ----------
@pytest.mark.parametrize("idx", [1, 2, 3, 4], ids=[WORKLOADS[i].name for i in (1, 2, 3, 4)])
def test_full_size_every_head(gpu_lib, C, idx):
    w = WORKLOADS[idx].with_(chunk=C)
    inp = make_inputs(w)
    o, s = run_gpu(gpu_lib, inp)
    check(o, s, *oracle_full(inp), w.dtype, f"C={C} {w.name}")


# --------------------------------------------------- stage intermediates ---
PREP = [(0, {}), (1, dict(T=300)), (2, dict(B=1, T=300)), (3, dict(B=1, T=200))]


@pytest.mark.parametrize("idx,kw", PREP, ids=[WORKLOADS[i].name for i, _ in PREP])
def test_prep_intermediates(gpu_lib, C, idx, kw):
    """gamma, A_kk, A_qk and M^-1 of C-row chunks against the oracle's chunk
    form at the same C, with the bounds of the 64-row stage test (1e-5 for the
    fp32 prefix sum, 1e-4 for exact products summed in fp32, 1e-2 for the
    per-channel decayed dots from fp16-rounded operands, 8 * 2^-11 for the
    bf16 path's blocked inverse)."""
    import torch
    w = WORKLOADS[idx].with_(chunk=C, **kw)
    inp = make_inputs(w)
    t = to_device(inp)
    _, ins = gpu_lib.gdr_chunk_prep(t["q"], t["k"], t["g"], t["beta"], chunk=C,
                                    scale=inp.scale, V=w.V, inspect=True)
    torch.cuda.synchronize()
    ins = {k_: v_.cpu().numpy().astype(np.float64) for k_, v_ in ins.items()}
    ref = oracle.chunk_forward(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.scale, C, inp.s0)
    gam = ref["gamma"] if w.per_channel else ref["gamma"][..., 0]
    errs = dict(gamma=rel_err(ins["gamma"], gam),
                a_kk=rel_err(ins["a_kk"], ref["M"] - np.eye(C)),
                a_qk=rel_err(ins["a_qk"], ref["A_qk"]),
                m_inv=rel_err(ins["m_inv"], oracle.ut_inverse_solve(ref["M"])))
    print(C, w.name, {k_: f"{v_:.2e}" for k_, v_ in errs.items()}, flush=True)
    f32 = w.dtype == "fp32"
    bounds = dict(gamma=1e-5,
                  a_kk=1e-4 if (f32 or not w.per_channel) else 1e-2,
                  a_qk=1e-4 if (f32 or not w.per_channel) else 1e-2,
                  m_inv=1e-4 if f32 else 8 * 2.0 ** -11)
    for k_, e in errs.items():
        assert e <= bounds[k_], (k_, e, bounds[k_])


# ----------------------------------------------------------- edge cases ----
RAGGED = {"1": lambda C: 1, "17": lambda C: 17, "C-1": lambda C: C - 1, "C": lambda C: C,
          "C+1": lambda C: C + 1, "2C-1": lambda C: 2 * C - 1, "300": lambda C: 300}


@pytest.mark.parametrize("per_channel", [False, True])
@pytest.mark.parametrize("length", list(RAGGED))
def test_ragged_lengths(gpu_lib, C, per_channel, length):
    T = RAGGED[length](C)
    inp = make_inputs(small(C, per_channel=per_channel, T=T))
    o, s = run_gpu(gpu_lib, inp)
    check(o, s, *oracle_full(inp), "bf16", f"T={T} pc={per_channel}")


@pytest.mark.parametrize("K,V,dtype", [(64, 64, "bf16"), (128, 64, "bf16"), (64, 128, "bf16"),
                                       (128, 128, "fp32"), (64, 128, "fp32"), (128, 64, "fp32")])
@pytest.mark.parametrize("per_channel", [False, True])
def test_head_dims_and_dtypes(gpu_lib, C, K, V, dtype, per_channel):
    inp = make_inputs(small(C, per_channel=per_channel, dtype=dtype, K=K, V=V, T=300))
    o, s = run_gpu(gpu_lib, inp)
    check(o, s, *oracle_full(inp), dtype, f"K={K} V={V} {dtype} pc={per_channel}")


@pytest.mark.parametrize("per_channel", [False, True])
def test_reset_and_positive_g(gpu_lib, C, per_channel):
    inp = make_inputs(small(C, per_channel=per_channel, T=300))
    inp.g[...] = -800.0
    o, s = run_gpu(gpu_lib, inp)
    check(o, s, *oracle_full(inp), "bf16", f"reset pc={per_channel}")
    # positive g: the bound per row (see test_gpu_parity.test_positive_g)
    inp = make_inputs(small(C, per_channel=per_channel, T=300))
    rng = np.random.default_rng(3)
    inp.g[...] = (0.1 * rng.standard_normal(inp.g.shape)).astype(np.float32)
    o, s = run_gpu(gpu_lib, inp)
    ro, rs = oracle_full(inp)
    eo, es = rel_err_rows(o, s, ro, rs)
    print(f"C={C} positive g pc={per_channel}: per row err_o={eo:.3e} err_S={es:.3e}, "
          f"whole err_o={rel_err(o, ro):.3e} err_S={rel_err(s, rs):.3e}", flush=True)
    assert eo <= TOL["bf16"] and es <= TOL["bf16"], (eo, es)
    if not per_channel:
        check(o, s, ro, rs, "bf16", f"positive g pc={per_channel}")


@pytest.mark.parametrize("mu", [-1.0, -3.0])
def test_per_channel_strong_decay(gpu_lib, C, mu):
    inp = make_inputs(small(C, per_channel=True, T=300, mu=mu))
    o, s = run_gpu(gpu_lib, inp)
    check(o, s, *oracle_full(inp), "bf16", f"strong decay mu={mu}")


def test_per_channel_mixed_extreme_decay(gpu_lib, C):
    inp = make_inputs(small(C, per_channel=True, T=300, mu=4.0))
    rng = np.random.default_rng(11)
    inp.g[rng.random(inp.g.shape) < 0.05] = -30.0
    o, s = run_gpu(gpu_lib, inp)
    check(o, s, *oracle_full(inp), "bf16", "mixed extreme decay")


def test_beta0_g0_keeps_state(gpu_lib, C):
    inp = make_inputs(small(C, T=300))
    inp.g[...] = 0.0
    inp.beta[...] = 0.0
    o, s = run_gpu(gpu_lib, inp)
    assert np.array_equal(s, inp.s0)
    check(o, s, *oracle_full(inp), "bf16", "beta0 g0")


@pytest.mark.parametrize("G", [2, 4])
@pytest.mark.parametrize("per_channel", [False, True])
def test_grouped_heads(gpu_lib, C, G, per_channel):
    inp = make_inputs(small(C, per_channel=per_channel, H=2, HV=2 * G, T=300))
    o, s = run_gpu(gpu_lib, inp)
    check(o, s, *oracle_full(inp), "bf16", f"G={G} pc={per_channel}")


SEG_CASES = [
    (1, dict(T=1000), [1, 2, 3, 8]),    # a ragged last chunk at both lengths
    (2, dict(B=1, T=700), [1, 2, 3]),   # per-channel decay
    (3, dict(B=1, T=900), [1, 3, 7]),   # grouped heads + initial state
    (0, dict(T=700), [1, 2, 4]),        # fp32, K = V = 64
]


@pytest.mark.parametrize("idx,kw,segs", SEG_CASES, ids=[WORKLOADS[c[0]].name for c in SEG_CASES])
def test_scan_segments(gpu_lib, C, idx, kw, segs):
    w = WORKLOADS[idx].with_(chunk=C, **kw)
    inp = make_inputs(w)
    ro, rs = oracle_full(inp)
    slabs = (32, 64) if C == 32 else (0,)
    for nseg in segs:
        for slab in slabs:
            prob = gpu_lib.problem(w.B, w.T, w.H, w.HV, w.K, w.V, chunk=C,
                                   per_channel=w.per_channel, dtype=w.dtype, segments=nseg,
                                   slab=slab)
            used = gpu_lib.scan_segments(prob)
            assert 1 <= used <= nseg
            o, s = run_gpu(gpu_lib, inp, segments=nseg, slab=slab)
            check(o, s, ro, rs, w.dtype, f"C={C} {w.name} segments={nseg}->{used} slab={slab}")


def test_in_place_state_with_segments(gpu_lib, C):
    import torch
    w = WORKLOADS[3].with_(B=1, T=900, chunk=C)
    inp = make_inputs(w)
    t = to_device(inp)
    args = (t["q"], t["k"], t["v"], t["g"], t["beta"])
    o_ref, s_ref = gpu_lib.gdr_chunk_fwd(*args, t["initial_state"], chunk=C, scale=inp.scale,
                                         segments=3)
    st = t["initial_state"].clone()
    o = torch.empty_like(o_ref)
    gpu_lib.gdr_chunk_fwd(*args, st, chunk=C, scale=inp.scale, segments=3, out=(o, st))
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(st, s_ref)


# --------------------------------- the linear rule, in-kernel normalisation -
LIN = [(1, dict(T=1000), 3), (2, dict(B=1, T=700), 1), (3, dict(B=1, T=640), 2), (0, {}, 1)]


@pytest.mark.parametrize("idx,kw,segs", LIN, ids=[f"{WORKLOADS[i].name}-seg{s_}" for i, _, s_ in LIN])
def test_linear_rule(gpu_lib, C, idx, kw, segs):
    w = WORKLOADS[idx].with_(chunk=C, **kw)
    inp = make_inputs(w)
    o, s = run_gpu(gpu_lib, inp, segments=segs, rule="linear")
    check(o, s, *oracle_full(inp, rule="linear"), w.dtype, f"C={C} linear {w.name}")


@pytest.mark.parametrize("idx,kw", [(1, dict(T=1000)), (2, dict(B=1, T=500))],
                         ids=["scalar", "per-channel"])
def test_in_kernel_l2norm(gpu_lib, C, idx, kw):
    w = WORKLOADS[idx].with_(chunk=C, normalize_qk=False, **kw)
    inp = make_inputs(w)
    o, s = run_gpu(gpu_lib, inp, qk_l2norm=True)
    ro, rs = oracle.recurrence(oracle.l2norm_rows(inp.q), oracle.l2norm_rows(inp.k), inp.v, inp.g,
                               inp.beta, inp.scale, inp.s0)
    check(o, s, ro, rs, w.dtype, f"C={C} l2norm {w.name}")


def test_chunk_lengths_agree(gpu_lib, C):
    """64-row chunks and C-row chunks compute the same recurrence: both within
    the bound of the oracle, and of each other."""
    w = WORKLOADS[3].with_(T=1000)
    inp = make_inputs(w)
    o64, s64 = run_gpu(gpu_lib, inp)
    inpc = make_inputs(w.with_(chunk=C))
    oc, sc = run_gpu(gpu_lib, inpc)
    assert rel_err(oc, o64) <= TOL["bf16"] and rel_err(sc, s64) <= TOL["bf16"]
