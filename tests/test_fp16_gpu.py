"""fp16 inputs and fp16 o (GDR_F16) on the GPU, against the fp64 oracle.

With fp16 q, k and v the kernels use the input values as fp16 MFMA operands
without conversion; every other operand and every rounding is that of the
bf16 path, so the bound is the 16-bit one (2e-2, max|delta| / rms(ref) on o
and the final state).  The inputs are the seeded workloads rounded once to
fp16 (round to nearest even), and the oracle consumes exactly those values.

Covered: both decay forms, grouped heads with an initial state, ragged
lengths, 32-, 64- and 128-row chunks, forced scan segments, the linear rule,
in-kernel q/k normalisation, the grouped-head workload at full size (every
value head of one batch), the prep stage's intermediates, fp16 o (the fp32
result rounded once), the decode step, and the input check's fp16 encoding.
"""
import numpy as np
import pytest

import oracle
from chunkwise_gated_delta_cumsum_amd.inputs import WORKLOADS, Workload, make_inputs
from helpers import TOL, rel_err, run_gpu, to_device

pytestmark = pytest.mark.gpu


def small(per_channel=False, T=300, B=2, H=2, HV=4, chunk=64, s0=0.1, seed=61, norm=True):
    return Workload("h16", B=B, T=T, H=H, HV=HV, K=128, V=128, chunk=chunk,
                    per_channel=per_channel, dtype="fp16", g_mu=4.0 if per_channel else 3.0,
                    s0_std=s0, seed=seed, normalize_qk=norm)


def check(o, s, ro, rs, label):
    eo, es = rel_err(o, ro), rel_err(s, rs)
    print(f"{label}: err_o={eo:.3e} err_S={es:.3e} (tol {TOL['fp16']})", flush=True)
    assert np.isfinite(o).all() and np.isfinite(s).all()
    assert eo <= TOL["fp16"] and es <= TOL["fp16"], (eo, es)


CASES = [
    (dict(), dict()),
    (dict(per_channel=True), dict()),
    (dict(T=1), dict()),
    (dict(T=129, H=1, HV=4), dict()),
    (dict(T=777), dict(segments=4)),
    (dict(per_channel=True, T=500), dict(segments=3)),
    (dict(chunk=32, T=301), dict()),
    (dict(chunk=128, T=301), dict()),
    (dict(chunk=128, T=301, per_channel=True), dict()),
    (dict(chunk=32, T=201, per_channel=True), dict()),
    (dict(T=300), dict(slab=32)),
    (dict(T=300), dict(rule="linear")),
    (dict(T=300, per_channel=True), dict(rule="linear", segments=2)),
    (dict(T=300, norm=False), dict(qk_l2norm=True)),
    (dict(T=300, norm=False, per_channel=True), dict(qk_l2norm=True)),
]


@pytest.mark.parametrize("wkw,kw", CASES, ids=[f"{i}" for i in range(len(CASES))])
def test_fp16_inputs_match_the_oracle(gpu_lib, wkw, kw):
    w = small(**wkw)
    inp = make_inputs(w)
    o, s = run_gpu(gpu_lib, inp, **kw)
    q, k = inp.q, inp.k
    if kw.get("qk_l2norm"):
        q, k = oracle.l2norm_rows(q), oracle.l2norm_rows(k)
    ro, rs = oracle.recurrence(q, k, inp.v, inp.g, inp.beta, inp.scale, inp.s0,
                               rule=kw.get("rule", "delta"))
    check(o, s, ro, rs, f"fp16 {wkw} {kw}")


def test_fp16_full_size_grouped_heads(gpu_lib):
    """The grouped-head workload (B2 T16000 H16 HV32) in fp16, in the bench's
    launch configuration, against the oracle on every value head of batch 1."""
    import torch
    w = WORKLOADS[3].with_(dtype="fp16")
    inp = make_inputs(w)
    t = to_device(inp)
    o, s = gpu_lib.gdr_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["initial_state"],
                                 scale=inp.scale)
    torch.cuda.synchronize()
    o, s = o.cpu().numpy(), s.cpu().numpy()
    ref = oracle.recurrence_heads(inp, [(1, hv) for hv in range(w.HV)])
    for (b, hv), (ro, rs) in ref.items():
        check(o[b, :, hv], s[b, hv], ro, rs, f"full size head ({b}, {hv})")


@pytest.mark.parametrize("per_channel", [False, True], ids=["row", "pc"])
def test_fp16_prep_intermediates(gpu_lib, per_channel):
    """gamma, A_kk, A_qk and M^-1 from fp16 inputs: the Gram products take the
    raw fp16 values (exact products), so A_kk and A_qk meet 1e-4 with one
    decay per row; the per-channel and inverse bounds are the bf16 path's."""
    import torch
    w = small(per_channel=per_channel, B=1, T=200)
    inp = make_inputs(w)
    t = to_device(inp)
    _, ins = gpu_lib.gdr_chunk_prep(t["q"], t["k"], t["g"], t["beta"], scale=inp.scale,
                                    V=w.V, inspect=True)
    torch.cuda.synchronize()
    ins = {k_: v_.cpu().numpy().astype(np.float64) for k_, v_ in ins.items()}
    ref = oracle.chunk_forward(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.scale, w.chunk, inp.s0)
    gam = ref["gamma"] if per_channel else ref["gamma"][..., 0]
    errs = dict(gamma=rel_err(ins["gamma"], gam),
                a_kk=rel_err(ins["a_kk"], ref["M"] - np.eye(w.chunk)),
                a_qk=rel_err(ins["a_qk"], ref["A_qk"]),
                m_inv=rel_err(ins["m_inv"], oracle.ut_inverse_solve(ref["M"])))
    print({k_: f"{v_:.2e}" for k_, v_ in errs.items()}, flush=True)
    bounds = dict(gamma=1e-5, a_kk=1e-2 if per_channel else 1e-4,
                  a_qk=1e-2 if per_channel else 1e-4, m_inv=8 * 2.0 ** -11)
    for k_, e in errs.items():
        assert e <= bounds[k_], (k_, e)


def test_fp16_o_is_the_rounded_fp32_o(gpu_lib):
    import torch
    inp = make_inputs(small(T=333))
    t = to_device(inp)
    args = (t["q"], t["k"], t["v"], t["g"], t["beta"], t["initial_state"])
    o32, s32 = gpu_lib.gdr_chunk_fwd(*args, scale=inp.scale)
    oh, sh = gpu_lib.gdr_chunk_fwd(*args, scale=inp.scale, o_dtype="fp16")
    torch.cuda.synchronize()
    assert oh.dtype == torch.float16
    assert torch.equal(oh, o32.to(torch.float16)) and torch.equal(sh, s32)


@pytest.mark.parametrize("per_channel", [False, True], ids=["row", "pc"])
def test_fp16_decode_step(gpu_lib, per_channel):
    import torch
    w = small(per_channel=per_channel, B=3, T=1)
    inp = make_inputs(w)
    t = to_device(inp)
    one = lambda x: x[:, 0].contiguous()
    o, s = gpu_lib.gdr_decode_step(one(t["q"]), one(t["k"]), one(t["v"]), one(t["g"]),
                                   one(t["beta"]), t["initial_state"], scale=inp.scale)
    oh, _ = gpu_lib.gdr_decode_step(one(t["q"]), one(t["k"]), one(t["v"]), one(t["g"]),
                                    one(t["beta"]), t["initial_state"], scale=inp.scale,
                                    o_dtype="fp16")
    torch.cuda.synchronize()
    ro, rs = oracle.recurrence(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.scale, inp.s0)
    check(o.cpu().numpy(), s.cpu().numpy(), ro[:, 0], rs, f"decode pc={per_channel}")
    assert torch.equal(oh, o.to(torch.float16))


def test_fp16_input_check(gpu_lib):
    """The input check reads fp16 encodings: large finite fp16 values are in
    range, an fp16 infinity or NaN is non-finite, and the decay bound applies."""
    inp = make_inputs(small(T=130))
    t = to_device(inp)
    flags = lambda: int(gpu_lib.gdr_check_inputs(t["q"], t["k"], t["v"], t["g"],
                                                 t["beta"])[0].item())
    assert flags() == 0
    t["q"][0, 3, 1, 5] = 60000.0                 # finite fp16: no range problem
    t["v"][1, 7, 2, 9] = -65504.0
    assert flags() == 0
    t["k"][1, 100, 0, 127] = float("inf")
    assert flags() == 1
    t["k"][1, 100, 0, 127] = float("nan")
    assert flags() == 1
    t["k"][1, 100, 0, 127] = 0.0
    t["g"][0, 70:102, 3] = 0.3                   # 9.6 within one 64-row chunk
    assert flags() == 4
