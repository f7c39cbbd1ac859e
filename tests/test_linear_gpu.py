"""GPU parity of the decayed linear-attention rule (gdr_problem.rule =
GDR_RULE_LINEAR: no erase term, the Mamba2 state-space-duality form of the
"Chunkwise parallel algorithms" page, section 1.1) against the fp64 oracle's
linear recurrence.  Bounds as for the delta rule: 1e-3 for fp32 inputs,
2e-2 for bf16 inputs, on o and the final state.
"""
import numpy as np
import pytest

import oracle
from chunkwise_gated_delta_cumsum_amd.inputs import WORKLOADS, make_inputs
from helpers import TOL, rel_err, to_device

pytestmark = pytest.mark.gpu


def check(o, s, ro, rs, dtype, label):
    eo, es = rel_err(o, ro), rel_err(s, rs)
    print(f"{label}: err_o={eo:.3e} err_S={es:.3e} (tol {TOL[dtype]})", flush=True)
    assert np.isfinite(o).all() and np.isfinite(s).all()
    assert eo <= TOL[dtype] and es <= TOL[dtype], (eo, es)


def oracle_linear(inp):
    return oracle.recurrence(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.scale, inp.s0,
                             rule="linear")


CASES = [
    (WORKLOADS[1].with_(T=300), 0, 0),
    (WORKLOADS[1].with_(T=1000), 5, 32),                 # ragged, segmented, 32-column slabs
    (WORKLOADS[2].with_(B=1, T=200), 0, 0),              # per-channel decay (gated linear attention)
    (WORKLOADS[2].with_(B=1, T=700), 3, 0),
    (WORKLOADS[3].with_(B=1, T=640), 3, 0),              # grouped heads, initial state
    (WORKLOADS[0], 2, 0),                                # fp32
    (WORKLOADS[3].with_(B=1, T=450, K=64, V=128), 1, 0),
]


@pytest.mark.parametrize("w,segs,slab", CASES,
                         ids=[f"{w.name}-T{w.T}-K{w.K}V{w.V}-seg{s_}" for w, s_, _ in CASES])
def test_chunk_fwd_linear(gpu_lib, w, segs, slab):
    import torch
    inp = make_inputs(w)
    t = to_device(inp)
    o, s = gpu_lib.gdr_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["initial_state"],
                                 scale=inp.scale, segments=segs, slab=slab, rule="linear")
    torch.cuda.synchronize()
    ro, rs = oracle_linear(inp)
    check(o.cpu().numpy(), s.cpu().numpy(), ro, rs, w.dtype, f"linear {w.name} T={w.T}")


@pytest.mark.parametrize("w", [WORKLOADS[1].with_(T=200), WORKLOADS[2].with_(B=1, T=130)],
                         ids=["scalar", "per_channel"])
def test_linear_prep_has_no_ut_transform(gpu_lib, w):
    """With the linear rule the prep stage's A_kk is zero and M^-1 = I exactly."""
    import torch
    inp = make_inputs(w)
    t = to_device(inp)
    _, ins = gpu_lib.gdr_chunk_prep(t["q"], t["k"], t["g"], t["beta"], scale=inp.scale, V=w.V,
                                    inspect=True, rule="linear")
    torch.cuda.synchronize()
    assert not ins["a_kk"].any()
    eye = torch.eye(w.chunk, device=ins["m_inv"].device).expand_as(ins["m_inv"])
    assert torch.equal(ins["m_inv"], eye)


FULL = [(1, [(0, 0), (0, 5), (0, 11)]), (2, [(0, 3), (3, 15)]), (3, [(0, 1), (1, 30)]),
        (4, [(0, 7)])]


@pytest.mark.parametrize("idx,heads", FULL, ids=[WORKLOADS[i].name for i, _ in FULL])
def test_linear_full_size_sampled_heads(gpu_lib, idx, heads):
    """Every large workload at full size, in the bench's launch configuration
    (automatic segments and slabs: the linear rule's own scan), against
    sampled (batch, value head) scans."""
    import torch
    w = WORKLOADS[idx]
    inp = make_inputs(w)
    t = to_device(inp)
    o, s = gpu_lib.gdr_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["initial_state"],
                                 scale=inp.scale, rule="linear")
    torch.cuda.synchronize()
    o, s = o.cpu().numpy(), s.cpu().numpy()
    ref = oracle.recurrence_heads(inp, heads, rule="linear")
    for (b, hv), (ro, rs) in ref.items():
        check(o[b, :, hv], s[b, hv], ro, rs, w.dtype, f"linear {w.name} head ({b}, {hv})")


@pytest.mark.parametrize("w", [WORKLOADS[3].with_(B=2, T=12), WORKLOADS[2].with_(B=1, T=12)],
                         ids=["gqa", "kda"])
def test_decode_linear_token_by_token(gpu_lib, w):
    import torch
    inp = make_inputs(w)
    t = to_device(inp)
    s = t["initial_state"]
    outs = []
    for i in range(w.T):
        o, s = gpu_lib.gdr_decode_step(t["q"][:, i].contiguous(), t["k"][:, i].contiguous(),
                                       t["v"][:, i].contiguous(), t["g"][:, i].contiguous(),
                                       t["beta"][:, i].contiguous(), s, scale=inp.scale,
                                       rule="linear")
        outs.append(o)
    torch.cuda.synchronize()
    ro, rs = oracle_linear(inp)
    check(torch.stack(outs, 1).cpu().numpy(), s.cpu().numpy(), ro, rs, w.dtype,
          f"linear decode {w.name}")
