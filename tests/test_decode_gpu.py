"""GPU parity of the decode step (gdr_decode_step, through the C ABI) against
the fp64 oracle: the per-token recurrence itself, run for one token from the
same state (or for several tokens, step by step).

Bounds (max|delta| / rms(ref) on o and on the new state): 1e-3 for fp32
inputs and 2e-2 for bf16 inputs, as for the chunked path.
"""
import numpy as np
import pytest

import oracle
from chunkwise_gated_delta_cumsum_amd.inputs import DECODE_WORKLOADS, WORKLOADS, make_inputs
from helpers import TOL, rel_err

pytestmark = pytest.mark.gpu


def dev(a):
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def token(inp, t):
    """Device tensors of token t: q, k [B, H, K]; v [B, HV, V]; g; beta."""
    return (dev(inp.q_dev[:, t]), dev(inp.k_dev[:, t]), dev(inp.v_dev[:, t]),
            dev(inp.g[:, t]), dev(inp.beta[:, t]))


def check(o, s, ro, rs, dtype, label):
    eo, es = rel_err(o, ro), rel_err(s, rs)
    print(f"{label}: err_o={eo:.3e} err_S={es:.3e} (tol {TOL[dtype]})", flush=True)
    assert np.isfinite(o).all() and np.isfinite(s).all()
    assert eo <= TOL[dtype] and es <= TOL[dtype], (eo, es)


CASES = [
    WORKLOADS[3].with_(B=3, T=1, s0_std=0.1),                          # grouped heads, bf16
    WORKLOADS[2].with_(B=2, T=1, s0_std=0.1),                          # per-channel, bf16
    WORKLOADS[0].with_(B=2, T=1, s0_std=0.1),                          # fp32, K = V = 64
    WORKLOADS[3].with_(B=2, T=1, K=64, V=128, s0_std=0.1),
    WORKLOADS[3].with_(B=2, T=1, K=128, V=64, s0_std=0.1, dtype="fp32"),
    WORKLOADS[2].with_(B=2, T=1, K=64, V=64, s0_std=0.1, dtype="fp32"),
    WORKLOADS[2].with_(B=2, T=1, H=4, HV=16, s0_std=0.1),              # per-channel, G = 4
    WORKLOADS[2].with_(B=2, T=1, H=2, HV=4, s0_std=0.1, dtype="fp32"),  # per-channel, G = 2
]


@pytest.mark.parametrize("w", CASES, ids=[f"{w.name}-K{w.K}V{w.V}-{w.dtype}" for w in CASES])
def test_decode_one_token(gpu_lib, w):
    import torch
    inp = make_inputs(w)
    o, s = gpu_lib.gdr_decode_step(*token(inp, 0), dev(inp.s0), scale=inp.scale)
    torch.cuda.synchronize()
    ro, rs = oracle.recurrence(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.scale, inp.s0)
    check(o.cpu().numpy(), s.cpu().numpy(), ro[:, 0], rs, w.dtype, w.name)


@pytest.mark.parametrize("w", [WORKLOADS[3].with_(B=2, T=24), WORKLOADS[2].with_(B=1, T=24),
                               WORKLOADS[0].with_(T=24)], ids=["gqa", "kda", "fp32"])
def test_decode_token_by_token(gpu_lib, w):
    """T decode steps from the initial (or zero) state equal the recurrence over T tokens."""
    import torch
    inp = make_inputs(w)
    s = None if inp.s0 is None else dev(inp.s0)
    outs = []
    for t in range(w.T):
        o, s = gpu_lib.gdr_decode_step(*token(inp, t), s, scale=inp.scale)
        outs.append(o)
    torch.cuda.synchronize()
    o = torch.stack(outs, 1).cpu().numpy()
    ro, rs = oracle.recurrence(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.scale, inp.s0)
    check(o, s.cpu().numpy(), ro, rs, w.dtype, f"{w.name} x{w.T}")


@pytest.mark.parametrize("w", [WORKLOADS[1].with_(T=306), WORKLOADS[2].with_(B=1, T=200)],
                         ids=["scalar", "per_channel"])
def test_prefill_then_decode(gpu_lib, w):
    """The chunked forward over a prefix, then decode steps from its final state."""
    import torch
    inp = make_inputs(w)
    T1 = w.T - 6
    cut = lambda a: dev(np.ascontiguousarray(a[:, :T1]))
    o1, s = gpu_lib.gdr_chunk_fwd(cut(inp.q_dev), cut(inp.k_dev), cut(inp.v_dev), cut(inp.g),
                                  cut(inp.beta), None, scale=inp.scale)
    outs = [o1]
    for t in range(T1, w.T):
        o, s = gpu_lib.gdr_decode_step(*token(inp, t), s, scale=inp.scale)
        outs.append(o[:, None])
    torch.cuda.synchronize()
    o = torch.cat(outs, 1).cpu().numpy()
    ro, rs = oracle.recurrence(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.scale, inp.s0)
    check(o[:, T1:], s.cpu().numpy(), ro[:, T1:], rs, w.dtype, f"{w.name} prefill {T1} + 6")


@pytest.mark.parametrize("slab", [32, 64, 128])
@pytest.mark.parametrize("w", [WORKLOADS[3].with_(B=2, T=1, s0_std=0.1),
                               WORKLOADS[2].with_(B=2, T=1, K=64, V=64, s0_std=0.1)],
                         ids=["gqa", "kda_K64V64"])
def test_decode_column_slabs(gpu_lib, w, slab):
    """Every workgroup width gives the oracle's result (the widths sum a
    column's rows in different orders, so the bits may differ)."""
    import torch
    inp = make_inputs(w)
    o, s = gpu_lib.gdr_decode_step(*token(inp, 0), dev(inp.s0), scale=inp.scale, slab=slab)
    torch.cuda.synchronize()
    ro, rs = oracle.recurrence(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.scale, inp.s0)
    check(o.cpu().numpy(), s.cpu().numpy(), ro[:, 0], rs, w.dtype, f"{w.name} slab={slab}")


def test_decode_inplace_and_zero_state(gpu_lib):
    import torch
    w = WORKLOADS[3].with_(B=2, T=1, s0_std=0.1)
    inp = make_inputs(w)
    args = token(inp, 0)
    o1, s1 = gpu_lib.gdr_decode_step(*args, dev(inp.s0), scale=inp.scale)
    st = dev(inp.s0)
    o2, s2 = gpu_lib.gdr_decode_step(*args, st, scale=inp.scale, inplace=True)
    assert s2.data_ptr() == st.data_ptr()
    z = torch.zeros_like(st)
    o3, s3 = gpu_lib.gdr_decode_step(*args, z, scale=inp.scale)
    o4, s4 = gpu_lib.gdr_decode_step(*args, None, scale=inp.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    assert torch.equal(o3, o4) and torch.equal(s3, s4)


@pytest.mark.parametrize("w", DECODE_WORKLOADS, ids=[w.name for w in DECODE_WORKLOADS])
def test_decode_full_size(gpu_lib, w):
    """The decode batches the bench measures, every head checked."""
    import torch
    inp = make_inputs(w)
    o, s = gpu_lib.gdr_decode_step(*token(inp, 0), dev(inp.s0), scale=inp.scale)
    torch.cuda.synchronize()
    ro, rs = oracle.recurrence(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.scale, inp.s0)
    check(o.cpu().numpy(), s.cpu().numpy(), ro[:, 0], rs, w.dtype, w.name)
