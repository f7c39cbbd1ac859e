"""Maximum-size parity: one sequence long enough that q, k and v hold more
than 2^31 elements each and o spans more than 8 GiB, so every byte offset
past 4 GiB and every element index past 2^31 is exercised in the prep and
scan kernels.

The oracle cannot run 2^20 tokens of 17 heads, so the inputs are built so
that exact answers are cheap (a property that holds at any size):
  * before the last W tokens, beta = 0 and g = 0.  The state then stays the
    initial state S0 exactly (decay 1, write 0), so o_t = scale S0^T q_t for
    every such token: checked token by token on samples placed across the
    2^30- and 2^31-element points of o, q and k, and just before the window;
  * the last W tokens carry ordinary random beta and g; their o and the final
    state are the oracle recurrence over those W tokens started from S0.
The window starts mid-chunk, so one chunk mixes both kinds of rows.
Inputs are drawn on the device from a seeded generator; only the sampled rows
and the window come back to the host.
"""
import numpy as np
import pytest

import oracle
from helpers import TOL, rel_err

pytestmark = pytest.mark.gpu

T = (1 << 20) + 37     # a ragged tail at every chunk length (16385 chunks of 64)
H = HV = 17            # T * H * K = 2.28e9 elements > 2^31
K = V = 128
W = 256                # active tokens at the end


def _samples():
    per_tok = HV * V
    s = set(range(0, 64))
    for elems in (1 << 30, 1 << 31):                  # byte offset 4 GiB, element 2^31 of o
        t = elems // per_tok
        s.update(range(t - 32, t + 32))
    s.update(range(T - W - 64, T - W))                 # just before the window
    return np.array(sorted(s))


@pytest.mark.parametrize("per_channel,chunk", [(False, 64), (True, 64), (False, 32), (True, 128)],
                         ids=["scalar_g", "per_channel_g", "scalar_g_C32", "per_channel_g_C128"])
def test_max_size_offsets(gpu_lib, per_channel, chunk):
    import torch
    print(f"max-size case: B=1 T={T} H=HV={H} K=V={K} per_channel={per_channel} C={chunk}",
          flush=True)
    dev = "cuda"
    gen = torch.Generator(device=dev)
    gen.manual_seed(91 + int(per_channel))
    assert T * H * K > 2 ** 31 and T * HV * V * 4 > 2 ** 33

    def randn(*shape, dtype=torch.bfloat16):
        return torch.randn(*shape, generator=gen, device=dev, dtype=torch.float32).to(dtype)

    q = randn(1, T, H, K)
    k = randn(1, T, H, K)
    v = randn(1, T, HV, V)
    # unit-norm keys and queries in the window (the delta rule's usual inputs)
    t0 = T - W
    for x in (q, k):
        xw = x[:, t0:].float()
        x[:, t0:] = (xw / xw.norm(dim=-1, keepdim=True)).to(torch.bfloat16)
    gshape = (1, T, HV, K) if per_channel else (1, T, HV)
    g = torch.zeros(gshape, device=dev, dtype=torch.float32)
    g[:, t0:] = -0.1 * torch.rand(g[:, t0:].shape, generator=gen, device=dev)
    beta = torch.zeros(1, T, HV, device=dev, dtype=torch.float32)
    beta[:, t0:] = torch.rand(1, W, HV, generator=gen, device=dev)
    s0 = 0.1 * torch.randn(1, HV, K, V, generator=gen, device=dev)
    scale = K ** -0.5

    prob = gpu_lib.problem(1, T, H, HV, K, V, per_channel=per_channel, scale=scale, chunk=chunk)
    print(f"scan segments: {gpu_lib.scan_segments(prob)}, workspace "
          f"{gpu_lib.workspace_size(prob) / 2**30:.1f} GiB", flush=True)
    o, s = gpu_lib.gdr_chunk_fwd(q, k, v, g, beta, s0, chunk=chunk, scale=scale)
    torch.cuda.synchronize()

    def host(x):
        return x.float().cpu().numpy().astype(np.float64)

    # before the window: o_t = scale S0^T q_t exactly
    idx = torch.from_numpy(_samples()).to(dev)
    qs = host(q[0].index_select(0, idx))                # [n, H, K]
    os_ = host(o[0].index_select(0, idx))               # [n, HV, V]
    ref = scale * np.einsum("thk,hkv->thv", qs, host(s0[0]))
    e_pre = rel_err(os_, ref)
    assert np.isfinite(os_).all()

    # the window: the recurrence over its W tokens from S0
    ro, rs = oracle.recurrence(host(q[:, t0:]), host(k[:, t0:]), host(v[:, t0:]),
                               host(g[:, t0:]), host(beta[:, t0:]), scale, host(s0))
    go, gs = host(o[:, t0:]), host(s)
    e_o, e_s = rel_err(go, ro), rel_err(gs, rs)
    print(f"err_pre={e_pre:.3e} err_o_window={e_o:.3e} err_S={e_s:.3e} (tol {TOL['bf16']})",
          flush=True)
    del q, k, v, g, beta, o, s, s0
    torch.cuda.empty_cache()
    assert np.isfinite(go).all() and np.isfinite(gs).all()
    assert e_pre <= TOL["bf16"], e_pre
    assert e_o <= TOL["bf16"], e_o
    assert e_s <= TOL["bf16"], e_s
