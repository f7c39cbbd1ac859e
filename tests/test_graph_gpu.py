"""The entry points under HIP graph capture (torch.cuda.CUDAGraph on torch's
current stream, which the binding passes to the C ABI).

The library enqueues kernel launches only (no memsets, copies or
synchronisations), so a captured call must replay exactly what the eager call
computes.  Each replay runs with new contents in the captured input buffers,
with eager work and a synchronisation in between; every replay is compared
with an eager call on the same inputs (bit-exact: same kernels, same grids)
and the first one with the oracle as well.
"""
import numpy as np
import pytest

import oracle
from chunkwise_gated_delta_cumsum_amd.inputs import WORKLOADS, make_inputs
from helpers import TOL, rel_err, to_device

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _capture(fn):
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm-up outside the capture
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    torch.cuda.synchronize()
    return graph


CHUNK_CASES = [
    (WORKLOADS[3].with_(B=1, T=1000), 3),     # grouped heads, initial state, chain + full pass
    (WORKLOADS[2].with_(B=1, T=777), 0),      # per-channel decay
    (WORKLOADS[0].with_(T=300), 2),           # fp32
]


@pytest.mark.parametrize("w,segs", CHUNK_CASES, ids=[w.name for w, _ in CHUNK_CASES])
def test_chunk_fwd_graph_replays(gpu_lib, w, segs):
    import torch
    print(f"graph chunk_fwd: {w.name} B={w.B} T={w.T} segments={segs}", flush=True)
    static = to_device(make_inputs(w))
    prob = gpu_lib.problem(w.B, w.T, w.H, w.HV, w.K, w.V, per_channel=w.per_channel,
                           dtype=w.dtype, segments=segs)
    ws = torch.empty(gpu_lib.workspace_size(prob), dtype=torch.uint8, device="cuda")
    o = torch.empty((w.B, w.T, w.HV, w.V), dtype=torch.float32, device="cuda")
    s = torch.empty((w.B, w.HV, w.K, w.V), dtype=torch.float32, device="cuda")
    scale = w.K ** -0.5

    def args():
        return (static["q"], static["k"], static["v"], static["g"], static["beta"],
                static["initial_state"])

    graph = _capture(lambda: gpu_lib.gdr_chunk_fwd(*args(), chunk=w.chunk, scale=scale,
                                                   workspace=ws, out=(o, s), segments=segs))
    for rep in range(REPLAYS):
        inp = make_inputs(w.with_(seed=w.seed + 100 + rep))
        fresh = to_device(inp)
        for name, x in fresh.items():
            if x is not None:
                static[name].copy_(x)
        o.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        oe, se = gpu_lib.gdr_chunk_fwd(*args(), chunk=w.chunk, scale=scale, segments=segs)
        torch.cuda.synchronize()
        assert torch.equal(o, oe) and torch.equal(s, se), f"replay {rep} differs from eager"
        if rep == 0:
            ro, rs = oracle.recurrence(inp.q, inp.k, inp.v, inp.g, inp.beta, scale, inp.s0)
            eo, es = rel_err(o.cpu().numpy(), ro), rel_err(s.cpu().numpy(), rs)
            print(f"  replay 0 vs oracle: err_o={eo:.3e} err_S={es:.3e}", flush=True)
            assert eo <= TOL[w.dtype] and es <= TOL[w.dtype], (eo, es)


@pytest.mark.parametrize("w", [WORKLOADS[3].with_(B=2, T=8, s0_std=0.1),
                               WORKLOADS[2].with_(B=2, T=8, s0_std=0.1)], ids=["gqa", "kda"])
def test_decode_graph_replays(gpu_lib, w):
    """T decode steps captured as one graph, updating one state in place."""
    import torch
    print(f"graph decode: {w.name} B={w.B} steps={w.T}", flush=True)
    inp = make_inputs(w)
    t = to_device(inp)
    steps = [tuple(t[n][:, i].contiguous() for n in ("q", "k", "v", "g", "beta"))
             for i in range(w.T)]
    s_init = t["initial_state"]
    state = s_init.clone()
    outs = [torch.empty((w.B, w.HV, w.V), dtype=torch.float32, device="cuda") for _ in steps]
    scale = w.K ** -0.5

    def run(st, os_):
        for x, oi in zip(steps, os_):
            gpu_lib.gdr_decode_step(*x, st, scale=scale, out=(oi, st), inplace=True)

    graph = _capture(lambda: run(state, outs))
    for rep in range(REPLAYS):
        start = s_init * (1.0 + 0.5 * rep)
        state.copy_(start)
        for oi in outs:
            oi.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        se = start.clone()
        oe = [torch.empty_like(oi) for oi in outs]
        run(se, oe)
        torch.cuda.synchronize()
        assert torch.equal(state, se), f"replay {rep}: state differs from eager"
        assert all(torch.equal(a, b) for a, b in zip(outs, oe)), f"replay {rep}: o differs"
        if rep == 0:
            ro, rs = oracle.recurrence(inp.q, inp.k, inp.v, inp.g, inp.beta, scale, inp.s0)
            go = np.stack([oi.cpu().numpy() for oi in outs], axis=1)
            eo, es = rel_err(go, ro), rel_err(state.cpu().numpy(), rs)
            print(f"  replay 0 vs oracle: err_o={eo:.3e} err_S={es:.3e}", flush=True)
            assert eo <= TOL[w.dtype] and es <= TOL[w.dtype], (eo, es)
