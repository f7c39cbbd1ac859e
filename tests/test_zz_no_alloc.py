"""gdr_chunk_fwd_noalloc (the entry point without a workspace argument, on
the library's own device scratch array) against gdr_chunk_fwd, through the
C ABI: calls in a row on one GPU (the second with a smaller problem, the
third with per-channel decay and fp16 inputs), each equal to gdr_chunk_fwd
bit for bit and to the fp64 oracle within the bounds of the parity tests."""
import numpy as np
import pytest

import oracle
from chunkwise_gated_delta_cumsum_amd.inputs import WORKLOADS, make_inputs
from helpers import TOL, rel_err, to_device

pytestmark = pytest.mark.gpu


def _run_both(gdr, inp, **kw):
    import torch
    t = to_device(inp)
    args = (t["q"], t["k"], t["v"], t["g"], t["beta"], t["initial_state"])
    o1, s1 = gdr.gdr_chunk_fwd(*args, scale=inp.scale, **kw)
    o2 = torch.empty_like(o1)
    s2 = torch.empty_like(s1)
    gdr.gdr_chunk_fwd_noalloc(*args, scale=inp.scale, out=(o2, s2), **kw)
    torch.cuda.synchronize()
    return o1.cpu().numpy(), s1.cpu().numpy(), o2.cpu().numpy(), s2.cpu().numpy()


def test_noalloc_two_calls_match_chunk_fwd(gpu_lib):
    cases = [
        # the largest problem the scratch array takes: 4096 tokens, 12 heads,
        # a 6-segment scan (transitions and segment states in the scratch)
        (WORKLOADS[1], {}),
        # then a smaller one with grouped heads, an initial state and 3 segments
        (WORKLOADS[3].with_(B=1, T=700), dict(segments=3)),
        # and a third on the same array: per-channel decay, fp16 inputs, 2 segments
        (WORKLOADS[2].with_(B=1, T=300, dtype="fp16"), dict(segments=2)),
    ]
    for w, kw in cases:
        inp = make_inputs(w)
        prob = gpu_lib.problem(w.B, w.T, w.H, w.HV, w.K, w.V, per_channel=w.per_channel,
                               dtype=w.dtype, **kw)
        assert gpu_lib.workspace_size(prob) <= gpu_lib.NOALLOC_SCRATCH_BYTES
        o1, s1, o2, s2 = _run_both(gpu_lib, inp, **kw)
        assert np.array_equal(o1, o2) and np.array_equal(s1, s2), w.name
        ro, rs = oracle.recurrence(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.scale, inp.s0)
        eo, es = rel_err(o2, ro), rel_err(s2, rs)
        print(f"noalloc {w.name} {kw}: err_o={eo:.3e} err_S={es:.3e}", flush=True)
        assert eo <= TOL[w.dtype] and es <= TOL[w.dtype]


def test_noalloc_refuses_large_problem(gpu_lib):
    import torch
    w = WORKLOADS[3].with_(T=4096)
    prob = gpu_lib.problem(w.B, w.T, w.H, w.HV, w.K, w.V)
    assert gpu_lib.workspace_size(prob) > gpu_lib.NOALLOC_SCRATCH_BYTES
    inp = make_inputs(w)
    t = to_device(inp)
    with pytest.raises(gpu_lib.GdrError) as e:
        gpu_lib.gdr_chunk_fwd_noalloc(t["q"], t["k"], t["v"], t["g"], t["beta"],
                                      t["initial_state"], scale=inp.scale)
    assert e.value.name == "GDR_ERR_SCRATCH"
    torch.cuda.synchronize()


def test_noalloc_under_graph_capture(gpu_lib):
    """The callers the entry point is for: captured into a HIP graph with
    caller-owned outputs (nothing is allocated during the capture), replayed
    with new contents in the captured input buffers and eager work in
    between, each replay equal to gdr_chunk_fwd bit for bit."""
    import torch
    w = WORKLOADS[3].with_(B=1, T=700)
    static = to_device(make_inputs(w))
    o = torch.empty((w.B, w.T, w.HV, w.V), dtype=torch.float32, device="cuda")
    s = torch.empty((w.B, w.HV, w.K, w.V), dtype=torch.float32, device="cuda")
    scale = w.K ** -0.5

    def args():
        return (static["q"], static["k"], static["v"], static["g"], static["beta"],
                static["initial_state"])

    def call():
        gpu_lib.gdr_chunk_fwd_noalloc(*args(), scale=scale, out=(o, s), segments=3)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm-up outside the capture
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    for rep in range(3):
        fresh = to_device(make_inputs(w.with_(seed=w.seed + 200 + rep)))
        for name, x in fresh.items():
            if x is not None:
                static[name].copy_(x)
        o.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        oe, se = gpu_lib.gdr_chunk_fwd(*args(), scale=scale, segments=3)
        torch.cuda.synchronize()
        print(f"noalloc graph replay {rep}: equal {torch.equal(o, oe) and torch.equal(s, se)}",
              flush=True)
        assert torch.equal(o, oe) and torch.equal(s, se), rep
