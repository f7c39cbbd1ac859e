"""Shared helpers for the GPU tests: device copies of generated inputs and the
parity metric.  The metric is the one the method's accuracy target uses:
max |x_gpu - x_ref| / sqrt(mean(x_ref^2)) over all valid elements."""
from __future__ import annotations

import numpy as np

# max|delta| / rms(ref) bounds for o and the final state
TOL = {"fp32": 1e-3, "bf16": 2e-2, "fp16": 2e-2}


def rel_err(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert x.shape == ref.shape, (x.shape, ref.shape)
    rms = np.sqrt((ref ** 2).mean())
    if rms == 0:
        return float(np.abs(x).max())
    return float(np.abs(x - ref).max() / rms)


def rel_err_rows(o, s, ro, rs):
    """The same metric taken row by row: the final state per (batch, value
    head, key channel) row and o per token, each against the rms of its own
    reference row (the worst row is returned for each).  For decays above 1
    per key channel the state's channel rows grow at different rates, as the
    exp of each channel's own decay sum, so their magnitudes spread over
    orders and max|delta| / rms over the whole tensor compares the error of
    the largest rows with the rms of all; per row, every value is compared
    with values of its own scale."""
    o, s, ro, rs = (np.asarray(x, dtype=np.float64) for x in (o, s, ro, rs))
    ds = np.abs(s - rs).max(axis=-1) / np.sqrt((rs ** 2).mean(axis=-1))
    do = np.abs(o - ro).max(axis=(0, 2, 3)) / np.sqrt((ro ** 2).mean(axis=(0, 2, 3)))
    return float(do.max()), float(ds.max())


def to_device(inp, device="cuda"):
    """torch tensors on `device` holding exactly the generated values."""
    import torch

    half = torch.float16 if inp.w.dtype == "fp16" else torch.bfloat16

    def dev(a):
        if a.dtype == np.uint16:          # 16-bit storage: bf16 or fp16 bits
            return torch.from_numpy(a.view(np.int16)).view(half).to(device)
        return torch.from_numpy(np.ascontiguousarray(a)).to(device)

    s0 = None if inp.s0 is None else dev(inp.s0)
    return dict(q=dev(inp.q_dev), k=dev(inp.k_dev), v=dev(inp.v_dev), g=dev(inp.g),
                beta=dev(inp.beta), initial_state=s0)


def run_gpu(gdr, inp, **kw):
    import torch
    t = to_device(inp)
    o, s = gdr.gdr_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["initial_state"],
                             chunk=inp.w.chunk, scale=inp.scale, **kw)
    torch.cuda.synchronize()
    return o.cpu().numpy(), None if s is None else s.cpu().numpy()
