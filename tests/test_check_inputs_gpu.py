"""gdr_check_inputs on the GPU: the flags it sets against a host evaluation
of the same preconditions (include/gdr.h, numerics notes), bit for bit.

The host side states each precondition directly on the tensors' values:
non-finite values anywhere; bf16 q, k, v whose bits encode a magnitude of
65536 or more (fp16 overflow); with bf16 inputs, a chunk (of the problem's
chunk length) in which the positive g of one channel, or of the row decay,
sum to more than 8.  Planted values stay well away from the limit of 8, so
the device's fp32 sums and the host's fp64 sums cannot decide differently.
"""
import numpy as np
import pytest

from chunkwise_gated_delta_cumsum_amd.inputs import Workload, make_inputs
from helpers import to_device

pytestmark = pytest.mark.gpu

NONFINITE, RANGE, DECAY = 1, 2, 4


def host_flags(t, chunk=64, qk_l2norm=False):
    import torch
    bits = 0
    bf16 = t["q"].dtype == torch.bfloat16
    for name in ("q", "k", "v"):
        x = t[name].cpu()
        if bf16:
            u = x.view(torch.int16).numpy().view(np.uint16) & 0x7FFF
            if (u >= 0x7F80).any():
                bits |= NONFINITE
            if (name == "v" or not qk_l2norm) and ((u >= 0x4780) & (u < 0x7F80)).any():
                bits |= RANGE
        elif not torch.isfinite(x).all():
            bits |= NONFINITE
    g = t["g"].cpu().numpy().astype(np.float64)
    beta = t["beta"].cpu().numpy()
    if not (np.isfinite(g).all() and np.isfinite(beta).all()):
        bits |= NONFINITE
    if bf16:
        B, T = g.shape[:2]
        N = -(-T // chunk)
        pos = np.zeros((B, N * chunk) + g.shape[2:])
        pos[:, :T] = np.fmax(g, 0.0)
        sums = pos.reshape((B, N, chunk) + g.shape[2:]).sum(axis=2)
        if (sums > 8.0).any():
            bits |= DECAY
    return bits


def device_flags(gdr, t, chunk=0, qk_l2norm=False, flags=None):
    f = gdr.gdr_check_inputs(t["q"], t["k"], t["v"], t["g"], t["beta"], chunk=chunk,
                             qk_l2norm=qk_l2norm, flags=flags)
    return int(f[0].item())


def small(per_channel=False, dtype="bf16", T=130, B=2, H=2, HV=4, seed=5):
    return Workload("check", B=B, T=T, H=H, HV=HV, K=128, V=128, per_channel=per_channel,
                    dtype=dtype, g_mu=3.0, s0_std=0.0, seed=seed)


CLEAN = [dict(), dict(per_channel=True), dict(T=1), dict(T=64), dict(T=300, per_channel=True),
         dict(dtype="fp32"), dict(dtype="fp32", per_channel=True, T=77)]


@pytest.mark.parametrize("kw", CLEAN, ids=[str(i) for i in range(len(CLEAN))])
def test_generated_inputs_are_clean(gpu_lib, kw):
    t = to_device(make_inputs(small(**kw)))
    print(f"clean inputs {kw}", flush=True)
    assert host_flags(t) == 0
    assert device_flags(gpu_lib, t) == 0


def _set(name, idx, value):
    def f(t):
        t[name][idx] = value
    return f


PLANTED = [
    ("q just below fp16 max", dict(), _set("q", (0, 5, 1, 7), 65280.0), 0),
    ("q past fp16 max", dict(), _set("q", (0, 5, 1, 7), 65536.0), RANGE),
    ("k past fp16 max", dict(), _set("k", (1, 129, 0, 127), -70000.0), RANGE),
    ("v past fp16 max", dict(), _set("v", (1, 3, 3, 0), 1e6), RANGE),
    ("q inf", dict(), _set("q", (0, 0, 0, 0), float("inf")), NONFINITE),
    ("v nan", dict(), _set("v", (1, 129, 3, 127), float("nan")), NONFINITE),
    ("beta nan", dict(), _set("beta", (1, 77, 2), float("nan")), NONFINITE),
    ("g inf", dict(), _set("g", (0, 64, 1), float("inf")), NONFINITE | DECAY),
    ("g -inf", dict(), _set("g", (0, 64, 1), float("-inf")), NONFINITE),
    ("row decay 0.3 x 32 rows", dict(), _set("g", (1, slice(70, 102), 2), 0.3), DECAY),
    ("row decay 0.1 x 64 rows", dict(), _set("g", (1, slice(64, 128), 2), 0.1), 0),
    ("channel decay 0.3 x 32 rows", dict(per_channel=True),
     _set("g", (0, slice(0, 32), 3, 77), 0.3), DECAY),
    ("channel decay in the ragged tail", dict(per_channel=True, T=150),
     _set("g", (1, slice(130, 150), 0, 5), 0.5), DECAY),
    ("channel decay spread over two chunks", dict(per_channel=True),
     _set("g", (0, slice(44, 84), 3, 77), 0.3), 0),
    ("fp32: large q, positive g", dict(dtype="fp32"),
     lambda t: (_set("q", (0, 5, 1, 7), 1e6)(t), _set("g", (1, slice(0, 64), 2), 1.0)(t)), 0),
    ("fp32: nan k", dict(dtype="fp32"), _set("k", (1, 100, 1, 9), float("nan")), NONFINITE),
]


@pytest.mark.parametrize("name,kw,plant,bits", PLANTED, ids=[p[0] for p in PLANTED])
def test_planted_violations(gpu_lib, name, kw, plant, bits):
    t = to_device(make_inputs(small(**kw)))
    plant(t)
    print(f"planted: {name}", flush=True)
    assert host_flags(t) == bits
    assert device_flags(gpu_lib, t) == bits


def test_l2norm_exempts_q_and_k(gpu_lib):
    t = to_device(make_inputs(small()))
    t["q"][0, 5, 1, 7] = 70000.0
    assert device_flags(gpu_lib, t, qk_l2norm=False) == RANGE
    assert device_flags(gpu_lib, t, qk_l2norm=True) == 0
    t["v"][0, 5, 1, 7] = 70000.0
    assert device_flags(gpu_lib, t, qk_l2norm=True) == RANGE


@pytest.mark.parametrize("chunk,bits", [(32, 0), (64, DECAY), (128, DECAY)])
def test_decay_bound_follows_the_chunk_length(gpu_lib, chunk, bits):
    # 0.3 on rows 24..55: one 64-row chunk sums 9.6; at 32 rows it splits 2.4 + 7.2
    t = to_device(make_inputs(small(per_channel=True)))
    t["g"][1, 24:56, 2, 100] = 0.3
    assert host_flags(t, chunk=chunk) == bits
    assert device_flags(gpu_lib, t, chunk=chunk) == bits


def test_flags_word_is_cleared_by_each_call(gpu_lib):
    import torch
    flags = torch.full((1,), 0x7F, dtype=torch.int32, device="cuda")
    t = to_device(make_inputs(small()))
    assert device_flags(gpu_lib, t, flags=flags) == 0
    t["v"][0, 0, 0, 0] = float("nan")
    assert device_flags(gpu_lib, t, flags=flags) == NONFINITE
    t["v"][0, 0, 0, 0] = 0.0
    assert device_flags(gpu_lib, t, flags=flags) == 0


def test_full_size_last_elements(gpu_lib):
    """The grouped-head workload at full size (B2 T16000 H16 HV32): clean, then
    a violation in the last element of v, of k, and in the last chunk of g."""
    w = Workload("gqa_check", B=2, T=16000, H=16, HV=32, K=128, V=128, g_mu=3.0,
                 s0_std=0.0, seed=11)
    t = to_device(make_inputs(w))
    print("full size: clean", flush=True)
    assert device_flags(gpu_lib, t) == 0
    t["v"][-1, -1, -1, -1] = float("nan")
    assert device_flags(gpu_lib, t) == NONFINITE
    t["v"][-1, -1, -1, -1] = 0.0
    t["k"][-1, -1, -1, -1] = 1e5
    assert device_flags(gpu_lib, t) == RANGE
    t["k"][-1, -1, -1, -1] = 0.0
    t["g"][-1, -20:, -1] = 0.5          # sums to 10 in the last 64-row chunk
    assert device_flags(gpu_lib, t) == DECAY
    assert host_flags(t) == DECAY
