#!/usr/bin/env python3
"""Throughput of the chunkwise gated delta rule forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one forward pass over one batch of the workload: the chunk-prep
kernel then the state-scan kernel (exactly the launch sequence of
gdr_chunk_fwd, issued through the two stage entry points so that HIP events
can bracket each kernel on the stream they run on).  Inputs are resident in
HBM before the timed region; the step rotates through several copies of the
inputs and outputs so that no step finds its data in the 256 MB last-level
cache.  Prints one JSON line.

Workload (default): the largest single-GPU configuration, grouped heads with
an initial state: B=2, T=16000, H=16 q/k heads, HV=32 value heads,
K=V=128, chunk 64, scalar decay, bf16 q/k/v, fp32 g/beta/initial state/o/
final state.  The other workloads run with --workload NAME.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

WORKLOAD_DEFAULT = "gqa_bf16_B2_T16000_H16_HV32_D128"
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, GB/s
MFMA_F16_PEAK_TFLOPS = 2500.0   # dense fp16/bf16 MFMA
MFMA_F32_PEAK_TFLOPS = 157.3


def traffic_model(w):
    """Bytes per launch of each stage and of the whole method.

    compulsory: the method's own inputs and outputs, each counted once (q/k
    once per q/k head, o in fp32, the states): for the path, for the prep
    stage (q, k, g, beta) and for the scan stage (q, k, v, o and the states).
    design: what each stage of this implementation is built to move, i.e.
    the compulsory bytes plus the workspace the prep kernel hands to the
    scan kernel: W^, the compact A^, the row scalars and the fragment-order
    q/k copies (per q/k head with one decay per row, per value head with
    per-channel decay), which the scan reads in place of q and k.
    """
    C = w.chunk
    N = -(-w.T // C)
    nch = w.B * w.HV * N
    tok = w.B * w.T
    es = 4 if w.dtype == "fp32" else 2          # q/k/v element
    wes = es                                    # workspace fragment element
    qk = 2 * tok * w.H * w.K * es
    v = tok * w.HV * w.V * es
    g = tok * w.HV * (w.K if w.per_channel else 1) * 4
    beta = tok * w.HV * 4
    o = tok * w.HV * w.V * 4
    state = w.B * w.HV * w.K * w.V * 4
    s0 = state if w.s0_std > 0 else 0
    ah_frags = (C // 16) * (C // 16 + 2) // 4        # lower-triangular A^ fragments
    rs = (C + (w.K if w.per_channel else 1)) * 4      # row scalars written and read
    ws = nch * (C * w.K * wes + ah_frags * 512 * wes + rs)
    qkh = 2 * (nch if w.per_channel else w.B * w.H * N) * C * w.K * wes
    design = dict(chunk_prep=qk + g + beta + ws + qkh,
                  state_scan=qkh + v + ws + s0 + o + state)
    stage = dict(chunk_prep=qk + g + beta, state_scan=qk + v + o + s0 + state)
    compulsory = qk + v + g + beta + o + s0 + state
    return dict(design=design, stage=stage, compulsory=compulsory)


def algorithmic_flops(w):
    """2 x MACs of the chunk algorithm (lower triangles only, no dense C x C work)."""
    C, K, V, G = w.chunk, w.K, w.V, w.HV // w.H
    mac = (((C - 1) / 2 * K + (C + 1) / 2 * K) / G + (C - 1) / 2 * (K + V) + 3 * K * V
           + (C + 1) / 2 * V)
    return 2.0 * mac * w.B * w.T * w.HV


ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "chunkwise_gated_delta_cumsum_amd", "csrc")


def kernel_sources_sha256():
    """Hash of the HIP sources, to tell whether stored counters still apply."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".hpp")):
            h.update(name.encode())
            h.update(open(os.path.join(CSRC, name), "rb").read())
    return h.hexdigest()


# the bench settings the stored counters were taken with (bench.py's defaults)
COUNTER_SETTING = {"rule": "delta", "chunk": 64, "segments": 0, "slab": 0}


def _counter_record(w, setting):
    """The stored rocprofv3 counter record of a workload, or None when there is
    none, the kernels changed since it was taken, or this run's settings
    (rule, chunk length, forced segments or slab) differ from its own."""
    path = os.path.join(ROOT, "profiles", f"counters_{w.name}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("sources_sha256") != kernel_sources_sha256():
        return None
    if rec.get("setting", COUNTER_SETTING) != setting:
        return None
    return rec


def measured_traffic(w, stage_kernels, setting=COUNTER_SETTING):
    """HBM bytes per launch of a stage from the stored rocprofv3 FETCH_SIZE and
    WRITE_SIZE counts (already scaled by the plain-copy calibration), or None
    (see _counter_record)."""
    rec = _counter_record(w, setting)
    if rec is None:
        return None
    total = 0.0
    found = False
    for name, v in rec["kernels"].items():
        if any(s in name for s in stage_kernels):
            total += v["fetch_bytes"] + v["write_bytes"]
            found = True
    return total if found else None


def measured_mfma(w, setting=COUNTER_SETTING):
    """MFMA busy fraction per kernel from the stored rocprofv3 counters
    (SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE x compute units), or None
    (see _counter_record)."""
    rec = _counter_record(w, setting)
    if rec is None:
        return None
    out = {name: v["mfma_busy_frac"] for name, v in rec["kernels"].items()
           if "mfma_busy_frac" in v}
    return out or None


class Ranges:
    """roctx ranges (torch.cuda.nvtx is roctx on ROCm) around launches, when
    enabled: ``with ranges(name):`` pushes the range before the launch and
    pops it after.  Host-side marks only; used outside the timed steps."""

    def __init__(self, enabled):
        self.enabled = enabled

    def __call__(self, name, active=True):
        import contextlib
        if not (self.enabled and active):
            return contextlib.nullcontext()
        import torch

        @contextlib.contextmanager
        def rng():
            torch.cuda.nvtx.range_push(name)
            try:
                yield
            finally:
                torch.cuda.nvtx.range_pop()
        return rng()


# the small workloads whose oracle time is also reported on one thread
SINGLE_THREAD_BASELINE = ("tiny_fp32_T256_H2_D64", "gdn_bf16_T4096_H12_D128")


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def usable_cores():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    omp = os.environ.get("OMP_NUM_THREADS", "")
    return min(n, int(omp)) if omp.isdigit() and int(omp) > 0 else n


# Parity bound of the GPU result against the oracle, max |delta| / rms(ref)
# (the 16-bit bound covers the fp16 MFMA operands; fp32 inputs keep fp32).
PARITY_TOL = {"fp32": 1e-3, "bf16": 2e-2, "fp16": 2e-2}


def _rel_err(x, ref):
    import numpy as np
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt((ref ** 2).mean()))
    d = float(np.abs(x - ref).max()) if x.size else 0.0
    return d / rms if rms > 0 else d


def cpu_baseline(inp, budget_s, rule="delta", single_thread=False, gpu_out=None,
                 gpu_what="o of a timed call"):
    """The fp64 oracle recurrence on the host cores, over a bounded sample of
    the workload: all (batch, value head) scans over a token prefix sized to
    about budget_s / 2 seconds per pass, repeated to about budget_s.  Reports
    the median pass as tokens/s, with the fastest pass, the thread count and
    the CPU model; with single_thread, also one thread on a short prefix.

    gpu_out(Ts) -> (o [B, Ts, HV, V], final state or None) gives the GPU's
    result (``gpu_what``) on the same prefix (o is causal, so the prefix of
    the full sequence's o is the prefix's o; the final state only where the
    prefix is the whole sequence): it is compared with the last pass's
    result under ``parity``."""
    import oracle
    w = inp.w
    threads = min(usable_cores(), w.B * w.HV)
    last = {}

    def run(Ts, nthreads):
        t0 = time.perf_counter()
        last["res"] = oracle.recurrence(inp.q[:, :Ts], inp.k[:, :Ts], inp.v[:, :Ts],
                                        inp.g[:, :Ts], inp.beta[:, :Ts], inp.scale, inp.s0,
                                        threads=nthreads, rule=rule)
        return time.perf_counter() - t0

    probe_T = min(w.T, 256)
    rate = probe_T / max(run(probe_T, threads), 1e-9)          # token positions / s
    Ts = min(w.T, max(probe_T, int(rate * budget_s / 2)))
    times = []
    while sum(times) < budget_s * 0.5 or len(times) < 2:
        times.append(run(Ts, threads))
    times.sort()
    med = times[len(times) // 2] if len(times) % 2 else 0.5 * (times[len(times) // 2 - 1] +
                                                              times[len(times) // 2])
    rec = {"value": w.B * Ts / med, "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "min_time_value": w.B * Ts / times[0], "cpu_model": cpu_model(),
           "sample": (f"fp64 {rule}-rule recurrence (C, -O2, OpenMP over scans) on all "
                      f"{w.B * w.HV} (batch, value head) scans, "
                      f"{'all' if Ts == w.T else 'first'} {Ts} of {w.T} tokens, "
                      f"{len(times)} passes, median {med:.2f} s, min {times[0]:.2f} s")}
    if gpu_out is not None:
        ro, rs = last["res"]
        o_gpu, s_gpu = gpu_out(Ts)
        tol = PARITY_TOL[w.dtype]
        err_o = _rel_err(o_gpu, ro)
        err_s = None if s_gpu is None else _rel_err(s_gpu, rs)
        rec["parity"] = {
            "what": ("max |GPU - oracle| / rms(oracle) over every (batch, value head) scan, "
                     f"on {gpu_what}" + (" and its final state" if s_gpu is not None
                                          else "") + f", first {Ts} of {w.T} tokens"),
            "err_o": err_o, "err_state": err_s, "tol": tol,
            "pass": bool(err_o <= tol and (err_s is None or err_s <= tol))}
        last.clear()
    if single_thread:
        T1 = min(w.T, 256)
        t1 = sorted(run(T1, 1) for _ in range(3))[1]
        rec["single_thread"] = {"value": w.B * T1 / t1, "unit": "tokens/s",
                                "sample": f"first {T1} tokens, median of 3 passes, {t1:.3f} s"}
    return rec


def decode_traffic(w):
    """Algorithmic bytes of one decode step: the state read and written once,
    the token's q, k (per q/k head), v, g, beta read and o written."""
    es = 4 if w.dtype == "fp32" else 2
    heads = w.B * w.HV
    state = heads * w.K * w.V * 4
    vec = (2 * w.B * w.H * w.K * es + heads * w.V * es
           + heads * (w.K if w.per_channel else 1) * 4 + heads * 4 + heads * w.V * 4)
    return 2 * state + vec


def bench_decode(args, w, inp):
    """Decode steps (one token per sequence, state updated in place), each
    one launch of the decode kernel over the whole batch."""
    import numpy as np
    import torch
    import chunkwise_gated_delta_cumsum_amd as gdr

    from chunkwise_gated_delta_cumsum_amd.inputs import workload
    half = torch.float16 if w.dtype == "fp16" else torch.bfloat16

    def to_dev(a):
        if a.dtype == np.uint16:          # 16-bit storage: bf16 or fp16 bits
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(half).cuda()
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    tok = dict(q=to_dev(inp.q_dev[:, 0]), k=to_dev(inp.k_dev[:, 0]), v=to_dev(inp.v_dev[:, 0]),
               g=to_dev(inp.g[:, 0]), beta=to_dev(inp.beta[:, 0]))
    s0 = to_dev(inp.s0)
    per_set = 2 * s0.numel() * 4
    nsets = args.sets or max(2, -(-(640 << 20) // per_set))
    sets = []
    for i in range(nsets):
        d = {k_: (t if i == 0 else t.clone()) for k_, t in tok.items()}
        d["s"] = s0.clone()
        d["o"] = torch.empty((w.B, w.HV, w.V), dtype=torch.float32, device="cuda")
        sets.append(d)

    def step(d):
        gdr.gdr_decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s"], scale=inp.scale,
                            out=(d["o"], d["s"]), slab=args.slab, rule=args.rule)

    for i in range(args.warmup):
        step(sets[i % nsets])
    K = args.steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(sets[i % nsets])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # the kernel's launch duration: back-to-back launches between one pair of
    # events on the launch stream
    KI = max(K, 20)
    a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ranges = Ranges(args.trace)
    a0.record()
    for i in range(KI):
        with ranges("decode_step"):
            step(sets[i % nsets])
    a1.record()
    torch.cuda.synchronize()
    kernel_ms = a0.elapsed_time(a1) / KI
    nbytes = decode_traffic(w)
    achieved = nbytes / (kernel_ms * 1e-3) / 1e9
    ms_per_step = elapsed / K * 1e3
    rec = {
        "metric": "tokens/sec of gated-delta-rule decode step at 1 GPU; % HBM roofline",
        "value": w.B / (elapsed / K),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "T": 1, "H": w.H, "HV": w.HV, "K": w.K,
                   "V": w.V, "decay": "per-channel" if w.per_channel else "scalar",
                   "inputs": w.dtype, "state": "fp32, updated in place",
                   "columns_per_workgroup": args.slab or "auto", "rule": args.rule,
                   "rotating_sets": nsets},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic(w, ("decode_step_kernel",), {
                         **COUNTER_SETTING, "rule": args.rule, "slab": args.slab,
                         **({"dtype": w.dtype} if w.dtype != workload(args.workload).dtype
                            else {})}),
                     "kernel": "decode_step", "kernels": ["decode_step_kernel"],
                     "algorithmic_bytes": nbytes, "kernel_ms": {"decode_step": kernel_ms}},
    }
    if not args.no_cpu_baseline:
        # one more step in the timed configuration from the initial state
        d = sets[0]
        o1 = torch.empty_like(d["o"])
        s1 = torch.empty_like(s0)
        gdr.gdr_decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], s0, scale=inp.scale,
                            out=(o1, s1), slab=args.slab, rule=args.rule)
        torch.cuda.synchronize()
        rec["cpu_baseline"] = cpu_baseline(
            inp, args.cpu_budget, args.rule,
            gpu_out=lambda Ts: (o1.cpu().numpy()[:, None], s1.cpu().numpy()),
            gpu_what="o of one step in the timed configuration from the initial state")
    print(json.dumps(rec), flush=True)


def copy_calibration(mib, reps):
    """Plain device copy of known size, for scaling rocprof FETCH/WRITE_SIZE;
    also reports the copy's own rate (bytes read plus written per second), the
    HBM rate a plain streaming kernel reaches on this GPU."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    print(json.dumps({"calibration_copy_bytes": n * 4, "reps": reps, "ms_per_copy": ms,
                      "copy_GBps": 2 * n * 4 / (ms * 1e-3) / 1e9}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[1])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # 10 warmup steps (6 ms on the grouped-head workload) left the timed mean
    # 3% above the per-step event median; from 100 on the two agree
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default=WORKLOAD_DEFAULT)
    ap.add_argument("--config", type=int, default=-1,
                    help="the workload by its index in the workload table (0-4: tiny fp32, "
                         "4096 tokens, per channel, grouped heads, 65536 tokens); "
                         "overrides --workload")
    ap.add_argument("--trace", action="store_true",
                    help="roctx ranges around each stage of the untimed per-stage run "
                         "(chunk_prep, state_scan; decode_step), for rocprofv3 --marker-trace")
    ap.add_argument("--sets", type=int, default=0,
                    help="rotating input/output copies (0: enough to exceed 640 MiB)")
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--chunk", type=int, default=0, choices=(0, 32, 64, 128),
                    help="chunk length (0: the workload's, 64)")
    ap.add_argument("--dtype", default="", choices=("", "bf16", "fp16", "fp32"),
                    help="storage type of q, k, v (default: the workload's)")
    ap.add_argument("--seed", type=int, default=-1,
                    help="seed of the synthetic inputs (default: the workload's)")
    ap.add_argument("--segments", type=int, default=0,
                    help="sequence segments of the state scan (0: the library's choice)")
    ap.add_argument("--slab", type=int, default=0, choices=(0, 32, 64, 128),
                    help="state columns per scan (32, 64) or decode (32, 64, 128) "
                         "workgroup (0: the library's choice)")
    ap.add_argument("--rule", default="delta", choices=("delta", "linear"),
                    help="state update: gated delta rule, or decayed linear attention "
                         "(no erase term)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="only run a plain copy of this many MiB (counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this library runs the forward pass on one GPU; there is no "
              "multi-GPU path to measure (independent heads and batches would shard "
              "across GPUs with no communication).  Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.calib_copy_mib:
        copy_calibration(args.calib_copy_mib, max(args.steps, 1))
        return

    import chunkwise_gated_delta_cumsum_amd as gdr
    from chunkwise_gated_delta_cumsum_amd.inputs import make_inputs, workload

    gdr.load()
    if args.config >= 0:
        args.workload = workload(args.config).name
    w = workload(args.workload)
    own_dtype = w.dtype
    if args.chunk:
        w = w.with_(chunk=args.chunk)
    if args.dtype:
        w = w.with_(dtype=args.dtype)
    if args.seed >= 0:
        w = w.with_(seed=args.seed)
    inp = make_inputs(w)
    if w.T == 1:
        bench_decode(args, w, inp)
        return
    dev = torch.device("cuda", 0)

    half = torch.float16 if w.dtype == "fp16" else torch.bfloat16

    def to_dev(a):
        import numpy as np
        if a.dtype == np.uint16:          # 16-bit storage: bf16 or fp16 bits
            return torch.from_numpy(a.view(np.int16)).view(half).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    base = dict(q=to_dev(inp.q_dev), k=to_dev(inp.k_dev), v=to_dev(inp.v_dev),
                g=to_dev(inp.g), beta=to_dev(inp.beta),
                s0=None if inp.s0 is None else to_dev(inp.s0))
    prob = gdr.problem(w.B, w.T, w.H, w.HV, w.K, w.V, chunk=w.chunk,
                       per_channel=w.per_channel, scale=inp.scale, dtype=w.dtype,
                       segments=args.segments, slab=args.slab, rule=args.rule)
    knobs = dict(segments=args.segments, slab=args.slab, rule=args.rule)
    ws_bytes = gdr.workspace_size(prob)
    per_set = sum(t.numel() * t.element_size() for t in base.values() if t is not None)
    per_set += ws_bytes + w.B * w.T * w.HV * w.V * 4 + w.B * w.HV * w.K * w.V * 4
    nsets = args.sets or max(1, -(-(640 << 20) // per_set))
    sets = []
    for i in range(nsets):
        d = base if i == 0 else {k_: (None if t is None else t.clone()) for k_, t in base.items()}
        d = dict(d)
        d["ws"] = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        d["o"] = torch.empty((w.B, w.T, w.HV, w.V), dtype=torch.float32, device=dev)
        d["sT"] = torch.empty((w.B, w.HV, w.K, w.V), dtype=torch.float32, device=dev)
        sets.append(d)

    ranges = Ranges(args.trace)

    def step(d, e0=None, e1=None, e2=None):
        if e0 is not None:
            e0.record()
        with ranges("chunk_prep", e0 is not None):
            gdr.gdr_chunk_prep(d["q"], d["k"], d["g"], d["beta"], chunk=w.chunk,
                               scale=inp.scale, V=w.V, workspace=d["ws"], **knobs)
        if e1 is not None:
            e1.record()
        with ranges("state_scan", e0 is not None):
            gdr.gdr_chunk_scan(d["q"], d["k"], d["v"], d["g"], d["beta"], d["ws"], d["s0"],
                               chunk=w.chunk, scale=inp.scale, out=(d["o"], d["sT"]), **knobs)
        if e2 is not None:
            e2.record()

    for i in range(args.warmup):
        step(sets[i % nsets])
    K = args.steps
    # the timed steps carry no events of their own: an event recorded between
    # two launches costs the stream several microseconds
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(sets[i % nsets])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # the split of a step between the two stages, from a separate untimed run
    # of the same steps with events around each stage
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    for i in range(K):
        step(sets[i % nsets], *evs[i])
    torch.cuda.synchronize()
    step_prep_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / K
    step_scan_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / K
    # per-step durations of that run (events on the launch stream), for the
    # median and fastest step beside the timed mean
    step_each = sorted(e[0].elapsed_time(e[2]) for e in evs)

    # Per-stage launch durations: each stage alone, launched back to back over
    # the rotating sets between one pair of events on the launch stream (the
    # per-step events above also count the launch gaps inside a step).
    def stage_ms(fn):
        KI = max(K, 20)
        for i in range(3):
            fn(sets[i % nsets])
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record()
        for i in range(KI):
            fn(sets[i % nsets])
        a1.record()
        torch.cuda.synchronize()
        return a0.elapsed_time(a1) / KI

    prep_ms = stage_ms(lambda d: gdr.gdr_chunk_prep(d["q"], d["k"], d["g"], d["beta"], chunk=w.chunk,
                                                   scale=inp.scale, V=w.V, workspace=d["ws"],
                                                   **knobs))
    scan_ms = stage_ms(lambda d: gdr.gdr_chunk_scan(d["q"], d["k"], d["v"], d["g"], d["beta"],
                                                   d["ws"], d["s0"], chunk=w.chunk, scale=inp.scale,
                                                   out=(d["o"], d["sT"]), **knobs))

    # the path check: one more pass through the single-call entry point
    d = sets[0]
    o_ref = d["o"].clone()
    gdr.gdr_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"], chunk=w.chunk,
                      scale=inp.scale, workspace=d["ws"], out=(d["o"], d["sT"]), **knobs)
    torch.cuda.synchronize()
    same = bool(torch.equal(o_ref, d["o"]))

    tm = traffic_model(w)
    # the two stages of the path; the scan stage is up to two kernels (chain
    # pass, then the full pass that also combines the segment transitions)
    # launched by one gdr_chunk_scan call
    stages = {"chunk_prep": (prep_ms, ("chunk_prep",)),
              "state_scan": (scan_ms, ("chunk_scan_kernel",))}
    dom = max(stages, key=lambda k_: stages[k_][0])
    dom_ms, dom_kernels = stages[dom]
    dom_bytes = tm["stage"][dom]
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    setting = {"rule": args.rule, "chunk": w.chunk, "segments": args.segments, "slab": args.slab}
    if w.dtype != own_dtype:   # the stored counters were taken in the workload's own dtype
        setting["dtype"] = w.dtype
    traffic = measured_traffic(w, dom_kernels, setting)
    nseg = gdr.scan_segments(prob)
    slab = gdr.scan_slab(prob)
    ms_per_step = elapsed / K * 1e3
    tokens = w.B * w.T
    flops = algorithmic_flops(w)
    mfma_peak = MFMA_F32_PEAK_TFLOPS if w.dtype == "fp32" else MFMA_F16_PEAK_TFLOPS

    rec = {
        "metric": "tokens/sec of chunked gated-delta-rule fwd at 1 GPU; % HBM/MFMA roofline",
        "value": tokens / (elapsed / K),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "T": w.T, "H": w.H, "HV": w.HV, "K": w.K,
                   "V": w.V, "chunk": w.chunk,
                   "decay": "per-channel" if w.per_channel else "scalar",
                   "inputs": w.dtype, "initial_state": w.s0_std > 0,
                   "compute": ("fp32 MFMA" if w.dtype == "fp32" else
                               "fp16 MFMA operands (exact for bf16 inputs), fp32 accumulation")
                              + ", fp32 state, gamma and o",
                   "rotating_sets": nsets, "rule": args.rule},
        # roofline of the dominant stage: the method's compulsory bytes that
        # stage must move (its inputs read once, its outputs written once)
        # over its launch duration; the whole path's fraction beside it, and
        # the fraction on the bytes this implementation is built to move
        # (compulsory plus the prep-to-scan workspace) under its own name
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic, "kernel": dom,
                     "kernels": list(dom_kernels), "algorithmic_bytes": dom_bytes,
                     "kernel_ms": {"chunk_prep": prep_ms, "state_scan": scan_ms},
                     "step_stage_ms": {"chunk_prep": step_prep_ms, "state_scan": step_scan_ms},
                     "scan_segments": nseg, "scan_slab": slab,
                     "path_compulsory_bytes": tm["compulsory"],
                     "path_hbm_frac": tm["compulsory"] / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
                     "path_mfma_frac": flops / (ms_per_step * 1e-3) / 1e12 / mfma_peak,
                     "design_bytes": tm["design"][dom],
                     "design_bytes_frac": tm["design"][dom] / (dom_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                     "mfma_busy": measured_mfma(w, setting)},
        "fwd_entry_point_matches": same,
        # the same steps one by one with events around each (a separate,
        # untimed run): median and fastest step, and the tokens/s and path
        # fraction of the median step
        "step_events": {"median_ms": step_each[len(step_each) // 2], "min_ms": step_each[0],
                        "tokens_per_s_median": tokens / (step_each[len(step_each) // 2] * 1e-3),
                        "path_hbm_frac_median": tm["compulsory"] / (
                            step_each[len(step_each) // 2] * 1e-3) / 1e9 / HBM_PEAK_GBS},
    }
    if not args.no_cpu_baseline:
        d = sets[0]   # o and the final state of the path check above
        rec["cpu_baseline"] = cpu_baseline(
            inp, args.cpu_budget, args.rule, single_thread=w.name in SINGLE_THREAD_BASELINE,
            gpu_out=lambda Ts: (d["o"][:, :Ts].cpu().numpy(),
                                d["sT"].cpu().numpy() if Ts == w.T else None))
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
