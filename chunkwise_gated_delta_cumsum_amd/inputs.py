"""Seeded synthetic inputs for the chunkwise gated delta rule forward pass.

This module only draws random numbers and rounds them to the storage types the
device path consumes.  It holds none of the method's arithmetic, so both the
HIP path and the fp64 oracle can take their inputs from here.

Distributions follow the workloads the source pages describe (page "Chunkwise
parallel algorithms" / page "sec-03 chunkwise" notes, and the scalar-g
DeltaNet chunk kernel page, whose demo uses seed 42, normal q/k/v, sigmoid
beta and a state scaled by 0.1):

* q, k ~ N(0, 1) on [B, T, H, K], then each row is L2-normalised with
  x * rsqrt(sum(x^2) + 1e-6) (the normaliser of the scalar-g kernel page),
  unless the workload asks for raw rows (normalize_qk=False, for the
  in-kernel normalisation tests, where the rows are normalised on the
  device and in the oracle instead);
* v ~ N(0, 1) on [B, T, HV, V];
* beta = sigmoid(N(0, 1)) on [B, T, HV];
* g = logsigmoid(N(mu, 1)) on [B, T, HV] (one log-decay per value head) or on
  [B, T, HV, K] (one per key channel, the KDA form);
* initial state = std * N(0, 1) on [B, HV, K, V] when std > 0, else absent.

q, k and v are rounded once (round-to-nearest-even) to the storage dtype
("fp32", "bf16" or "fp16"); g, beta and the state are fp32.  Both sides then consume
exactly these rounded values (the oracle upcasts them to fp64).
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional

import numpy as np

__all__ = ["Workload", "WORKLOADS", "DECODE_WORKLOADS", "Inputs", "make_inputs", "workload",
           "bf16_round", "bf16_bits_to_f64"]


@dataclass(frozen=True)
class Workload:
    """One synthetic problem: shapes, decay form, dtype and distributions."""
    name: str
    B: int
    T: int
    H: int
    HV: int
    K: int
    V: int
    chunk: int = 64
    per_channel: bool = False
    dtype: str = "bf16"          # storage type of q, k, v: "fp32", "bf16" or "fp16"
    g_mu: float = 3.0            # g = logsigmoid(N(g_mu, 1))
    s0_std: float = 0.0          # 0 -> no initial state
    seed: int = 42
    normalize_qk: bool = True    # False: raw N(0, 1) q and k (for in-kernel normalisation)

    @property
    def G(self) -> int:
        return self.HV // self.H

    @property
    def tokens(self) -> int:
        return self.B * self.T

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads of the method's benchmark table: a tiny fp32 case, the
# 4096-token 12-head shape of the scalar-g kernel page's memory estimate, a
# per-channel (KDA) batch, a grouped-head batch with an initial state, and a
# 65536-token single sequence that stresses the serial inter-chunk scan.
WORKLOADS = (
    Workload("tiny_fp32_T256_H2_D64", B=1, T=256, H=2, HV=2, K=64, V=64,
             dtype="fp32", g_mu=3.0, seed=42),
    Workload("gdn_bf16_T4096_H12_D128", B=1, T=4096, H=12, HV=12, K=128,
             V=128, dtype="bf16", g_mu=3.0, seed=43),
    Workload("kda_bf16_B4_T8192_H16_D128", B=4, T=8192, H=16, HV=16, K=128,
             V=128, per_channel=True, dtype="bf16", g_mu=4.0, seed=44),
    Workload("gqa_bf16_B2_T16000_H16_HV32_D128", B=2, T=16000, H=16, HV=32,
             K=128, V=128, dtype="bf16", g_mu=3.0, s0_std=0.1, seed=45),
    Workload("long_bf16_T65536_H12_D128", B=1, T=65536, H=12, HV=12, K=128,
             V=128, dtype="bf16", g_mu=5.0, seed=46),
)


# Decode batches: one token per sequence (T = 1) against a state carried
# over from earlier tokens, drawn as 0.1 N(0, 1) like the grouped-head
# workload's initial state.  The shapes are the grouped-head and the
# per-channel workloads' heads at serving batch sizes.
DECODE_WORKLOADS = (
    Workload("decode_bf16_B64_H16_HV32_D128", B=64, T=1, H=16, HV=32, K=128, V=128,
             dtype="bf16", g_mu=3.0, s0_std=0.1, seed=47),
    Workload("decode_kda_bf16_B32_H16_D128", B=32, T=1, H=16, HV=16, K=128, V=128,
             per_channel=True, dtype="bf16", g_mu=4.0, s0_std=0.1, seed=48),
)


def workload(i_or_name) -> Workload:
    if isinstance(i_or_name, int):
        return WORKLOADS[i_or_name]
    for w in WORKLOADS + DECODE_WORKLOADS:
        if w.name == i_or_name:
            return w
    raise KeyError(i_or_name)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round to bfloat16 (nearest-even, via fp32) and return the raw uint16 bits."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    u = bits.astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


@dataclass
class Inputs:
    w: Workload
    # exact values the device consumes, upcast to fp64 (for the oracle)
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    g: np.ndarray                # fp32
    beta: np.ndarray             # fp32
    s0: Optional[np.ndarray]     # fp32 or None
    # raw device storage of q, k, v: float32 arrays or uint16 bf16 bits
    q_dev: np.ndarray
    k_dev: np.ndarray
    v_dev: np.ndarray

    @property
    def scale(self) -> float:
        return float(self.w.K) ** -0.5


def _l2norm_rows(x: np.ndarray) -> np.ndarray:
    return x / np.sqrt((x * x).sum(axis=-1, keepdims=True) + 1e-6)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return 0.5 * (1.0 + np.tanh(0.5 * x))


def _logsigmoid(x: np.ndarray) -> np.ndarray:
    return -np.logaddexp(0.0, -x)


def _store(x: np.ndarray, dtype: str):
    if dtype == "fp32":
        dev = np.ascontiguousarray(x, dtype=np.float32)
        return dev.astype(np.float64), dev
    if dtype == "bf16":
        bits = bf16_round(x)
        return bf16_bits_to_f64(bits), bits
    if dtype == "fp16":
        h = np.ascontiguousarray(x, dtype=np.float16)    # round to nearest even
        return h.astype(np.float64), h.view(np.uint16)
    raise ValueError(f"unknown dtype {dtype!r}")


def make_inputs(w: Workload, T: Optional[int] = None) -> Inputs:
    """Draw the inputs of workload ``w`` (optionally cut to the first T tokens).

    The draw order is fixed (q, k, v, beta, g, state) so a given seed always
    yields the same tensors; cutting T re-draws at the smaller shape.
    """
    if T is not None:
        w = w.with_(T=T)
    rng = np.random.default_rng(w.seed)
    B, T_, H, HV, K, V = w.B, w.T, w.H, w.HV, w.K, w.V
    q = rng.standard_normal((B, T_, H, K))
    k = rng.standard_normal((B, T_, H, K))
    if w.normalize_qk:
        q, k = _l2norm_rows(q), _l2norm_rows(k)
    v = rng.standard_normal((B, T_, HV, V))
    beta = _sigmoid(rng.standard_normal((B, T_, HV))).astype(np.float32)
    gshape = (B, T_, HV, K) if w.per_channel else (B, T_, HV)
    g = _logsigmoid(rng.normal(w.g_mu, 1.0, gshape)).astype(np.float32)
    s0 = None
    if w.s0_std > 0:
        s0 = (w.s0_std * rng.standard_normal((B, HV, K, V))).astype(np.float32)
    q64, qd = _store(q, w.dtype)
    k64, kd = _store(k, w.dtype)
    v64, vd = _store(v, w.dtype)
    return Inputs(w, q64, k64, v64, g, beta, s0, qd, kd, vd)
