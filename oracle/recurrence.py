"""ctypes wrapper of the fp64 per-token recurrence in gdr_oracle.c (the gated
delta rule, or the decayed linear attention without the erase term).

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the product path.

The recurrence is the plain definition the chunkwise algorithm must reproduce
(sec-03 notes: the chunk form equals the naive recurrent form; "Chunkwise
parallel algorithms" page, section 2.1, the delta rule):

    S <- diag(exp(g_t)) S
    S <- S + beta_t k_t (v_t - S^T k_t)^T
    o_t = scale * S^T q_t
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdr_oracle.c")
_LIB = os.path.join(_HERE, "libgdr_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile gdr_oracle.c with gcc (-O2, no fast-math, OpenMP)."""
    if force or not os.path.exists(_LIB) or (
            os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared",
                               "-std=c11", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build(force=False)
        lib = ctypes.CDLL(_LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.gdr_oracle_recurrence.argtypes = (
            [ctypes.c_int] * 7 + [ctypes.c_double] + [dp] * 8 + [ctypes.c_int])
        lib.gdr_oracle_recurrence.restype = ctypes.c_int
        lib.gdr_oracle_recurrence_rule.argtypes = (
            [ctypes.c_int] * 8 + [ctypes.c_double] + [dp] * 8 + [ctypes.c_int])
        lib.gdr_oracle_recurrence_rule.restype = ctypes.c_int
        lib.gdr_oracle_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def num_threads() -> int:
    return _load().gdr_oracle_num_threads()


def _f64(x):
    return None if x is None else np.ascontiguousarray(x, dtype=np.float64)


def _ptr(x):
    if x is None:
        return None
    return x.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def recurrence(q, k, v, g, beta, scale: float, s0=None,
               threads: int = 0, rule: str = "delta") -> Tuple[np.ndarray, np.ndarray]:
    """Run the fp64 recurrence.

    q, k: [B, T, H, K]; v: [B, T, HV, V]; g: [B, T, HV] or [B, T, HV, K];
    beta: [B, T, HV]; s0: [B, HV, K, V] or None.  rule "delta" is the gated
    delta rule; "linear" drops the prediction term (S <- S + beta k v^T, the
    decayed linear attention of the page's Mamba2 SSD section).
    Returns (o [B, T, HV, V], final_state [B, HV, K, V]) in fp64.
    """
    q, k, v, g, beta, s0 = map(_f64, (q, k, v, g, beta, s0))
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    per_channel = g.ndim == 4
    assert k.shape == q.shape and v.shape[:2] == (B, T)
    assert g.shape == ((B, T, HV, K) if per_channel else (B, T, HV))
    assert beta.shape == (B, T, HV)
    if s0 is not None:
        assert s0.shape == (B, HV, K, V)
    o = np.empty((B, T, HV, V), np.float64)
    s = np.empty((B, HV, K, V), np.float64)
    if rule not in ("delta", "linear"):
        raise ValueError(f"unknown rule {rule!r}")
    rc = _load().gdr_oracle_recurrence_rule(
        B, T, H, HV, K, V, int(per_channel), int(rule == "linear"), float(scale),
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(s0), _ptr(o),
        _ptr(s), int(threads))
    if rc != 0:
        raise RuntimeError(f"gdr_oracle_recurrence failed ({rc})")
    return o, s


def recurrence_heads(inp, heads, T: Optional[int] = None, threads: int = 0,
                     rule: str = "delta"):
    """Recurrence on a subset of (b, hv) pairs of an ``inputs.Inputs``.

    Returns {(b, hv): (o [T, V], S [K, V])}.  Used to check full-size runs on
    sampled heads, each of which is an independent scan.
    """
    w = inp.w
    T = w.T if T is None else T
    out = {}
    for b, hv in heads:
        h = hv // w.G
        q = inp.q[b:b + 1, :T, h:h + 1]
        k = inp.k[b:b + 1, :T, h:h + 1]
        v = inp.v[b:b + 1, :T, hv:hv + 1]
        g = inp.g[b:b + 1, :T, hv:hv + 1]
        be = inp.beta[b:b + 1, :T, hv:hv + 1]
        s0 = None if inp.s0 is None else inp.s0[b:b + 1, hv:hv + 1]
        o, s = recurrence(q, k, v, g, be, inp.scale, s0, threads, rule=rule)
        out[(b, hv)] = (o[0, :, 0], s[0, 0])
    return out
