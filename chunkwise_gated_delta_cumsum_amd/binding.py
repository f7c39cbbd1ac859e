"""Thin ctypes binding of libgdr.so (include/gdr.h).

Argument marshalling only: shapes, dtypes and devices are checked, outputs
and the workspace are allocated with torch on the inputs' device, and the
C entry point is called on torch's current stream.  Every step of the
computation runs in the HIP kernels; there is no fallback.  If the library
is missing, load() raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Tuple

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgdr.so")

GDR_F32, GDR_BF16 = 0, 1
RULES = {"delta": 0, "linear": 1}   # gdr_rule: gated delta rule, decayed linear attention
GDR_OK = 0
STATUS_NAMES = {
    0: "GDR_OK", 1: "GDR_ERR_NULL", 2: "GDR_ERR_SHAPE", 3: "GDR_ERR_DTYPE",
    4: "GDR_ERR_UNSUPPORTED", 5: "GDR_ERR_ALIGN", 6: "GDR_ERR_WORKSPACE",
    7: "GDR_ERR_DEVICE", 8: "GDR_ERR_HIP", 9: "GDR_ERR_ARG", 10: "GDR_ERR_ALIAS",
}
EXPORTED = ("gdr_chunk_fwd_workspace_size", "gdr_chunk_fwd", "gdr_chunk_prep",
            "gdr_chunk_scan", "gdr_chunk_scan_segments", "gdr_chunk_scan_slab",
            "gdr_decode_step", "gdr_status_string", "gdr_version")


class GdrProblem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32),
                ("HV", ctypes.c_int32), ("K", ctypes.c_int32), ("V", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("g_per_channel", ctypes.c_int32),
                ("scale", ctypes.c_float), ("qkv_dtype", ctypes.c_int32),
                ("scan_segments", ctypes.c_int32), ("scan_slab", ctypes.c_int32),
                ("qk_l2norm", ctypes.c_int32), ("rule", ctypes.c_int32)]


class GdrError(RuntimeError):
    def __init__(self, status: int, text: str):
        super().__init__(text)
        self.status = status
        self.name = STATUS_NAMES.get(status, "GDR_ERR_UNKNOWN")


_lib = None


def load():
    """Load libgdr.so from the package directory (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run "
                           "`python -m chunkwise_gated_delta_cumsum_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(GdrProblem)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    lib.gdr_chunk_fwd_workspace_size.argtypes = [P]
    lib.gdr_chunk_fwd_workspace_size.restype = sz
    lib.gdr_chunk_fwd.argtypes = [P] + [vp] * 8 + [vp, sz, vp]
    lib.gdr_chunk_fwd.restype = ctypes.c_int
    lib.gdr_chunk_prep.argtypes = [P] + [vp] * 4 + [vp, sz] + [vp] * 4 + [vp]
    lib.gdr_chunk_prep.restype = ctypes.c_int
    lib.gdr_chunk_scan.argtypes = [P] + [vp] * 6 + [vp, sz, vp]
    lib.gdr_chunk_scan.restype = ctypes.c_int
    lib.gdr_status_string.argtypes = [ctypes.c_int]
    lib.gdr_status_string.restype = ctypes.c_char_p
    lib.gdr_chunk_scan_segments.argtypes = [P]
    lib.gdr_chunk_scan_segments.restype = ctypes.c_int
    lib.gdr_chunk_scan_slab.argtypes = [P]
    lib.gdr_decode_step.argtypes = [P] + [vp] * 8 + [vp]
    lib.gdr_decode_step.restype = ctypes.c_int
    lib.gdr_chunk_scan_slab.restype = ctypes.c_int
    lib.gdr_version.argtypes = []
    lib.gdr_version.restype = ctypes.c_int
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().gdr_status_string(int(status)).decode()


def check(status: int) -> None:
    if status != GDR_OK:
        raise GdrError(status, status_string(status))


def problem(B: int, T: int, H: int, HV: int, K: int, V: int, *, chunk: int = 64,
            per_channel: bool = False, scale: Optional[float] = None,
            dtype: str = "bf16", segments: int = 0, slab: int = 0,
            qk_l2norm: bool = False, rule: str = "delta") -> GdrProblem:
    return GdrProblem(B, T, H, HV, K, V, chunk, int(bool(per_channel)),
                      float(K ** -0.5 if scale is None else scale),
                      {"fp32": GDR_F32, "bf16": GDR_BF16}[dtype], int(segments), int(slab),
                      int(bool(qk_l2norm)), RULES[rule])


def scan_segments(prob: GdrProblem) -> int:
    """Segments the state scan uses for this problem (0: invalid problem)."""
    return int(load().gdr_chunk_scan_segments(ctypes.byref(prob)))


def scan_slab(prob: GdrProblem) -> int:
    """State columns per scan workgroup for this problem (0: invalid problem)."""
    return int(load().gdr_chunk_scan_slab(ctypes.byref(prob)))


def workspace_size(prob: GdrProblem) -> int:
    return int(load().gdr_chunk_fwd_workspace_size(ctypes.byref(prob)))


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _problem_from(q, k, v, g, beta, chunk, scale, segments=0, slab=0,
                  qk_l2norm=False, rule="delta") -> GdrProblem:
    import torch
    if q.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError(f"q/k/v must be float32 or bfloat16, got {q.dtype}")
    if k.dtype != q.dtype or (v is not None and v.dtype != q.dtype):
        raise TypeError("q, k and v must share one dtype")
    if q.dim() != 4 or k.shape != q.shape:
        raise ValueError(f"q and k must be [B, T, H, K] of one shape: {tuple(q.shape)}, {tuple(k.shape)}")
    B, T, H, K = q.shape
    if beta.dim() != 3 or beta.shape[:2] != (B, T):
        raise ValueError(f"beta must be [B, T, HV], got {tuple(beta.shape)}")
    HV = beta.shape[2]
    if v is not None:
        if v.dim() != 4 or v.shape[:3] != (B, T, HV):
            raise ValueError(f"v must be [B, T, HV, V], got {tuple(v.shape)}")
        V = v.shape[3]
    else:
        V = K
    if g.shape == (B, T, HV):
        per_channel = False
    elif g.shape == (B, T, HV, K):
        per_channel = True
    else:
        raise ValueError(f"g must be [B, T, HV] or [B, T, HV, K], got {tuple(g.shape)}")
    for name, t in (("g", g), ("beta", beta)):
        if t.dtype != torch.float32:
            raise TypeError(f"{name} must be float32")
    return problem(B, T, H, HV, K, V, chunk=chunk, per_channel=per_channel, scale=scale,
                   dtype="fp32" if q.dtype == torch.float32 else "bf16", segments=segments,
                   slab=slab, qk_l2norm=qk_l2norm, rule=rule)


def _check_tensors(dev, **ts):
    for name, t in ts.items():
        if t is None:
            continue
        if t.device != dev:
            raise ValueError(f"{name} is on {t.device}, expected {dev}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")


def _stream(dev) -> ctypes.c_void_p:
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def gdr_chunk_fwd(q, k, v, g, beta, initial_state=None, chunk: int = 64,
                  scale: Optional[float] = None, *, output_final_state: bool = True,
                  workspace=None, out=None, segments: int = 0, slab: int = 0,
                  qk_l2norm: bool = False, rule: str = "delta"
                  ) -> Tuple["torch.Tensor", Optional["torch.Tensor"]]:
    """Chunkwise gated delta rule forward on the GPU.

    q, k: [B, T, H, K]; v: [B, T, HV, V] (float32 or bfloat16, one dtype);
    g: [B, T, HV] or [B, T, HV, K] float32 log-decay; beta: [B, T, HV] float32;
    initial_state: [B, HV, K, V] float32 or None.  scale defaults to K**-0.5.
    Returns (o [B, T, HV, V] float32, final_state [B, HV, K, V] float32 or None).
    ``workspace`` (uint8, at least workspace_size bytes) and ``out`` = (o, S)
    may be passed to avoid allocations.  ``segments`` > 0 asks for that many
    sequence segments in the state scan (0: automatic); ``slab`` (32 or 64)
    sets the state columns per scan workgroup (0: automatic).  ``qk_l2norm``
    L2-normalises every q and k row inside the kernels first.  ``rule`` is
    "delta" (the gated delta rule) or "linear" (decayed linear attention,
    no erase term).
    """
    import torch
    lib = load()
    dev = q.device
    _check_tensors(dev, q=q, k=k, v=v, g=g, beta=beta, initial_state=initial_state)
    prob = _problem_from(q, k, v, g, beta, chunk, scale, segments, slab, qk_l2norm, rule)
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    if initial_state is not None and (initial_state.dtype != torch.float32 or
                                      initial_state.shape != (B, HV, K, V)):
        raise ValueError("initial_state must be float32 [B, HV, K, V]")
    nbytes = workspace_size(prob)
    if nbytes == 0:
        check(lib.gdr_chunk_fwd(ctypes.byref(prob), *([None] * 8), None, 0, None))
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    if out is not None:
        o, s = out
    else:
        o = torch.empty((B, T, HV, V), dtype=torch.float32, device=dev)
        s = (torch.empty((B, HV, K, V), dtype=torch.float32, device=dev)
             if output_final_state else None)
    st = lib.gdr_chunk_fwd(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                           _ptr(initial_state), _ptr(o), _ptr(s), _ptr(workspace),
                           workspace.numel() * workspace.element_size(), _stream(dev))
    check(st)
    return o, s


def gdr_chunk_prep(q, k, g, beta, chunk: int = 64, scale: Optional[float] = None, *,
                   V: Optional[int] = None, inspect: bool = False,
                   workspace=None, segments: int = 0, slab: int = 0,
                   qk_l2norm: bool = False, rule: str = "delta"
                   ) -> Tuple["torch.Tensor", Dict[str, "torch.Tensor"]]:
    """Run the chunk-preparation stage alone.

    Returns (workspace, inspection dict).  With inspect=True the dict holds
    fp32 gamma [B,HV,N,C(,K)], a_kk, a_qk and m_inv [B,HV,N,C,C].
    """
    import torch
    lib = load()
    dev = q.device
    _check_tensors(dev, q=q, k=k, g=g, beta=beta)
    prob = _problem_from(q, k, None, g, beta, chunk, scale, segments, slab, qk_l2norm, rule)
    if V is not None:
        prob.V = V
    nbytes = workspace_size(prob)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    ins: Dict[str, torch.Tensor] = {}
    if inspect:
        B, T, H, K = q.shape
        HV = beta.shape[2]
        N = -(-T // chunk)
        gshape = (B, HV, N, chunk, K) if prob.g_per_channel else (B, HV, N, chunk)
        ins = dict(gamma=torch.empty(gshape, dtype=torch.float32, device=dev),
                   a_kk=torch.empty((B, HV, N, chunk, chunk), dtype=torch.float32, device=dev),
                   a_qk=torch.empty((B, HV, N, chunk, chunk), dtype=torch.float32, device=dev),
                   m_inv=torch.empty((B, HV, N, chunk, chunk), dtype=torch.float32, device=dev))
    st = lib.gdr_chunk_prep(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(g), _ptr(beta),
                            _ptr(workspace), workspace.numel(), _ptr(ins.get("gamma")),
                            _ptr(ins.get("a_kk")), _ptr(ins.get("a_qk")), _ptr(ins.get("m_inv")),
                            _stream(dev))
    check(st)
    return workspace, ins


def gdr_chunk_scan(q, k, v, g, beta, workspace, initial_state=None, chunk: int = 64,
                   scale: Optional[float] = None, *, out=None, segments: int = 0,
                   slab: int = 0, qk_l2norm: bool = False, rule: str = "delta"):
    """Run the state-scan stage on a workspace filled by gdr_chunk_prep.

    ``out`` = (o, final_state) reuses caller tensors (final_state may be None).
    """
    import torch
    lib = load()
    dev = q.device
    _check_tensors(dev, q=q, k=k, v=v, initial_state=initial_state)
    prob = _problem_from(q, k, v, g, beta, chunk, scale, segments, slab, qk_l2norm, rule)
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    if out is not None:
        o, s = out
    else:
        o = torch.empty((B, T, HV, V), dtype=torch.float32, device=dev)
        s = torch.empty((B, HV, K, V), dtype=torch.float32, device=dev)
    st = lib.gdr_chunk_scan(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(initial_state),
                            _ptr(o), _ptr(s), _ptr(workspace), workspace.numel(), _stream(dev))
    check(st)
    return o, s


def gdr_decode_step(q, k, v, g, beta, state=None, scale: Optional[float] = None, *,
                    out=None, inplace: bool = False, slab: int = 0, qk_l2norm: bool = False,
                    rule: str = "delta") -> Tuple["torch.Tensor", "torch.Tensor"]:
    """One decode step (one token per sequence) on the GPU.

    q, k: [B, H, K]; v: [B, HV, V] (float32 or bfloat16, one dtype);
    g: [B, HV] or [B, HV, K] float32 log-decay; beta: [B, HV] float32;
    state: [B, HV, K, V] float32 or None (zero state).  scale defaults to
    K**-0.5.  Returns (o [B, HV, V] float32, new state [B, HV, K, V] float32).
    With ``inplace`` the new state overwrites ``state``; ``out`` = (o, S) may
    be passed to avoid allocations.  ``slab`` (32, 64 or 128) sets the state
    columns per workgroup (0: automatic).  ``qk_l2norm`` L2-normalises q and
    k inside the kernel first; ``rule`` "linear" drops the erase term.
    """
    import torch
    lib = load()
    dev = q.device
    _check_tensors(dev, q=q, k=k, v=v, g=g, beta=beta, state=state)
    if q.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError(f"q/k/v must be float32 or bfloat16, got {q.dtype}")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k and v must share one dtype")
    if q.dim() != 3 or k.shape != q.shape:
        raise ValueError(f"q and k must be [B, H, K] of one shape: {tuple(q.shape)}, {tuple(k.shape)}")
    B, H, K = q.shape
    if v.dim() != 3 or v.shape[0] != B:
        raise ValueError(f"v must be [B, HV, V], got {tuple(v.shape)}")
    HV, V = v.shape[1], v.shape[2]
    if g.shape == (B, HV):
        per_channel = False
    elif g.shape == (B, HV, K):
        per_channel = True
    else:
        raise ValueError(f"g must be [B, HV] or [B, HV, K], got {tuple(g.shape)}")
    if beta.shape != (B, HV):
        raise ValueError(f"beta must be [B, HV], got {tuple(beta.shape)}")
    for name, t in (("g", g), ("beta", beta)):
        if t.dtype != torch.float32:
            raise TypeError(f"{name} must be float32")
    if state is not None and (state.dtype != torch.float32 or state.shape != (B, HV, K, V)):
        raise ValueError("state must be float32 [B, HV, K, V]")
    if inplace and state is None:
        raise ValueError("inplace needs a state")
    prob = problem(B, 1, H, HV, K, V, per_channel=per_channel, scale=scale,
                   dtype="fp32" if q.dtype == torch.float32 else "bf16", slab=slab,
                   qk_l2norm=qk_l2norm, rule=rule)
    if out is not None:
        o, s = out
    else:
        o = torch.empty((B, HV, V), dtype=torch.float32, device=dev)
        s = state if inplace else torch.empty((B, HV, K, V), dtype=torch.float32, device=dev)
    st = lib.gdr_decode_step(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                             _ptr(beta), _ptr(state), _ptr(s), _ptr(o), _stream(dev))
    check(st)
    return o, s
