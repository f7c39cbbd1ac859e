"""Thin ctypes binding of libgdr.so (include/gdr.h).

Argument marshalling only: shapes, dtypes and devices of inputs, caller
outputs and caller workspaces are checked (host tensors are refused before
the call, since the library takes device pointers), missing outputs and the
workspace are allocated with torch on the inputs' device, and the C entry
point is called on torch's current stream.  Every step of the
computation runs in the HIP kernels; there is no fallback.  If the library
is missing, load() raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Tuple

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgdr.so")

GDR_F32, GDR_BF16, GDR_F16 = 0, 1, 2
DTYPES = {"fp32": GDR_F32, "bf16": GDR_BF16, "fp16": GDR_F16}   # gdr_dtype of q/k/v and of o
RULES = {"delta": 0, "linear": 1}   # gdr_rule: gated delta rule, decayed linear attention
GDR_OK = 0
STATUS_NAMES = {
    0: "GDR_OK", 1: "GDR_ERR_NULL", 2: "GDR_ERR_SHAPE", 3: "GDR_ERR_DTYPE",
    4: "GDR_ERR_UNSUPPORTED", 5: "GDR_ERR_ALIGN", 6: "GDR_ERR_WORKSPACE",
    7: "GDR_ERR_DEVICE", 8: "GDR_ERR_HIP", 9: "GDR_ERR_ARG", 10: "GDR_ERR_ALIAS",
    11: "GDR_ERR_SCRATCH",
}
NOALLOC_SCRATCH_BYTES = 64 << 20    # GDR_NOALLOC_SCRATCH_BYTES in gdr.h
# gdr_check_bit: the bits gdr_check_inputs sets
CHECK_BITS = {1: "GDR_CHECK_NONFINITE", 2: "GDR_CHECK_FP16_RANGE", 4: "GDR_CHECK_DECAY_RANGE"}
EXPORTED = ("gdr_chunk_fwd_workspace_size", "gdr_chunk_fwd", "gdr_chunk_fwd_noalloc",
            "gdr_chunk_prep",
            "gdr_chunk_scan", "gdr_chunk_scan_segments", "gdr_chunk_scan_slab",
            "gdr_decode_step", "gdr_check_inputs", "gdr_status_string", "gdr_version")


class GdrProblem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32),
                ("HV", ctypes.c_int32), ("K", ctypes.c_int32), ("V", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("g_per_channel", ctypes.c_int32),
                ("scale", ctypes.c_float), ("qkv_dtype", ctypes.c_int32),
                ("scan_segments", ctypes.c_int32), ("scan_slab", ctypes.c_int32),
                ("qk_l2norm", ctypes.c_int32), ("rule", ctypes.c_int32),
                ("o_dtype", ctypes.c_int32)]


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
    lib.gdr_chunk_fwd_noalloc.argtypes = [P] + [vp] * 8 + [vp]
    lib.gdr_chunk_fwd_noalloc.restype = ctypes.c_int
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
    lib.gdr_check_inputs.argtypes = [P] + [vp] * 6 + [vp]
    lib.gdr_check_inputs.restype = ctypes.c_int
    lib.gdr_version.argtypes = []
    lib.gdr_version.restype = ctypes.c_int
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().gdr_status_string(int(status)).decode()


def check(status: int) -> None:
    if status != GDR_OK:
        raise GdrError(status, status_string(status))


def problem(B: int, T: int, H: int, HV: int, K: int, V: int, *, chunk: int = 0,
            per_channel: bool = False, scale: Optional[float] = None,
            dtype: str = "bf16", segments: int = 0, slab: int = 0,
            qk_l2norm: bool = False, rule: str = "delta",
            o_dtype: str = "fp32") -> GdrProblem:
    return GdrProblem(B, T, H, HV, K, V, chunk, int(bool(per_channel)),
                      float(K ** -0.5 if scale is None else scale),
                      DTYPES[dtype], int(segments), int(slab),
                      int(bool(qk_l2norm)), RULES[rule], DTYPES[o_dtype])


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


def _torch_dtype(name: str):
    import torch
    return {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}[name]


def _dtype_name(t) -> str:
    """The gdr dtype name of a q/k/v tensor (float32, bfloat16 or float16)."""
    import torch
    names = {torch.float32: "fp32", torch.bfloat16: "bf16", torch.float16: "fp16"}
    if t.dtype not in names:
        raise TypeError(f"q/k/v must be float32, bfloat16 or float16, got {t.dtype}")
    return names[t.dtype]


def _problem_from(q, k, v, g, beta, chunk, scale, segments=0, slab=0,
                  qk_l2norm=False, rule="delta", o_dtype="fp32") -> GdrProblem:
    import torch
    _dtype_name(q)
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
                   dtype=_dtype_name(q), segments=segments,
                   slab=slab, qk_l2norm=qk_l2norm, rule=rule, o_dtype=o_dtype)


def _check_tensors(dev, **ts):
    for name, t in ts.items():
        if t is None:
            continue
        if t.device != dev:
            raise ValueError(f"{name} is on {t.device}, expected {dev}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")


def _check_out(dev, name, t, shape, dtype):
    """An output the kernels write: exactly `shape` and `dtype`, contiguous, on `dev`."""
    if t is None:
        return
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    _check_tensors(dev, **{name: t})


def _check_workspace(dev, ws, nbytes):
    """A caller workspace: uint8, contiguous, on `dev`, at least `nbytes` bytes."""
    import torch
    if ws.dtype != torch.uint8:
        raise TypeError(f"workspace must be uint8, got {ws.dtype}")
    _check_tensors(dev, workspace=ws)
    if _nbytes(ws) < nbytes:
        raise ValueError(f"workspace holds {_nbytes(ws)} bytes, the problem needs {nbytes}")


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _require_gpu(dev):
    """The library takes device pointers: refuse host tensors before the call."""
    if dev.type != "cuda":
        raise ValueError(f"tensors must be on a GPU, got {dev}")


def _stream(dev) -> ctypes.c_void_p:
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _check_state(name, t, B, HV, K, V):
    import torch
    if t is not None and (t.dtype != torch.float32 or tuple(t.shape) != (B, HV, K, V)):
        raise ValueError(f"{name} must be float32 [B, HV, K, V] = {(B, HV, K, V)}")


def gdr_chunk_fwd(q, k, v, g, beta, initial_state=None, chunk: int = 0,
                  scale: Optional[float] = None, *, output_final_state: bool = True,
                  workspace=None, out=None, segments: int = 0, slab: int = 0,
                  qk_l2norm: bool = False, rule: str = "delta", o_dtype: str = "fp32"
                  ) -> Tuple["torch.Tensor", Optional["torch.Tensor"]]:
    """Chunkwise gated delta rule forward on the GPU.

    q, k: [B, T, H, K]; v: [B, T, HV, V] (float32, bfloat16 or float16, one dtype);
    g: [B, T, HV] or [B, T, HV, K] float32 log-decay; beta: [B, T, HV] float32;
    initial_state: [B, HV, K, V] float32 or None.  scale defaults to K**-0.5;
    chunk is 32, 64 or 128, or 0 for the automatic choice (64).
    Returns (o [B, T, HV, V], final_state [B, HV, K, V] float32 or None); o is
    float32, or bfloat16 / float16 with ``o_dtype="bf16"`` / ``"fp16"`` (the fp32 result rounded
    once, to nearest even).
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
    prob = _problem_from(q, k, v, g, beta, chunk, scale, segments, slab, qk_l2norm, rule,
                         o_dtype)
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    _check_state("initial_state", initial_state, B, HV, K, V)
    nbytes = workspace_size(prob)
    if nbytes == 0:
        check(lib.gdr_chunk_fwd(ctypes.byref(prob), *([None] * 8), None, 0, None))
    odt = _torch_dtype(o_dtype)
    if workspace is not None:
        _check_workspace(dev, workspace, nbytes)
    if out is not None:
        o, s = out
        _check_out(dev, "o", o, (B, T, HV, V), odt)
        _check_out(dev, "final_state", s, (B, HV, K, V), torch.float32)
    _require_gpu(dev)
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    if out is None:
        o = torch.empty((B, T, HV, V), dtype=odt, device=dev)
        s = (torch.empty((B, HV, K, V), dtype=torch.float32, device=dev)
             if output_final_state else None)
    st = lib.gdr_chunk_fwd(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                           _ptr(initial_state), _ptr(o), _ptr(s), _ptr(workspace),
                           _nbytes(workspace), _stream(dev))
    check(st)
    return o, s


def gdr_check_inputs(q, k, v, g, beta, chunk: int = 0, *, qk_l2norm: bool = False,
                     flags=None) -> "torch.Tensor":
    """Checks the forward pass's inputs against its numeric preconditions on
    the device (gdr_check_inputs in gdr.h).  Returns the one-element int32
    device tensor (``flags`` if given) that the library sets, on torch's
    current stream, to the OR of the violated CHECK_BITS (0: none); reading it
    synchronises.  ``chunk`` and ``qk_l2norm`` are those of the forward call
    the inputs are meant for."""
    import torch
    lib = load()
    dev = q.device
    _check_tensors(dev, q=q, k=k, v=v, g=g, beta=beta)
    prob = _problem_from(q, k, v, g, beta, chunk, None, qk_l2norm=qk_l2norm)
    if flags is None:
        _require_gpu(dev)
        flags = torch.empty(1, dtype=torch.int32, device=dev)
    elif flags.dtype != torch.int32 or flags.numel() < 1:
        raise TypeError("flags must be an int32 tensor of at least one element")
    else:
        _check_tensors(dev, flags=flags)
        _require_gpu(dev)
    check(lib.gdr_check_inputs(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                               _ptr(beta), _ptr(flags), _stream(dev)))
    return flags


def check_bit_names(bits: int) -> list:
    """Names of the CHECK_BITS set in ``bits``."""
    return [name for bit, name in CHECK_BITS.items() if bits & bit]


def gdr_chunk_fwd_noalloc(q, k, v, g, beta, initial_state=None, chunk: int = 0,
                          scale: Optional[float] = None, *, output_final_state: bool = True,
                          out=None, segments: int = 0, slab: int = 0,
                          qk_l2norm: bool = False, rule: str = "delta", o_dtype: str = "fp32"
                          ) -> Tuple["torch.Tensor", Optional["torch.Tensor"]]:
    """gdr_chunk_fwd on the library's own device scratch array instead of a
    workspace (the C entry point allocates nothing; with ``out`` given this
    wrapper allocates nothing either).  Problems whose workspace exceeds
    NOALLOC_SCRATCH_BYTES raise GDR_ERR_SCRATCH.  Calls that overlap in time
    on one GPU share the array and race."""
    import torch
    lib = load()
    dev = q.device
    _check_tensors(dev, q=q, k=k, v=v, g=g, beta=beta, initial_state=initial_state)
    prob = _problem_from(q, k, v, g, beta, chunk, scale, segments, slab, qk_l2norm, rule,
                         o_dtype)
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    _check_state("initial_state", initial_state, B, HV, K, V)
    nbytes = workspace_size(prob)
    if nbytes == 0:     # an invalid problem: the library names the reason
        check(lib.gdr_chunk_fwd_noalloc(ctypes.byref(prob), *([None] * 8), None))
    if nbytes > NOALLOC_SCRATCH_BYTES:
        check(11)       # GDR_ERR_SCRATCH, as the library would return
    odt = _torch_dtype(o_dtype)
    if out is not None:
        o, s = out
        _check_out(dev, "o", o, (B, T, HV, V), odt)
        _check_out(dev, "final_state", s, (B, HV, K, V), torch.float32)
    _require_gpu(dev)
    if out is None:
        o = torch.empty((B, T, HV, V), dtype=odt, device=dev)
        s = (torch.empty((B, HV, K, V), dtype=torch.float32, device=dev)
             if output_final_state else None)
    st = lib.gdr_chunk_fwd_noalloc(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                   _ptr(beta), _ptr(initial_state), _ptr(o), _ptr(s),
                                   _stream(dev))
    check(st)
    return o, s


def gdr_chunk_prep(q, k, g, beta, chunk: int = 0, scale: Optional[float] = None, *,
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
    if nbytes == 0:
        check(lib.gdr_chunk_prep(ctypes.byref(prob), *([None] * 4), None, 0,
                                 *([None] * 4), None))
    if workspace is not None:
        _check_workspace(dev, workspace, nbytes)
    _require_gpu(dev)
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    ins: Dict[str, torch.Tensor] = {}
    if inspect:
        B, T, H, K = q.shape
        HV = beta.shape[2]
        chunk = chunk or 64               # the automatic chunk length
        N = -(-T // chunk)
        gshape = (B, HV, N, chunk, K) if prob.g_per_channel else (B, HV, N, chunk)
        ins = dict(gamma=torch.empty(gshape, dtype=torch.float32, device=dev),
                   a_kk=torch.empty((B, HV, N, chunk, chunk), dtype=torch.float32, device=dev),
                   a_qk=torch.empty((B, HV, N, chunk, chunk), dtype=torch.float32, device=dev),
                   m_inv=torch.empty((B, HV, N, chunk, chunk), dtype=torch.float32, device=dev))
    st = lib.gdr_chunk_prep(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(g), _ptr(beta),
                            _ptr(workspace), _nbytes(workspace), _ptr(ins.get("gamma")),
                            _ptr(ins.get("a_kk")), _ptr(ins.get("a_qk")), _ptr(ins.get("m_inv")),
                            _stream(dev))
    check(st)
    return workspace, ins


def gdr_chunk_scan(q, k, v, g, beta, workspace, initial_state=None, chunk: int = 0,
                   scale: Optional[float] = None, *, out=None, segments: int = 0,
                   slab: int = 0, qk_l2norm: bool = False, rule: str = "delta",
                   o_dtype: str = "fp32"):
    """Run the state-scan stage on a workspace filled by gdr_chunk_prep.

    ``out`` = (o, final_state) reuses caller tensors (final_state may be None).
    """
    import torch
    lib = load()
    dev = q.device
    _check_tensors(dev, q=q, k=k, v=v, initial_state=initial_state)
    prob = _problem_from(q, k, v, g, beta, chunk, scale, segments, slab, qk_l2norm, rule,
                         o_dtype)
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    _check_state("initial_state", initial_state, B, HV, K, V)
    nbytes = workspace_size(prob)
    if nbytes == 0:
        check(lib.gdr_chunk_scan(ctypes.byref(prob), *([None] * 6), None, 0, None))
    _check_workspace(dev, workspace, nbytes)
    odt = _torch_dtype(o_dtype)
    if out is not None:
        o, s = out
        _check_out(dev, "o", o, (B, T, HV, V), odt)
        _check_out(dev, "final_state", s, (B, HV, K, V), torch.float32)
    _require_gpu(dev)
    if out is None:
        o = torch.empty((B, T, HV, V), dtype=odt, device=dev)
        s = torch.empty((B, HV, K, V), dtype=torch.float32, device=dev)
    st = lib.gdr_chunk_scan(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(initial_state),
                            _ptr(o), _ptr(s), _ptr(workspace), _nbytes(workspace), _stream(dev))
    check(st)
    return o, s


def gdr_decode_step(q, k, v, g, beta, state=None, scale: Optional[float] = None, *,
                    out=None, inplace: bool = False, slab: int = 0, qk_l2norm: bool = False,
                    rule: str = "delta", o_dtype: str = "fp32"
                    ) -> Tuple["torch.Tensor", "torch.Tensor"]:
    """One decode step (one token per sequence) on the GPU.

    q, k: [B, H, K]; v: [B, HV, V] (float32, bfloat16 or float16, one dtype);
    g: [B, HV] or [B, HV, K] float32 log-decay; beta: [B, HV] float32;
    state: [B, HV, K, V] float32 or None (zero state).  scale defaults to
    K**-0.5.  Returns (o [B, HV, V] float32 (bfloat16 / float16 with o_dtype),
    new state [B, HV, K, V] float32).
    With ``inplace`` the new state overwrites ``state``; ``out`` = (o, S) may
    be passed to avoid allocations.  ``slab`` (32, 64 or 128) sets the state
    columns per workgroup (0: automatic).  ``qk_l2norm`` L2-normalises q and
    k inside the kernel first; ``rule`` "linear" drops the erase term.
    """
    import torch
    lib = load()
    dev = q.device
    _check_tensors(dev, q=q, k=k, v=v, g=g, beta=beta, state=state)
    _dtype_name(q)
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
    _check_state("state", state, B, HV, K, V)
    if inplace and state is None:
        raise ValueError("inplace needs a state")
    prob = problem(B, 1, H, HV, K, V, per_channel=per_channel, scale=scale,
                   dtype=_dtype_name(q), slab=slab,
                   qk_l2norm=qk_l2norm, rule=rule, o_dtype=o_dtype)
    odt = _torch_dtype(o_dtype)
    if out is not None:
        o, s = out
        _check_out(dev, "o", o, (B, HV, V), odt)
        if s is None:
            raise ValueError("out must hold a state tensor")
        _check_out(dev, "state_out", s, (B, HV, K, V), torch.float32)
    _require_gpu(dev)
    if out is None:
        o = torch.empty((B, HV, V), dtype=odt, device=dev)
        s = state if inplace else torch.empty((B, HV, K, V), dtype=torch.float32, device=dev)
    st = lib.gdr_decode_step(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                             _ptr(beta), _ptr(state), _ptr(s), _ptr(o), _stream(dev))
    check(st)
    return o, s
