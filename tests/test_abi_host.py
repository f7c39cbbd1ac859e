"""Host-side checks of the C ABI (no GPU needed, nothing is launched).

The library must load, export every function include/gdr.h declares, and
reject bad arguments with the documented status before any HIP call.  All
calls here fail validation, so they return before touching a device; the
pointers are fake, 16-byte-aligned addresses that are never dereferenced.
"""
import ctypes
import os
import re

import pytest

import chunkwise_gated_delta_cumsum_amd as gdr
from chunkwise_gated_delta_cumsum_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdr.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        from chunkwise_gated_delta_cumsum_amd import build
        build.build()
    return gdr.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdr_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(binding.EXPORTED)


def test_header_is_plain_c(tmp_path):
    """include/gdr.h compiles as strict C99 (the ABI carries no C++ types)."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    src = tmp_path / "use_gdr.c"
    src.write_text('#include "gdr.h"\n'
                   "int probe(const gdr_problem* p, void* s) {\n"
                   "  uint32_t* f = 0;\n"
                   "  return (int)gdr_check_inputs(p, 0, 0, 0, 0, 0, f, s) + (int)GDR_CHECK_DECAY_RANGE"
                   " + (int)gdr_chunk_fwd_workspace_size(p) + gdr_version();\n}\n")
    subprocess.check_call(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
                           "-I", os.path.join(ROOT, "include"), "-c", str(src),
                           "-o", str(tmp_path / "use_gdr.o")])


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_library_is_gfx950_code_object(lib):
    data = open(binding.LIB_PATH, "rb").read()
    assert b"gfx950" in data


def test_status_strings(lib):
    for code, name in binding.STATUS_NAMES.items():
        assert gdr.status_string(code).startswith(name)
    assert gdr.status_string(12345).startswith("GDR_ERR_UNKNOWN")
    assert lib.gdr_version() >= 200
    # the binding's struct must match the header's field for field
    import re as _re
    body = open(HEADER).read().split("typedef struct gdr_problem {")[1].split("} gdr_problem;")[0]
    body = _re.sub(r"/\*.*?\*/", "", body, flags=_re.S)
    names = [n for decl in body.split(";") for n in _re.findall(r"\b(\w+)\s*(?:,|$)", decl.strip())
             if n not in ("int32_t", "float")]
    assert names == [f[0] for f in binding.GdrProblem._fields_]


A = 1 << 20   # fake device addresses, spaced far apart, 16-byte aligned


def call_fwd(lib, prob, q=A, k=2 * A, v=3 * A, g=4 * A, beta=5 * A, s0=None,
             o=6 * A, sT=7 * A, ws=8 * A, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = gdr.workspace_size(prob) if gdr.workspace_size(prob) else 1 << 30
    return lib.gdr_chunk_fwd(ctypes.byref(prob), q, k, v, g, beta, s0, o, sT, ws,
                             ws_bytes, None)


def base(**kw):
    args = dict(B=1, T=100, H=2, HV=4, K=128, V=128)
    args.update(kw)
    return gdr.problem(**args)


def test_workspace_size(lib):
    p = base()
    n = 1 * 4 * 2   # B * HV * ceil(100 / 64)
    nq = 1 * 2 * 2  # B * H * ceil(100 / 64): q and k fragments per query head
    # per chunk: W^ (K x C), the 6 lower-triangular fragments of A^, row scalars
    expect_min = n * (128 * 64 * 2 + 6 * 512 * 2 + 256 * 4) + nq * 2 * (64 * 128 * 2)
    assert gdr.workspace_size(p) >= expect_min
    assert gdr.workspace_size(base(per_channel=True)) > gdr.workspace_size(p)
    assert gdr.workspace_size(base(dtype="fp32")) > gdr.workspace_size(p)
    assert gdr.workspace_size(base(HV=3)) == 0          # invalid -> 0
    assert lib.gdr_chunk_fwd_workspace_size(None) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), "GDR_ERR_SHAPE"),
    (dict(T=0), "GDR_ERR_SHAPE"),
    (dict(H=3, HV=4), "GDR_ERR_SHAPE"),
    (dict(K=96), "GDR_ERR_UNSUPPORTED"),
    (dict(V=256), "GDR_ERR_UNSUPPORTED"),
    (dict(chunk=48), "GDR_ERR_UNSUPPORTED"),
    (dict(scale=float("nan")), "GDR_ERR_ARG"),
    (dict(scale=float("inf")), "GDR_ERR_ARG"),
])
def test_invalid_problem(lib, kw, status):
    assert binding.STATUS_NAMES[call_fwd(lib, base(**kw))] == status


def test_invalid_dtype_and_flag(lib):
    p = base()
    p.qkv_dtype = 7
    assert binding.STATUS_NAMES[call_fwd(lib, p)] == "GDR_ERR_DTYPE"
    p = base()
    p.g_per_channel = 2
    assert binding.STATUS_NAMES[call_fwd(lib, p)] == "GDR_ERR_ARG"


def test_null_pointers(lib):
    assert binding.STATUS_NAMES[lib.gdr_chunk_fwd(None, *([A] * 8), A, 1 << 30, None)] == "GDR_ERR_NULL"
    for kw in (dict(q=None), dict(k=None), dict(v=None), dict(g=None), dict(beta=None), dict(o=None)):
        assert binding.STATUS_NAMES[call_fwd(lib, base(), **kw)] == "GDR_ERR_NULL", kw


def test_alignment(lib):
    for kw in (dict(q=A + 8), dict(v=3 * A + 2), dict(o=6 * A + 4), dict(s0=9 * A + 8),
               dict(sT=7 * A + 12), dict(ws=8 * A + 8)):
        assert binding.STATUS_NAMES[call_fwd(lib, base(), **kw)] == "GDR_ERR_ALIGN", kw


def call_check(lib, prob, q=A, k=2 * A, v=3 * A, g=4 * A, beta=5 * A, flags=6 * A):
    return lib.gdr_check_inputs(None if prob is None else ctypes.byref(prob), q, k, v, g, beta,
                                flags, None)


def test_check_inputs_validates(lib):
    name = lambda st: binding.STATUS_NAMES[st]
    assert name(call_check(lib, None)) == "GDR_ERR_NULL"
    assert name(call_check(lib, base(B=0))) == "GDR_ERR_SHAPE"
    assert name(call_check(lib, base(K=96))) == "GDR_ERR_UNSUPPORTED"
    assert name(call_check(lib, base(chunk=-64))) == "GDR_ERR_ARG"
    p = base()
    p.qkv_dtype = 5
    assert name(call_check(lib, p)) == "GDR_ERR_DTYPE"
    for kw in (dict(q=None), dict(k=None), dict(v=None), dict(g=None), dict(beta=None),
               dict(flags=None)):
        assert name(call_check(lib, base(), **kw)) == "GDR_ERR_NULL", kw
    for kw in (dict(q=A + 8), dict(g=4 * A + 4), dict(beta=5 * A + 8), dict(flags=6 * A + 2)):
        assert name(call_check(lib, base(), **kw)) == "GDR_ERR_ALIGN", kw
    # the flags word must not overlap an input: q holds 1*100*2*128*2 bytes
    assert name(call_check(lib, base(), flags=A + 4096)) == "GDR_ERR_ALIAS"
    assert name(call_check(lib, base(), flags=5 * A + 1596)) == "GDR_ERR_ALIAS"  # last beta
    assert name(call_check(lib, base(per_channel=True), flags=4 * A + 400 * 512 - 4)) == \
        "GDR_ERR_ALIAS"                                                # last per-channel g


def test_workspace_checks(lib):
    p = base()
    need = gdr.workspace_size(p)
    assert binding.STATUS_NAMES[call_fwd(lib, p, ws=None)] == "GDR_ERR_WORKSPACE"
    assert binding.STATUS_NAMES[call_fwd(lib, p, ws_bytes=need - 1)] == "GDR_ERR_WORKSPACE"


def test_aliasing(lib):
    p = base()
    assert binding.STATUS_NAMES[call_fwd(lib, p, o=A)] == "GDR_ERR_ALIAS"          # o == q
    assert binding.STATUS_NAMES[call_fwd(lib, p, o=3 * A + 4096)] == "GDR_ERR_ALIAS"  # inside v
    assert binding.STATUS_NAMES[call_fwd(lib, p, ws=5 * A)] == "GDR_ERR_ALIAS"     # ws == beta
    assert binding.STATUS_NAMES[call_fwd(lib, p, sT=2 * A)] == "GDR_ERR_ALIAS"     # S == k
    assert binding.STATUS_NAMES[call_fwd(lib, p, s0=9 * A, sT=9 * A + 64)] == "GDR_ERR_ALIAS"


def test_stage_entry_points_validate(lib):
    p = base()
    ws = gdr.workspace_size(p)
    st = lib.gdr_chunk_prep(ctypes.byref(p), None, 2 * A, 4 * A, 5 * A, 8 * A, ws,
                            None, None, None, None, None)
    assert binding.STATUS_NAMES[st] == "GDR_ERR_NULL"
    st = lib.gdr_chunk_prep(ctypes.byref(p), A, 2 * A, 4 * A, 5 * A, 8 * A, ws,
                            9 * A + 4, None, None, None, None)
    assert binding.STATUS_NAMES[st] == "GDR_ERR_ALIGN"
    st = lib.gdr_chunk_prep(ctypes.byref(p), A, 2 * A, 4 * A, 5 * A, 8 * A, ws,
                            A, None, None, None, None)
    assert binding.STATUS_NAMES[st] == "GDR_ERR_ALIAS"
    st = lib.gdr_chunk_scan(ctypes.byref(p), A, 2 * A, 3 * A, None, 6 * A, 7 * A,
                            8 * A, ws - 1, None)
    assert binding.STATUS_NAMES[st] == "GDR_ERR_WORKSPACE"
    st = lib.gdr_chunk_scan(ctypes.byref(p), A, 2 * A, 3 * A, None, 8 * A, 7 * A,
                            8 * A, ws, None)
    assert binding.STATUS_NAMES[st] == "GDR_ERR_ALIAS"


def test_binding_refuses_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        binding.load()


def test_scan_segment_query(lib):
    p = base(T=4096, H=12, HV=12)
    auto = gdr.scan_segments(p)
    assert auto >= 1
    for want, N in ((1, 64), (3, 64), (64, 64), (1000, 64)):
        q = base(T=64 * N, H=12, HV=12, segments=want)
        got = gdr.scan_segments(q)
        L = -(-N // min(want, N))
        assert got == -(-N // L)
        assert gdr.workspace_size(q) > 0
    bad = base(segments=-1)
    assert gdr.scan_segments(bad) == 0
    assert binding.STATUS_NAMES[call_fwd(lib, bad)] == "GDR_ERR_ARG"
    # more segments need more workspace (transitions and states)
    assert gdr.workspace_size(base(T=4096, segments=8)) > gdr.workspace_size(base(T=4096, segments=1))


def test_scan_slab_query(lib):
    assert gdr.scan_slab(base(T=4096, H=12, HV=12)) in (32, 64)
    for want in (32, 64):
        p = base(T=4096, H=12, HV=12, slab=want)
        assert gdr.scan_slab(p) == want
        assert gdr.workspace_size(p) > 0
    for bad_slab in (-1, 16, 48, 128):
        bad = base(slab=bad_slab)
        assert gdr.scan_slab(bad) == 0
        assert binding.STATUS_NAMES[call_fwd(lib, bad)] == "GDR_ERR_ARG"


def test_scan_width_choice(lib):
    """The automatic slab width and segment count of the cost model: narrow
    slabs in one segment where 48-64 scans would leave most compute units
    idle at 64 columns, 64 columns with segments for few long scans, and 64
    columns whenever the choice was not measured (fp32, the linear rule,
    head dims of 64)."""
    def pick(**kw):
        p = base(**kw)
        return gdr.scan_slab(p), gdr.scan_segments(p)
    assert pick(B=2, T=16000, H=16, HV=32, K=128, V=128) == (32, 1)
    assert pick(B=4, T=8192, H=16, HV=16, K=128, V=128, per_channel=True) == (32, 1)
    assert pick(B=1, T=4096, H=12, HV=12, K=128, V=128) == (64, 6)
    assert pick(B=1, T=65536, H=12, HV=12, K=128, V=128) == (64, 10)
    assert pick(B=8, T=4000, H=16, HV=32, K=128, V=128) == (64, 1)
    assert pick(B=2, T=16000, H=16, HV=32, K=128, V=128, dtype="fp32")[0] == 64
    assert pick(B=2, T=16000, H=16, HV=32, K=128, V=128, rule="linear")[0] == 64
    assert pick(B=2, T=16000, H=16, HV=32, K=64, V=64)[0] == 64
    # a forced width is kept; forced segments let the width follow the model
    assert pick(B=2, T=16000, H=16, HV=32, K=128, V=128, slab=64)[0] == 64
    assert pick(B=2, T=16000, H=16, HV=32, K=128, V=128, segments=1) == (32, 1)


def call_decode(lib, prob, q=A, k=2 * A, v=3 * A, g=4 * A, beta=5 * A, s_in=6 * A,
                s_out=7 * A, o=8 * A):
    ref = None if prob is None else ctypes.byref(prob)
    return lib.gdr_decode_step(ref, q, k, v, g, beta, s_in, s_out, o, None)


def test_decode_validation(lib):
    """Each bad argument of gdr_decode_step gets its status before any HIP call."""
    name = lambda st: binding.STATUS_NAMES[st]
    ok = base(T=1, B=2, H=2, HV=4)
    assert name(call_decode(lib, None)) == "GDR_ERR_NULL"
    assert name(call_decode(lib, base(T=2))) == "GDR_ERR_SHAPE"          # one token only
    assert name(call_decode(lib, base(T=1, H=3, HV=4))) == "GDR_ERR_SHAPE"
    assert name(call_decode(lib, base(T=1, K=96))) == "GDR_ERR_UNSUPPORTED"
    bad_dtype = base(T=1)
    bad_dtype.qkv_dtype = 7
    assert name(call_decode(lib, bad_dtype)) == "GDR_ERR_DTYPE"
    bad_scale = base(T=1, scale=float("nan"))
    assert name(call_decode(lib, bad_scale)) == "GDR_ERR_ARG"
    for kw in ("q", "k", "v", "g", "beta", "s_out", "o"):
        assert name(call_decode(lib, ok, **{kw: None})) == "GDR_ERR_NULL", kw
    assert name(call_decode(lib, ok, q=A + 4)) == "GDR_ERR_ALIGN"
    # o must not overlap anything; the new state must not overlap the inputs;
    # the state may be updated exactly in place but not with a partial overlap
    assert name(call_decode(lib, ok, o=7 * A)) == "GDR_ERR_ALIAS"
    assert name(call_decode(lib, ok, s_out=A)) == "GDR_ERR_ALIAS"
    assert name(call_decode(lib, ok, s_out=6 * A + 1024)) == "GDR_ERR_ALIAS"
    assert name(call_decode(lib, base(T=1, slab=48))) == "GDR_ERR_ARG"
    # the chunk settings do not apply to a single token
    odd = base(T=1, B=2, H=2, HV=4, chunk=32, segments=5)
    assert name(call_decode(lib, odd, q=A + 4)) == "GDR_ERR_ALIGN"


def test_qk_l2norm_flag_validation(lib):
    bad = base(T=100)
    bad.qk_l2norm = 2
    assert binding.STATUS_NAMES[call_fwd(lib, bad)] == "GDR_ERR_ARG"
    assert gdr.workspace_size(bad) == 0
    bad1 = base(T=1)
    bad1.qk_l2norm = -1
    assert binding.STATUS_NAMES[call_decode(lib, bad1)] == "GDR_ERR_ARG"
    ok = base(T=100, qk_l2norm=True)
    assert ok.qk_l2norm == 1 and gdr.workspace_size(ok) == gdr.workspace_size(base(T=100))


def test_rule_validation(lib):
    bad = base(T=100)
    bad.rule = 2
    assert binding.STATUS_NAMES[call_fwd(lib, bad)] == "GDR_ERR_ARG"
    bad1 = base(T=1)
    bad1.rule = -1
    assert binding.STATUS_NAMES[call_decode(lib, bad1)] == "GDR_ERR_ARG"
    lin = base(T=100, rule="linear")
    assert lin.rule == 1 and gdr.workspace_size(lin) == gdr.workspace_size(base(T=100))


def test_o_dtype_validation(lib):
    """o_dtype and qkv_dtype must be gdr_dtypes (fp32, bf16, fp16); a 16-bit o
    spans half the bytes of an fp32 one."""
    name = lambda st: binding.STATUS_NAMES[st]
    bad = base(T=100)
    bad.o_dtype = 3
    assert name(call_fwd(lib, bad)) == "GDR_ERR_DTYPE"
    assert gdr.workspace_size(bad) == 0
    bad.o_dtype = 2                     # fp16 o
    assert gdr.workspace_size(bad) == gdr.workspace_size(base(T=100))
    h16 = base(T=100, dtype="fp16")
    assert gdr.workspace_size(h16) == gdr.workspace_size(base(T=100))
    h16.qkv_dtype = 3
    assert name(call_fwd(lib, h16)) == "GDR_ERR_DTYPE"
    bad1 = base(T=1)
    bad1.o_dtype = -1
    assert name(call_decode(lib, bad1)) == "GDR_ERR_DTYPE"
    # o placed just below v: B*T*HV*V = 51200 elements, 204800 bytes in fp32
    # (overlaps v) and 102400 in bf16 (does not)
    p32, p16, ph = base(T=100), base(T=100, o_dtype="bf16"), base(T=100, o_dtype="fp16")
    o_at = 3 * A - 150000
    assert name(call_fwd(lib, p32, o=o_at)) == "GDR_ERR_ALIAS"
    assert name(call_fwd(lib, p16, o=o_at)) != "GDR_ERR_ALIAS"
    assert name(call_fwd(lib, ph, o=o_at)) != "GDR_ERR_ALIAS"
    assert gdr.workspace_size(p16) == gdr.workspace_size(p32)


def _cpu_inputs(B=1, T=40, H=2, HV=4, K=64, V=64):
    import torch
    q = torch.zeros(B, T, H, K, dtype=torch.bfloat16)
    return dict(q=q, k=q.clone(), v=torch.zeros(B, T, HV, V, dtype=torch.bfloat16),
                g=torch.zeros(B, T, HV), beta=torch.zeros(B, T, HV))


def test_binding_checks_outputs_and_workspace(lib):
    """The binding refuses caller outputs and workspaces of the wrong dtype,
    shape or layout, and host tensors, before the library is called."""
    import torch
    t = _cpu_inputs()
    args = (t["q"], t["k"], t["v"], t["g"], t["beta"])
    o = torch.empty(1, 40, 4, 64)
    s = torch.empty(1, 4, 64, 64)
    with pytest.raises(TypeError, match="o must be"):
        gdr.gdr_chunk_fwd(*args, out=(o.to(torch.bfloat16), s))
    with pytest.raises(TypeError, match="o must be"):
        gdr.gdr_chunk_fwd(*args, out=(o, s), o_dtype="bf16")
    with pytest.raises(ValueError, match="o must have shape"):
        gdr.gdr_chunk_fwd(*args, out=(torch.empty(1, 39, 4, 64), s))
    with pytest.raises(ValueError, match="final_state must have shape"):
        gdr.gdr_chunk_fwd(*args, out=(o, torch.empty(1, 4, 64, 32)))
    with pytest.raises(TypeError, match="final_state must be"):
        gdr.gdr_chunk_fwd(*args, out=(o, s.double()))
    with pytest.raises(ValueError, match="contiguous"):
        gdr.gdr_chunk_fwd(*args, out=(torch.empty(1, 40, 64, 4).transpose(2, 3), s))
    need = gdr.workspace_size(gdr.problem(1, 40, 2, 4, 64, 64))
    with pytest.raises(TypeError, match="workspace must be uint8"):
        gdr.gdr_chunk_fwd(*args, workspace=torch.empty(need, dtype=torch.float32))
    with pytest.raises(ValueError, match="workspace holds"):
        gdr.gdr_chunk_fwd(*args, workspace=torch.empty(need - 1, dtype=torch.uint8))
    with pytest.raises(ValueError, match="initial_state must be"):
        gdr.gdr_chunk_fwd(*args, torch.empty(1, 4, 64, 63))
    # a well-formed call on host tensors is refused: the library takes device pointers
    with pytest.raises(ValueError, match="on a GPU"):
        gdr.gdr_chunk_fwd(*args, out=(o, s), workspace=torch.empty(need, dtype=torch.uint8))
    # the stage entry points and decode check the same way
    with pytest.raises(ValueError, match="workspace holds"):
        gdr.gdr_chunk_prep(t["q"], t["k"], t["g"], t["beta"], V=64,
                           workspace=torch.empty(need - 1, dtype=torch.uint8))
    with pytest.raises(ValueError, match="workspace holds"):
        gdr.gdr_chunk_scan(*args, torch.empty(need - 16, dtype=torch.uint8))
    with pytest.raises(ValueError, match="o must have shape"):
        gdr.gdr_chunk_scan(*args, torch.empty(need, dtype=torch.uint8),
                           out=(torch.empty(1, 40, 4, 32), s))
    with pytest.raises(ValueError, match="on a GPU"):
        gdr.gdr_chunk_scan(*args, torch.empty(need, dtype=torch.uint8), out=(o, s))
    with pytest.raises(ValueError, match="on a GPU"):
        gdr.gdr_check_inputs(*args)
    with pytest.raises(TypeError, match="flags must be an int32"):
        gdr.gdr_check_inputs(*args, flags=torch.zeros(1, dtype=torch.int64))
    d = {k_: v_[:, 0].contiguous() for k_, v_ in t.items()}
    dargs = (d["q"], d["k"], d["v"], d["g"], d["beta"])
    st = torch.zeros(1, 4, 64, 64)
    with pytest.raises(ValueError, match="o must have shape"):
        gdr.gdr_decode_step(*dargs, st, out=(torch.empty(1, 4, 32), st))
    with pytest.raises(TypeError, match="state_out must be"):
        gdr.gdr_decode_step(*dargs, st, out=(torch.empty(1, 4, 64), st.double()))
    with pytest.raises(ValueError, match="on a GPU"):
        gdr.gdr_decode_step(*dargs, st, out=(torch.empty(1, 4, 64), st))


def call_noalloc(lib, prob, q=A, k=2 * A, v=3 * A, g=4 * A, beta=5 * A, s0=None,
                 o=6 * A, sT=7 * A):
    return lib.gdr_chunk_fwd_noalloc(ctypes.byref(prob), q, k, v, g, beta, s0, o, sT, None)


def test_noalloc_validation(lib):
    """gdr_chunk_fwd_noalloc validates like gdr_chunk_fwd, and refuses a
    problem whose workspace exceeds the built-in scratch array before any
    device call."""
    name = lambda st: binding.STATUS_NAMES[st]
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    m = re.search(r"#define\s+GDR_NOALLOC_SCRATCH_BYTES\s+\(\(size_t\)(\d+)\s*<<\s*(\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == binding.NOALLOC_SCRATCH_BYTES
    assert lib.gdr_chunk_fwd_noalloc(None, *([A] * 8), None) == 1            # GDR_ERR_NULL
    assert name(call_noalloc(lib, base(B=0))) == "GDR_ERR_SHAPE"
    assert name(call_noalloc(lib, base(), q=None)) == "GDR_ERR_NULL"
    assert name(call_noalloc(lib, base(), v=3 * A + 4)) == "GDR_ERR_ALIGN"
    assert name(call_noalloc(lib, base(), o=A)) == "GDR_ERR_ALIAS"
    assert name(call_noalloc(lib, base(), sT=2 * A)) == "GDR_ERR_ALIAS"
    big = base(B=2, T=16000, H=16, HV=32)
    assert gdr.workspace_size(big) > binding.NOALLOC_SCRATCH_BYTES
    assert name(call_noalloc(lib, big)) == "GDR_ERR_SCRATCH"
    assert gdr.status_string(11).startswith("GDR_ERR_SCRATCH")
    # the 4096-token, 12-head problem fits
    assert gdr.workspace_size(base(T=4096, H=12, HV=12)) <= binding.NOALLOC_SCRATCH_BYTES


def test_chunk_length_problems(lib):
    """Chunk lengths 32, 64 and 128 are built; 128-row chunks use one slab
    width per key dimension (32 columns for K = 128, 64 for K = 64)."""
    name = lambda st: binding.STATUS_NAMES[st]
    for K, bv in ((128, 32), (64, 64)):
        p = base(T=1000, K=K, V=128, chunk=128)
        assert gdr.workspace_size(p) > 0
        assert gdr.scan_slab(p) == bv
        assert gdr.scan_slab(base(T=1000, K=K, chunk=128, slab=bv)) == bv
        other = 64 if bv == 32 else 32
        assert name(call_fwd(lib, base(T=1000, K=K, chunk=128, slab=other))) == "GDR_ERR_UNSUPPORTED"
    for C in (16, 48, 96, 256):
        assert name(call_fwd(lib, base(chunk=C))) == "GDR_ERR_UNSUPPORTED"
    # 32-row chunks: the general kernels at 32 or 64 columns (64 by default)
    for K in (64, 128):
        p = base(T=1000, K=K, V=128, chunk=32)
        assert gdr.workspace_size(p) > 0
        assert gdr.scan_slab(p) == 64
        for bv in (32, 64):
            assert gdr.scan_slab(base(T=1000, K=K, chunk=32, slab=bv)) == bv
    assert name(call_fwd(lib, base(chunk=-64))) == "GDR_ERR_ARG"
    # chunk 0 is the automatic choice: 64-row chunks, the same workspace,
    # segments and slab as asking for 64
    for kw in (dict(T=4096, H=12, HV=12), dict(T=16000, B=2, H=16, HV=32),
               dict(T=8192, B=4, H=16, HV=16, per_channel=True), dict(T=300, K=64, V=64)):
        auto, c64 = base(chunk=0, **kw), base(chunk=64, **kw)
        assert gdr.workspace_size(auto) == gdr.workspace_size(c64) > 0
        assert gdr.scan_segments(auto) == gdr.scan_segments(c64)
        assert gdr.scan_slab(auto) == gdr.scan_slab(c64)
    # the workspace per token: the same W^ and q/k fragments, A^ keeps the
    # lower-triangular k-blocks (20 of 32 fragments at C = 128, 6 of 8 at 64)
    w64 = gdr.workspace_size(base(T=4096, H=12, HV=12, segments=1))
    w128 = gdr.workspace_size(base(T=4096, H=12, HV=12, segments=1, chunk=128))
    nc = 12 * 64                       # value-head chunks of 64 rows
    assert w128 - w64 == (nc // 2) * (20 - 2 * 6) * 512 * 2 - (nc // 2) * 256 * 4
    assert gdr.scan_segments(base(T=4096, H=12, HV=12, chunk=128, segments=3)) == 3


def test_grid_limit_cannot_wrap(lib):
    """Shapes whose workgroup count B HV N passes 2^31 are GDR_ERR_SHAPE, also
    where the 64-bit product B HV N would wrap to a small value (B = HV = 2^19
    with N = 2^26 chunks of 32 rows is exactly 2^64) and where T + C - 1 passes
    INT_MAX; the largest single sequence stays valid."""
    M = 2 ** 31 - 1
    wrap = gdr.problem(2 ** 19, M, 2 ** 19, 2 ** 19, 128, 128, chunk=32)
    assert gdr.workspace_size(wrap) == 0
    assert lib.gdr_chunk_scan_segments(ctypes.byref(wrap)) == 0
    assert call_fwd(lib, wrap) == 2
    assert gdr.workspace_size(gdr.problem(2 ** 16, 64, 1, 2 ** 16, 128, 128)) == 0
    assert gdr.workspace_size(gdr.problem(M, M, M, M, 128, 128)) == 0
    for chunk in (0, 32, 64, 128):
        one = gdr.problem(1, M, 1, 1, 128, 128, chunk=chunk)
        C = chunk or 64
        assert gdr.workspace_size(one) >= -(-M // C) * 128 * C * 2   # W^ alone
        assert 1 <= lib.gdr_chunk_scan_segments(ctypes.byref(one)) <= -(-M // C)


def _valid_by_the_header(B, T, H, HV, K, V, chunk, pc, scale, dtype, seg, slab, l2, rule, odt):
    """The validity rules gdr.h states for gdr_problem, written out."""
    import math
    if min(B, T, H, HV, K, V) < 1 or HV % H:
        return False
    if dtype not in (0, 1, 2) or odt not in (0, 1, 2):
        return False
    if pc not in (0, 1) or l2 not in (0, 1) or rule not in (0, 1) or not math.isfinite(scale):
        return False
    if chunk not in (0, 32, 64, 128) or K not in (64, 128) or V not in (64, 128):
        return False
    if seg < 0 or slab not in (0, 32, 64):
        return False
    C = chunk or 64
    if C == 128 and slab not in (0, 32 if K == 128 else 64):
        return False
    N = -(-T // C)
    return B * HV * N + 8 * HV <= 2 ** 31 - 1


def test_validation_fuzz(lib):
    """Arbitrary field values, extreme ones included: the size, segment and
    slab queries agree with each other and with the header's validity rules,
    no call crashes, and a call with NULL buffers never reports success."""
    from hypothesis import given, settings, strategies as st, HealthCheck
    edge = st.sampled_from([-2 ** 31, -1, 0, 1, 2, 3, 32, 63, 64, 65, 127, 128, 2 ** 16,
                            2 ** 19, 2 ** 24, 2 ** 31 - 1])
    small = st.one_of(st.integers(-2, 300), edge)
    field = st.one_of(st.integers(-2, 3), edge)
    kv = st.one_of(st.sampled_from([64, 128]), small)

    @settings(max_examples=600, deadline=None, derandomize=True,
              suppress_health_check=list(HealthCheck))
    @given(B=small, T=small, H=small, HV=small, K=kv, V=kv,
           chunk=st.one_of(st.sampled_from([0, 32, 64, 128]), small), pc=field,
           scale=st.floats(width=32), dtype=field, seg=small,
           slab=st.one_of(st.sampled_from([0, 32, 64]), small), l2=field, rule=field,
           odt=field)
    def run(B, T, H, HV, K, V, chunk, pc, scale, dtype, seg, slab, l2, rule, odt):
        p = binding.GdrProblem(B, T, H, HV, K, V, chunk, pc, scale, dtype, seg, slab, l2, rule,
                               odt)
        ws = lib.gdr_chunk_fwd_workspace_size(ctypes.byref(p))
        nseg = lib.gdr_chunk_scan_segments(ctypes.byref(p))
        width = lib.gdr_chunk_scan_slab(ctypes.byref(p))
        valid = _valid_by_the_header(B, T, H, HV, K, V, chunk, pc, scale, dtype, seg, slab, l2,
                                     rule, odt)
        assert (ws > 0) == valid and (nseg > 0) == valid and (width > 0) == valid
        if valid:
            N = -(-T // (chunk or 64))
            assert 1 <= nseg <= N and width in (32, 64)
            assert ws >= B * HV * N * K * (chunk or 64) * 2   # W^ alone
        st_fwd = lib.gdr_chunk_fwd(ctypes.byref(p), *([None] * 8), None, 0, None)
        st_dec = lib.gdr_decode_step(ctypes.byref(p), *([None] * 8), None)
        st_chk = lib.gdr_check_inputs(ctypes.byref(p), *([None] * 6), None)
        for s in (st_fwd, st_dec, st_chk):
            assert s != 0 and lib.gdr_status_string(s)

    run()
