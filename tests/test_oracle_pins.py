"""Pins of the fp64 oracle against what the pages and the mathematics fix.

CPU only.  Every function in oracle/ is checked here against something other
than itself: hand-derived golden values, closed forms, a Kronecker-product
brute force, the page's claim that the chunk form equals the recurrence, the
three UT inverse forms the pages give, and structural properties (segment
split, linearity, grouped-head equivalence).
"""
import glob
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd_problem(rng, B=1, T=40, H=2, HV=2, K=8, V=6, per_channel=False,
                s0=False, g_lo=-0.6, g_hi=0.0, normalize=True):
    q = rng.standard_normal((B, T, H, K))
    k = rng.standard_normal((B, T, H, K))
    if normalize:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, HV, V))
    gshape = (B, T, HV, K) if per_channel else (B, T, HV)
    g = rng.uniform(g_lo, g_hi, gshape)
    beta = rng.uniform(0.05, 1.0, (B, T, HV))
    S0 = 0.3 * rng.standard_normal((B, HV, K, V)) if s0 else None
    return q, k, v, g, beta, S0


def rel(a, b):
    return np.abs(a - b).max() / max(np.sqrt((b ** 2).mean()), 1e-300)


# ---------------------------------------------------------------- golden ----
@pytest.mark.parametrize("path", sorted(glob.glob(os.path.join(GOLDEN, "hand_*.json"))))
def test_golden_hand_derived(path):
    d = json.load(open(path))
    arr = lambda x: None if x is None else np.array(x, dtype=np.float64)
    q, k, v, g, beta, s0 = (arr(d[n]) for n in ("q", "k", "v", "g", "beta", "s0"))
    o_ref, s_ref = arr(d["o"]), arr(d["final_state"])
    o, s = oracle.recurrence(q, k, v, g, beta, d["scale"], s0)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(s, s_ref, rtol=0, atol=1e-12)
    for C in (1, 2, 4):
        r = oracle.chunk_forward(q, k, v, g, beta, d["scale"], C, s0)
        np.testing.assert_allclose(r["o"], o_ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(r["final_state"], s_ref, rtol=0, atol=1e-12)


# ------------------------------------------- chunk form == recurrence -------
@pytest.mark.parametrize("per_channel", [False, True])
@pytest.mark.parametrize("C", [1, 16, 32, 64, 128, 200])
@pytest.mark.parametrize("T,H,HV,s0", [(200, 2, 2, False), (130, 1, 2, True),
                                       (77, 2, 4, True)])
def test_chunk_form_equals_recurrence(per_channel, C, T, H, HV, s0):
    """sec-03 notes: the chunk form reproduces the naive recurrence exactly."""
    rng = np.random.default_rng(T * 7 + C + HV)
    q, k, v, g, beta, S0 = rnd_problem(rng, B=2, T=T, H=H, HV=HV,
                                       per_channel=per_channel, s0=s0)
    o, s = oracle.recurrence(q, k, v, g, beta, 0.35, S0)
    r = oracle.chunk_forward(q, k, v, g, beta, 0.35, C, S0)
    assert rel(r["o"], o) < 1e-12
    assert rel(r["final_state"], s) < 1e-12


def test_chunk_form_positive_g():
    """g may be positive (the scalar-g page's demo draws g = 0.1 N(0,1))."""
    rng = np.random.default_rng(5)
    q, k, v, g, beta, S0 = rnd_problem(rng, T=96, g_lo=-0.2, g_hi=0.2, s0=True)
    o, s = oracle.recurrence(q, k, v, g, beta, 0.5, S0)
    r = oracle.chunk_forward(q, k, v, g, beta, 0.5, 32, S0)
    assert rel(r["o"], o) < 1e-12 and rel(r["final_state"], s) < 1e-12


# ------------------------------------------------------- closed forms -------
def test_beta0_g0_keeps_state():
    rng = np.random.default_rng(1)
    q, k, v, g, beta, S0 = rnd_problem(rng, B=1, T=50, s0=True)
    g[:] = 0.0
    beta[:] = 0.0
    o, s = oracle.recurrence(q, k, v, g, beta, 0.7, S0)
    assert np.array_equal(s, S0)
    G = 1
    o_ref = 0.7 * np.einsum("bthk,bhkv->bthv", q, S0)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-14)
    r = oracle.chunk_forward(q, k, v, g, beta, 0.7, 16, S0)
    np.testing.assert_allclose(r["final_state"], S0, rtol=0, atol=1e-14)
    np.testing.assert_allclose(r["o"], o_ref, rtol=0, atol=1e-14)


def test_orthonormal_keys_closed_form():
    """With orthonormal keys the erase term only sees the initial state."""
    rng = np.random.default_rng(2)
    K, V, T = 12, 5, 10
    Qm, _ = np.linalg.qr(rng.standard_normal((K, K)))
    k = Qm[:, :T].T.reshape(1, T, 1, K)
    q = rng.standard_normal((1, T, 1, K))
    v = rng.standard_normal((1, T, 1, V))
    g = rng.uniform(-0.5, 0.0, (1, T, 1))
    beta = rng.uniform(0.1, 1.0, (1, T, 1))
    S0 = rng.standard_normal((1, 1, K, V))
    scale = 0.9
    Gam = np.cumsum(g[0, :, 0])
    u = np.stack([beta[0, t, 0] * (v[0, t, 0] - np.exp(Gam[t]) * S0[0, 0].T @ k[0, t, 0])
                  for t in range(T)])
    S_T = np.exp(Gam[-1]) * S0[0, 0] + sum(
        np.exp(Gam[-1] - Gam[t]) * np.outer(k[0, t, 0], u[t]) for t in range(T))
    o_ref = np.stack([scale * (np.exp(Gam[t]) * S0[0, 0].T @ q[0, t, 0] + sum(
        np.exp(Gam[t] - Gam[s]) * u[s] * (k[0, s, 0] @ q[0, t, 0]) for s in range(t + 1)))
        for t in range(T)])
    o, s = oracle.recurrence(q, k, v, g, beta, scale, S0)
    np.testing.assert_allclose(s[0, 0], S_T, rtol=0, atol=1e-13)
    np.testing.assert_allclose(o[0, :, 0], o_ref, rtol=0, atol=1e-13)
    r = oracle.chunk_forward(q, k, v, g, beta, scale, 4, S0)
    np.testing.assert_allclose(r["final_state"][0, 0], S_T, rtol=0, atol=1e-13)
    np.testing.assert_allclose(r["o"][0, :, 0], o_ref, rtol=0, atol=1e-13)


def test_repeated_unit_key_recalls_value():
    """beta = 1, g = 0, one repeated unit key: S^T k = v_t after each step."""
    rng = np.random.default_rng(3)
    K, V, T = 16, 8, 70
    kk = rng.standard_normal(K)
    kk /= np.linalg.norm(kk)
    k = np.broadcast_to(kk, (1, T, 1, K)).copy()
    q = k.copy()
    v = rng.standard_normal((1, T, 1, V))
    g = np.zeros((1, T, 1))
    beta = np.ones((1, T, 1))
    S0 = rng.standard_normal((1, 1, K, V))
    o, s = oracle.recurrence(q, k, v, g, beta, 0.25, S0)
    np.testing.assert_allclose(o, 0.25 * v, rtol=0, atol=1e-13)
    r = oracle.chunk_forward(q, k, v, g, beta, 0.25, 32, S0)
    np.testing.assert_allclose(r["o"], 0.25 * v, rtol=0, atol=1e-12)


@pytest.mark.parametrize("per_channel", [False, True])
def test_reset_by_large_negative_g(per_channel):
    """g = -800 wipes the state each step: o_t = scale beta_t <q_t,k_t> v_t."""
    rng = np.random.default_rng(4)
    q, k, v, g, beta, S0 = rnd_problem(rng, T=70, per_channel=per_channel, s0=True)
    g[:] = -800.0
    scale = 0.6
    o, s = oracle.recurrence(q, k, v, g, beta, scale, S0)
    qk = np.einsum("bthk,bthk->bth", q, k)
    o_ref = scale * (beta * qk)[..., None] * v
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-13)
    s_ref = np.einsum("bhk,bhv->bhkv", beta[:, -1, :, None] * k[:, -1], v[:, -1])
    np.testing.assert_allclose(s, s_ref, rtol=0, atol=1e-13)
    r = oracle.chunk_forward(q, k, v, g, beta, scale, 64, S0)
    assert np.isfinite(r["o"]).all()
    np.testing.assert_allclose(r["o"], o_ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(r["final_state"], s_ref, rtol=0, atol=1e-13)


def test_standard_basis_keys_per_channel_closed_form():
    """Per-channel decay with standard-basis keys: every state row evolves alone.

    Row d decays by exp(g_t[d]) each step; when k_t = e_d the write blends
    that row towards v_t: row <- (1 - beta_t) row + beta_t v_t.
    """
    rng = np.random.default_rng(6)
    K, V, T = 6, 4, 30
    idx = rng.integers(0, K, T)
    k = np.zeros((1, T, 1, K))
    k[0, np.arange(T), 0, idx] = 1.0
    q = rng.standard_normal((1, T, 1, K))
    v = rng.standard_normal((1, T, 1, V))
    g = rng.uniform(-0.7, 0.0, (1, T, 1, K))
    beta = rng.uniform(0.1, 1.0, (1, T, 1))
    S0 = rng.standard_normal((1, 1, K, V))
    rows = S0[0, 0].copy()
    o_ref = np.zeros((T, V))
    for t in range(T):
        rows = np.exp(g[0, t, 0])[:, None] * rows
        d = idx[t]
        rows[d] = (1.0 - beta[0, t, 0]) * rows[d] + beta[0, t, 0] * v[0, t, 0]
        o_ref[t] = 0.8 * q[0, t, 0] @ rows
    o, s = oracle.recurrence(q, k, v, g, beta, 0.8, S0)
    np.testing.assert_allclose(s[0, 0], rows, rtol=0, atol=1e-13)
    np.testing.assert_allclose(o[0, :, 0], o_ref, rtol=0, atol=1e-13)
    r = oracle.chunk_forward(q, k, v, g, beta, 0.8, 8, S0)
    np.testing.assert_allclose(r["o"][0, :, 0], o_ref, rtol=0, atol=1e-12)


# ---------------------------------------------- Kronecker brute force -------
@pytest.mark.parametrize("per_channel", [False, True])
def test_kronecker_brute_force(per_channel):
    """vec(S_t) = (I_V kron (I - beta k k^T) diag(exp g_t)) vec(S_{t-1}) + beta (v kron k)."""
    rng = np.random.default_rng(7 + per_channel)
    K, V, T = 3, 2, 6
    q, k, v, g, beta, S0 = rnd_problem(rng, B=1, T=T, H=1, HV=1, K=K, V=V,
                                       per_channel=per_channel, s0=True,
                                       normalize=False)
    x = S0[0, 0].reshape(-1, order="F")            # column-major vec
    o_ref = []
    for t in range(T):
        kt, qt, vt, bt = k[0, t, 0], q[0, t, 0], v[0, t, 0], beta[0, t, 0]
        dg = np.exp(g[0, t, 0]) * np.ones(K)
        Amat = (np.eye(K) - bt * np.outer(kt, kt)) @ np.diag(dg)
        x = np.kron(np.eye(V), Amat) @ x + bt * np.kron(vt, kt)
        o_ref.append(1.3 * np.kron(np.eye(V), qt[None, :]) @ x)
    o, s = oracle.recurrence(q, k, v, g, beta, 1.3, S0)
    np.testing.assert_allclose(s[0, 0].reshape(-1, order="F"), x, rtol=0, atol=1e-12)
    np.testing.assert_allclose(o[0, :, 0], np.array(o_ref), rtol=0, atol=1e-12)


# ----------------------------------------------- structural properties ------
@pytest.mark.parametrize("per_channel", [False, True])
def test_segment_split(per_channel):
    rng = np.random.default_rng(8)
    q, k, v, g, beta, S0 = rnd_problem(rng, B=1, T=150, H=1, HV=2,
                                       per_channel=per_channel, s0=True)
    T1 = 37
    o, s = oracle.recurrence(q, k, v, g, beta, 0.5, S0)
    cut = lambda a, sl: a[:, sl]
    o1, s1 = oracle.recurrence(*(cut(a, slice(0, T1)) for a in (q, k, v, g, beta)), 0.5, S0)
    o2, s2 = oracle.recurrence(*(cut(a, slice(T1, None)) for a in (q, k, v, g, beta)), 0.5, s1)
    np.testing.assert_allclose(np.concatenate([o1, o2], 1), o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(s2, s, rtol=0, atol=1e-12)
    r1 = oracle.chunk_forward(*(cut(a, slice(0, T1)) for a in (q, k, v, g, beta)), 0.5, 16, S0)
    r2 = oracle.chunk_forward(*(cut(a, slice(T1, None)) for a in (q, k, v, g, beta)), 0.5, 16,
                              r1["final_state"])
    np.testing.assert_allclose(r2["final_state"], s, rtol=0, atol=1e-12)


def test_joint_linearity_in_state_and_values():
    rng = np.random.default_rng(9)
    q, k, v, g, beta, S0 = rnd_problem(rng, T=60, s0=True)
    v2 = rng.standard_normal(v.shape)
    S02 = rng.standard_normal(S0.shape)
    a, b = 0.7, -1.9
    oa, sa = oracle.recurrence(q, k, v, g, beta, 0.4, S0)
    ob, sb = oracle.recurrence(q, k, v2, g, beta, 0.4, S02)
    oc, sc = oracle.recurrence(q, k, a * v + b * v2, g, beta, 0.4, a * S0 + b * S02)
    np.testing.assert_allclose(oc, a * oa + b * ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(sc, a * sa + b * sb, rtol=0, atol=1e-12)


def test_grouped_heads_equal_explicit_repeat():
    """HV = G*H with q/k head h = hv // G equals running with repeated q/k."""
    rng = np.random.default_rng(10)
    q, k, v, g, beta, S0 = rnd_problem(rng, B=2, T=45, H=2, HV=6, s0=True)
    o, s = oracle.recurrence(q, k, v, g, beta, 0.3, S0)
    rep = lambda x: np.repeat(x, 3, axis=2)        # repeat_interleave
    o2, s2 = oracle.recurrence(rep(q), rep(k), v, g, beta, 0.3, S0)
    np.testing.assert_allclose(o, o2, rtol=0, atol=0)
    np.testing.assert_allclose(s, s2, rtol=0, atol=0)
    # the modulo grouping (hv % H) is a different method: it must disagree
    tile = lambda x: np.tile(x, (1, 1, 3, 1))
    o3, _ = oracle.recurrence(tile(q), tile(k), v, g, beta, 0.3, S0)
    assert rel(o3, o) > 1e-3


def test_per_channel_with_equal_channels_is_scalar():
    rng = np.random.default_rng(11)
    q, k, v, g, beta, S0 = rnd_problem(rng, T=50, s0=True)
    gpc = np.repeat(g[..., None], k.shape[-1], axis=-1)
    o, s = oracle.recurrence(q, k, v, g, beta, 0.3, S0)
    o2, s2 = oracle.recurrence(q, k, v, gpc, beta, 0.3, S0)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-13)
    r = oracle.chunk_forward(q, k, v, gpc, beta, 0.3, 16, S0)
    np.testing.assert_allclose(r["o"], o, rtol=0, atol=1e-12)


# ---------------------------------------------------- chunk intermediates ---
def test_decayed_dot_definition_and_scalar_factoring():
    """decayed_dot vs a triple loop, and (x k^T) * exp(gam_i - gam_j) for scalar g."""
    rng = np.random.default_rng(12)
    C, K = 9, 5
    x = rng.standard_normal((C, K))
    kk = rng.standard_normal((C, K))
    gpc = np.cumsum(rng.uniform(-0.5, 0.1, (C, K)), axis=0)
    A = oracle.decayed_dot(x, kk, gpc)
    ref = np.zeros((C, C))
    for i in range(C):
        for j in range(i + 1):
            ref[i, j] = sum(x[i, d] * np.exp(gpc[i, d] - gpc[j, d]) * kk[j, d]
                            for d in range(K))
    np.testing.assert_allclose(A, ref, rtol=0, atol=1e-13)
    gs = np.cumsum(rng.uniform(-0.5, 0.1, (C, 1)), axis=0)
    As = oracle.decayed_dot(x, kk, gs)
    fact = np.tril((x @ kk.T) * np.exp(gs - gs.T))
    np.testing.assert_allclose(As, fact, rtol=0, atol=1e-13)


def test_ut_inverse_forms_agree():
    """Triangular solve == Neumann series == row iteration (pages' UT identities)."""
    rng = np.random.default_rng(13)
    q, k, v, g, beta, _ = rnd_problem(rng, B=1, T=64, H=1, HV=1, K=16, V=4)
    r = oracle.chunk_forward(q, k, v, g, beta, 0.25, 64)
    M = r["M"]
    L = M - np.eye(64)
    assert np.array_equal(np.triu(L), np.zeros_like(L))     # strictly lower
    Xs = oracle.ut_inverse_solve(M)
    Xn = oracle.ut_inverse_neumann(L)
    Xr = oracle.ut_inverse_rowloop(L)
    np.testing.assert_allclose(Xs @ M, np.broadcast_to(np.eye(64), M.shape), atol=1e-12)
    np.testing.assert_allclose(Xn, Xs, rtol=0, atol=1e-12)
    np.testing.assert_allclose(Xr, Xs, rtol=0, atol=1e-12)
    # and the UT outputs are that inverse applied to the right-hand sides
    kc = k.transpose(0, 2, 1, 3).reshape(1, 1, 1, 64, 16)
    W = Xs @ (np.exp(r["gamma"]) * kc)
    np.testing.assert_allclose(r["W"], W, rtol=0, atol=1e-12)


def test_chunk_intermediate_masks():
    rng = np.random.default_rng(14)
    q, k, v, g, beta, _ = rnd_problem(rng, B=1, T=128, H=1, HV=1, K=8, V=4)
    r = oracle.chunk_forward(q, k, v, g, beta, 0.3, 64)
    C = 64
    iu = np.triu_indices(C, 0)
    assert np.all(r["M"][..., iu[0], iu[1]] == np.eye(C)[iu])     # unit upper part
    assert np.all(np.triu(r["A_qk"], 1) == 0)                     # diagonal kept
    assert np.any(np.diagonal(r["A_qk"], axis1=-2, axis2=-1) != 0)
    gam = r["gamma"][0, 0, :, :, 0]
    np.testing.assert_allclose(gam, np.cumsum(g[0, :, 0].reshape(2, 64), axis=1), atol=1e-14)


def test_l2norm_rows_pins():
    """The row normaliser of in-kernel q/k normalisation: a hand-derived row
    ((3, 4) -> (3, 4) / sqrt(25 + 1e-6)), the closed-form norm of any output
    row, ||x|| / sqrt(||x||^2 + 1e-6), the zero row staying zero, and
    independence of the rows."""
    import math
    from oracle import l2norm_rows
    got = l2norm_rows(np.array([[3.0, 4.0]]))
    d = math.sqrt(25.0 + 1e-6)
    assert got[0, 0] == 3.0 / d and got[0, 1] == 4.0 / d
    rng = np.random.default_rng(5)
    x = rng.standard_normal((3, 5, 2, 16)) * rng.uniform(0.01, 10, (3, 5, 2, 1))
    y = l2norm_rows(x)
    nx = np.sqrt((x ** 2).sum(-1))
    np.testing.assert_allclose(np.sqrt((y ** 2).sum(-1)), nx / np.sqrt(nx ** 2 + 1e-6),
                               rtol=1e-13)
    # direction kept: y is a positive multiple of x, row by row
    np.testing.assert_allclose(y * (np.sqrt(nx ** 2 + 1e-6))[..., None], x, rtol=1e-12)
    assert not l2norm_rows(np.zeros((2, 8))).any()
    x2 = x.copy()
    x2[0, 0, 0] *= 7.0
    y2 = l2norm_rows(x2)
    np.testing.assert_array_equal(y2[1:], y[1:])


def _masked_attention(q, k, v, g, beta, scale, s0):
    """Decayed linear attention in its quadratic form (the Mamba2 SSD section
    of the "Chunkwise parallel algorithms" page, section 1.1: O = ((Q K^T) .
    Gamma) V, Gamma[t, i] = gamma_t / gamma_i for i <= t), with beta on the
    columns, the query scale, per-channel decay allowed, and the initial
    state's decayed contribution; written as dense per-head sums."""
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    G = HV // H
    o = np.zeros((B, T, HV, V))
    sT = np.zeros((B, HV, K, V))
    for b in range(B):
        for hv in range(HV):
            h = hv // G
            gg = g[b, :, hv] if g.ndim == 4 else np.repeat(g[b, :, hv][:, None], K, 1)
            Gam = np.cumsum(gg, axis=0)                     # [T, K], inclusive
            for t in range(T):
                for i in range(t + 1):
                    w = (q[b, t, h] * np.exp(Gam[t] - Gam[i]) * k[b, i, h]).sum()
                    o[b, t, hv] += scale * beta[b, i, hv] * w * v[b, i, hv]
                if s0 is not None:
                    o[b, t, hv] += scale * (q[b, t, h] * np.exp(Gam[t])) @ s0[b, hv]
            for i in range(T):
                sT[b, hv] += beta[b, i, hv] * np.outer(np.exp(Gam[T - 1] - Gam[i]) * k[b, i, h],
                                                      v[b, i, hv])
            if s0 is not None:
                sT[b, hv] += np.exp(Gam[T - 1])[:, None] * s0[b, hv]
    return o, sT


@pytest.mark.parametrize("per_channel", [False, True])
def test_linear_rule_equals_masked_attention(per_channel):
    """The linear rule (no erase) equals the quadratic masked-attention form,
    o and final state, with grouped heads and an initial state."""
    rng = np.random.default_rng(11)
    B, T, H, HV, K, V = 1, 23, 1, 2, 5, 3
    q, k = rng.standard_normal((2, B, T, H, K))
    v = rng.standard_normal((B, T, HV, V))
    beta = rng.uniform(0.1, 1.0, (B, T, HV))
    g = -rng.uniform(0.0, 0.5, (B, T, HV, K) if per_channel else (B, T, HV))
    s0 = rng.standard_normal((B, HV, K, V))
    o, s = oracle.recurrence(q, k, v, g, beta, 0.7, s0, rule="linear")
    ro, rs = _masked_attention(q, k, v, g, beta, 0.7, s0)
    np.testing.assert_allclose(o, ro, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(s, rs, rtol=1e-12, atol=1e-12)


def test_linear_rule_page_form_and_delta_difference():
    """beta = 1, scale = 1, zero state: exactly the page's O = ((Q K^T) . Gamma) V;
    and the delta rule differs from it as soon as a key meets the state."""
    rng = np.random.default_rng(12)
    B, T, H, K, V = 1, 9, 1, 4, 4
    q, k = rng.standard_normal((2, B, T, H, K))
    v = rng.standard_normal((B, T, H, V))
    g = np.log(rng.uniform(0.5, 1.0, (B, T, H)))
    one = np.ones((B, T, H))
    o, _ = oracle.recurrence(q, k, v, g, one, 1.0, None, rule="linear")
    gam = np.exp(np.cumsum(g[0, :, 0]))
    Gmask = np.tril(gam[:, None] / gam[None, :])
    page = ((q[0, :, 0] @ k[0, :, 0].T) * Gmask) @ v[0, :, 0]
    np.testing.assert_allclose(o[0, :, 0], page, rtol=1e-12, atol=1e-12)
    od, _ = oracle.recurrence(q, k, v, g, one, 1.0, None)
    assert np.abs(od - o).max() > 1e-3
    # with one token from a zero state the two rules coincide
    o1, s1 = oracle.recurrence(q[:, :1], k[:, :1], v[:, :1], g[:, :1], one[:, :1], 1.0, None,
                               rule="linear")
    o2, s2 = oracle.recurrence(q[:, :1], k[:, :1], v[:, :1], g[:, :1], one[:, :1], 1.0, None)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(s1, s2)


# ------------------------------------------- DeltaNet without decay -------
def test_deltanet_without_decay_page_chunk_form():
    """Chunkwise parallel algorithms page, section 2.4 (the matrix iteration
    form of DeltaNet, no decay), with the UT transform of section 2.3: per
    chunk, with T = (I + strictLower(diag(beta) K K^T))^-1 diag(beta),
    W = T K and U = T V, and the state S' in the page's orientation (d_v x
    d_k, the transpose of the oracle's),
        O = Q S'^T + (Q K^T * M)(U - W S'^T),   S' <- S' + (U - W S'^T)^T K,
    with M the causal mask.  The mask is read as including its diagonal (each
    token's output sees its own write, as in the recurrence).  With g = 0 and
    a unit scale the oracle's recurrence gives the same o and final state,
    chunk after chunk; excluding the diagonal from M does not."""
    rng = np.random.default_rng(24)
    K, V, C, nch = 8, 6, 5, 3
    T = C * nch
    q, k, v, _, beta, S0 = rnd_problem(rng, B=1, T=T, H=1, HV=1, K=K, V=V, s0=True)
    g = np.zeros((1, T, 1))
    o, s = oracle.recurrence(q, k, v, g, beta, 1.0, S0)

    def page_form(diag):
        Sp = S0[0, 0].T.copy()
        M = np.tril(np.ones((C, C)), 0 if diag else -1)
        outs = []
        for c in range(nch):
            sl = slice(c * C, (c + 1) * C)
            Qc, Kc, Vc, b = q[0, sl, 0], k[0, sl, 0], v[0, sl, 0], beta[0, sl, 0]
            Tm = np.linalg.inv(np.eye(C) + np.tril(np.diag(b) @ Kc @ Kc.T, -1)) @ np.diag(b)
            R = Tm @ Vc - (Tm @ Kc) @ Sp.T
            outs.append(Qc @ Sp.T + (Qc @ Kc.T * M) @ R)
            Sp = Sp + R.T @ Kc
        return np.concatenate(outs)[None, :, None], Sp.T[None, None]

    po, ps = page_form(True)
    assert rel(po, o) < 1e-12 and rel(ps, s) < 1e-12
    assert rel(page_form(False)[0], o) > 1e-2


# ------------------------------------------------- per-head recurrence ------
@pytest.mark.parametrize("per_channel", [False, True])
def test_recurrence_heads_equals_full_recurrence(per_channel):
    """recurrence_heads (the reference of the full-size sampled-head GPU tests)
    slices one (b, hv) scan at a time, with q/k head h = hv // G (the
    repeat_interleave grouping of the sec-03 rearrange step) and the initial
    state of that head.  Every head, and a cut T, must equal the recurrence
    run on all heads at once bit for bit (each scan is independent)."""
    from chunkwise_gated_delta_cumsum_amd.inputs import Workload, make_inputs
    w = Workload("pin_heads", B=2, T=70, H=2, HV=4, K=8, V=8, per_channel=per_channel,
                 dtype="fp32", g_mu=1.0, s0_std=0.1, seed=5)
    inp = make_inputs(w)
    heads = [(b, hv) for b in range(w.B) for hv in range(w.HV)]
    for T in (w.T, 33):
        o, s = oracle.recurrence(inp.q[:, :T], inp.k[:, :T], inp.v[:, :T], inp.g[:, :T],
                                 inp.beta[:, :T], inp.scale, inp.s0)
        got = oracle.recurrence_heads(inp, heads, T=T)
        assert sorted(got) == heads
        for b, hv in heads:
            go, gs = got[(b, hv)]
            assert go.shape == (T, w.V) and gs.shape == (w.K, w.V)
            np.testing.assert_array_equal(go, o[b, :, hv])
            np.testing.assert_array_equal(gs, s[b, hv])
    # the modulo grouping (h = hv % H) is a different map: value head 1 of
    # batch 0 would read q/k head 1 instead of 0, and must disagree
    o, _ = oracle.recurrence(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.scale, inp.s0)
    wrong = oracle.recurrence(inp.q[:1, :, 1:2], inp.k[:1, :, 1:2], inp.v[:1, :, 1:2],
                              inp.g[:1, :, 1:2], inp.beta[:1, :, 1:2], inp.scale,
                              inp.s0[:1, 1:2])[0]
    assert rel(wrong[0, :, 0], o[0, :, 1]) > 1e-3
