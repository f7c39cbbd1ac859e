"""Property tests of the fp64 oracle on tiny shapes (CPU only, Hypothesis).

Each property holds for every shape and value the strategies can draw, so a
mistake that only shows on some shapes (an index off by one at a chunk edge,
a transposed operand that happens to be square, a grouped-head map that
agrees at G = 1) fails one of them.  The draws are derandomized: every run
checks the same examples, and a failure shrinks to a small one.

* The chunk form equals the recurrence at any chunk length, ragged T,
  grouped heads, one decay per row or per key channel, with or without an
  initial state (the chunkwise page's claim that the chunk form is the
  recurrence regrouped).
* The recurrence equals its Kronecker-product form, vec(S_t) = A_t vec(S_{t-1})
  + beta_t (v_t kron k_t), for the delta and the linear rule.
* Relabelling key channels permutes the state's rows and leaves o unchanged;
  relabelling value channels permutes o's and the state's columns.
* Cutting the sequence anywhere and carrying the state gives the same o and
  final state; batches are independent; o is linear in the query scale.
* beta = 0 leaves only the decay: closed forms for o and the final state.
* The linear rule equals the masked quadratic form O = ((Q K^T) . Gamma) V.
* The three UT inverse forms agree and invert I + L for any strictly lower L.

The GPU side has its own seeded random draws (test_random_configs_gpu.py).
"""
import numpy as np
from hypothesis import given, settings, strategies as st, HealthCheck

import oracle
from test_oracle_pins import _masked_attention

PROP = settings(max_examples=60, deadline=None, derandomize=True, database=None,
                suppress_health_check=[HealthCheck.too_slow])


@st.composite
def problems(draw, max_T=48, max_K=9, max_V=7):
    """A tiny problem: (q, k, v, g, beta, s0 or None, scale) in fp64."""
    B = draw(st.integers(1, 2))
    H = draw(st.integers(1, 2))
    G = draw(st.integers(1, 3))
    K = draw(st.integers(1, max_K))
    V = draw(st.integers(1, max_V))
    T = draw(st.integers(1, max_T))
    per_channel = draw(st.booleans())
    with_s0 = draw(st.booleans())
    g_lo = draw(st.sampled_from([-0.05, -0.6, -3.0]))
    seed = draw(st.integers(0, 2 ** 31 - 1))
    rng = np.random.default_rng(seed)
    HV = H * G
    q = rng.standard_normal((B, T, H, K))
    k = rng.standard_normal((B, T, H, K))
    k /= np.maximum(np.linalg.norm(k, axis=-1, keepdims=True), 1e-3)
    v = rng.standard_normal((B, T, HV, V))
    g = rng.uniform(g_lo, 0.0, (B, T, HV, K) if per_channel else (B, T, HV))
    beta = rng.uniform(0.0, 1.0, (B, T, HV))
    s0 = 0.5 * rng.standard_normal((B, HV, K, V)) if with_s0 else None
    scale = float(rng.uniform(0.1, 2.0))
    return q, k, v, g, beta, s0, scale


def close(a, b, tol=1e-10):
    """Max abs difference within tol times the reference's rms (and 1e-300)."""
    a, b = np.asarray(a), np.asarray(b)
    assert a.shape == b.shape
    den = max(np.sqrt((b ** 2).mean()) if b.size else 0.0, 1e-300)
    err = np.abs(a - b).max() / den if b.size else 0.0
    assert err <= tol, err


@PROP
@given(problems(), st.integers(1, 56))
def test_chunk_form_equals_recurrence(p, C):
    q, k, v, g, beta, s0, scale = p
    o, s = oracle.recurrence(q, k, v, g, beta, scale, s0)
    r = oracle.chunk_forward(q, k, v, g, beta, scale, C, s0)
    close(r["o"], o)
    close(r["final_state"], s)


@PROP
@given(st.integers(1, 4), st.integers(1, 3), st.integers(1, 7), st.booleans(),
       st.sampled_from(["delta", "linear"]), st.integers(0, 2 ** 31 - 1))
def test_kronecker_form(K, V, T, per_channel, rule, seed):
    rng = np.random.default_rng(seed)
    q, k = rng.standard_normal((2, 1, T, 1, K))
    v = rng.standard_normal((1, T, 1, V))
    g = rng.uniform(-1.0, 0.2, (1, T, 1, K) if per_channel else (1, T, 1))
    beta = rng.uniform(0.0, 1.0, (1, T, 1))
    s0 = rng.standard_normal((1, 1, K, V))
    scale = 0.8
    x = s0[0, 0].reshape(-1, order="F")              # column-major vec of K x V
    o_ref = []
    for t in range(T):
        kt, qt, vt, bt = k[0, t, 0], q[0, t, 0], v[0, t, 0], beta[0, t, 0]
        D = np.diag(np.exp(g[0, t, 0]) * np.ones(K))
        erase = np.eye(K) - bt * np.outer(kt, kt) if rule == "delta" else np.eye(K)
        x = np.kron(np.eye(V), erase @ D) @ x + bt * np.kron(vt, kt)
        o_ref.append(scale * np.kron(np.eye(V), qt[None, :]) @ x)
    o, s = oracle.recurrence(q, k, v, g, beta, scale, s0, rule=rule)
    close(s[0, 0].reshape(-1, order="F"), x, 1e-12)
    close(o[0, :, 0], np.array(o_ref), 1e-12)


@PROP
@given(problems(), st.integers(0, 2 ** 31 - 1))
def test_key_channel_relabelling(p, seed):
    q, k, v, g, beta, s0, scale = p
    K = q.shape[-1]
    perm = np.random.default_rng(seed).permutation(K)
    o, s = oracle.recurrence(q, k, v, g, beta, scale, s0)
    gp = g[..., perm] if g.ndim == 4 else g
    s0p = s0[:, :, perm, :] if s0 is not None else None
    o2, s2 = oracle.recurrence(q[..., perm], k[..., perm], v, gp, beta, scale, s0p)
    close(o2, o, 1e-12)
    close(s2, s[:, :, perm, :], 1e-12)


@PROP
@given(problems(), st.integers(0, 2 ** 31 - 1))
def test_value_channel_relabelling(p, seed):
    q, k, v, g, beta, s0, scale = p
    V = v.shape[-1]
    perm = np.random.default_rng(seed).permutation(V)
    o, s = oracle.recurrence(q, k, v, g, beta, scale, s0)
    s0p = s0[..., perm] if s0 is not None else None
    o2, s2 = oracle.recurrence(q, k, v[..., perm], g, beta, scale, s0p)
    close(o2, o[..., perm], 1e-13)
    close(s2, s[..., perm], 1e-13)


@PROP
@given(problems(), st.floats(0.0, 1.0), st.sampled_from(["delta", "linear"]))
def test_sequence_cut_carries_state(p, frac, rule):
    q, k, v, g, beta, s0, scale = p
    T = q.shape[1]
    t = int(round(frac * T))
    o, s = oracle.recurrence(q, k, v, g, beta, scale, s0, rule=rule)
    parts = [a[:, :t] for a in (q, k, v, g, beta)], [a[:, t:] for a in (q, k, v, g, beta)]
    if t == 0:
        o1, s1 = np.zeros((q.shape[0], 0) + o.shape[2:]), (
            s0 if s0 is not None else np.zeros_like(s))
    else:
        o1, s1 = oracle.recurrence(*parts[0], scale, s0, rule=rule)
    if t == T:
        o2, s2 = np.zeros((q.shape[0], 0) + o.shape[2:]), s1
    else:
        o2, s2 = oracle.recurrence(*parts[1], scale, s1, rule=rule)
    close(np.concatenate([o1, o2], axis=1), o, 1e-12)
    close(s2, s, 1e-12)


@PROP
@given(problems())
def test_batches_independent_and_scale_linear(p):
    q, k, v, g, beta, s0, scale = p
    o, s = oracle.recurrence(q, k, v, g, beta, scale, s0)
    for b in range(q.shape[0]):
        sl = slice(b, b + 1)
        ob, sb = oracle.recurrence(q[sl], k[sl], v[sl], g[sl], beta[sl], scale,
                                   s0[sl] if s0 is not None else None)
        np.testing.assert_array_equal(ob, o[sl])
        np.testing.assert_array_equal(sb, s[sl])
    o3, s3 = oracle.recurrence(q, k, v, g, beta, 3.0 * scale, s0)
    np.testing.assert_array_equal(s3, s)         # the state never sees the scale
    close(o3, 3.0 * o, 1e-13)


@PROP
@given(problems(), st.sampled_from(["delta", "linear"]))
def test_beta_zero_is_pure_decay(p, rule):
    """beta = 0: S_t = diag(exp(G_t)) S0 with G_t the running sum of g, and
    o_t = scale q_t^T S_t (zero without an initial state)."""
    q, k, v, g, beta, s0, scale = p
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    G = HV // H
    o, s = oracle.recurrence(q, k, v, g, np.zeros_like(beta), scale, s0, rule=rule)
    base = s0 if s0 is not None else np.zeros((B, HV, K, V))
    gg = g if g.ndim == 4 else np.repeat(g[..., None], K, axis=3)   # [B, T, HV, K]
    Gam = np.cumsum(gg, axis=1)
    S_t = np.exp(Gam)[..., None] * base[:, None]                      # [B, T, HV, K, V]
    qh = np.repeat(q, G, axis=2)                                      # h = hv // G
    o_ref = scale * np.einsum("bthk,bthkv->bthv", qh, S_t)
    close(s, S_t[:, -1], 1e-12)
    if s0 is None:
        np.testing.assert_array_equal(o, np.zeros_like(o))
    else:
        close(o, o_ref, 1e-12)


@settings(max_examples=25, deadline=None, derandomize=True, database=None)
@given(problems(max_T=14, max_K=5, max_V=4))
def test_linear_rule_is_masked_attention(p):
    q, k, v, g, beta, s0, scale = p
    o, s = oracle.recurrence(q, k, v, g, beta, scale, s0, rule="linear")
    ro, rs = _masked_attention(q, k, v, g, beta, scale, s0)
    close(o, ro, 1e-11)
    close(s, rs, 1e-11)


@PROP
@given(st.integers(1, 40), st.floats(0.01, 0.5), st.integers(0, 2 ** 31 - 1))
def test_ut_inverse_forms(n, mag, seed):
    rng = np.random.default_rng(seed)
    L = np.tril(mag * rng.standard_normal((n, n)), -1)
    M = np.eye(n) + L
    a = oracle.ut_inverse_solve(M)
    b = oracle.ut_inverse_neumann(L)
    c = oracle.ut_inverse_rowloop(L)
    close(a @ M, np.eye(n), 1e-11)
    close(b, a, 1e-11)
    close(c, a, 1e-11)
    np.testing.assert_array_equal(np.triu(a, 1), np.zeros((n, n)))
    np.testing.assert_array_equal(np.diag(a), np.ones(n))
