"""fp64 NumPy/SciPy chunkwise form of the gated delta rule, step by step.

TEST INFRASTRUCTURE ONLY: imported by tests/ (and smoke/bench checks), never
by the product path.  It shares nothing with the HIP path.

It takes the steps in the order and notation of the sec-03 notes ("Chunkwise",
sections "in-chunk cumsum and lower-triangular solve", "code comparison",
"inter-chunk recurrence" and "decayed dot function"), written from the
equations there, and exposes every intermediate so the device kernels can be
checked step by step:

  1. split T into N chunks of C rows; q/k head h serves value heads
     h*G .. h*G+G-1 (repeat_interleave grouping); q <- q * scale
  2. gamma = inclusive cumsum of g inside each chunk
  3. A_kk = decayed_dot(k, k, gamma),  A_ij = <x_i, exp(gamma_i - gamma_j) k_j>
  4. M = I + strictly_lower(A_kk * beta_j)          (beta scales columns)
  5. W = M^-1 (exp(gamma) k),  U = M^-1 v           (UT transform, a
                                                     triangular solve)
  6. A_qk = lower_with_diagonal(decayed_dot(q, k, gamma) * beta_j)
  7. for each chunk, serially:
        r  = U - W S
        o  = (q exp(gamma)) S + A_qk r
        S <- diag(exp(gamma_last)) S + (exp(gamma_last - gamma) k)^T (beta r)

Readings where the listing is loose:
  * ``(decay * k_n).T`` transposes the last two axes; ``r * beta_n`` scales
    row j of r by beta_j.
  * T not a multiple of C: pad q, k, v, g, beta with zeros (the scalar-g
    kernel page pads the same way), then drop the padded rows of o.  Padded
    rows have beta = 0 and g = 0, so they leave S unchanged.
  * decayed_dot only forms entries with j <= i: both uses mask j > i away,
    and exp(gamma_i - gamma_j) for j > i can overflow (the scalar-g page
    masks before exp for the same reason).
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np
from scipy.linalg import solve_triangular

__all__ = ["decayed_dot", "chunk_forward", "ut_inverse_solve",
           "ut_inverse_neumann", "ut_inverse_rowloop"]


def decayed_dot(x: np.ndarray, k: np.ndarray, gam: np.ndarray) -> np.ndarray:
    """A[..., i, j] = <x_i, exp(gam_i - gam_j) * k_j> for j <= i, else 0.

    x, k: [..., C, K]; gam: [..., C, K] (per-channel) or [..., C, 1] (one
    log-decay per row, broadcast over K).  Row i is built from its own decay
    vector, one row at a time, as the sec-03 "decayed dot function" defines.
    """
    C = x.shape[-2]
    A = np.zeros(x.shape[:-2] + (C, C), dtype=np.float64)
    for i in range(C):
        decay = np.exp(gam[..., i:i + 1, :] - gam[..., :i + 1, :])
        A[..., i, :i + 1] = np.einsum("...jd,...jd->...j",
                                      x[..., i:i + 1, :] * decay,
                                      k[..., :i + 1, :])
    return A


def ut_inverse_solve(M: np.ndarray) -> np.ndarray:
    """M^-1 for a batch of unit-lower-triangular M by a triangular solve."""
    C = M.shape[-1]
    flat = M.reshape(-1, C, C)
    out = np.empty_like(flat)
    eye = np.eye(C)
    for i in range(flat.shape[0]):
        out[i] = solve_triangular(flat[i], eye, lower=True)
    return out.reshape(M.shape)


def ut_inverse_neumann(L: np.ndarray) -> np.ndarray:
    """(I + L)^-1 = sum_{n < C} (-L)^n for strictly lower L (nilpotent).

    The Neumann series of the "Chunkwise parallel algorithms" page, section
    2.3, taken with N = -L so that (I - N)^-1 = sum N^n.
    """
    C = L.shape[-1]
    N = -L
    term = np.broadcast_to(np.eye(C), L.shape).copy()
    acc = term.copy()
    for _ in range(1, C):
        term = term @ N
        acc = acc + term
    return acc


def ut_inverse_rowloop(L: np.ndarray) -> np.ndarray:
    """(I + L)^-1 built one row at a time (the row iteration with Q = -N).

    Starting from Q = -L, row i becomes Q[i,:i] + sum_m Q[i,m] Q[m,:i] using
    the rows m < i already finished; the inverse is Q + I.  This is the
    iteration of the "Chunkwise parallel algorithms" page, section 2.3, and
    the row loop that the scalar-g kernel page replaces by one solve.
    """
    C = L.shape[-1]
    Q = -np.array(L, dtype=np.float64)
    for i in range(1, C):
        row = Q[..., i, :i].copy()
        sub = Q[..., :i, :i].copy()
        Q[..., i, :i] = row + (row[..., :, None] * sub).sum(-2)
    return Q + np.eye(C)


def _to_chunks(x: np.ndarray, C: int) -> np.ndarray:
    """[B, T, Hx, D] -> [B, Hx, N, C, D] (T already a multiple of C)."""
    B, T, Hx, D = x.shape
    return x.transpose(0, 2, 1, 3).reshape(B, Hx, T // C, C, D)


def chunk_forward(q, k, v, g, beta, scale: float, C: int = 64,
                  s0: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """Chunkwise forward in fp64.  Returns o, final_state and intermediates.

    q, k: [B, T, H, K]; v: [B, T, HV, V]; g: [B, T, HV] or [B, T, HV, K];
    beta: [B, T, HV]; s0: [B, HV, K, V] or None.
    Intermediates are on the padded chunk grid [B, HV, N, C, ...]:
    gamma, A_kk, M, W, U, A_qk (gamma is [..., C, 1] for one decay per row).
    """
    q, k, v, g, beta = (np.asarray(a, dtype=np.float64)
                        for a in (q, k, v, g, beta))
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    G = HV // H
    per_channel = g.ndim == 4
    N = -(-T // C)
    pad = N * C - T
    if pad:
        zpad = lambda a: np.concatenate(
            [a, np.zeros((B, pad) + a.shape[2:], a.dtype)], axis=1)
        q, k, v, g, beta = map(zpad, (q, k, v, g, beta))

    # step 1: chunk, group heads, scale q
    head_of = np.arange(HV) // G
    qc = _to_chunks(q[:, :, head_of], C) * scale
    kc = _to_chunks(k[:, :, head_of], C)
    vc = _to_chunks(v, C)
    gc = _to_chunks(g if per_channel else g[..., None], C)
    bc = beta.transpose(0, 2, 1).reshape(B, HV, N, C)

    # step 2: in-chunk inclusive cumsum
    gam = np.cumsum(gc, axis=-2)

    # steps 3-5: triangular system and UT transform
    A_kk = decayed_dot(kc, kc, gam)
    eye = np.eye(C)
    M = eye + np.tril(A_kk * bc[..., None, :], -1)
    rhs = np.concatenate([np.exp(gam) * kc, vc], axis=-1)
    flatM = M.reshape(-1, C, C)
    flatR = rhs.reshape(-1, C, K + V)
    sol = np.empty_like(flatR)
    for i in range(flatM.shape[0]):
        sol[i] = solve_triangular(flatM[i], flatR[i], lower=True)
    sol = sol.reshape(rhs.shape)
    W, U = sol[..., :K], sol[..., K:]

    # step 6: query-key decayed dot, diagonal kept
    A_qk = np.tril(decayed_dot(qc, kc, gam) * bc[..., None, :])

    # step 7: inter-chunk recurrence
    S = (np.zeros((B, HV, K, V)) if s0 is None
         else np.array(s0, dtype=np.float64))
    o = np.empty((B, HV, N, C, V))
    for n in range(N):
        gn = gam[:, :, n]                                   # [B,HV,C,K|1]
        r = U[:, :, n] - W[:, :, n] @ S
        o[:, :, n] = (qc[:, :, n] * np.exp(gn)) @ S + A_qk[:, :, n] @ r
        decay = np.exp(gn[:, :, -1:, :] - gn)               # to chunk end
        last = np.broadcast_to(np.exp(gn[:, :, -1, :]), (B, HV, K))
        S = S * last[..., None]
        S = S + np.swapaxes(decay * kc[:, :, n], -1, -2) @ (
            r * bc[:, :, n, :, None])
    o = o.reshape(B, HV, N * C, V)[:, :, :T].transpose(0, 2, 1, 3)
    return dict(o=np.ascontiguousarray(o), final_state=S, gamma=gam,
                A_kk=A_kk, M=M, W=W, U=U, A_qk=A_qk)
