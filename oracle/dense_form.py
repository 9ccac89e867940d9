"""Whole-sequence triangular-solve form of the gated delta rule — TEST INFRASTRUCTURE ONLY.

Used only to pin the token recurrence (``oracle.recurrence``) on tiny inputs; it is an
independent formulation, not a re-typing of the recurrence.

Derivation (one (sequence, head) pair; h = S^T is Dk x Dv, h0 the initial state).
Write the update as h_t = e^{g_t} h_{t-1} + k_t d_t^T with the "delta"
d_t = beta_t (v_t - e^{g_t} h_{t-1}^T k_t).  With G the inclusive cumulative sum of g over
the whole sequence, unrolling gives h_i = e^{G_i} h0 + sum_{j<=i} e^{G_i - G_j} k_j d_j^T.
Substituting h_{i-1} into d_i gives the lower-triangular system

    (I + A) D = diag(beta) V - diag(beta e^G) K h0,   A_ij = beta_i e^{G_i - G_j} k_i.k_j (i > j)

and then  O = scale (diag(e^G) Q h0 + (Q K^T * e^{G_i - G_j} * [i >= j]) D),
          h_T = e^{G_T} h0 + K^T diag(e^{G_T - G}) D.

This is the "chunk" algebra of the MegaGDN-PTO page (section 1.1, stages scaled_dot_kkt,
solve_tril, wy_fast, chunk_o) applied with a single chunk that spans the sequence, solved
here by scipy's triangular solver rather than by an explicit inverse.
"""
from __future__ import annotations

import numpy as np
import scipy.linalg


def pair_dense(q, k, v, g, beta, h0, scale):
    """q, k: [T, Dk]; v: [T, Dv]; g, beta: [T]; h0: [Dk, Dv] (or None).  fp64 in/out.
    Returns (o [T, Dv], ht [Dk, Dv])."""
    q, k, v, g, beta = (np.asarray(x, np.float64) for x in (q, k, v, g, beta))
    T, Dk = k.shape
    Dv = v.shape[1]
    h0 = np.zeros((Dk, Dv)) if h0 is None else np.asarray(h0, np.float64)
    if T == 0:
        return np.zeros((0, Dv)), h0.copy()
    G = np.cumsum(g)
    diff = G[:, None] - G[None, :]
    causal_strict = np.tril(np.ones((T, T), dtype=bool), -1)
    causal = np.tril(np.ones((T, T), dtype=bool), 0)
    gate = np.where(causal, np.exp(np.where(causal, diff, 0.0)), 0.0)
    A = np.where(causal_strict, beta[:, None] * gate * (k @ k.T), 0.0)
    rhs = beta[:, None] * v - (beta * np.exp(G))[:, None] * (k @ h0)
    D = scipy.linalg.solve_triangular(np.eye(T) + A, rhs, lower=True, unit_diagonal=True)
    o = scale * (np.exp(G)[:, None] * (q @ h0) + ((q @ k.T) * gate) @ D)
    ht = np.exp(G[-1]) * h0 + k.T @ (np.exp(G[-1] - G)[:, None] * D)
    return o, ht


def dense(q, k, v, g, beta, h0=None, scale=None, cu_seqlens=None):
    """Same signature and layouts as ``oracle.recurrence`` (numpy fp64 arrays)."""
    q, k, v, g, beta = (np.asarray(x, np.float64) for x in (q, k, v, g, beta))
    B, T, Hg, Dk = q.shape
    H, Dv = v.shape[2], v.shape[3]
    group = H // Hg
    if scale is None:
        scale = Dk ** -0.5
    if cu_seqlens is None:
        spans = [(b * T, T) for b in range(B)]
    else:
        cu = np.asarray(cu_seqlens, np.int64)
        spans = [(int(cu[i]), int(cu[i + 1] - cu[i])) for i in range(len(cu) - 1)]
    qf, kf = q.reshape(B * T, Hg, Dk), k.reshape(B * T, Hg, Dk)
    vf, gf, bf = v.reshape(B * T, H, Dv), g.reshape(B * T, H), beta.reshape(B * T, H)
    o = np.zeros((B * T, H, Dv))
    ht = np.zeros((len(spans), H, Dk, Dv))
    for n, (s, L) in enumerate(spans):
        for h in range(H):
            hk = h // group
            sl = slice(s, s + L)
            on, hn = pair_dense(qf[sl, hk], kf[sl, hk], vf[sl, h], gf[sl, h], bf[sl, h],
                                None if h0 is None else h0[n, h], scale)
            o[sl, h] = on
            ht[n, h] = hn
    return o.reshape(B, T, H, Dv), ht
