"""The seven chunk stages in fp64 numpy — TEST INFRASTRUCTURE ONLY.

Follows the stage list of the MegaGDN-PTO page (section 1.1, "the seven-stage pipeline"),
in its order:  cumsum -> transpose -> scaled_dot_kkt -> solve_tril -> wy_fast -> chunk_h
-> chunk_o.  It exists to give every stage intermediate for per-stage parity of the staged
GPU variant; the result it reaches is pinned to the token recurrence (``oracle.recurrence``)
by the tests, at several chunk sizes.

Stage outputs use the layouts the staged GPU variant writes to its workspace:

  chunk table    list of (sequence, first token, length) in sequence order; chunks restart
                 at every sequence start (the page's per-sequence state offsets, section 5.3)
  g_cum          [Ttot, H]      in-chunk inclusive prefix sum of g              (stage 1)
  g_t, beta_t    [H, Ttot]      head-major copies of g_cum and beta             (stage 2)
  A              [Ttot, H, C]   row = token, column = position j in its chunk   (stage 3)
  Tinv           [Ttot, H, C]   rows of (I + A_chunk)^-1                         (stage 4)
  W, U           [Ttot, H, Dk] / [Ttot, H, Dv]                                   (stage 5)
  h_c            [NC, H, Dk, Dv] state at the start of every chunk               (stage 6)
  v_new          [Ttot, H, Dv]  U - W h_c  (before the e^{G_last - G} weighting)  (stage 6)
  o              [Ttot, H, Dv]                                                    (stage 7)
  ht             [N, H, Dk, Dv]

Readings (where the page is silent): A is strictly lower (i > j) while chunk_o's in-chunk
term includes the diagonal (i >= j); solve_tril inverts the unit-lower matrix I + A; the
clamp max=0 of the gate exponent is a guard for the masked triangle and is written here as
the exact product beta_i e^{G_i - G_j}; a partial last chunk uses only its valid rows and
takes G_last at its last valid token.
"""
from __future__ import annotations

import numpy as np


def chunk_table(starts, lens, C):
    """Stage 0 (the varlen chunk list): every sequence is cut into ceil(len / C) chunks."""
    table = []
    for n, (s, L) in enumerate(zip(starts, lens)):
        s, L = int(s), int(L)
        for m in range((L + C - 1) // C):
            table.append((n, s + m * C, min(C, L - m * C)))
    return table


def stage_cumsum(g, table):
    """Stage 1 (page section 4.1): g_cum[t, h] = sum of g[i, h] over the chunk's tokens up to t."""
    out = np.zeros_like(g)
    for _, s, L in table:
        out[s:s + L] = np.cumsum(g[s:s + L], axis=0)
    return out


def stage_transpose(g_cum, beta):
    """Stage 2 (page section 4.5): [T, H] -> [H, T] so each head reads contiguously."""
    return np.ascontiguousarray(g_cum.T), np.ascontiguousarray(beta.T)


def stage_kkt(k, g_t, beta_t, table, H, C):
    """Stage 3 (page section 4.2): A = (K K^T) * beta_i e^{G_i - G_j}, strictly lower."""
    Ttot, Hg, _ = k.shape
    group = H // Hg
    A = np.zeros((Ttot, H, C))
    for _, s, L in table:
        for h in range(H):
            kc = k[s:s + L, h // group]
            G = g_t[h, s:s + L]
            b = beta_t[h, s:s + L]
            gate = b[:, None] * np.exp(G[:, None] - G[None, :])
            A[s:s + L, h, :L] = np.tril((kc @ kc.T) * gate, -1)
    return A


def stage_solve_tril(A, table, H):
    """Stage 4 (page section 4.4): Tinv = (I + A)^-1 for every chunk and head, by forward
    substitution on the unit-lower system (I + A) X = I, one row of X at a time:
    X[i, :] = e_i - sum_{m < i} A[i, m] X[m, :]."""
    Tinv = np.zeros_like(A)
    for _, s, L in table:
        for h in range(H):
            Ac = A[s:s + L, h, :L]
            X = np.zeros((L, L))
            for i in range(L):
                X[i] = -(Ac[i, :i] @ X[:i])
                X[i, i] += 1.0
            Tinv[s:s + L, h, :L] = X
    return Tinv


def stage_wy(Tinv, k, v, g_t, beta_t, table, H):
    """Stage 5 (page section 4.3): U = (Tinv * beta_col) V and W = (Tinv * (e^G beta)_col) K,
    where x_col[i, j] = x[j]."""
    Ttot, Hg, Dk = k.shape
    Dv = v.shape[2]
    group = H // Hg
    W = np.zeros((Ttot, H, Dk))
    U = np.zeros((Ttot, H, Dv))
    for _, s, L in table:
        for h in range(H):
            Ti = Tinv[s:s + L, h, :L]
            b = beta_t[h, s:s + L]
            eg = np.exp(g_t[h, s:s + L])
            U[s:s + L, h] = (Ti * b[None, :]) @ v[s:s + L, h]
            W[s:s + L, h] = (Ti * (eg * b)[None, :]) @ k[s:s + L, h // group]
    return W, U


def stage_chunk_h(k, W, U, g_t, h0, table, N, H):
    """Stage 6 (TileLang chunk_gated_delta_rule_fwd_h kernel, TileLang x xLLM page, step 1):
    per chunk, record h, v_new = U - W h, then h = e^{G_last} h + K^T (e^{G_last - G} v_new)."""
    Ttot, Hg, Dk = k.shape
    Dv = U.shape[2]
    group = H // Hg
    NC = len(table)
    h_c = np.zeros((NC, H, Dk, Dv))
    v_new = np.zeros((Ttot, H, Dv))
    state = np.zeros((N, H, Dk, Dv)) if h0 is None else np.array(h0, np.float64)
    for c, (n, s, L) in enumerate(table):
        for h in range(H):
            hs = state[n, h]
            h_c[c, h] = hs
            vn = U[s:s + L, h] - W[s:s + L, h] @ hs
            v_new[s:s + L, h] = vn
            G = g_t[h, s:s + L]
            glast = G[L - 1]
            state[n, h] = np.exp(glast) * hs + k[s:s + L, h // group].T @ (
                np.exp(glast - G)[:, None] * vn)
    return h_c, v_new, state


def stage_chunk_o(q, k, v_new, h_c, g_t, table, H, scale):
    """Stage 7 (page section 1.1, chunk_o): O = scale (diag(e^G) Q h_c
    + (Q K^T * e^{G_i - G_j} * [i >= j]) v_new)."""
    Ttot, Hg, Dk = q.shape
    Dv = v_new.shape[2]
    group = H // Hg
    o = np.zeros((Ttot, H, Dv))
    for c, (_, s, L) in enumerate(table):
        for h in range(H):
            qc, kc = q[s:s + L, h // group], k[s:s + L, h // group]
            G = g_t[h, s:s + L]
            decay = np.tril(np.exp(G[:, None] - G[None, :]))
            o[s:s + L, h] = scale * (np.exp(G)[:, None] * (qc @ h_c[c, h])
                                     + ((qc @ kc.T) * decay) @ v_new[s:s + L, h])
    return o


def chunked(q, k, v, g, beta, h0=None, scale=None, cu_seqlens=None, C=64):
    """Run all stages.  Same inputs and layouts as ``oracle.recurrence``.  Returns a dict of
    every stage output (token axis flattened to Ttot) plus ``o`` [B, T, H, Dv] and ``ht``."""
    from . import sequences
    q, k, v, g, beta = (np.asarray(x, np.float64) for x in (q, k, v, g, beta))
    B, T, Hg, Dk = q.shape
    H, Dv = v.shape[2], v.shape[3]
    if scale is None:
        scale = Dk ** -0.5
    starts, lens = sequences(B, T, cu_seqlens)
    N = len(starts)
    qf, kf = q.reshape(B * T, Hg, Dk), k.reshape(B * T, Hg, Dk)
    vf, gf, bf = v.reshape(B * T, H, Dv), g.reshape(B * T, H), beta.reshape(B * T, H)
    table = chunk_table(starts, lens, C)
    g_cum = stage_cumsum(gf, table)
    g_t, beta_t = stage_transpose(g_cum, bf)
    A = stage_kkt(kf, g_t, beta_t, table, H, C)
    Tinv = stage_solve_tril(A, table, H)
    W, U = stage_wy(Tinv, kf, vf, g_t, beta_t, table, H)
    h_c, v_new, ht = stage_chunk_h(kf, W, U, g_t, h0, table, N, H)
    o = stage_chunk_o(qf, kf, v_new, h_c, g_t, table, H, scale)
    return dict(table=table, g_cum=g_cum, g_t=g_t, beta_t=beta_t, A=A, Tinv=Tinv, W=W,
                U=U, h_c=h_c, v_new=v_new, o=o.reshape(B, T, H, Dv), ht=ht)
