"""Gradients of the gated delta rule forward — TEST INFRASTRUCTURE ONLY (the same import
rules as the rest of ``oracle/``).

The pages cite forward and backward speedups of the chunked operator (the FlashQLA how-to,
its performance section) but print no backward formulas.  The backward here is the exact
reverse-mode derivative of the forward recurrence (the definition the forward oracle
computes), written out step by step in fp64.  With the state held as H = S^T (Dk x Dv,
``ht``'s layout) and e_t = exp(g_t), the forward step is

    s_t = H_{t-1}^T k_t,   u_t = beta_t (v_t - e_t s_t),   H_t = e_t H_{t-1} + k_t u_t^T,
    o_t = scale H_t^T q_t,

and, with dH the gradient of the loss with respect to H_t, one reverse step is

    dH   += scale q_t do_t^T                 dq_t  = scale H_t do_t
    du    = dH^T k_t                         dk_t  = dH u_t + H_{t-1} ds
    dv_t  = beta_t du                        dbeta = du . (v_t - e_t s_t)
    ds    = -beta_t e_t du                   de    = <dH, H_{t-1}> - beta_t du . s_t
    dg_t  = e_t de                           dH   <- e_t dH + k_t ds^T

starting from dH = dht and ending with dh0 = dH.  Value heads that share a q/k head add
their dq and dk.  Pinned by central finite differences of a random scalar loss in
tests/test_oracle.py (no kernel computes it yet).
"""
from __future__ import annotations

import numpy as np


def _pair_forward(q, k, v, g, beta, H0, scale):
    """Forward of one (sequence, head): returns the states H_0 .. H_T and the outputs."""
    T = q.shape[0]
    Hs = [H0]
    o = np.zeros((T, v.shape[1]))
    H = H0
    for t in range(T):
        e = np.exp(g[t])
        s = H.T @ k[t]
        u = beta[t] * (v[t] - e * s)
        H = e * H + np.outer(k[t], u)
        o[t] = scale * (H.T @ q[t])
        Hs.append(H)
    return Hs, o


def _pair_backward(q, k, v, g, beta, Hs, scale, do, dH):
    T = q.shape[0]
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    dg, db = np.zeros(T), np.zeros(T)
    for t in range(T - 1, -1, -1):
        Hp, Ht = Hs[t], Hs[t + 1]
        e = np.exp(g[t])
        s = Hp.T @ k[t]
        r = v[t] - e * s
        u = beta[t] * r
        dH = dH + scale * np.outer(q[t], do[t])
        dq[t] = scale * (Ht @ do[t])
        du = dH.T @ k[t]
        dv[t] = beta[t] * du
        db[t] = du @ r
        ds = -beta[t] * e * du
        de = np.sum(dH * Hp) - beta[t] * (du @ s)
        dk[t] = dH @ u + Hp @ ds
        dg[t] = e * de
        dH = e * dH + np.outer(k[t], ds)
    return dq, dk, dv, dg, db, dH


def recurrence_backward(q, k, v, g, beta, h0, scale, do, dht, cu_seqlens=None):
    """Gradients of (o, ht) = forward(q, k, v, g, beta, h0) against upstream do and dht.

    Layouts as the forward: q, k [B, T, Hg, Dk]; v, do [B, T, H, Dv]; g, beta [B, T, H];
    h0, dht [N, H, Dk, Dv] or None (zero state / no gradient through ht); packed batches via
    cu_seqlens with B = 1.  Returns dq, dk, dv, dg, dbeta (input shapes) and dh0
    [N, H, Dk, Dv], all fp64."""
    q, k, v, g, beta, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta, do))
    B, T, Hg, Dk = q.shape
    H, Dv = v.shape[2], v.shape[3]
    grp = H // Hg
    if cu_seqlens is None:
        seqs = [(n, n, 0, T) for n in range(B)]
    else:
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        seqs = [(n, 0, int(cu[n]), int(cu[n + 1])) for n in range(len(cu) - 1)]
    N = len(seqs)
    out = [np.zeros_like(x) for x in (q, k, v, g, beta)]
    dh0 = np.zeros((N, H, Dk, Dv))
    for n, b, s0, s1 in seqs:
        for h in range(H):
            hk = h // grp
            H0 = np.zeros((Dk, Dv)) if h0 is None else np.asarray(h0[n, h], dtype=np.float64)
            dH = np.zeros((Dk, Dv)) if dht is None else np.asarray(dht[n, h], dtype=np.float64)
            args = (q[b, s0:s1, hk], k[b, s0:s1, hk], v[b, s0:s1, h], g[b, s0:s1, h],
                    beta[b, s0:s1, h])
            Hs, _ = _pair_forward(*args, H0, scale)
            dq, dk, dv, dg, db, dH0 = _pair_backward(*args, Hs, scale, do[b, s0:s1, h], dH)
            out[0][b, s0:s1, hk] += dq
            out[1][b, s0:s1, hk] += dk
            out[2][b, s0:s1, h] = dv
            out[3][b, s0:s1, h] = dg
            out[4][b, s0:s1, h] = db
            dh0[n, h] = dH0
    return (*out, dh0)
