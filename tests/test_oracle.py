"""Pins for the oracle (CPU only).

The oracle is the token recurrence (``oracle.recurrence``).  Nothing here compares it with
itself: every test checks it against a value fixed by hand, a closed form, an independent
formulation (dense triangular solve; the page's seven chunk stages), a library routine or
an invariant of the mathematics.  Each is chosen so that a plausible slip (dropped decay,
wrong sign, transposed state, diagonal in the mask, wrong GQA grouping, wrong chunk
restart) fails at least one test; the ``planted`` tests show that on mutated copies.
"""
import json
import os

import numpy as np
import pytest
import scipy.linalg

import oracle
from oracle import chunked as ch
from oracle import dense_form

HERE = os.path.dirname(os.path.abspath(__file__))


def rand_case(seed, B=1, T=37, H=2, Hg=None, Dk=6, Dv=5, h0=True, normalise=True):
    rng = np.random.default_rng(seed)
    Hg = Hg or H
    q = rng.standard_normal((B, T, Hg, Dk))
    k = rng.standard_normal((B, T, Hg, Dk))
    if normalise:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, Dv))
    g = -np.log1p(np.exp(-(rng.standard_normal((B, T, H)) + 3.0)))  # logsigmoid(N(3,1))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    hs = 0.1 * rng.standard_normal((B, H, Dk, Dv)) if h0 else None
    return q, k, v, g, beta, hs


def close(a, b, tol=1e-11):
    a, b = np.asarray(a), np.asarray(b)
    scale = max(1.0, float(np.abs(b).max()) if b.size else 1.0)
    assert a.shape == b.shape
    err = float(np.abs(a - b).max()) if a.size else 0.0
    assert err <= tol * scale, "max abs err %g (scale %g)" % (err, scale)


# --------------------------------------------------------------------------- hand-worked
def test_hand_worked_golden():
    with open(os.path.join(HERE, "golden", "hand_worked.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        T = len(c["g"])
        q = np.array(c["q"]).reshape(1, T, 1, c["Dk"])
        k = np.array(c["k"]).reshape(1, T, 1, c["Dk"])
        v = np.array(c["v"]).reshape(1, T, 1, c["Dv"])
        g = np.array(c["g"]).reshape(1, T, 1)
        beta = np.array(c["beta"]).reshape(1, T, 1)
        h0 = None if c["h0"] is None else np.array(c["h0"]).reshape(1, 1, c["Dk"], c["Dv"])
        o, ht = oracle.recurrence(q, k, v, g, beta, h0, scale=c["scale"])
        close(o.reshape(T, c["Dv"]), np.array(c["o"]), 1e-12)
        close(ht.reshape(c["Dk"], c["Dv"]), np.array(c["ht"]), 1e-12)


# --------------------------------------------------------------------------- closed forms
def test_beta0_g0_keeps_state():
    """beta = 0, g = 0: the state never changes, ht = h0 and o_t = scale h0^T q_t.
    Dk != Dv and a non-symmetric h0 pin the state orientation."""
    q, k, v, g, beta, h0 = rand_case(1, B=2, T=19, H=3, Dk=7, Dv=4)
    o, ht = oracle.recurrence(q, k, v, 0 * g, 0 * beta, h0, scale=0.3)
    close(ht, h0)
    close(o, 0.3 * np.einsum("bhkv,bthk->bthv", h0, q))


def test_beta0_pure_decay():
    """beta = 0: ht = e^{G_T} h0 and o_t = scale e^{G_t} h0^T q_t, G the running sum of g."""
    q, k, v, g, beta, h0 = rand_case(2, B=1, T=23, H=2, Dk=5, Dv=3)
    o, ht = oracle.recurrence(q, k, v, g, 0 * beta, h0, scale=0.7)
    G = np.cumsum(g, axis=1)                                    # [B, T, H]
    close(ht, np.exp(G[:, -1])[:, :, None, None] * h0)
    close(o, 0.7 * np.exp(G)[..., None] * np.einsum("bhkv,bthk->bthv", h0, q))


def test_delta_rule_overwrites_orthonormal_keys():
    """beta = 1, g = 0, orthonormal keys: each write replaces the value stored under its key
    (S k_t = v_t right after token t) and leaves the other keys' values alone, so at the end
    S k_i = v_i for all i, and o_t = scale v_t when q_t = k_t.  Holds for any h0."""
    rng = np.random.default_rng(3)
    Dk, Dv, T = 8, 5, 6
    Qm, _ = np.linalg.qr(rng.standard_normal((Dk, Dk)))
    keys = Qm[:, :T].T                                           # T orthonormal rows
    v = rng.standard_normal((1, T, 1, Dv))
    h0 = rng.standard_normal((1, 1, Dk, Dv))
    k = keys.reshape(1, T, 1, Dk)
    o, ht = oracle.recurrence(k, k, v, np.zeros((1, T, 1)), np.ones((1, T, 1)), h0, scale=1.5)
    close(o, 1.5 * v)
    S = ht[0, 0].T                                               # Dv x Dk
    close(keys @ S.T, v[0, :, 0])
    # directions orthogonal to every key keep their h0 values
    rest = Qm[:, T:].T
    close(rest @ S.T, rest @ h0[0, 0])


def test_single_token_from_zero_state():
    """One token, h0 = 0: S = beta v k^T, so o = scale beta (k . q) v and ht = beta k v^T."""
    q, k, v, g, beta, _ = rand_case(4, B=1, T=1, H=1, Dk=6, Dv=4, h0=False)
    o, ht = oracle.recurrence(q, k, v, g, beta, None, scale=0.9)
    b = beta[0, 0, 0]
    close(o[0, 0, 0], 0.9 * b * (k[0, 0, 0] @ q[0, 0, 0]) * v[0, 0, 0])
    close(ht[0, 0], b * np.outer(k[0, 0, 0], v[0, 0, 0]))


# ----------------------------------------------------------------- independent formulations
@pytest.mark.parametrize("T,H,Hg,Dk,Dv,h0", [(1, 1, 1, 4, 4, True), (2, 2, 1, 5, 3, True),
                                             (17, 4, 2, 6, 6, False), (64, 2, 2, 8, 5, True),
                                             (200, 2, 1, 16, 16, True)])
def test_recurrence_equals_dense_solve(T, H, Hg, Dk, Dv, h0):
    q, k, v, g, beta, hs = rand_case(10 + T, B=2, T=T, H=H, Hg=Hg, Dk=Dk, Dv=Dv, h0=h0)
    o, ht = oracle.recurrence(q, k, v, g, beta, hs)
    od, htd = dense_form.dense(q, k, v, g, beta, hs)
    close(o, od, 1e-10)
    close(ht, htd, 1e-10)


@pytest.mark.parametrize("C", [1, 2, 7, 16, 64, 97])
def test_chunked_stages_equal_recurrence(C):
    """The page's seven stages reach the recurrence at every chunk size, including a
    ragged last chunk (T = 97 is not a multiple of 2, 7, 16 or 64)."""
    q, k, v, g, beta, hs = rand_case(20 + C, B=2, T=97, H=4, Hg=2, Dk=6, Dv=5)
    o, ht = oracle.recurrence(q, k, v, g, beta, hs)
    r = ch.chunked(q, k, v, g, beta, hs, C=C)
    close(r["o"], o, 1e-10)
    close(r["ht"], ht, 1e-10)


def test_chunked_varlen_equals_recurrence():
    rng = np.random.default_rng(5)
    lens = [1, 63, 64, 65, 130, 7]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v, g, beta, _ = rand_case(6, B=1, T=int(cu[-1]), H=2, Dk=8, Dv=4, h0=False)
    hs = 0.1 * rng.standard_normal((len(lens), 2, 8, 4))
    o, ht = oracle.recurrence(q, k, v, g, beta, hs, cu_seqlens=cu)
    r = ch.chunked(q, k, v, g, beta, hs, cu_seqlens=cu, C=64)
    close(r["o"], o, 1e-10)
    close(r["ht"], ht, 1e-10)
    # chunks restart at every sequence start
    assert [(n, s, L) for n, s, L in r["table"]][:4] == [(0, 0, 1), (1, 1, 63), (2, 64, 64),
                                                         (3, 128, 64)]


def test_solve_stage_matches_library_and_inverts():
    q, k, v, g, beta, hs = rand_case(7, B=1, T=128, H=2, Dk=16, Dv=8)
    r = ch.chunked(q, k, v, g, beta, hs, C=64)
    for _, s, L in r["table"]:
        for h in range(2):
            A = r["A"][s:s + L, h, :L]
            assert np.all(np.triu(A) == 0.0)                     # strictly lower
            Ti = r["Tinv"][s:s + L, h, :L]
            close(Ti @ (np.eye(L) + A), np.eye(L), 1e-12)
            ref = scipy.linalg.solve_triangular(np.eye(L) + A, np.eye(L), lower=True,
                                                unit_diagonal=True)
            close(Ti, ref, 1e-12)


def test_cumsum_stage_matches_numpy_per_chunk():
    q, k, v, g, beta, hs = rand_case(8, B=1, T=100, H=3, Dk=4, Dv=4)
    r = ch.chunked(q, k, v, g, beta, hs, C=32)
    gf = g.reshape(100, 3)
    for _, s, L in r["table"]:
        close(r["g_cum"][s:s + L], np.add.accumulate(gf[s:s + L], axis=0), 1e-14)
    close(r["g_t"], r["g_cum"].T, 0)
    close(r["beta_t"], beta.reshape(100, 3).T, 0)


# --------------------------------------------------------------------------- invariants
def test_varlen_equals_per_sequence_runs():
    lens = [5, 70, 1, 33]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v, g, beta, _ = rand_case(9, B=1, T=int(cu[-1]), H=2, Dk=6, Dv=4, h0=False)
    hs = 0.1 * np.random.default_rng(9).standard_normal((4, 2, 6, 4))
    o, ht = oracle.recurrence(q, k, v, g, beta, hs, cu_seqlens=cu)
    for n in range(4):
        sl = slice(cu[n], cu[n + 1])
        on, hn = oracle.recurrence(q[:, sl], k[:, sl], v[:, sl], g[:, sl], beta[:, sl],
                                   hs[n:n + 1])
        close(o[:, sl], on, 1e-14)
        close(ht[n:n + 1], hn, 1e-14)


def test_dense_batch_equals_packed():
    q, k, v, g, beta, hs = rand_case(11, B=3, T=20, H=2, Dk=5, Dv=5)
    o, ht = oracle.recurrence(q, k, v, g, beta, hs)
    flat = lambda x: x.reshape((1, 60) + x.shape[2:])
    op, htp = oracle.recurrence(flat(q), flat(k), flat(v), flat(g), flat(beta), hs,
                                cu_seqlens=[0, 20, 40, 60])
    close(flat(o), op, 0)
    close(ht, htp, 0)


def test_gqa_equals_repeated_heads():
    """Value head h reads q/k head h // (H / Hg) (contiguous groups, MegaGDN-PTO page
    section 5.2) — a GQA run equals a plain run with q, k repeated along heads."""
    q, k, v, g, beta, hs = rand_case(12, B=2, T=30, H=6, Hg=2, Dk=4, Dv=3)
    o, ht = oracle.recurrence(q, k, v, g, beta, hs)
    rep = lambda x: np.repeat(x, 3, axis=2)
    o2, ht2 = oracle.recurrence(rep(q), rep(k), v, g, beta, hs)
    close(o, o2, 0)
    close(ht, ht2, 0)


def test_continuation_through_final_state():
    """Feeding the final state of a prefix as h0 of the suffix equals one run."""
    q, k, v, g, beta, hs = rand_case(13, B=2, T=50, H=2, Dk=5, Dv=4)
    o, ht = oracle.recurrence(q, k, v, g, beta, hs)
    a, b = slice(0, 21), slice(21, 50)
    o1, h1 = oracle.recurrence(q[:, a], k[:, a], v[:, a], g[:, a], beta[:, a], hs)
    o2, h2 = oracle.recurrence(q[:, b], k[:, b], v[:, b], g[:, b], beta[:, b], h1)
    close(np.concatenate([o1, o2], axis=1), o, 1e-14)
    close(h2, ht, 1e-14)


def test_linear_in_values_and_initial_state():
    q, k, v, g, beta, hs = rand_case(14, B=1, T=40, H=2, Dk=5, Dv=4)
    _, _, v2, _, _, hs2 = rand_case(15, B=1, T=40, H=2, Dk=5, Dv=4)
    a = -1.7
    o1, h1 = oracle.recurrence(q, k, v, g, beta, hs)
    o2, h2 = oracle.recurrence(q, k, v2, g, beta, hs2)
    o3, h3 = oracle.recurrence(q, k, v + a * v2, g, beta, hs + a * hs2)
    close(o3, o1 + a * o2, 1e-12)
    close(h3, h1 + a * h2, 1e-12)


def test_value_columns_are_independent():
    """Column j of v (and of h0) only reaches o[..., j] and ht[..., j]."""
    q, k, v, g, beta, hs = rand_case(16, B=1, T=30, H=1, Dk=4, Dv=6)
    o, ht = oracle.recurrence(q, k, v, g, beta, hs)
    o2, ht2 = oracle.recurrence(q, k, v[..., 2:4], g, beta, hs[..., 2:4])
    close(o2, o[..., 2:4], 0)
    close(ht2, ht[..., 2:4], 0)


def test_pairs_subset_matches_full_run():
    q, k, v, g, beta, hs = rand_case(17, B=2, T=12, H=3, Dk=4, Dv=4)
    o, ht = oracle.recurrence(q, k, v, g, beta, hs)
    pairs = [1, 5]
    os_, hts = oracle.recurrence(q, k, v, g, beta, hs, pairs=pairs)
    for p in pairs:
        n, h = divmod(p, 3)
        close(os_[n, :, h], o[n, :, h], 0)
        close(hts[n, h], ht[n, h], 0)
    assert np.all(os_[0, :, 0] == 0)


def test_empty_sequence_passes_state_through():
    """A length-0 sequence writes no output and returns its h0 as the final state."""
    q, k, v, g, beta, _ = rand_case(18, B=1, T=10, H=1, Dk=4, Dv=4, h0=False)
    hs = np.random.default_rng(18).standard_normal((3, 1, 4, 4))
    o, ht = oracle.recurrence(q, k, v, g, beta, hs, cu_seqlens=[0, 4, 4, 10])
    close(ht[1], hs[1], 0)


# --------------------------------------------------------------------- planted mistakes
def _recurrence_py(q, k, v, g, beta, h0, scale, *, transpose_h0=False, decay_write=False,
                   sign=-1.0, o_before=False, group_mod=False):
    """A mutable pure-Python copy of the recurrence, used only to show that the pins above
    catch each plausible mistake (the real oracle is the C one)."""
    B, T, Hg, Dk = q.shape
    H, Dv = v.shape[2], v.shape[3]
    grp = H // Hg
    o = np.zeros((B, T, H, Dv))
    ht = np.zeros((B, H, Dk, Dv))
    for b in range(B):
        for h in range(H):
            hk = h % Hg if group_mod else h // grp
            S = np.zeros((Dv, Dk)) if h0 is None else (
                h0[b, h].reshape(Dv, Dk) if transpose_h0 else h0[b, h].T.copy())
            for t in range(T):
                kt, qt, vt = k[b, t, hk], q[b, t, hk], v[b, t, h]
                d, bt = np.exp(g[b, t, h]), beta[b, t, h]
                if o_before:
                    o[b, t, h] = scale * S @ qt
                upd = S + sign * bt * np.outer(S @ kt, kt)
                S = d * upd + (d if decay_write else 1.0) * bt * np.outer(vt, kt)
                if not o_before:
                    o[b, t, h] = scale * S @ qt
            ht[b, h] = S.T
    return o, ht


@pytest.mark.parametrize("mutation", ["transpose_h0", "decay_write", "sign", "o_before",
                                      "group_mod"])
def test_planted_mistakes_are_caught(mutation):
    q, k, v, g, beta, hs = rand_case(19, B=1, T=24, H=4, Hg=2, Dk=5, Dv=5)
    kw = {"sign": {"sign": +1.0}}.get(mutation, {mutation: True})
    # the unmutated copy agrees with the oracle ...
    o, ht = _recurrence_py(q, k, v, g, beta, hs, 0.5)
    od, htd = dense_form.dense(q, k, v, g, beta, hs, scale=0.5)
    close(o, od, 1e-10)
    close(ht, htd, 1e-10)
    # ... and each mutation is caught by the independent dense formulation
    om, htm = _recurrence_py(q, k, v, g, beta, hs, 0.5, **kw)
    err = max(np.abs(om - od).max(), np.abs(htm - htd).max())
    assert err > 1e-3, mutation


def test_planted_diagonal_in_kkt_mask_is_caught(monkeypatch):
    """Reading the KKT mask as lower *including* the diagonal breaks agreement with the
    recurrence, which pins the strictly-lower reading."""
    q, k, v, g, beta, hs = rand_case(21, B=1, T=64, H=2, Dk=8, Dv=8)
    o, _ = oracle.recurrence(q, k, v, g, beta, hs)
    orig = ch.stage_kkt

    def kkt_with_diag(kf, g_t, beta_t, table, H, C):
        A = orig(kf, g_t, beta_t, table, H, C)
        for _, s, L in table:
            for h in range(H):
                kc = kf[s:s + L, h // (H // kf.shape[1])]
                A[s:s + L, h, :L] += np.diag(beta_t[h, s:s + L] * np.sum(kc * kc, axis=1))
        return A

    def solve_general(A, table, H):
        # the mistaken reading solves with the diagonal of A included (not unit-lower)
        Tinv = np.zeros_like(A)
        for _, s, L in table:
            for h in range(H):
                M = np.eye(L) + A[s:s + L, h, :L]
                Tinv[s:s + L, h, :L] = scipy.linalg.solve_triangular(M, np.eye(L), lower=True)
        return Tinv

    monkeypatch.setattr(ch, "stage_kkt", kkt_with_diag)
    monkeypatch.setattr(ch, "stage_solve_tril", solve_general)
    r = ch.chunked(q, k, v, g, beta, hs, C=16)
    rel = np.linalg.norm(r["o"] - o) / np.linalg.norm(o)
    assert rel > 0.05


def test_sampled_pairs_helper_matches_full_run():
    import gdn_inputs
    # the packed single-head form used for sampled full-size checks returns the same values
    from gdn_testlib import oracle_full, oracle_pairs, pair_slices
    inp = gdn_inputs.draw(gdn_inputs.small(T=0, n_varlen=5, max_len=90, H=4, Hg=2, Dk=16,
                                           C=16, seed=11, h0_std=0.1), device="cpu")
    o_ref, ht_ref = oracle_full(inp)
    pairs = [(0, 0), (4, 3), (2, 1), (3, 2)]
    got = oracle_pairs(inp, pairs, nthreads=2)
    for (n, h), (o, ht) in got.items():
        ts, b, _ = pair_slices(inp, n, h)
        np.testing.assert_allclose(o, o_ref[b, ts, h], rtol=0, atol=1e-14)
        np.testing.assert_allclose(ht, ht_ref[n, h], rtol=0, atol=1e-14)


# ------------------------------------------------------------ affine segment composition
@pytest.mark.parametrize("bounds", [(0, 13, 37), (0, 1, 20, 21, 37), (0, 37)])
def test_segments_compose_as_affine_maps(bounds):
    """The segmented evaluation's algebra, on the oracle alone: the final state is affine in
    the initial state, h_end = M h_in + b, with M the final state from h_in = I and v = 0
    (M acts on the key index) and b the final state from h_in = 0.  Composing the segments'
    maps in order gives the whole sequence's final state, and each segment run from its
    composed h_in gives the whole sequence's outputs."""
    q, k, v, g, beta, hs = rand_case(77, B=1, T=37, H=3, Hg=1, Dk=5, Dv=5)
    o_full, ht_full = oracle.recurrence(q, k, v, g, beta, hs)
    eye = np.broadcast_to(np.eye(5), (1, 3, 5, 5)).copy()
    h = hs.copy()
    for a, b_ in zip(bounds[:-1], bounds[1:]):
        sl = (slice(None), slice(a, b_))
        _, bseg = oracle.recurrence(q[sl], k[sl], v[sl], g[sl], beta[sl], None)
        _, mseg = oracle.recurrence(q[sl], k[sl], 0 * v[sl], g[sl], beta[sl], eye)
        oseg, _ = oracle.recurrence(q[sl], k[sl], v[sl], g[sl], beta[sl], h)
        close(oseg, o_full[sl], 1e-11)
        h = np.einsum("nhac,nhcb->nhab", mseg, h) + bseg
    close(h, ht_full, 1e-11)


def test_segment_map_orientation_is_pinned():
    """A planted mistake: applying M on the value index (h M instead of M h) breaks the
    composition, so the test above pins the orientation."""
    q, k, v, g, beta, hs = rand_case(78, B=1, T=20, H=1, Dk=4, Dv=4)
    _, ht_full = oracle.recurrence(q, k, v, g, beta, hs)
    eye = np.eye(4)[None, None]
    _, b1 = oracle.recurrence(q[:, :9], k[:, :9], v[:, :9], g[:, :9], beta[:, :9], None)
    _, m1 = oracle.recurrence(q[:, :9], k[:, :9], 0 * v[:, :9], g[:, :9], beta[:, :9], eye)
    _, b2 = oracle.recurrence(q[:, 9:], k[:, 9:], v[:, 9:], g[:, 9:], beta[:, 9:], None)
    _, m2 = oracle.recurrence(q[:, 9:], k[:, 9:], 0 * v[:, 9:], g[:, 9:], beta[:, 9:], eye)
    h1 = hs @ m1 + b1
    wrong = h1 @ m2 + b2
    assert np.abs(wrong - ht_full).max() > 1e-6


# ------------------------------------------------------------------ causal conv1d oracle
from oracle import conv1d as cv  # noqa: E402


def conv_case(seed, T=23, C=6, W=4, B=1):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, T, C)), rng.standard_normal((C, W)),
            rng.standard_normal(C))


@pytest.mark.parametrize("W", [2, 3, 4])
def test_conv1d_matches_numpy_convolution(W):
    """With no state the causal convolution is numpy's full convolution with the reversed
    taps, truncated to the first T outputs, plus the bias."""
    x, w, b = conv_case(40 + W, W=W)
    y, st = cv.causal_conv1d(x, w, b)
    assert st is None
    for c in range(x.shape[2]):
        ref = np.convolve(x[0, :, c], w[c, ::-1])[:x.shape[1]] + b[c]
        close(y[0, :, c], ref, 1e-12)


def test_conv1d_impulse_response():
    """A unit impulse at position p in channel c gives y[p + i, c] = weight[c, W - 1 - i]:
    the last tap multiplies the current token, the first the oldest."""
    W, T, C, p, c = 4, 12, 3, 5, 1
    x = np.zeros((1, T, C))
    x[0, p, c] = 1.0
    w = np.arange(1.0, 1.0 + C * W).reshape(C, W)
    y, _ = cv.causal_conv1d(x, w)
    expect = np.zeros((1, T, C))
    for i in range(W):
        expect[0, p + i, c] = w[c, W - 1 - i]
    close(y, expect, 0)


@pytest.mark.parametrize("split", [1, 2, 3, 7])
def test_conv1d_continues_across_calls(split):
    """Two calls with the state carried (including a first piece shorter than W - 1) give
    the outputs and final state of one call over the whole sequence."""
    x, w, b = conv_case(50 + split, T=15, W=4)
    rng = np.random.default_rng(9)
    st0 = rng.standard_normal((1, 3, x.shape[2]))
    y_all, st_all = cv.causal_conv1d(x, w, b, conv_state=st0, activation="silu")
    y1, st1 = cv.causal_conv1d(x[:, :split], w, b, conv_state=st0, activation="silu")
    y2, st2 = cv.causal_conv1d(x[:, split:], w, b, conv_state=st1, activation="silu")
    close(np.concatenate([y1, y2], axis=1), y_all, 1e-12)
    close(st2, st_all, 0)


def test_conv1d_state_holds_the_last_inputs():
    x, w, b = conv_case(61, T=9, W=4)
    st0 = np.full((1, 3, x.shape[2]), 7.0)
    _, st = cv.causal_conv1d(x, w, b, conv_state=st0)
    close(st[0], x[0, -3:], 0)
    # a sequence of one token shifts the old state by one
    _, st = cv.causal_conv1d(x[:, :1], w, b, conv_state=st0)
    close(st[0], np.concatenate([st0[0, 1:], x[0, :1]]), 0)


def test_silu_values_and_odd_identity():
    z = np.linspace(-30, 30, 121)
    close(cv.silu(z) - cv.silu(-z), z, 1e-12)  # z s(z) + z s(-z) = z
    assert cv.silu(0.0) == 0.0
    close(cv.silu(1.0), 0.7310585786300049, 1e-15)  # the logistic function at 1
    close(cv.silu(40.0), 40.0, 1e-12)
    assert abs(cv.silu(-40.0)) < 1e-15


def test_conv1d_packed_equals_per_sequence_runs():
    """A packed batch with permuted cache lines, a sequence that starts from zeros and an
    empty sequence equals per-sequence runs on the matching lines."""
    rng = np.random.default_rng(71)
    C, W = 5, 3
    lens = [4, 0, 1, 6]
    x = rng.standard_normal((1, sum(lens), C))
    w, b = rng.standard_normal((C, W)), rng.standard_normal(C)
    st0 = rng.standard_normal((6, W - 1, C))
    idx = np.array([5, 0, 2, 3])
    init = np.array([1, 1, 0, 1])
    cu = np.concatenate([[0], np.cumsum(lens)])
    y, st = cv.causal_conv1d(x, w, b, conv_state=st0, cache_indices=idx,
                             has_initial_state=init, cu_seqlens=cu, activation="silu")
    for n in range(len(lens)):
        s, e = cu[n], cu[n + 1]
        head = st0[idx[n]] if init[n] else np.zeros((W - 1, C))
        yn, stn = cv.causal_conv1d(x[:, s:e], w, b, conv_state=head[None],
                                   activation="silu")
        close(y[0, s:e], yn[0], 0)
        close(st[idx[n]], stn[0], 0)
    close(st[1], st0[1], 0)  # an unused line is untouched
    close(st[4], st0[4], 0)
    close(st[0], st0[0], 0)  # the empty sequence leaves its line as it was


# ------------------------------------------------------------------ backward oracle
from oracle import backward as bw  # noqa: E402


def _loss_and_grads(case, scale, cu=None, seed=0):
    """A random linear loss L = <Wo, o> + <Wh, ht> of the C forward oracle, its analytic
    gradients from oracle.backward, and a central finite-difference check of each."""
    q, k, v, g, beta, h0 = case
    rng = np.random.default_rng(seed)
    o, ht = oracle.recurrence(q, k, v, g, beta, h0, scale=scale, cu_seqlens=cu)
    Wo, Wh = rng.standard_normal(o.shape), rng.standard_normal(ht.shape)

    def loss(q_, k_, v_, g_, b_, h_):
        o_, ht_ = oracle.recurrence(q_, k_, v_, g_, b_, h_, scale=scale, cu_seqlens=cu)
        return float(np.sum(Wo * o_) + np.sum(Wh * ht_))

    grads = bw.recurrence_backward(q, k, v, g, beta, h0, scale, Wo, Wh, cu_seqlens=cu)
    inputs = [q, k, v, g, beta, h0]
    eps = 1e-6
    for which, (x, dx) in enumerate(zip(inputs, grads)):
        if x is None:
            continue
        flat = x.reshape(-1)
        idx = rng.choice(flat.size, size=min(flat.size, 12), replace=False)
        for i in idx:
            keep = flat[i]
            flat[i] = keep + eps
            lp = loss(*inputs)
            flat[i] = keep - eps
            lm = loss(*inputs)
            flat[i] = keep
            fd = (lp - lm) / (2 * eps)
            an = dx.reshape(-1)[i]
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), (which, int(i), fd, an)
    return grads


@pytest.mark.parametrize("H,Hg", [(2, 2), (4, 2)])
def test_backward_matches_finite_differences(H, Hg):
    """Every input's gradient (q, k, v, g, beta, h0; GQA groups summing dq and dk) against
    central differences of the forward oracle."""
    case = rand_case(81 + H, B=2, T=9, H=H, Hg=Hg, Dk=4, Dv=3)
    _loss_and_grads(case, scale=0.7, seed=H)


def test_backward_packed_batch_matches_finite_differences():
    case = rand_case(85, B=1, T=11, H=2, Dk=3, Dv=4, h0=False)
    q, k, v, g, beta, _ = case
    cu = np.array([0, 4, 4, 11])
    h0 = 0.1 * np.random.default_rng(3).standard_normal((3, 2, 3, 4))
    grads = _loss_and_grads((q, k, v, g, beta, h0), scale=0.5, cu=cu, seed=9)
    # the empty sequence passes the ht gradient straight to h0
    _, _, _, _, _, dh0 = grads
    rng = np.random.default_rng(9)
    o, ht = oracle.recurrence(q, k, v, g, beta, h0, scale=0.5, cu_seqlens=cu)
    rng.standard_normal(o.shape)
    Wh = rng.standard_normal(ht.shape)
    close(dh0[1], Wh[1], 0)


def test_backward_planted_sign_error_is_caught():
    """A wrong sign in the decay gradient makes the finite-difference check fail."""
    case = rand_case(87, B=1, T=6, H=1, Dk=3, Dv=3)
    orig = bw._pair_backward

    def planted(*a):
        dq, dk, dv, dg, db, dH = orig(*a)
        return dq, dk, dv, -dg, db, dH

    bw._pair_backward = planted
    try:
        with pytest.raises(AssertionError):
            _loss_and_grads(case, scale=1.0, seed=1)
    finally:
        bw._pair_backward = orig


# ------------------------------------------------------------------ decode gating (f2)
from oracle import gating  # noqa: E402


def test_gating_functions_match_library_routines_everywhere():
    import scipy.special
    x = np.concatenate([np.linspace(-800, 800, 4001), [-1e-300, 0.0, 1e-300, 35.0, -35.0]])
    # softplus(x) = log(e^0 + e^x): numpy's logaddexp; sigmoid: scipy's expit
    assert np.allclose(gating.softplus(x), np.logaddexp(0.0, x), rtol=1e-14, atol=0)
    assert np.allclose(gating.sigmoid(x), scipy.special.expit(x), rtol=1e-14, atol=1e-300)
    assert np.all(np.isfinite(gating.softplus(x))) and np.all(np.isfinite(gating.sigmoid(x)))


def test_gating_identities():
    x = np.linspace(-30, 30, 601)
    close(gating.softplus(x) - gating.softplus(-x), x, 1e-12)   # softplus is x + s(-x)
    close(gating.sigmoid(x) + gating.sigmoid(-x), np.ones_like(x), 1e-15)
    h = 1e-6                                                             # d softplus = sigmoid
    close((gating.softplus(x + h) - gating.softplus(x - h)) / (2 * h), gating.sigmoid(x), 1e-8)
    assert gating.softplus(0.0) == np.log(2.0) and gating.sigmoid(0.0) == 0.5


def test_gates_closed_forms():
    z = np.zeros((1, 3, 2))
    g, beta = gating.gates(z, z, np.zeros(2))
    close(g, np.full_like(g, -np.log(2.0)), 1e-15)
    close(beta, np.full_like(beta, 0.5), 1e-15)
    # the rate exp(A_log) multiplies; dt_bias shifts a; both per head
    A_log = np.array([np.log(3.0), 0.0])
    dt_bias = np.array([0.0, 2.0])
    a = np.full((1, 1, 2), -2.0)
    g, _ = gating.gates(a, np.zeros((1, 1, 2)), A_log, dt_bias)
    close(g[0, 0], np.array([-3.0 * np.log1p(np.exp(-2.0)), -np.log(2.0)]), 1e-15)
    # a vanishing rate gives no decay whatever a is; the decay e^g always lies in (0, 1]
    g, _ = gating.gates(np.full((1, 4, 1), 40.0), np.zeros((1, 4, 1)), np.array([-800.0]))
    assert np.all(g == 0.0)
    rng = np.random.default_rng(3)
    g, beta = gating.gates(rng.standard_normal((2, 50, 4)) * 5, rng.standard_normal((2, 50, 4)),
                           rng.standard_normal(4), rng.standard_normal(4))
    assert np.all(g < 0) and np.all((beta > 0) & (beta < 1))


def test_gated_recurrence_hand_worked_token():
    """One token, Dk = Dv = 2, h0 = I, k = (1, 0), q = (0, 1), v = (2, 3), scale 1,
    A_log = a = dt_bias = b = 0: e^g = exp(-ln 2) = 1/2 and beta = 1/2, so
    S1 = 1/2 I (I - 1/2 k k^T) + 1/2 v k^T = [[1/4 + 1, 0], [3/2, 1/2]],
    o = S1 q = (0, 1/2) and ht = S1^T."""
    q = np.array([0.0, 1.0]).reshape(1, 1, 1, 2)
    k = np.array([1.0, 0.0]).reshape(1, 1, 1, 2)
    v = np.array([2.0, 3.0]).reshape(1, 1, 1, 2)
    z = np.zeros((1, 1, 1))
    h0 = np.eye(2).reshape(1, 1, 2, 2)
    o, ht = gating.gated_recurrence(q, k, v, z, z, np.zeros(1), np.zeros(1), h0, scale=1.0)
    close(o[0, 0, 0], np.array([0.0, 0.5]), 1e-15)
    close(ht[0, 0], np.array([[1.25, 1.5], [0.0, 0.5]]), 1e-15)


@pytest.mark.parametrize("mutation", ["rate_not_exponentiated", "beta_not_activated",
                                      "bias_ignored", "decay_sign"])
def test_gating_planted_mistakes_are_caught(mutation):
    """Copies of the gate map with one plausible slip each disagree with the closed forms."""
    def wrong(a, b, A_log, dt_bias):
        x = a + dt_bias
        if mutation == "rate_not_exponentiated":
            return -A_log * gating.softplus(x), gating.sigmoid(b)
        if mutation == "beta_not_activated":
            return -np.exp(A_log) * gating.softplus(x), b
        if mutation == "bias_ignored":
            return -np.exp(A_log) * gating.softplus(a), gating.sigmoid(b)
        return np.exp(A_log) * gating.softplus(x), gating.sigmoid(b)
    A_log = np.array([np.log(3.0)])
    dt_bias = np.array([2.0])
    a = np.full((1, 1, 1), -2.0)
    b = np.full((1, 1, 1), 0.7)
    g_ok, b_ok = gating.gates(a, b, A_log, dt_bias)
    close(g_ok, np.full_like(g_ok, -3.0 * np.log(2.0)), 1e-15)       # softplus(0) = ln 2
    close(b_ok, np.full_like(b_ok, 1.0 / (1.0 + np.exp(-0.7))), 1e-15)
    g_bad, b_bad = wrong(a, b, A_log, dt_bias)
    assert not (np.allclose(g_bad, g_ok) and np.allclose(b_bad, b_ok))


def test_gated_recurrence_is_the_recurrence_with_mapped_gates():
    """With g and beta from the gate map given directly, the plain recurrence agrees, and a
    vanishing rate with b -> +inf is the undecayed full-overwrite delta rule."""
    q, k, v, _, _, h0 = rand_case(31, B=2, T=9, H=4, Hg=2)
    rng = np.random.default_rng(32)
    a, b = rng.standard_normal((2, 9, 4)), rng.standard_normal((2, 9, 4))
    A_log, dt_bias = np.log(rng.uniform(1, 16, 4)), rng.standard_normal(4)
    o, ht = gating.gated_recurrence(q, k, v, a, b, A_log, dt_bias, h0)
    g = -np.exp(A_log) * np.logaddexp(0.0, a + dt_bias)
    beta = 1.0 / (1.0 + np.exp(-b))
    o2, ht2 = oracle.recurrence(q, k, v, g, beta, h0)
    close(o, o2, 1e-13)
    close(ht, ht2, 1e-13)
    big = np.full_like(b, 800.0)
    o3, ht3 = gating.gated_recurrence(q, k, v, a, big, np.full(4, -800.0), None, h0)
    o4, ht4 = oracle.recurrence(q, k, v, np.zeros_like(a), np.ones_like(b), h0)
    close(o3, o4, 1e-13)
    close(ht3, ht4, 1e-13)
