"""GPU checks of properties the mathematics fixes, on every variant, through the C ABI.

* Magnitude: every output is linear in (v, h0) jointly (the state recurrence and o are
  linear in them for fixed q, k, g, beta).  Scaling both by a power of two a must scale o
  and ht by exactly a, and every variant must stay within the bf16 tolerances of the fp64
  oracle at any magnitude bf16 holds, far outside fp16's range included.
* beta = 0: nothing is written into the state, so ht = e^{G_T} h0 and
  o_t = scale e^{G_t} h0^T q_t, with G_t the prefix sum of g over the sequence.  The
  expected values are that closed form evaluated in fp64 here, not the oracle.
"""
import numpy as np
import pytest
import torch

import gdn_inputs
from gdn_testlib import check_against_oracle, log, oracle_full, rel_l2, run_gdn, to64

pytestmark = pytest.mark.gpu

VARIANTS = ["fused", "segmented", "staged", "recurrent"]
SCALES = [2.0 ** -20, 2.0 ** -12, 2.0 ** 12, 2.0 ** 17]


def draw(**kw):
    return gdn_inputs.draw(gdn_inputs.small(**kw), device="cpu")


def scaled(inp, a):
    out = dict(inp)
    out["v"] = (inp["v"].float() * a).to(inp["v"].dtype)  # exact: a is a power of two
    out["h0"] = inp["h0"] * a
    return out


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("variant", VARIANTS)
def test_joint_linearity_in_v_and_h0(variant, D):
    inp = draw(B=2, T=200, H=2, Hg=1, Dk=D, C=64, seed=300 + D, h0_std=0.05)
    o1, ht1 = run_gdn(inp, variant=variant)
    o1, ht1 = to64(o1), to64(ht1)
    for a in SCALES:
        sa = scaled(inp, a)
        o_ref, ht_ref = oracle_full(sa)
        o, ht = run_gdn(sa, variant=variant)
        assert torch.isfinite(o.float()).all() and torch.isfinite(ht).all(), (variant, a)
        eo, eh = check_against_oracle(sa, o, ht, o_ref, ht_ref, "%s a=%g" % (variant, a))
        # linearity of the GPU path itself: o(a v, a h0) = a o(v, h0)
        lo = rel_l2(to64(o) / a, o1)
        lh = rel_l2(to64(ht) / a, ht1)
        log(test="linearity", variant=variant, D=D, a=a, o_rel=eo, ht_rel=eh, lin_o=lo,
            lin_ht=lh)
        assert lo <= 1e-6 and lh <= 1e-6, (variant, a, lo, lh)


@pytest.mark.parametrize("variant", VARIANTS)
def test_large_and_small_values_in_one_batch(variant):
    """Sequences of very different magnitude side by side in one packed batch (each
    sequence's own v and h0 scaled): every sequence stays within the tolerances."""
    lens = [150, 1, 70, 200]
    mags = [2.0 ** 16, 2.0 ** -16, 1.0, 2.0 ** 10]
    w = gdn_inputs.small(H=2, Hg=2, Dk=128, C=64, seed=77, h0_std=0.05)
    inp = gdn_inputs.draw(w.with_(B=1, T=sum(lens)), device="cpu")
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    inp["cu_seqlens"] = torch.from_numpy(cu)
    h0 = torch.randn(len(lens), 2, 128, 128, generator=torch.Generator().manual_seed(9)) * 0.05
    v = inp["v"].float().clone()
    for n, a in enumerate(mags):
        v[:, cu[n]:cu[n + 1]] *= a
        h0[n] *= a
    inp["v"], inp["h0"] = v.to(inp["v"].dtype), h0
    o_ref, ht_ref = oracle_full(inp)
    o, ht = run_gdn(inp, variant=variant)
    o64, ht64 = to64(o), to64(ht)
    assert np.isfinite(o64).all() and np.isfinite(ht64).all()
    for n in range(len(lens)):
        for h in range(2):
            ts = slice(int(cu[n]), int(cu[n + 1]))
            assert rel_l2(o64[0, ts, h], o_ref[0, ts, h]) <= 5e-3, (n, h)
            assert rel_l2(ht64[n, h], ht_ref[n, h]) <= 1e-2, (n, h)


def beta_zero_closed_form(inp):
    """ht = e^{G_T} h0 and o_t = scale e^{G_t} h0^T q_t (fp64, per sequence and head)."""
    q = to64(inp["q"])
    g = to64(inp["g"])
    h0 = to64(inp["h0"])
    B, T, Hg, D = q.shape
    H = g.shape[2]
    grp = H // Hg
    o = np.zeros((B, T, H, D))
    ht = np.zeros_like(h0)
    for n in range(B):
        for h in range(H):
            G = np.cumsum(g[n, :, h])
            o[n, :, h] = inp["scale"] * np.exp(G)[:, None] * (q[n, :, h // grp] @ h0[n, h])
            ht[n, h] = np.exp(G[-1]) * h0[n, h]
    return o, ht


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("variant", VARIANTS)
def test_beta_zero_is_pure_decay(variant, D):
    inp = draw(B=2, T=150, H=4, Hg=2, Dk=D, C=64, seed=400 + D, h0_std=0.1)
    inp["beta"] = torch.zeros_like(inp["beta"])
    o_ref, ht_ref = beta_zero_closed_form(inp)
    o, ht = run_gdn(inp, variant=variant)
    eo, eh = check_against_oracle(inp, o, ht, o_ref, ht_ref, "beta=0 %s D%d" % (variant, D))
    log(test="beta_zero", variant=variant, D=D, o_rel=eo, ht_rel=eh)
