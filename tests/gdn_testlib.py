"""Shared helpers for the libgdn tests: metrics, oracle calls on sampled (sequence, head)
pairs, and running the HIP path through the C ABI binding."""
from __future__ import annotations

import json
import os

import numpy as np
import torch

import oracle


def log(**kw):
    """Print one JSON record; also append it to $GDN_PARITY_LOG when that is set (pytest
    captures the output of passing tests)."""
    print(json.dumps(kw), flush=True)
    path = os.environ.get("GDN_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(kw) + "\n")

# Tolerances (stated for the workloads): fp32 max-abs on o and ht; bf16 relative L2 error
# over the whole tensor.
TOL_F32_MAXABS = 1e-4
TOL_BF16_O = 5e-3
TOL_BF16_HT = 1e-2


def rel_l2(x, ref) -> float:
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / (den if den > 0 else 1.0))


def max_abs(x, ref) -> float:
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.abs(x - ref).max()) if x.size else 0.0


def to64(t):
    return None if t is None else t.detach().to("cpu", torch.float64).numpy()


def oracle_full(inp):
    """Oracle on every pair of a (small) input dict from gdn_inputs.draw."""
    return oracle.recurrence(inp["q"].cpu(), inp["k"].cpu(), inp["v"].cpu(), inp["g"].cpu(),
                             inp["beta"].cpu(),
                             None if inp["h0"] is None else inp["h0"].cpu(),
                             scale=inp["scale"],
                             cu_seqlens=None if inp["cu_seqlens"] is None
                             else inp["cu_seqlens"].cpu().numpy())


def pair_slices(inp, n, h):
    """Index the tokens and heads of pair (n, h): returns (token slice, batch row, q/k head)."""
    q = inp["q"]
    B, T, Hg, _ = q.shape
    H = inp["v"].shape[2]
    hk = h // (H // Hg)
    if inp["cu_seqlens"] is None:
        return slice(0, T), n, hk
    cu = inp["cu_seqlens"].cpu().numpy()
    return slice(int(cu[n]), int(cu[n + 1])), 0, hk


def oracle_pairs(inp, pairs, nthreads=0):
    """Oracle for sampled (n, h) pairs only.  The pairs' tokens are copied to the host and
    packed as one variable-length batch with a single head, so the oracle's parallel loop
    over (sequence, head) runs them side by side.
    Returns {(n, h): (o [L, Dv], ht [Dk, Dv])}."""
    pairs = list(pairs)
    if not pairs:
        return {}
    qs, ks, vs, gs, bs, h0s, lens = [], [], [], [], [], [], []
    for n, h in pairs:
        ts, b, hk = pair_slices(inp, n, h)
        qs.append(inp["q"][b, ts, hk].detach().cpu())
        ks.append(inp["k"][b, ts, hk].detach().cpu())
        vs.append(inp["v"][b, ts, h].detach().cpu())
        gs.append(inp["g"][b, ts, h].detach().cpu())
        bs.append(inp["beta"][b, ts, h].detach().cpu())
        if inp["h0"] is not None:
            h0s.append(inp["h0"][n, h].detach().cpu())
        lens.append(qs[-1].shape[0])
    cat = lambda xs: torch.cat(xs, 0)[None, :, None]
    cu = np.zeros(len(pairs) + 1, np.int64)
    cu[1:] = np.cumsum(lens)
    h0 = torch.stack(h0s)[:, None] if h0s else None
    o, ht = oracle.recurrence(cat(qs), cat(ks), cat(vs), cat(gs), cat(bs), h0,
                              scale=inp["scale"], cu_seqlens=cu, nthreads=nthreads)
    return {p: (o[0, cu[i]:cu[i + 1], 0], ht[i, 0]) for i, p in enumerate(pairs)}


def run_gdn(inp, variant="auto", C=None, output_final_state=True, **kw):
    from gated_deltanet_chunked_02_amd import chunk_gated_delta_rule
    dev = torch.device("cuda")
    mv = lambda t: None if t is None else t.to(dev)
    o, ht = chunk_gated_delta_rule(mv(inp["q"]), mv(inp["k"]), mv(inp["v"]), mv(inp["g"]),
                                   mv(inp["beta"]), scale=inp["scale"],
                                   initial_state=mv(inp["h0"]),
                                   output_final_state=output_final_state,
                                   cu_seqlens=mv(inp["cu_seqlens"]),
                                   chunk_size=C or inp["C"], variant=variant, **kw)
    torch.cuda.synchronize()
    return o, ht


def check_against_oracle(inp, o, ht, o_ref, ht_ref, label=""):
    """Apply the tolerance of the workload's dtype; returns the measured errors."""
    o64, ht64 = to64(o), to64(ht)
    if inp["q"].dtype == torch.float32:
        eo, eh = max_abs(o64, o_ref), max_abs(ht64, ht_ref)
        assert eo <= TOL_F32_MAXABS, "%s o max-abs %.3g" % (label, eo)
        assert eh <= TOL_F32_MAXABS, "%s ht max-abs %.3g" % (label, eh)
    else:
        eo, eh = rel_l2(o64, o_ref), rel_l2(ht64, ht_ref)
        assert eo <= TOL_BF16_O, "%s o rel-L2 %.3g" % (label, eo)
        assert eh <= TOL_BF16_HT, "%s ht rel-L2 %.3g" % (label, eh)
    assert np.isfinite(o64).all() and np.isfinite(ht64).all()
    return eo, eh
