"""GPU parity of the decode operator with in-kernel gates (gdn_fused_sigmoid_gating_delta_rule)
against the fp64 oracle (oracle.gating: the gate map, then the token recurrence), through
the C ABI, at the tolerances of the input dtype (fp32: max-abs 1e-4; bf16: relative L2
5e-3 on o and 1e-2 on ht)."""
import numpy as np
import pytest
import torch

import gdn_inputs
from gdn_testlib import check_against_oracle, log, rel_l2, to64

pytestmark = pytest.mark.gpu


def case(B=4, T=1, H=4, Hg=2, D=128, dtype="bf16", seed=0, h0_std=0.05, lens=None,
         beta_dtype=""):
    w = gdn_inputs.small(B=B, T=T, H=H, Hg=Hg, Dk=D, dtype=dtype, seed=seed, h0_std=h0_std,
                         beta_dtype=beta_dtype)
    if lens is not None:
        w = w.with_(B=1, T=sum(lens))
    inp = gdn_inputs.draw(w, device="cpu")
    if lens is not None:
        inp["cu_seqlens"] = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32))
        if h0_std is not None:
            inp["h0"] = torch.randn(len(lens), H, D, D,
                                    generator=torch.Generator().manual_seed(seed)) * h0_std
    Bx, Tx = inp["g"].shape[:2]
    inp.update(gdn_inputs.draw_gating(w, Bx, Tx, device="cpu"))
    return inp


def oracle_gated(inp, dt_bias=True):
    from oracle import gating
    return gating.gated_recurrence(
        inp["q"], inp["k"], inp["v"], inp["a"], inp["b"], inp["A_log"],
        inp["dt_bias"] if dt_bias else None, inp["h0"], scale=inp["scale"],
        cu_seqlens=None if inp["cu_seqlens"] is None else inp["cu_seqlens"].numpy())


def run_gated(inp, dt_bias=True, **kw):
    from gated_deltanet_chunked_02_amd import fused_sigmoid_gating_delta_rule
    dev = torch.device("cuda")
    mv = lambda t: None if t is None else t.to(dev)
    o, ht = fused_sigmoid_gating_delta_rule(
        mv(inp["q"]), mv(inp["k"]), mv(inp["v"]), mv(inp["a"]), mv(inp["b"]),
        mv(inp["A_log"]), mv(inp["dt_bias"]) if dt_bias else None, scale=inp["scale"],
        initial_state=mv(inp["h0"]), cu_seqlens=mv(inp["cu_seqlens"]), **kw)
    torch.cuda.synchronize()
    return o, ht


CASES = [
    # B, T, H, Hg, D, dtype, h0
    (8, 1, 4, 2, 128, "bf16", True),
    (3, 5, 4, 4, 128, "bf16", True),
    (2, 40, 2, 1, 128, "f32", False),
    (4, 1, 4, 1, 64, "bf16", True),
    (2, 7, 2, 2, 64, "f32", True),
    (2, 3, 2, 1, 256, "bf16", True),
    (1, 4, 2, 2, 256, "f32", True),
]


@pytest.mark.parametrize("B,T,H,Hg,D,dtype,h0", CASES)
def test_gated_decode_matches_oracle(B, T, H, Hg, D, dtype, h0):
    inp = case(B=B, T=T, H=H, Hg=Hg, D=D, dtype=dtype, seed=D + T + B,
               h0_std=0.05 if h0 else None)
    o_ref, ht_ref = oracle_gated(inp)
    o, ht = run_gated(inp)
    eo, eh = check_against_oracle(inp, o, ht, o_ref, ht_ref, "gated D%d %s" % (D, dtype))
    log(test="gated", D=D, dtype=dtype, B=B, T=T, o_err=eo, ht_err=eh)


def test_gated_without_dt_bias_and_with_fp32_gate_inputs():
    inp = case(B=4, T=3, D=128, seed=5, beta_dtype="f32")
    assert inp["a"].dtype == torch.float32 and inp["q"].dtype == torch.bfloat16
    o_ref, ht_ref = oracle_gated(inp, dt_bias=False)
    o, ht = run_gated(inp, dt_bias=False)
    check_against_oracle(inp, o, ht, o_ref, ht_ref, "gated, no dt_bias, fp32 a/b")


@pytest.mark.parametrize("D,dtype", [(64, "bf16"), (128, "bf16"), (256, "bf16"), (128, "f32")])
def test_gated_varlen_edge_lengths(D, dtype):
    lens = [1, 0, 3, 1, 17, 2]
    inp = case(H=4, Hg=2, D=D, dtype=dtype, seed=13, lens=lens)
    o_ref, ht_ref = oracle_gated(inp)
    o, ht = run_gated(inp)
    check_against_oracle(inp, o, ht, o_ref, ht_ref, "gated varlen D%d" % D)
    assert torch.equal(ht[1].cpu(), inp["h0"][1])  # the empty sequence keeps its state


@pytest.mark.parametrize("regime", ["fast_decay", "no_decay", "beta_saturated"])
def test_gated_extremes(regime):
    """Large rates and steps (the decay e^g underflows), a vanishing rate (no decay), and
    |b| = 30 (beta at 0 and 1 to fp32 precision): finite and at the tolerances."""
    inp = case(B=3, T=6, D=128, seed=71)
    if regime == "fast_decay":
        inp["A_log"] = torch.full_like(inp["A_log"], np.log(16.0))
        inp["a"] = (inp["a"].float() * 4 + 8).to(inp["a"].dtype)
    elif regime == "no_decay":
        inp["A_log"] = torch.full_like(inp["A_log"], -60.0)
    else:
        sign = torch.sign(torch.randn(inp["b"].shape, generator=torch.Generator().manual_seed(1)))
        inp["b"] = (30.0 * sign).to(inp["b"].dtype)
    o_ref, ht_ref = oracle_gated(inp)
    o, ht = run_gated(inp)
    assert torch.isfinite(o.float()).all() and torch.isfinite(ht).all()
    check_against_oracle(inp, o, ht, o_ref, ht_ref, "gated " + regime)


def test_gated_decode_loop_in_place_equals_one_call():
    """One token per call with the state updated in place (a serving loop) equals one call
    over all tokens, bit for bit, and the oracle."""
    from gated_deltanet_chunked_02_amd import fused_sigmoid_gating_delta_rule
    inp = case(B=3, T=6, H=4, Hg=2, D=128, seed=17)
    o_ref, ht_ref = oracle_gated(inp)
    dev = torch.device("cuda")
    state = inp["h0"].clone().to(dev)
    A_log, dt_bias = inp["A_log"].to(dev), inp["dt_bias"].to(dev)
    outs = []
    for t in range(6):
        sl = lambda x: x[:, t:t + 1].contiguous().to(dev)
        o, st = fused_sigmoid_gating_delta_rule(
            sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), sl(inp["a"]), sl(inp["b"]), A_log,
            dt_bias, scale=inp["scale"], initial_state=state, inplace_final_state=True)
        assert st is state
        outs.append(o)
    torch.cuda.synchronize()
    o_loop = torch.cat(outs, dim=1)
    check_against_oracle(inp, o_loop, state, o_ref, ht_ref, "gated loop")
    o_one, ht_one = run_gated(inp)
    assert torch.equal(o_one, o_loop) and torch.equal(ht_one, state)


def test_gated_equals_recurrent_with_the_mapped_gates():
    """The same decode step through gdn_chunk_fwd's recurrent variant, fed the gates the
    oracle's map makes (rounded to fp32): the two kernels agree to fp32 rounding of g."""
    from gated_deltanet_chunked_02_amd import chunk_gated_delta_rule
    from oracle import gating
    inp = case(B=8, T=2, D=128, seed=23, beta_dtype="f32")
    g, beta = gating.gates(inp["a"], inp["b"], inp["A_log"], inp["dt_bias"])
    dev = torch.device("cuda")
    o1, ht1 = chunk_gated_delta_rule(
        inp["q"].to(dev), inp["k"].to(dev), inp["v"].to(dev),
        torch.from_numpy(g).float().to(dev), torch.from_numpy(beta).float().to(dev),
        scale=inp["scale"], initial_state=inp["h0"].to(dev), variant="recurrent")
    o2, ht2 = run_gated(inp)
    assert rel_l2(to64(o1), to64(o2)) <= 1e-3 and rel_l2(to64(ht1), to64(ht2)) <= 1e-5


def test_gated_empty_token_axis_passes_state():
    from gated_deltanet_chunked_02_amd import fused_sigmoid_gating_delta_rule
    dev = torch.device("cuda")
    q = torch.empty(2, 0, 2, 64, dtype=torch.bfloat16, device=dev)
    ab = torch.empty(2, 0, 2, dtype=torch.bfloat16, device=dev)
    A_log = torch.zeros(2, device=dev)
    h0 = torch.randn(2, 2, 64, 64, generator=torch.Generator().manual_seed(3)).to(dev)
    o, ht = fused_sigmoid_gating_delta_rule(q, q, q, ab, ab, A_log, initial_state=h0)
    torch.cuda.synchronize()
    assert o.shape == (2, 0, 2, 64) and torch.equal(ht, h0)
