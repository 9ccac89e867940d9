"""GPU parity of the backward pass (gdn_chunk_bwd) against the fp64 oracle's reverse-mode
derivative of the token recurrence (oracle.backward, itself pinned by finite differences),
through the C ABI.  Every gradient is compared over the whole tensor by relative L2 error:
fp32 inputs at 1e-5 (fp32 matrix-core products throughout), bf16 inputs at 1e-2 (the
backward rounds its matrix-core operands and its stored intermediates to bf16, as the
forward does: a relative error of about 2^-9 per rounding, a few roundings deep).  Sizes
span several 64-token chunks and a ragged tail; varlen batches hold empty and one-token
sequences; the full-size case samples (sequence, head) pairs of the 16 x 8192 workload."""
import numpy as np
import pytest
import torch

import gdn_inputs
from gdn_testlib import log, rel_l2, to64

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dg", "dbeta", "dh0")


def tol(dtype, name):
    return 1e-5 if dtype == "f32" else 1e-2


def draw(B=1, T=200, H=4, Hg=2, D=128, dtype="bf16", seed=0, h0=True, dht=True, lens=None,
         beta_dtype=""):
    w = gdn_inputs.small(B=B, T=T, H=H, Hg=Hg, Dk=D, dtype=dtype, seed=seed,
                         h0_std=0.05 if h0 else None, beta_dtype=beta_dtype)
    N = B
    if lens is not None:
        w = w.with_(B=1, T=int(sum(lens)))
        N = len(lens)
    inp = gdn_inputs.draw(w, device="cpu")
    if lens is not None:
        inp["cu_seqlens"] = torch.from_numpy(
            np.concatenate([[0], np.cumsum(lens)]).astype(np.int32))
        if h0:
            inp["h0"] = torch.randn(N, H, D, D, generator=torch.Generator().manual_seed(seed)) * 0.05
    Bx, Tx = inp["g"].shape[:2]
    inp.update(gdn_inputs.draw_grads(w, Bx, Tx, N, dht_std=0.1 if dht else None))
    return inp


def oracle_bwd(inp):
    from oracle import backward
    cu = None if inp["cu_seqlens"] is None else inp["cu_seqlens"].numpy()
    h0 = None if inp["h0"] is None else inp["h0"].double().numpy()
    dht = None if inp["dht"] is None else inp["dht"].double().numpy()
    f = lambda x: x.double().numpy()
    return backward.recurrence_backward(f(inp["q"]), f(inp["k"]), f(inp["v"]), f(inp["g"]),
                                        f(inp["beta"]), h0, inp["scale"], f(inp["do"]), dht,
                                        cu_seqlens=cu)


def run_bwd(inp, variant="auto", grad_dtype=None):
    from gated_deltanet_chunked_02_amd import chunk_gated_delta_rule_bwd
    dev = torch.device("cuda")
    mv = lambda t: None if t is None else t.to(dev)
    out = chunk_gated_delta_rule_bwd(
        mv(inp["q"]), mv(inp["k"]), mv(inp["v"]), mv(inp["g"]), mv(inp["beta"]),
        mv(inp["do"]), dht=mv(inp["dht"]), scale=inp["scale"], initial_state=mv(inp["h0"]),
        cu_seqlens=mv(inp["cu_seqlens"]), variant=variant, grad_dtype=grad_dtype)
    torch.cuda.synchronize()
    return out


def compare(inp, got, ref, dtype, label):
    errs = {}
    for name, x, r in zip(NAMES, got, ref):
        if name == "dh0" and inp["h0"] is None:
            assert x is None
            continue
        x = to64(x)
        assert np.isfinite(x).all(), (label, name)
        errs[name] = rel_l2(x, r)
    log(test="backward", case=label, **errs)
    for name, e in errs.items():
        assert e <= tol(dtype, name), (label, name, e, errs)
    return errs


CASES = [
    # B, T, H, Hg, D, dtype, h0, dht
    (2, 200, 4, 2, 128, "bf16", True, True),
    (2, 130, 2, 2, 64, "bf16", False, False),
    (1, 150, 4, 1, 64, "bf16", True, True),
    (1, 256, 2, 2, 64, "f32", True, True),
    (2, 77, 2, 1, 64, "f32", False, True),
    (3, 64, 2, 2, 128, "bf16", True, False),
]


@pytest.mark.parametrize("B,T,H,Hg,D,dtype,h0,dht", CASES)
def test_backward_matches_oracle(B, T, H, Hg, D, dtype, h0, dht):
    inp = draw(B=B, T=T, H=H, Hg=Hg, D=D, dtype=dtype, seed=B * 7 + T + D, h0=h0, dht=dht)
    compare(inp, run_bwd(inp), oracle_bwd(inp), dtype,
            "B%d T%d H%d Hg%d D%d %s" % (B, T, H, Hg, D, dtype))


@pytest.mark.parametrize("D,dtype", [(128, "bf16"), (64, "bf16"), (64, "f32")])
def test_backward_varlen_with_empty_and_short_sequences(D, dtype):
    lens = [70, 0, 1, 64, 129, 5]
    inp = draw(H=4, Hg=2, D=D, dtype=dtype, seed=31, lens=lens)
    got = run_bwd(inp)
    ref = oracle_bwd(inp)
    compare(inp, got, ref, dtype, "varlen D%d %s" % (D, dtype))
    # the empty sequence's state passes through: its dh0 is its dht, exactly
    assert torch.equal(got[5][1].cpu(), inp["dht"][1])
    # per-sequence errors (a short sequence must not hide behind the long ones)
    cu = inp["cu_seqlens"].numpy()
    for n in range(len(lens)):
        s0, s1 = int(cu[n]), int(cu[n + 1])
        if s1 == s0:
            continue
        e = rel_l2(to64(got[2])[:, s0:s1], ref[2][:, s0:s1])
        assert e <= tol(dtype, "dv"), (n, e)


def test_backward_many_pairs_two_workgroups_per_cu():
    # 72 sequences x 32 heads: enough (sequence, head) pairs (8 per CU) for the reverse pass
    # to run its two-workgroups-per-CU layout (four waves of two column blocks, tiles copied
    # straight into LDS); short sequences with empty and one-token ones among them
    rng = np.random.default_rng(5)
    lens = [int(x) for x in rng.integers(0, 41, size=72)]
    lens[3], lens[10] = 0, 1
    inp = draw(H=32, Hg=16, D=128, dtype="bf16", seed=53, lens=lens)
    got = run_bwd(inp)
    ref = oracle_bwd(inp)
    compare(inp, got, ref, "bf16", "many pairs")
    cu = inp["cu_seqlens"].numpy()
    for n in range(len(lens)):
        s0, s1 = int(cu[n]), int(cu[n + 1])
        if s1 == s0:
            continue
        for i in (0, 2):  # dq and dv of the sequence
            e = rel_l2(to64(got[i])[:, s0:s1], ref[i][:, s0:s1])
            assert e <= tol("bf16", NAMES[i]), (n, NAMES[i], e)


@pytest.mark.parametrize("lens", [None, [70, 0, 1, 64, 129, 5]])
def test_backward_bf16_gradients_are_the_fp32_ones_rounded(lens):
    # bf16 gradients round the kernel's fp32 values once, at the store: dq, dk and dv equal the
    # fp32 gradients rounded to bf16 bit for bit, dg, dbeta and dh0 stay fp32 and unchanged,
    # and all of them are within the bf16 tolerance of the oracle
    inp = draw(B=2 if lens is None else 1, T=200, H=4, Hg=2, D=128, seed=61, lens=lens)
    g32 = run_bwd(inp)
    g16 = run_bwd(inp, grad_dtype=torch.bfloat16)
    for i in (0, 1, 2):
        assert g16[i].dtype == torch.bfloat16, NAMES[i]
        assert torch.equal(g16[i], g32[i].to(torch.bfloat16)), NAMES[i]
    for i in (3, 4, 5):
        assert g16[i].dtype == torch.float32 and torch.equal(g16[i], g32[i]), NAMES[i]
    compare(inp, g16, oracle_bwd(inp), "bf16", "bf16 gradients %s" % ("dense" if lens is None
                                                                       else "varlen"))


def test_backward_fp32_beta_with_bf16_inputs():
    inp = draw(B=1, T=100, H=2, Hg=2, D=128, seed=41, beta_dtype="f32")
    assert inp["beta"].dtype == torch.float32 and inp["q"].dtype == torch.bfloat16
    compare(inp, run_bwd(inp), oracle_bwd(inp), "bf16", "bf16 fp32-beta")


def test_backward_beta_zero_closed_form():
    """beta = 0: the state only decays (h_t = e^{G_t} h0), so o_t = scale e^{G_t} h0^T q_t;
    then dq_t = scale e^{G_t} h0 do_t, dk = dv = 0 and dh0 = sum_t scale e^{G_t} q_t do_t^T +
    e^{G_T} dht, in closed form (fp32 inputs)."""
    inp = draw(B=1, T=90, H=2, Hg=2, D=64, dtype="f32", seed=43)
    inp["beta"] = torch.zeros_like(inp["beta"])
    dq, dk, dv, dg, dbeta, dh0 = run_bwd(inp)
    G = np.cumsum(inp["g"].double().numpy()[0], axis=0)  # [T, H]
    q, do = inp["q"].double().numpy()[0], inp["do"].double().numpy()[0]
    h0, dht = inp["h0"].double().numpy()[0], inp["dht"].double().numpy()[0]
    s = inp["scale"]
    for h in range(2):
        e = np.exp(G[:, h])
        dq_ref = s * e[:, None] * (do[:, h] @ h0[h].T)
        dh0_ref = s * (q[:, h] * e[:, None]).T @ do[:, h] + e[-1] * dht[h]
        assert rel_l2(to64(dq)[0, :, h], dq_ref) <= 1e-5
        assert rel_l2(to64(dh0)[0, h], dh0_ref) <= 1e-5
    assert float(dk.abs().max()) == 0.0
    assert float(dv.abs().max()) == 0.0


def test_backward_empty_token_axis_passes_dht():
    from gated_deltanet_chunked_02_amd import chunk_gated_delta_rule_bwd
    dev = torch.device("cuda")
    q = torch.empty(2, 0, 2, 64, dtype=torch.bfloat16, device=dev)
    g = torch.empty(2, 0, 2, device=dev)
    h0 = torch.zeros(2, 2, 64, 64, device=dev)
    dht = torch.randn(2, 2, 64, 64, generator=torch.Generator().manual_seed(3)).to(dev)
    out = chunk_gated_delta_rule_bwd(q, q, q, g, g.to(torch.bfloat16), q, dht=dht,
                                     initial_state=h0)
    torch.cuda.synchronize()
    assert out[0].shape == (2, 0, 2, 64) and torch.equal(out[5], dht)
    out = chunk_gated_delta_rule_bwd(q, q, q, g, g.to(torch.bfloat16), q, initial_state=h0)
    torch.cuda.synchronize()
    assert float(out[5].abs().max()) == 0.0


def test_backward_is_deterministic():
    inp = draw(B=2, T=300, H=4, Hg=1, D=128, seed=47)
    a = run_bwd(inp)
    b = run_bwd(inp)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_backward_full_size_sampled_pairs():
    """16 x 8192, H = 32, D = 128, bf16, no initial state: the whole backward on the GPU,
    two (sequence, head) pairs checked against the oracle (dq, dk, dv, dg, dbeta of the
    pair's tokens; q/k heads are not shared here, so a pair's dq and dk are its own)."""
    from oracle import backward
    w = gdn_inputs.WORKLOADS["headline"]
    inp = gdn_inputs.draw(w, device="cpu")
    inp.update(gdn_inputs.draw_grads(w, w.B, w.T, w.B, dht_std=None))
    got = run_bwd(inp)
    f = lambda x: x.double().numpy()
    for n, h in ((0, 0), (15, 31)):
        sl = lambda x: f(x[n:n + 1, :, h:h + 1])
        ref = backward.recurrence_backward(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]),
                                           sl(inp["g"]), sl(inp["beta"]), None, inp["scale"],
                                           sl(inp["do"]), None)
        errs = {}
        for name, x, r in zip(NAMES[:5], got[:5], ref[:5]):
            errs[name] = rel_l2(to64(x[n:n + 1, :, h:h + 1]), r)
        log(test="backward_fullsize", pair=[n, h], **errs)
        for name, e in errs.items():
            assert e <= tol("bf16", name), (n, h, name, e)


# ------------------------------------------------------------------ segmented reverse pass
SEG_CASES = [
    # B, T, H, Hg, D, h0, dht, lens: forced segments of 64 tokens and more, ragged last ones
    (1, 700, 2, 1, 128, True, True, None),
    (2, 333, 2, 2, 64, False, True, None),
    (1, 0, 4, 2, 128, True, True, [70, 0, 1, 300, 200, 64]),
    (1, 0, 2, 2, 64, True, False, [513, 129]),
]


@pytest.mark.parametrize("B,T,H,Hg,D,h0,dht,lens", SEG_CASES)
def test_backward_segmented_matches_oracle(B, T, H, Hg, D, h0, dht, lens):
    """Both sequential passes per segment (the state maps of the segmented forward, the
    adjoint maps composed last to first) against the oracle, and against the one-pass
    backward on the same inputs."""
    import gated_deltanet_chunked_02_amd as gdn
    inp = draw(B=B, T=T, H=H, Hg=Hg, D=D, seed=B * 11 + T + D + H, h0=h0, dht=dht, lens=lens)
    label = "segmented B%d T%d H%d Hg%d D%d lens %s" % (B, T, H, Hg, D, lens)
    print(label, flush=True)
    q, v, beta, cu = inp["q"], inp["v"], inp["beta"], inp["cu_seqlens"]
    desc = gdn.make_desc(q, v, beta, cu, 64, "segmented")
    assert gdn.gdn_chunk_bwd_resolved_variant(desc, cu) == "segmented"
    got = run_bwd(inp, "segmented")
    compare(inp, got, oracle_bwd(inp), "bf16", label)
    flat = run_bwd(inp, "fused")
    for name, x, y in zip(NAMES, got, flat):
        if x is not None:
            assert rel_l2(to64(x), to64(y)) <= 1e-2, (name, label)


@pytest.mark.parametrize("decay", ["workload", "slow"])
def test_backward_long_prompt_segments(decay):
    """1 x 65536 tokens, H = 32 over Hg = 16, D = 128, bf16: AUTO runs the passes per
    segment (8 segments of 8192 tokens); every gradient against the one-pass backward, and
    one (sequence, head) pair's dv, dg, dbeta against the oracle (dq and dk sum the two value
    heads of a q/k head).  With the workload's gates (about e^-0.05 per token) no trace of a
    segment's start state survives 8192 tokens in fp32, so both paths agree bit for bit;
    the slow decay (g / 500: about e^-0.8 over a segment) makes the composition across
    segments carry real weight."""
    import gated_deltanet_chunked_02_amd as gdn
    from oracle import backward
    w = gdn_inputs.WORKLOADS["long"].with_(T=65536)
    inp = gdn_inputs.draw(w, device="cpu")
    if decay == "slow":
        inp["g"] = inp["g"] / 500.0
    inp.update(gdn_inputs.draw_grads(w, w.B, w.T, w.B, dht_std=0.1))
    desc = gdn.make_desc(inp["q"], inp["v"], inp["beta"], None, 64, "auto")
    assert gdn.gdn_chunk_bwd_resolved_variant(desc) == "segmented"
    print("long prompt backward, segmented", flush=True)
    got = run_bwd(inp)
    print("long prompt backward, one pass per sequence", flush=True)
    flat = run_bwd(inp, "fused")
    errs = {}
    for name, x, y in zip(NAMES[:5], got[:5], flat[:5]):
        errs[name] = rel_l2(to64(x), to64(y))
    log(test="backward_long_segmented_vs_flat", decay=decay, **errs)
    for name, e in errs.items():
        assert e <= 1e-2, (name, e)
    f = lambda x: x.double().numpy()
    h = 5
    sl = lambda x: f(x[:, :, h:h + 1])
    hk = h // (w.H // w.Hg)
    ref = backward.recurrence_backward(f(inp["q"][:, :, hk:hk + 1]), f(inp["k"][:, :, hk:hk + 1]),
                                       sl(inp["v"]), sl(inp["g"]), sl(inp["beta"]), None,
                                       inp["scale"], sl(inp["do"]), None if inp["dht"] is None
                                       else f(inp["dht"][:, h:h + 1]))
    perr = {}
    for i, name in ((2, "dv"), (3, "dg"), (4, "dbeta")):
        perr[name] = rel_l2(to64(got[i][:, :, h:h + 1]), ref[i])
    log(test="backward_long_segmented_pair", decay=decay, head=h, **perr)
    for name, e in perr.items():
        assert e <= 1e-2, (name, e)


@pytest.mark.parametrize("kv,kd", [(-20, 0), (17, 0), (0, -20), (0, 17), (12, -12)])
def test_backward_power_of_two_scaling(kv, kd):
    """The gradients are linear in (do, dht) and, jointly with the forward, homogeneous in
    (v, h0): scaling v and h0 by 2^kv scales dq, dk, dg and dbeta by 2^kv and leaves dv and dh0
    alone; scaling do and dht by 2^kd scales every gradient by 2^kd.  Powers of two are exact
    in binary floating point and every operand of the path is bf16 or fp32 (exponent range
    of fp32), so the relations hold bit for bit far outside the range of fp16; a step that
    kept any of these values in fp16 would overflow or flush them."""
    inp = draw(B=1, T=200, H=4, Hg=2, D=128, seed=53)
    base = run_bwd(inp)
    s = dict(inp)
    s["v"] = (inp["v"].float() * 2.0 ** kv).to(inp["v"].dtype)
    s["h0"] = inp["h0"] * 2.0 ** kv
    s["do"] = (inp["do"].float() * 2.0 ** kd).to(inp["do"].dtype)
    s["dht"] = inp["dht"] * 2.0 ** kd
    got = run_bwd(s)
    for name, x, y in zip(NAMES, got, base):
        f = 2.0 ** kd * (2.0 ** kv if name in ("dq", "dk", "dg", "dbeta") else 1.0)
        assert torch.isfinite(x).all(), (name, kv, kd)
        assert torch.equal(x, y * f), (name, kv, kd, rel_l2(to64(x), to64(y) * f))
