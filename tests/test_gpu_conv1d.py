"""GPU parity of the causal conv1d (gdn_causal_conv1d_fwd, through the C ABI) against the
fp64 oracle on the same seeded inputs.

Tolerances: fp32 max-abs <= 1e-5; bf16 |y - ref| <= 2^-8 |ref| + 1e-6 per element (the
bf16 rounding of y is at most 2^-9 relative).  The state lines are copies of inputs and are
compared bit for bit.  Sizes span several 32-token blocks with a ragged tail and two
2048-channel slabs, the second one partial.
"""
import json

import numpy as np
import pytest
import torch

import gdn_inputs
from oracle import conv1d as oc

pytestmark = pytest.mark.gpu


def to64(t):
    return None if t is None else t.detach().cpu().to(torch.float64).numpy()


def run(inp, **over):
    import gated_deltanet_chunked_02_amd as gdn
    dev = torch.device("cuda")
    mv = lambda t: None if t is None else t.to(dev)
    state = mv(inp["conv_state"])
    y = gdn.causal_conv1d(mv(inp["x"]), mv(inp["weight"]), mv(inp["bias"]), state,
                          mv(inp["cache_indices"]), mv(inp["has_initial_state"]),
                          mv(inp["cu_seqlens"]), over.get("activation", inp["activation"]))
    torch.cuda.synchronize()
    return y, state


def oracle(inp):
    return oc.causal_conv1d(to64(inp["x"]), to64(inp["weight"]), to64(inp["bias"]),
                            to64(inp["conv_state"]),
                            None if inp["cache_indices"] is None else inp["cache_indices"].numpy(),
                            None if inp["has_initial_state"] is None
                            else inp["has_initial_state"].numpy(),
                            None if inp["cu_seqlens"] is None else inp["cu_seqlens"].numpy(),
                            inp["activation"] or "none")


def check(inp, y, state, y_ref, st_ref, label):
    y64 = to64(y)
    assert np.isfinite(y64).all()
    if inp["x"].dtype == torch.float32:
        err = float(np.max(np.abs(y64 - y_ref))) if y64.size else 0.0
        assert err <= 1e-5, "%s y max-abs %.3g" % (label, err)
    else:
        excess = np.abs(y64 - y_ref) - (2.0 ** -8 * np.abs(y_ref) + 1e-6)
        err = float(np.max(excess)) if y64.size else 0.0
        assert err <= 0, "%s y beyond the bf16 bound by %.3g" % (label, err)
    if st_ref is not None:
        assert np.array_equal(to64(state), st_ref), label + " state"
    return err


def conv_inputs(B, T, C, W, dtype, lines, seed, activation="silu", bias=True):
    w = gdn_inputs.ConvWorkload("t", channels=C, width=W, dtype=dtype, seed=seed, B=B, T=T,
                                lines=lines, activation=activation)
    inp = gdn_inputs.draw_conv(w, device="cpu")
    if not bias:
        inp["bias"] = None
    return inp


DENSE = [
    # B, T, C, W, dtype, lines, activation, bias
    (3, 70, 2112, 4, "bf16", 5, "silu", True),
    (2, 33, 2112, 3, "f32", 2, None, True),
    (2, 65, 64, 2, "bf16", 0, "silu", False),
    (1, 1, 8, 4, "f32", 1, "silu", True),
    (4, 2, 2048, 4, "bf16", 4, None, True),
    # many short sequences: each lies in one token block, which writes its own state line
    (2048, 2, 64, 3, "f32", 2048, None, True),    # one sequence per block
    (4096, 2, 64, 4, "bf16", 4096, "silu", True),  # two sequences per block
]


@pytest.mark.parametrize("B,T,C,W,dtype,lines,act,bias", DENSE)
def test_conv1d_dense_matches_oracle(B, T, C, W, dtype, lines, act, bias):
    inp = conv_inputs(B, T, C, W, dtype, lines, seed=B * 100 + T + W, activation=act,
                      bias=bias)
    if lines and B > 1:
        inp["has_initial_state"] = torch.tensor([n % 2 for n in range(B)], dtype=torch.int32)
    y_ref, st_ref = oracle(inp)
    y, state = run(inp)
    err = check(inp, y, state, y_ref, st_ref, "dense B%d T%d C%d W%d %s" % (B, T, C, W, dtype))
    print(json.dumps(dict(test="conv1d_dense", B=B, T=T, C=C, W=W, dtype=dtype, err=err)))


@pytest.mark.parametrize("W,dtype", [(2, "bf16"), (4, "bf16"), (3, "f32")])
def test_conv1d_packed_edges(W, dtype):
    """Ragged packed batch: empty sequences, sequences shorter than W - 1, block-crossing
    boundaries, permuted lines, a zero start, and a cache index outside the state."""
    lens = [1, 0, 2, 45, 3, 0, 33, 1]
    C = 136
    inp = conv_inputs(1, sum(lens), C, W, dtype, 10, seed=5 + W)
    inp["cu_seqlens"] = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32))
    inp["cache_indices"] = torch.tensor([9, 0, 3, 4, 1, 7, 2, -1], dtype=torch.int32)
    inp["has_initial_state"] = torch.tensor([1, 1, 0, 1, 1, 0, 1, 1], dtype=torch.int32)
    # the oracle has no notion of an invalid line: give it a private one for that sequence
    ref_inp = dict(inp)
    ref_inp["conv_state"] = torch.cat([inp["conv_state"],
                                       torch.zeros_like(inp["conv_state"][:1])])
    ref_inp["cache_indices"] = torch.tensor([9, 0, 3, 4, 1, 7, 2, 10], dtype=torch.int32)
    ref_inp["has_initial_state"] = torch.tensor([1, 1, 0, 1, 1, 0, 1, 0], dtype=torch.int32)
    y_ref, st_ref = oracle(ref_inp)
    y, state = run(inp)
    check(inp, y, state, y_ref, st_ref[:10], "packed W%d" % W)
    # lines no sequence names keep their contents
    for line in (5, 6, 8):
        assert torch.equal(state[line].cpu(), inp["conv_state"][line])


def test_conv1d_decode_loop_in_place_equals_one_call():
    B, T, C, W = 4, 5, 256, 4
    inp = conv_inputs(B, T, C, W, "bf16", 6, seed=31)
    y_ref, st_ref = oracle(inp)
    import gated_deltanet_chunked_02_amd as gdn
    dev = torch.device("cuda")
    state = inp["conv_state"].to(dev)
    ys = []
    for t in range(T):
        x_t = inp["x"][:, t:t + 1].contiguous().to(dev)
        ys.append(gdn.causal_conv1d(x_t, inp["weight"].to(dev), inp["bias"].to(dev), state,
                                    inp["cache_indices"].to(dev), activation="silu"))
    torch.cuda.synchronize()
    y = torch.cat(ys, dim=1)
    check(inp, y, state, y_ref, st_ref, "decode loop")
    y_one, st_one = run(inp)
    assert torch.equal(y_one, y) and torch.equal(st_one, state)


def test_conv1d_without_state_and_empty_batch():
    inp = conv_inputs(2, 40, 64, 4, "f32", 0, seed=41)
    y_ref, _ = oracle(inp)
    y, _ = run(inp)
    check(inp, y, None, y_ref, None, "no state")
    # a packed batch of zero sequences is a no-op
    import gated_deltanet_chunked_02_amd as gdn
    x = torch.zeros(1, 0, 64, device="cuda")
    w = torch.zeros(64, 4, device="cuda")
    y = gdn.causal_conv1d(x, w, cu_seqlens=torch.zeros(1, dtype=torch.int32, device="cuda"))
    assert y.shape == (1, 0, 64)


@pytest.mark.parametrize("name", ["conv_prefill", "conv_decode"])
def test_conv1d_full_size_sampled(name):
    """The bench workloads at full size, inputs drawn on the GPU; the oracle checks every
    token of a seeded sample of 48 channels (channels are independent) and every state
    line bit for bit."""
    w = gdn_inputs.CONV_WORKLOADS[name]
    inp = gdn_inputs.draw_conv(w, device="cuda")
    x0 = inp["x"]
    st0 = inp["conv_state"].clone()
    y, state = run(inp)
    rng = np.random.default_rng(w.seed)
    ch = np.sort(rng.choice(w.channels, 48, replace=False))
    ch[0], ch[-1] = 0, w.channels - 1
    cht = torch.from_numpy(ch).cuda()
    sub = dict(x=x0[..., cht].cpu(), weight=inp["weight"][cht].cpu(),
               bias=inp["bias"][cht].cpu(), conv_state=st0[..., cht].cpu(),
               cache_indices=inp["cache_indices"].cpu(), has_initial_state=None,
               cu_seqlens=None, activation=w.activation)
    y_ref, st_ref = oracle(sub)
    err = check(sub, y[..., cht], state[..., cht], y_ref, st_ref, name)
    # the whole state: every line is the last W - 1 inputs of its sequence
    W = w.width
    expect = st0.clone()
    for n in range(w.B):
        line = int(inp["cache_indices"][n])
        expect[line] = torch.cat([st0[line], x0[n]], dim=0)[-(W - 1):]
    assert torch.equal(state, expect)
    print(json.dumps(dict(test="conv1d_full_size", workload=w.name, channels_checked=48,
                          err=err)))
