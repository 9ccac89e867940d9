"""gdn_chunk_fwd_noalloc (the allocation-free entry point) against gdn_chunk_fwd, through
the C ABI, on the variants that use a workspace: two calls in a row, the second with a
smaller input, each bit for bit equal to the allocating entry point run with a workspace
of its own (the same kernels on the same inputs).  Also: a request whose variant needs more
than the library's scratch is refused before any launch."""
import pytest
import torch

import gdn_inputs

pytestmark = pytest.mark.gpu


def _inputs(w):
    inp = gdn_inputs.draw(w, device="cuda")
    return inp


def _both(inp, variant, C):
    """o and ht from gdn_chunk_fwd (workspace allocated here) and from the no-alloc entry."""
    import gated_deltanet_chunked_02_amd as gdn
    q, k, v, g, beta = (inp[n] for n in ("q", "k", "v", "g", "beta"))
    h0, cu = inp["h0"], inp["cu_seqlens"]
    desc = gdn.make_desc(q, v, beta, cu, C, variant)
    ws_bytes = gdn.gdn_chunk_fwd_workspace_size(desc)
    assert 0 < ws_bytes <= (64 << 20)
    N = desc.N
    out = []
    for entry in ("alloc", "noalloc"):
        o = torch.full_like(v, float("nan"))
        ht = torch.full((N, desc.H, desc.Dk, desc.Dv), float("nan"), device="cuda")
        d = gdn.make_desc(q, v, beta, cu, C, variant)
        if entry == "alloc":
            ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
            d.workspace, d.workspace_bytes = ws.data_ptr(), ws_bytes
            st = gdn.gdn_chunk_fwd(d, q, k, v, g, beta, h0, cu, inp["scale"], o, ht)
        else:
            st = gdn.gdn_chunk_fwd_noalloc(d, q, k, v, g, beta, h0, cu, inp["scale"], o, ht)
        torch.cuda.synchronize()
        assert st == 0, (entry, st)
        out.append((o, ht, gdn.gdn_resolved_variant(d, cu) if entry == "alloc" else None))
    return out


CASES = [
    # workload, overrides (first call), overrides (second, smaller call), variant, C
    ("long", dict(T=65536), dict(T=16384), "auto", 128),          # segmented under AUTO
    ("long", dict(T=8192, H=8, Hg=8), dict(T=2048, H=8, Hg=8), "segmented", 128),
    ("varlen", dict(n_varlen=300, max_len=300, H=4, Hg=4),
     dict(n_varlen=40, max_len=200, H=4, Hg=4), "fused", 128),    # longest-first order
    ("tiny_f32", dict(T=300, B=2), dict(T=100, B=2), "staged", 64),
    ("headline", dict(B=2, T=1000, H=4, Hg=4), dict(B=1, T=333, H=4, Hg=4), "staged", 128),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] + "-" + c[3] for c in CASES])
def test_noalloc_equals_alloc_on_two_calls(case):
    import gated_deltanet_chunked_02_amd as gdn
    name, first, second, variant, C = case
    for over in (first, second):
        w = gdn_inputs.WORKLOADS[name].with_(**over)
        print("[noalloc] %s %s %s" % (name, over, variant), flush=True)
        inp = _inputs(w)
        (o1, ht1, ran), (o2, ht2, _) = _both(inp, variant, C)
        if variant == "auto":
            assert ran == "segmented"
        assert torch.isfinite(o1.float()).all() and torch.isfinite(ht1).all()
        assert torch.equal(o1, o2) and torch.equal(ht1, ht2)


def test_noalloc_refuses_more_than_its_scratch():
    import gated_deltanet_chunked_02_amd as gdn
    w = gdn_inputs.WORKLOADS["headline"].with_(B=2, T=8192, H=8, Hg=8)
    inp = _inputs(w)
    q, k, v, g, beta = (inp[n] for n in ("q", "k", "v", "g", "beta"))
    d = gdn.make_desc(q, v, beta, None, 128, "staged")
    assert gdn.gdn_chunk_fwd_workspace_size(d) > (64 << 20)
    o = torch.full_like(v, 7.0)
    st = gdn.gdn_chunk_fwd_noalloc(d, q, k, v, g, beta, None, None, inp["scale"], o, None)
    torch.cuda.synchronize()
    assert st == 3 and torch.all(o == 7.0)            # GDN_ERR_WORKSPACE, nothing launched
    # AUTO on the same shapes runs the fused variant, which needs no workspace
    d = gdn.make_desc(q, v, beta, None, 128, "auto")
    st = gdn.gdn_chunk_fwd_noalloc(d, q, k, v, g, beta, None, None, inp["scale"], o, None)
    torch.cuda.synchronize()
    assert st == 0 and torch.isfinite(o.float()).all()
