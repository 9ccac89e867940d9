"""The C ABI on the host (no GPU needed): the library loads, exports every function the
header declares, validates descriptors before any launch and lays out the workspace."""
import ctypes
import os
import re

import pytest

import gated_deltanet_chunked_02_amd as gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gdn.LIB_PATH):
        pytest.fail("libgdn.so is not built (python -m gated_deltanet_chunked_02_amd.build)")
    return gdn.load()


def header_functions():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(gdn_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_exports_every_declared_function(lib):
    names = header_functions()
    assert {"gdn_chunk_fwd", "gdn_chunk_fwd_workspace_size", "gdn_stage_buffer",
            "gdn_status_string", "gdn_version"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for s in range(5):
        assert len(gdn.gdn_status_string(s)) > 0
    assert gdn.gdn_status_string(99) == "unknown status"
    assert gdn.gdn_version() >= 100


def desc(**kw):
    base = dict(B=2, T=256, N=2, H=4, Hg=2, Dk=128, Dv=128, chunk=128, qkv_dtype=1,
                beta_dtype=1, variant=0, stop_after=0, workspace=None, workspace_bytes=0)
    base.update(kw)
    return gdn.GdnDesc(**base)


def ws_status(d):
    st = ctypes.c_int(-1)
    n = gdn.load().gdn_chunk_fwd_workspace_size(ctypes.byref(d), ctypes.byref(st))
    return st.value, n


@pytest.mark.parametrize("kw,status", [
    (dict(), 0),
    (dict(H=3, Hg=2), 1),
    (dict(B=0), 1),
    (dict(T=-1), 1),
    (dict(Dk=128, Dv=64), 2),
    (dict(Dk=96, Dv=96), 2),
    (dict(chunk=32), 2),
    (dict(qkv_dtype=7), 1),
    (dict(variant=9), 1),
    (dict(stop_after=7), 1),
    (dict(qkv_dtype=0, beta_dtype=0, Dk=128, Dv=128, chunk=128), 2),
    (dict(qkv_dtype=0, beta_dtype=0, Dk=64, Dv=64, chunk=64), 0),
    (dict(variant=2, qkv_dtype=0, beta_dtype=0, Dk=64, Dv=64, chunk=64), 2),
    (dict(variant=2, Dk=256, Dv=256), 0),
    (dict(variant=3), 0),
    (dict(variant=3, Dk=256, Dv=256), 0),
    (dict(variant=3, N=1, B=1), 0),
    (dict(variant=3, B=1, N=3), 0),      # packed batches segment too
    (dict(variant=3, stop_after=3), 2),
    (dict(variant=2, stop_after=3), 2),
    (dict(variant=2, stop_after=6), 0),   # the fused stage stop: h_c and v_new only
    (dict(variant=2, stop_after=6, Dk=64, Dv=64), 0),
    (dict(variant=2, stop_after=6, Dk=256, Dv=256), 2),
    (dict(variant=2, stop_after=6, qkv_dtype=0, beta_dtype=0, Dk=64, Dv=64, chunk=64), 2),
    (dict(variant=4), 0),
    (dict(variant=4, qkv_dtype=0, beta_dtype=0, Dk=256, Dv=256), 0),
    (dict(variant=4, stop_after=3), 2),
    (dict(variant=5), 1),
    (dict(variant=1, qkv_dtype=0, beta_dtype=0, Dk=128, Dv=128, chunk=128), 2),
])
def test_descriptor_validation(lib, kw, status):
    st, n = ws_status(desc(**kw))
    assert st == status
    if st != 0:
        assert n == 0


def test_fused_needs_no_workspace_and_staged_does(lib):
    assert ws_status(desc(variant=2)) == (0, 0)
    st, n = ws_status(desc(variant=1))
    assert st == 0 and n > 0
    # AUTO resolves to fused where it is built (bf16, D in {64, 128, 256}), to staged
    # otherwise (fp32 operands), and to segmented for a few long sequences
    assert ws_status(desc(variant=0))[1] == 0
    assert ws_status(desc(variant=0, Dk=256, Dv=256))[1] == 0
    assert ws_status(desc(variant=0, qkv_dtype=0, beta_dtype=0, Dk=64, Dv=64, chunk=64))[1] > 0
    assert ws_status(desc(variant=0, B=1, N=1, T=65536, H=8, Hg=8))[1] > 0
    assert ws_status(desc(variant=3))[1] > 0


def test_auto_takes_recurrent_for_few_tokens_per_sequence(lib):
    A = 0x10000  # only the nullness of cu_seqlens is read
    assert gdn.gdn_resolved_variant(desc(T=1)) == "recurrent"
    assert gdn.gdn_resolved_variant(desc(T=8)) == "recurrent"
    assert gdn.gdn_resolved_variant(desc(T=9)) == "fused"
    assert gdn.gdn_resolved_variant(desc(T=8, qkv_dtype=0, beta_dtype=0)) == "recurrent"
    # packed batches: the mean length decides (64 sequences in 512 tokens, then 513)
    assert gdn.gdn_resolved_variant(desc(B=1, N=64, T=512), A) == "recurrent"
    assert gdn.gdn_resolved_variant(desc(B=1, N=64, T=513), A) == "fused"
    assert gdn.gdn_resolved_variant(desc(variant=4, T=4096)) == "recurrent"
    assert ws_status(desc(variant=4)) == (0, 0)
    assert ws_status(desc(T=8)) == (0, 0)


def test_auto_segments_from_four_segments_of_512_tokens(lib):
    """One sequence, 32 heads: 8 segments wanted (256 pairs); AUTO segments when they are at
    least 512 tokens long and the workspace is there (host-only, fake aligned address)."""
    for T, expect in ((2048, "fused"), (4096, "segmented"), (65536, "segmented")):
        d = desc(B=1, N=1, T=T, H=32, Hg=16)
        need = gdn.gdn_chunk_fwd_workspace_size(d)
        if expect == "fused":
            assert need == 0
        d.workspace, d.workspace_bytes = 0x10000, need
        assert gdn.gdn_resolved_variant(d) == expect, T


def test_packed_batches_segment_when_few_long_sequences(lib):
    A = 0x10000  # only the nullness of cu_seqlens is read; fake aligned workspace
    # one packed 65536-token sequence over 32 heads: segments of 8192 tokens
    d = desc(B=1, N=1, T=65536, H=32, Hg=16)
    need = gdn.gdn_chunk_fwd_workspace_size(d)  # covers the dense and the packed reading
    d.workspace, d.workspace_bytes = A, need
    assert gdn.gdn_resolved_variant(d, A) == "segmented"
    assert gdn.gdn_resolved_variant(d) == "segmented"
    # 64 packed sequences already give 2048 pairs: fused
    d2 = desc(B=1, N=64, T=65536, H=32, Hg=16)
    d2.workspace, d2.workspace_bytes = A, 1 << 40
    assert gdn.gdn_resolved_variant(d2, A) == "fused"
    # a few sequences averaging under four 512-token segments each: fused
    d3 = desc(B=1, N=4, T=4096, H=32, Hg=16)
    d3.workspace, d3.workspace_bytes = A, 1 << 40
    assert gdn.gdn_resolved_variant(d3, A) == "fused"


def test_staged_layout_is_aligned_and_disjoint(lib):
    d = desc(variant=1, B=3, T=1000, N=3, H=6, Hg=3, Dk=64, Dv=64, chunk=64)
    total = gdn.gdn_chunk_fwd_workspace_size(d)
    spans = []
    for name, b in gdn.BUFFERS.items():
        off, nb = gdn.gdn_stage_buffer(d, b)
        assert off % 256 == 0
        assert off + nb <= total
        spans.append((off, off + nb, name))
    spans.sort()
    for (a0, a1, _), (b0, b1, _) in zip(spans, spans[1:]):
        assert a1 <= b0
    Ttot, H, C, D = 3000, 6, 64, 64
    max_chunks = -(-Ttot // C) + 3
    sizes = {n: gdn.gdn_stage_buffer(d, n)[1] for n in gdn.BUFFERS}
    assert sizes["chunk_table"] == max_chunks * 16
    assert sizes["A"] == Ttot * H * C * 4
    assert sizes["Tinv"] == Ttot * H * C * 2
    assert sizes["h_c"] == max_chunks * H * D * D * 2
    with pytest.raises(gdn.GdnError):
        gdn.gdn_stage_buffer(d, 11)


def test_fused_stop_layout_holds_only_what_the_kernel_forms(lib):
    # C = 128 is requested; the fused kernel runs and lays out 64-token chunks
    d = desc(variant=2, stop_after=6, B=1, T=1000, N=3, H=6, Hg=3, Dk=128, Dv=128, chunk=128)
    total = gdn.gdn_chunk_fwd_workspace_size(d)
    sizes = {n: gdn.gdn_stage_buffer(d, n) for n in gdn.BUFFERS}
    Ttot, H, D = 1000, 6, 128
    max_chunks = -(-Ttot // 64) + 3
    kept = {"chunk_table": max_chunks * 16, "seq_chunks": 4 * 4,
            "h_c": max_chunks * H * D * D * 2, "v_new": Ttot * H * D * 2}
    for name, (off, nb) in sizes.items():
        assert off % 256 == 0 and off + nb <= total
        assert nb == kept.get(name, 0), name
    spans = sorted((off, off + nb) for off, nb in sizes.values() if nb)
    for (a0, a1), (b0, b1) in zip(spans, spans[1:]):
        assert a1 <= b0
    assert gdn.gdn_resolved_chunk(desc(variant=2, stop_after=6)) == 64
    # stops the fused kernel does not have
    for k in range(1, 6):
        with pytest.raises(gdn.GdnError):
            gdn.gdn_stage_buffer(desc(variant=2, stop_after=k), 5)


def test_noalloc_refuses_a_stage_stop(lib):
    A = 0x10000
    for v, k in ((1, 3), (2, 6)):
        d = desc(variant=v, stop_after=k)
        assert gdn.load().gdn_chunk_fwd_noalloc(ctypes.byref(d), A, A, A, A, A, None, None,
                                                1.0, A, None, None) == 1


def test_chunk_fwd_rejects_bad_arguments_before_any_launch(lib):
    # Fake, well-aligned addresses: validation must fail before anything touches them.
    A = 0x10000
    d = desc(variant=2)

    def call(dd=d, q=A, k=A, v=A, g=A, beta=A, h0=None, cu=None, o=A, ht=None):
        return gdn.load().gdn_chunk_fwd(ctypes.byref(dd), q, k, v, g, beta, h0, cu, 1.0, o, ht,
                                        None)

    assert call(q=None) == 1
    assert call(o=None) == 1
    assert call(beta=None) == 1
    assert call(q=A + 2) == 1             # misaligned q
    assert call(g=A + 2) == 1             # misaligned g
    assert call(h0=A + 8) == 1            # misaligned h0
    assert call(dd=desc(variant=2, H=3, Hg=2)) == 1
    assert call(dd=desc(variant=2, Dk=96, Dv=96)) == 2
    assert call(dd=desc(variant=2, N=3)) == 1             # dense batch: N must equal B
    assert call(dd=desc(variant=2, B=2), cu=A) == 1       # varlen needs B == 1
    assert call(dd=desc(variant=1)) == 3                  # staged without workspace
    assert call(dd=desc(variant=1, workspace=A, workspace_bytes=16)) == 3


def test_python_binding_refuses_cpu_tensors(lib):
    import torch
    x = torch.zeros(1, 4, 1, 64, dtype=torch.bfloat16)
    g = torch.zeros(1, 4, 1)
    with pytest.raises(ValueError):
        gdn.chunk_gated_delta_rule(x, x, x, g, g.to(torch.bfloat16))


def conv_status(**kw):
    base = dict(B=2, T=64, N=0, channels=64, width=4, dtype=1, activation=1, state_lines=2)
    base.update({k: v for k, v in kw.items() if k in base})
    d = gdn.GdnConvDesc(**base)
    A = 0x10000  # fake, aligned: every case below must fail (or finish) before any launch
    args = dict(x=A, weight=A, bias=None, state=A, idx=None, init=None, cu=None, y=A)
    args.update({k: v for k, v in kw.items() if k in args})
    return gdn.load().gdn_causal_conv1d_fwd(ctypes.byref(d), args["x"], args["weight"],
                                            args["bias"], args["state"], args["idx"],
                                            args["init"], args["cu"], args["y"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(width=1), 2),
    (dict(width=5), 2),
    (dict(channels=60), 2),
    (dict(dtype=7), 1),
    (dict(activation=5), 1),
    (dict(x=None), 1),
    (dict(y=None), 1),
    (dict(weight=None), 1),
    (dict(x=0x10000 + 8), 1),
    (dict(state=0x10000 + 4), 1),
    (dict(state_lines=0), 1),
    (dict(N=3), 1),                       # dense: N must be B (or 0)
    (dict(cu=0x10000), 1),                # packed needs B == 1
    (dict(B=1, N=0, cu=0x10000), 0),      # no sequences: nothing to do, no launch
    (dict(B=-1), 1),
])
def test_conv1d_rejects_bad_arguments_before_any_launch(lib, kw, status):
    assert conv_status(**kw) == status


# ------------------------------------------------------------------ binding validation
# Each case has one defect; shapes and dtypes are checked before devices, so every case is
# caught here on the host, before any pointer reaches the library.
def gdn_args(**over):
    import torch
    B, T, Hg, H, D = 1, 8, 2, 4, 64
    a = dict(q=torch.zeros(B, T, Hg, D, dtype=torch.bfloat16),
             k=torch.zeros(B, T, Hg, D, dtype=torch.bfloat16),
             v=torch.zeros(B, T, H, D, dtype=torch.bfloat16),
             g=torch.zeros(B, T, H), beta=torch.zeros(B, T, H, dtype=torch.bfloat16),
             initial_state=None, cu_seqlens=None, workspace=None)
    a.update(over)
    return a


def _bad_gdn_cases():
    import torch
    bf = torch.bfloat16
    return [
        (dict(k=torch.zeros(1, 8, 2, 64, dtype=torch.float32)), TypeError),   # k dtype
        (dict(v=torch.zeros(1, 8, 4, 64, dtype=torch.float32)), TypeError),   # v dtype
        (dict(q=torch.zeros(1, 8, 2, 64, dtype=torch.float16),
              k=torch.zeros(1, 8, 2, 64, dtype=torch.float16),
              v=torch.zeros(1, 8, 4, 64, dtype=torch.float16)), TypeError),   # fp16
        (dict(k=torch.zeros(1, 8, 2, 32, dtype=bf)), ValueError),             # k shape
        (dict(v=torch.zeros(1, 7, 4, 64, dtype=bf)), ValueError),             # v tokens
        (dict(v=torch.zeros(1, 8, 3, 64, dtype=bf)), ValueError),             # H % Hg
        (dict(q=torch.zeros(8, 2, 64, dtype=bf)), ValueError),                # q rank
        (dict(g=torch.zeros(1, 8, 4, dtype=bf)), TypeError),                  # g dtype
        (dict(g=torch.zeros(1, 8, 2)), ValueError),                           # g shape
        (dict(beta=torch.zeros(1, 8, 4, dtype=torch.float16)), TypeError),    # beta dtype
        (dict(beta=torch.zeros(1, 8, 4, 1, dtype=bf)), ValueError),           # beta shape
        (dict(initial_state=torch.zeros(1, 4, 64, 32)), ValueError),          # h0 shape
        (dict(initial_state=torch.zeros(2, 4, 64, 64)), ValueError),          # h0: N != B
        (dict(initial_state=torch.zeros(1, 4, 64, 64, dtype=torch.int32)), TypeError),
        (dict(cu_seqlens=torch.zeros(3)), TypeError),                         # float cu
        (dict(cu_seqlens=torch.zeros(1, 3, dtype=torch.int32)), ValueError),  # 2-D cu
        (dict(q=torch.zeros(2, 4, 2, 64, dtype=bf), k=torch.zeros(2, 4, 2, 64, dtype=bf),
              v=torch.zeros(2, 4, 4, 64, dtype=bf), g=torch.zeros(2, 4, 4),
              beta=torch.zeros(2, 4, 4, dtype=bf),
              cu_seqlens=torch.tensor([0, 4, 8], dtype=torch.int32)), ValueError),  # B != 1
        (dict(cu_seqlens=torch.tensor([0, 3, 8], dtype=torch.int32),
              initial_state=torch.zeros(1, 4, 64, 64)), ValueError),          # h0: N = 2
        (dict(workspace=torch.zeros(16)), TypeError),                         # not uint8
        (dict(), ValueError),                                                 # host tensors
        (dict(cu_seqlens=torch.tensor([0, 8], dtype=torch.int32)), ValueError),
        (dict(initial_state=torch.zeros(1, 4, 64, 64)), ValueError),
    ]


@pytest.mark.parametrize("case", range(22))
def test_binding_validates_every_tensor(lib, case):
    over, exc = _bad_gdn_cases()[case]
    a = gdn_args(**over)
    with pytest.raises(exc):
        gdn.chunk_gated_delta_rule(a["q"], a["k"], a["v"], a["g"], a["beta"],
                                   initial_state=a["initial_state"],
                                   cu_seqlens=a["cu_seqlens"], workspace=a["workspace"])


def test_binding_case_count():
    assert len(_bad_gdn_cases()) == 22


def _bad_conv_cases():
    import torch
    bf = torch.bfloat16
    x = torch.zeros(2, 8, 16, dtype=bf)
    w = torch.zeros(16, 4)
    return [
        (dict(x=torch.zeros(2, 8, 16, dtype=torch.float16)), TypeError),
        (dict(x=torch.zeros(16, 8, dtype=bf)), ValueError),
        (dict(x=torch.zeros(2, 16, 8, dtype=bf).transpose(1, 2)), ValueError),  # strided
        (dict(weight=torch.zeros(16, 4, dtype=bf)), TypeError),
        (dict(weight=torch.zeros(8, 4)), ValueError),
        (dict(bias=torch.zeros(16, dtype=bf)), TypeError),
        (dict(bias=torch.zeros(8)), ValueError),
        (dict(conv_state=torch.zeros(2, 3, 16)), TypeError),                  # state dtype
        (dict(conv_state=torch.zeros(2, 2, 16, dtype=bf)), ValueError),       # W - 1 rows
        (dict(conv_state=torch.zeros(2, 16, 3, dtype=bf).transpose(1, 2)), ValueError),
        (dict(cache_indices=torch.zeros(3, dtype=torch.int32)), ValueError),  # [N]
        (dict(cache_indices=torch.zeros(2)), TypeError),
        (dict(has_initial_state=torch.zeros(1, 2, dtype=torch.int32)), ValueError),
        (dict(cu_seqlens=torch.tensor([0, 8], dtype=torch.int32)), ValueError),  # B != 1
        (dict(), ValueError),                                                 # host tensors
    ], x, w


@pytest.mark.parametrize("case", range(15))
def test_conv_binding_validates_every_tensor(lib, case):
    cases, x, w = _bad_conv_cases()
    over, exc = cases[case]
    a = dict(x=x, weight=w, bias=None, conv_state=None, cache_indices=None,
             has_initial_state=None, cu_seqlens=None)
    a.update(over)
    with pytest.raises(exc):
        gdn.causal_conv1d(a["x"], a["weight"], bias=a["bias"], conv_state=a["conv_state"],
                          cache_indices=a["cache_indices"],
                          has_initial_state=a["has_initial_state"], cu_seqlens=a["cu_seqlens"])


def test_resolved_chunk_reports_what_runs(lib):
    A = 0x10000
    assert gdn.load().gdn_resolved_chunk(ctypes.byref(desc(variant=1, chunk=64)), None) == 64
    assert gdn.load().gdn_resolved_chunk(ctypes.byref(desc(variant=1, chunk=0)), None) == 128
    assert gdn.gdn_resolved_chunk(desc(variant=2, chunk=128)) == 64
    assert gdn.gdn_resolved_chunk(desc(variant=2, chunk=128, Dk=256, Dv=256)) == 32
    assert gdn.gdn_resolved_chunk(desc(variant=2, Dk=64, Dv=64)) == 64
    assert gdn.gdn_resolved_chunk(desc(variant=4)) == 1
    assert gdn.gdn_resolved_chunk(desc(T=4)) == 1                      # AUTO: recurrent
    assert gdn.gdn_resolved_chunk(desc(variant=3, B=1, N=1, T=65536)) == 64
    assert gdn.load().gdn_resolved_chunk(ctypes.byref(desc(Dk=96, Dv=96)), None) == -1
    assert gdn.load().gdn_resolved_chunk(ctypes.byref(desc(B=1, N=5, T=4096)), A) == 64


def test_fused_packed_batch_asks_for_its_order(lib):
    # a packed batch (N other than B): 4 bytes per sequence, 256-byte aligned
    assert gdn.gdn_chunk_fwd_workspace_size(desc(B=1, N=64, T=200000, variant=2)) == 256
    assert gdn.gdn_chunk_fwd_workspace_size(desc(B=1, N=100, T=200000, variant=2)) == 512
    assert gdn.gdn_chunk_fwd_workspace_size(desc(B=1, N=4096, T=1 << 20, variant=2)) == 16384
    # a dense batch needs nothing, and neither does one packed sequence
    assert gdn.gdn_chunk_fwd_workspace_size(desc(variant=2)) == 0
    assert gdn.gdn_chunk_fwd_workspace_size(desc(B=1, N=1, T=4096, variant=2)) == 0
    # beyond 65536 sequences they run in index order, without workspace
    assert gdn.gdn_chunk_fwd_workspace_size(desc(B=1, N=70000, T=1 << 22, variant=2)) == 0


def test_gating_entry_rejects_bad_arguments_before_any_launch(lib):
    A = 0x10000  # fake, aligned: every case below must fail before any launch

    def call(dd=None, **kw):
        args = dict(q=A, k=A, v=A, a=A, b=A, A_log=A, dt_bias=None, h0=None, cu=None, o=A,
                    ht=None)
        args.update(kw)
        return lib.gdn_fused_sigmoid_gating_delta_rule(
            ctypes.byref(dd or desc()), args["q"], args["k"], args["v"], args["a"], args["b"],
            args["A_log"], args["dt_bias"], args["h0"], args["cu"], 0.1, args["o"],
            args["ht"], None)

    assert call(desc(variant=2)) == 2                     # only AUTO or RECURRENT
    assert call(desc(variant=1)) == 2
    assert call(desc(stop_after=1)) == 1
    assert call(A_log=None) == 1
    assert call(a=None) == 1 and call(b=None) == 1 and call(q=None) == 1
    assert call(a=A + 1) == 1                             # bf16 a needs 2-byte alignment
    assert call(desc(beta_dtype=0), b=A + 2) == 1         # fp32 b needs 4 bytes
    assert call(dt_bias=A + 2) == 1
    assert call(desc(N=3)) == 1                           # dense: N must equal B
    assert call(desc(B=2, N=2), cu=A) == 1                # packed needs B == 1
    assert call(desc(Dk=96, Dv=96)) == 2
    assert call(desc(B=1, N=0, T=0), cu=A) == 0           # no sequences: nothing to do


def _gating_args(**over):
    import torch
    a = gdn_args()
    a.update(a=torch.zeros(1, 8, 4, dtype=torch.bfloat16), A_log=torch.zeros(4),
             dt_bias=None)
    a.update(over)
    return a


def test_gating_binding_validates_its_tensors(lib):
    import torch
    bad = [
        (dict(a=torch.zeros(1, 8, 4)), TypeError),                      # a dtype != b dtype
        (dict(a=torch.zeros(1, 8, 2, dtype=torch.bfloat16)), ValueError),  # a shape
        (dict(A_log=torch.zeros(4, dtype=torch.float64)), TypeError),
        (dict(A_log=torch.zeros(3)), ValueError),
        (dict(dt_bias=torch.zeros(4, dtype=torch.bfloat16)), TypeError),
        (dict(dt_bias=torch.zeros(2)), ValueError),
        (dict(beta=torch.zeros(1, 8, 4, dtype=torch.float16)), TypeError),
        (dict(), ValueError),                                           # host tensors
    ]
    for over, exc in bad:
        a = _gating_args(**over)
        with pytest.raises(exc):
            gdn.fused_sigmoid_gating_delta_rule(a["q"], a["k"], a["v"], a["a"], a["beta"],
                                                a["A_log"], a["dt_bias"])
    a = _gating_args()
    with pytest.raises(ValueError):
        gdn.fused_sigmoid_gating_delta_rule(a["q"], a["k"], a["v"], a["a"], a["beta"],
                                            a["A_log"], inplace_final_state=True)


# ------------------------------------------------------------------ backward entry
def bwd_ws(d):
    st = ctypes.c_int(-1)
    n = gdn.load().gdn_chunk_bwd_workspace_size(ctypes.byref(d), ctypes.byref(st))
    return st.value, n


def test_bwd_workspace_covers_the_staged_stages_and_its_gradient_buffers(lib):
    # bf16 D = 128, dense B = 2, T = 256, H = 4, Hg = 2: the staged layout at C = 64 without
    # A, W and U, then dR [Ttot, H, D] and the chunk-end state gradients [max_chunks, H, D, D]
    # in bf16 (grouped heads need nothing more: one workgroup sums a group's dq and dk)
    d = desc(chunk=128)
    st, n = bwd_ws(d)
    assert st == 0
    Ttot, H, D = 512, 4, 128
    tok = Ttot * H * D * 4
    # the staged layout without A (fp32 [Ttot, H, 64]: it stays on chip) and without W and U
    # (bf16 [Ttot, H, D] each: the fused recompute never forms them)
    staged = (gdn.gdn_chunk_fwd_workspace_size(desc(chunk=64, variant=1)) - Ttot * H * 64 * 4
              - 2 * (tok // 2))
    max_chunks = Ttot // 64 + 2
    # dR and dh' in bf16
    assert n == staged + tok // 2 + max_chunks * H * D * D * 2
    # the same without grouped heads
    st, n2 = bwd_ws(desc(Hg=4))
    assert st == 0 and n2 == n
    # supported: bf16 D 64 / 128, fp32 D 64
    assert bwd_ws(desc(Dk=256, Dv=256))[0] == 2
    assert bwd_ws(desc(qkv_dtype=0, Dk=128, Dv=128))[0] == 2
    # fp32 recomputes through the staged stages, so its workspace keeps W and U
    st, n32 = bwd_ws(desc(qkv_dtype=0, Dk=64, Dv=64, beta_dtype=0))
    tok32 = Ttot * H * 64 * 4
    staged32 = (gdn.gdn_chunk_fwd_workspace_size(desc(qkv_dtype=0, Dk=64, Dv=64, beta_dtype=0,
                                                      chunk=64, variant=1))
                - Ttot * H * 64 * 4)
    assert st == 0 and n32 == staged32 + tok32 + max_chunks * H * 64 * 64 * 4
    assert bwd_ws(desc(Dk=64, Dv=64))[0] == 0
    # the chunk and stop_after fields do not change it, nor a variant other than SEGMENTED
    # where AUTO keeps one pass per sequence
    assert bwd_ws(desc(chunk=64, variant=2))[1] == n
    assert bwd_ws(desc(stop_after=3))[1] == n
    # a packed batch of N sequences bounds its chunks by ceil(Ttot / 64) + N
    st, npk = bwd_ws(desc(B=1, T=512, N=5))
    assert st == 0 and npk > n


def test_bwd_segments_few_long_sequences(lib):
    # the long prompt: 32 (sequence, head) pairs, AUTO runs the passes per segment
    long = desc(B=1, T=65536, N=0, H=32, Hg=16)
    assert gdn.gdn_chunk_bwd_resolved_variant(long) == "segmented"
    assert gdn.gdn_chunk_bwd_resolved_variant(desc(B=1, T=65536, N=0, H=32, Hg=16,
                                                   variant=2)) == "fused"
    st, nseg = bwd_ws(long)
    st2, nflat = bwd_ws(desc(B=1, T=65536, N=0, H=32, Hg=16, variant=2))
    assert st == 0 and st2 == 0 and nseg > nflat
    # the segment buffers: 8 segments of 8192 tokens (256 segment-head pairs), b, M and h_in
    # fp32 per (segment, head)
    assert nseg - nflat >= 3 * 8 * 32 * 128 * 128 * 4
    # many pairs: one pass per sequence; SEGMENTED forces segments (bf16 only)
    assert gdn.gdn_chunk_bwd_resolved_variant(desc(B=16, T=8192, N=0, H=32, Hg=32)) == "fused"
    assert gdn.gdn_chunk_bwd_resolved_variant(desc(variant=3)) == "segmented"
    assert gdn.gdn_chunk_bwd_resolved_variant(
        desc(qkv_dtype=0, beta_dtype=0, Dk=64, Dv=64)) == "staged"
    with pytest.raises(gdn.GdnError):
        gdn.gdn_chunk_bwd_resolved_variant(desc(qkv_dtype=0, beta_dtype=0, Dk=64, Dv=64,
                                                variant=3))
    assert bwd_ws(desc(qkv_dtype=0, beta_dtype=0, Dk=64, Dv=64, variant=3))[0] == 2
    # a dense single sequence may come packed: the query covers both readings
    st, n1 = bwd_ws(desc(B=1, T=4096, N=0, H=32, Hg=16, variant=3))
    st, n2 = bwd_ws(desc(B=1, T=4096, N=2, H=32, Hg=16, variant=3))
    assert n1 > 0 and n2 > 0


def test_bwd_rejects_bad_arguments_before_any_launch(lib):
    A = 0x10000  # fake, aligned: every case below must fail (or finish) before any launch

    def call(dd=None, **kw):
        args = dict(q=A, k=A, v=A, g=A, beta=A, h0=None, cu=None, do=A, dht=None, dq=A, dk=A,
                    dv=A, dg=A, dbeta=A, dh0=None)
        args.update(kw)
        return lib.gdn_chunk_bwd(
            ctypes.byref(dd or desc()), args["q"], args["k"], args["v"], args["g"],
            args["beta"], args["h0"], args["cu"], 0.1, args["do"], args["dht"], args["dq"],
            args["dk"], args["dv"], args["dg"], args["dbeta"], args["dh0"], None)

    for name in ("q", "do", "dq", "dk", "dv", "dg", "dbeta"):
        assert call(**{name: None}) == 1, name
    assert call(do=A + 2) == 1                            # misaligned dout
    assert call(dg=A + 2) == 1                            # misaligned dg
    assert call(dh0=A + 8) == 1
    assert call(desc(Dk=256, Dv=256)) == 2
    assert call(desc(qkv_dtype=0)) == 2                   # fp32 only at D = 64
    assert call(desc(N=3)) == 1                           # dense: N must equal B
    assert call(desc(B=2, N=2), cu=A) == 1                # packed needs B == 1
    assert call() == 3                                    # no workspace
    assert call(desc(workspace=A, workspace_bytes=4096)) == 3
    assert call(desc(workspace=A + 16, workspace_bytes=1 << 40)) == 3  # misaligned
    assert call(desc(B=1, N=0, T=0), cu=A) == 0           # no sequences: nothing to do
    assert call(desc(T=0)) == 0                           # no tokens and no dh0: nothing
    assert call(desc(grad_dtype=7)) == 1                  # unknown gradient dtype
    assert call(desc(grad_dtype=1, qkv_dtype=0, beta_dtype=0, Dk=64, Dv=64)) == 2  # bf16
    # gradients need bf16 inputs; with them they are accepted (and fail on the workspace)
    assert call(desc(grad_dtype=1)) == 3


def test_bwd_binding_validates_its_tensors(lib):
    import torch
    bf = torch.bfloat16
    bad = [
        (dict(do=torch.zeros(1, 8, 4, 64)), TypeError),                 # do dtype
        (dict(do=torch.zeros(1, 8, 2, 64, dtype=bf)), ValueError),      # do shape
        (dict(dht=torch.zeros(1, 4, 64, 32)), ValueError),              # dht shape
        (dict(dht=torch.zeros(1, 4, 64, 64, dtype=torch.int32)), TypeError),
        (dict(g=torch.zeros(1, 8, 4, dtype=bf)), TypeError),            # forward checks too
        (dict(), ValueError),                                           # host tensors
    ]
    for over, exc in bad:
        a = gdn_args()
        a.update(do=torch.zeros(1, 8, 4, 64, dtype=bf), dht=None)
        a.update(over)
        with pytest.raises(exc):
            gdn.chunk_gated_delta_rule_bwd(a["q"], a["k"], a["v"], a["g"], a["beta"], a["do"],
                                           dht=a["dht"], initial_state=a["initial_state"])
    # the gradient dtype: fp32 or bf16, bf16 only with bf16 inputs (checked first)
    a = gdn_args()
    a.update(do=torch.zeros(1, 8, 4, 64, dtype=bf))
    with pytest.raises(TypeError):
        gdn.chunk_gated_delta_rule_bwd(a["q"], a["k"], a["v"], a["g"], a["beta"], a["do"],
                                       grad_dtype=torch.float16)
    f32 = {n: (t.float() if isinstance(t, torch.Tensor) and t.dtype == bf else t)
           for n, t in a.items()}
    with pytest.raises(TypeError):
        gdn.chunk_gated_delta_rule_bwd(f32["q"], f32["k"], f32["v"], f32["g"], f32["beta"],
                                       f32["do"], grad_dtype=torch.bfloat16)
