"""Python binding of libgdn — the chunked Gated DeltaNet forward for MI355X (gfx950).

Argument marshalling only: every step of the computation runs in libgdn's HIP kernels.
PyTorch supplies device memory and the current stream.  The binding refuses to run when
the library is missing; there is no fallback.

Low level (same names as the C ABI in include/gdn.h):
    gdn_chunk_fwd(desc, q, k, v, g, beta, h0, cu_seqlens, scale, o, ht, stream)
    gdn_chunk_fwd_workspace_size(desc) / gdn_stage_buffer(desc, buf) / gdn_status_string(s)
High level (the call shape of the FlashQLA how-to, step 5.2):
    o, ht = chunk_gated_delta_rule(q, k, v, g, beta, scale=None, initial_state=None,
                                   output_final_state=True, cu_seqlens=None, chunk_size=128)
The decode operator with its gates made in the kernel (low level
gdn_fused_sigmoid_gating_delta_rule):
    o, ht = fused_sigmoid_gating_delta_rule(q, k, v, a, b, A_log, dt_bias=None, ...)
The short convolution before it (low level gdn_causal_conv1d_fwd):
    y = causal_conv1d(x, weight, bias=None, conv_state=None, cache_indices=None,
                      has_initial_state=None, cu_seqlens=None, activation=None)
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "GdnDesc", "GdnError", "load", "gdn_chunk_fwd", "gdn_chunk_fwd_workspace_size",
    "gdn_stage_buffer", "gdn_status_string", "gdn_version", "chunk_gated_delta_rule",
    "make_desc", "STATUS", "BUFFERS", "VARIANTS", "LIB_PATH", "gdn_resolved_variant",
    "gdn_chunk_bwd_resolved_variant",
    "gdn_resolved_chunk", "gdn_chunk_fwd_noalloc", "gdn_fused_sigmoid_gating_delta_rule",
    "fused_sigmoid_gating_delta_rule", "gdn_chunk_bwd", "gdn_chunk_bwd_workspace_size",
    "chunk_gated_delta_rule_bwd",
    "GdnConvDesc", "gdn_causal_conv1d_fwd", "causal_conv1d", "ACTIVATIONS",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgdn.so")

STATUS = {0: "GDN_OK", 1: "GDN_ERR_INVALID_ARG", 2: "GDN_ERR_UNSUPPORTED",
          3: "GDN_ERR_WORKSPACE", 4: "GDN_ERR_HIP"}
F32, BF16 = 0, 1
VARIANTS = {"auto": 0, "staged": 1, "fused": 2, "segmented": 3, "recurrent": 4}
ACTIVATIONS = {None: 0, "none": 0, "silu": 1}
BUFFERS = {"chunk_table": 0, "seq_chunks": 1, "g_cum": 2, "g_t": 3, "beta_t": 4, "A": 5,
           "Tinv": 6, "W": 7, "U": 8, "h_c": 9, "v_new": 10}


class GdnError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__("%s%s (%s)" % (what + ": " if what else "", STATUS.get(status, status),
                                        gdn_status_string(status) if _lib else "?"))


class GdnDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("N", ctypes.c_int32),
                ("H", ctypes.c_int32), ("Hg", ctypes.c_int32), ("Dk", ctypes.c_int32),
                ("Dv", ctypes.c_int32), ("chunk", ctypes.c_int32),
                ("qkv_dtype", ctypes.c_int32), ("beta_dtype", ctypes.c_int32),
                ("variant", ctypes.c_int32), ("stop_after", ctypes.c_int32),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("grad_dtype", ctypes.c_int32)]


class GdnConvDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("N", ctypes.c_int32),
                ("channels", ctypes.c_int32), ("width", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("activation", ctypes.c_int32),
                ("state_lines", ctypes.c_int32)]


_lib = None


def load(path: str = LIB_PATH):
    """Load libgdn.so (built by ``gated_deltanet_chunked_02_amd.build``); raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("libgdn.so not found at %s — build it with "
                           "`python -m gated_deltanet_chunked_02_amd.build`" % path)
    lib = ctypes.CDLL(path)
    P, S = ctypes.c_void_p, ctypes.c_size_t
    lib.gdn_chunk_fwd.restype = ctypes.c_int
    lib.gdn_chunk_fwd.argtypes = [ctypes.POINTER(GdnDesc), P, P, P, P, P, P, P, ctypes.c_float,
                                  P, P, P]
    lib.gdn_chunk_fwd_workspace_size.restype = S
    lib.gdn_chunk_fwd_workspace_size.argtypes = [ctypes.POINTER(GdnDesc),
                                                 ctypes.POINTER(ctypes.c_int)]
    lib.gdn_stage_buffer.restype = ctypes.c_int
    lib.gdn_stage_buffer.argtypes = [ctypes.POINTER(GdnDesc), ctypes.c_int32,
                                     ctypes.POINTER(S), ctypes.POINTER(S)]
    lib.gdn_status_string.restype = ctypes.c_char_p
    lib.gdn_status_string.argtypes = [ctypes.c_int]
    lib.gdn_version.restype = ctypes.c_int32
    lib.gdn_version.argtypes = []
    lib.gdn_resolved_variant.restype = ctypes.c_int32
    lib.gdn_resolved_variant.argtypes = [ctypes.POINTER(GdnDesc), P]
    lib.gdn_chunk_bwd_resolved_variant.restype = ctypes.c_int32
    lib.gdn_chunk_bwd_resolved_variant.argtypes = [ctypes.POINTER(GdnDesc), P]
    lib.gdn_resolved_chunk.restype = ctypes.c_int32
    lib.gdn_resolved_chunk.argtypes = [ctypes.POINTER(GdnDesc), P]
    lib.gdn_chunk_fwd_noalloc.restype = ctypes.c_int
    lib.gdn_chunk_fwd_noalloc.argtypes = lib.gdn_chunk_fwd.argtypes
    lib.gdn_fused_sigmoid_gating_delta_rule.restype = ctypes.c_int
    lib.gdn_fused_sigmoid_gating_delta_rule.argtypes = [
        ctypes.POINTER(GdnDesc), P, P, P, P, P, P, P, P, P, ctypes.c_float, P, P, P]
    lib.gdn_chunk_bwd_workspace_size.restype = S
    lib.gdn_chunk_bwd_workspace_size.argtypes = lib.gdn_chunk_fwd_workspace_size.argtypes
    lib.gdn_chunk_bwd.restype = ctypes.c_int
    lib.gdn_chunk_bwd.argtypes = [ctypes.POINTER(GdnDesc), P, P, P, P, P, P, P, ctypes.c_float,
                                  P, P, P, P, P, P, P, P, P]
    lib.gdn_causal_conv1d_fwd.restype = ctypes.c_int
    lib.gdn_causal_conv1d_fwd.argtypes = [ctypes.POINTER(GdnConvDesc), P, P, P, P, P, P, P, P,
                                          P]
    _lib = lib
    return lib


def gdn_status_string(status: int) -> str:
    return load().gdn_status_string(int(status)).decode()


def gdn_version() -> int:
    return int(load().gdn_version())


def gdn_resolved_variant(desc: GdnDesc, cu_seqlens=None) -> str:
    """Name of the variant gdn_chunk_fwd runs with this descriptor (AUTO resolved)."""
    v = int(load().gdn_resolved_variant(ctypes.byref(desc), _ptr(cu_seqlens)))
    for name, code in VARIANTS.items():
        if code == v and name != "auto":
            return name
    raise GdnError(1, "gdn_resolved_variant")


def gdn_chunk_bwd_resolved_variant(desc: GdnDesc, cu_seqlens=None) -> str:
    """How gdn_chunk_bwd runs with this descriptor: "segmented", "fused" (the fused
    recompute, one reverse pass per sequence) or "staged" (the staged recompute)."""
    v = int(load().gdn_chunk_bwd_resolved_variant(ctypes.byref(desc), _ptr(cu_seqlens)))
    for name, code in VARIANTS.items():
        if code == v and name != "auto":
            return name
    raise GdnError(1, "gdn_chunk_bwd_resolved_variant")


def gdn_resolved_chunk(desc: GdnDesc, cu_seqlens=None) -> int:
    """Chunk length the variant gdn_chunk_fwd runs with this descriptor evaluates (the
    staged variant's C, the fused kernel's own chunk, 1 for token by token)."""
    c = int(load().gdn_resolved_chunk(ctypes.byref(desc), _ptr(cu_seqlens)))
    if c < 0:
        raise GdnError(1, "gdn_resolved_chunk")
    return c


def gdn_chunk_fwd_workspace_size(desc: GdnDesc) -> int:
    st = ctypes.c_int(0)
    n = load().gdn_chunk_fwd_workspace_size(ctypes.byref(desc), ctypes.byref(st))
    if st.value != 0:
        raise GdnError(st.value, "gdn_chunk_fwd_workspace_size")
    return int(n)


def gdn_stage_buffer(desc: GdnDesc, buf) -> tuple:
    """(offset, bytes) of intermediate ``buf`` (name or id) inside the staged workspace."""
    b = BUFFERS[buf] if isinstance(buf, str) else int(buf)
    off, nb = ctypes.c_size_t(0), ctypes.c_size_t(0)
    st = load().gdn_stage_buffer(ctypes.byref(desc), b, ctypes.byref(off), ctypes.byref(nb))
    if st != 0:
        raise GdnError(st, "gdn_stage_buffer")
    return int(off.value), int(nb.value)


def _ptr(x) -> int:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def gdn_chunk_fwd(desc: GdnDesc, q, k, v, g, beta, h0, cu_seqlens, scale, o, ht,
                  stream=None) -> int:
    """Raw call: tensors (or integer device addresses / None) are passed as pointers.
    Returns the status code (0 = ok) without raising."""
    import torch
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    return int(load().gdn_chunk_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                    _ptr(beta), _ptr(h0), _ptr(cu_seqlens), float(scale),
                                    _ptr(o), _ptr(ht), stream))


def gdn_chunk_fwd_noalloc(desc: GdnDesc, q, k, v, g, beta, h0, cu_seqlens, scale, o, ht,
                          stream=None) -> int:
    """Raw call of the allocation-free entry point: the library's own per-GPU device
    scratch is the workspace (desc.workspace is ignored).  Returns the status code."""
    import torch
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    return int(load().gdn_chunk_fwd_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v),
                                            _ptr(g), _ptr(beta), _ptr(h0), _ptr(cu_seqlens),
                                            float(scale), _ptr(o), _ptr(ht), stream))


def gdn_fused_sigmoid_gating_delta_rule(desc: GdnDesc, q, k, v, a, b, A_log, dt_bias, h0,
                                        cu_seqlens, scale, o, ht, stream=None) -> int:
    """Raw call of the decode operator with in-kernel gates; returns the status code."""
    import torch
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    return int(load().gdn_fused_sigmoid_gating_delta_rule(
        ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(A_log),
        _ptr(dt_bias), _ptr(h0), _ptr(cu_seqlens), float(scale), _ptr(o), _ptr(ht), stream))


def gdn_chunk_bwd_workspace_size(desc: GdnDesc) -> int:
    st = ctypes.c_int(0)
    n = load().gdn_chunk_bwd_workspace_size(ctypes.byref(desc), ctypes.byref(st))
    if st.value != 0:
        raise GdnError(st.value, "gdn_chunk_bwd_workspace_size")
    return int(n)


def gdn_chunk_bwd(desc: GdnDesc, q, k, v, g, beta, h0, cu_seqlens, scale, do, dht, dq, dk, dv,
                  dg, dbeta, dh0, stream=None) -> int:
    """Raw call of the backward pass; returns the status code (0 = ok) without raising."""
    import torch
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    return int(load().gdn_chunk_bwd(
        ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0),
        _ptr(cu_seqlens), float(scale), _ptr(do), _ptr(dht), _ptr(dq), _ptr(dk), _ptr(dv),
        _ptr(dg), _ptr(dbeta), _ptr(dh0), stream))


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError("libgdn takes bf16 or fp32 tensors, got %s" % t.dtype)


def make_desc(q, v, beta, cu_seqlens=None, chunk_size=128, variant="auto", stop_after=0,
              N=None) -> GdnDesc:
    B, T, Hg, Dk = q.shape
    H, Dv = v.shape[2], v.shape[3]
    if N is None:
        N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    return GdnDesc(B=B, T=T, N=N, H=H, Hg=Hg, Dk=Dk, Dv=Dv, chunk=chunk_size,
                   qkv_dtype=_dtype_code(q), beta_dtype=_dtype_code(beta),
                   variant=VARIANTS[variant] if isinstance(variant, str) else int(variant),
                   stop_after=stop_after, workspace=None, workspace_bytes=0)

_INT_DTYPES = ("torch.int32", "torch.int64", "torch.int16", "torch.int8", "torch.uint8")


def _need(cond, exc, msg):
    if not cond:
        raise exc(msg)


def _check_devices(named, ref):
    """Every tensor of ``named`` (name -> tensor or None) on ``ref``, a CUDA (HIP) device.
    Run after the shape and dtype checks, so those also run on a host without a GPU."""
    _need(ref.type == "cuda", ValueError,
          "the tensors must be device tensors (got %s)" % ref)
    for name, t in named.items():
        if t is not None:
            _need(t.device == ref, ValueError,
                  "%s must be on %s like the other tensors (got %s)" % (name, ref, t.device))


def _validate_gdn(q, k, v, g, beta, initial_state, cu_seqlens, workspace, devices=True):
    """Shapes, dtypes and devices of chunk_gated_delta_rule's tensors, checked before any
    pointer reaches the library (a host pointer or a short buffer read by a kernel would
    fault the GPU instead of raising)."""
    import torch
    named = dict(q=q, k=k, v=v, g=g, beta=beta, initial_state=initial_state,
                 cu_seqlens=cu_seqlens, workspace=workspace)
    for name, t in named.items():
        _need(t is None or isinstance(t, torch.Tensor), TypeError,
              "%s must be a torch tensor" % name)
    for name in ("q", "k", "v"):
        _need(named[name].dim() == 4, ValueError, "%s must be 4-D [B, T, heads, D]" % name)
    _need(q.dtype in (torch.bfloat16, torch.float32), TypeError,
          "q must be bf16 or fp32, got %s" % q.dtype)
    _need(k.dtype == q.dtype and v.dtype == q.dtype, TypeError,
          "q, k and v must share one dtype (got %s, %s, %s)" % (q.dtype, k.dtype, v.dtype))
    _need(k.shape == q.shape, ValueError, "k %s must have q's shape %s" % (tuple(k.shape),
                                                                          tuple(q.shape)))
    B, T, Hg, Dk = q.shape
    _need(tuple(v.shape[:2]) == (B, T), ValueError, "v must be [B, T, H, Dv] with q's B, T")
    H, Dv = v.shape[2], v.shape[3]
    _need(Hg > 0 and H % Hg == 0, ValueError, "v heads (%d) must be a multiple of q/k heads "
          "(%d)" % (H, Hg))
    if g is not None:  # None: the decode operator, whose gates are made in the kernel
        _need(g.dtype == torch.float32, TypeError, "g must be fp32, got %s" % g.dtype)
        _need(tuple(g.shape) == (B, T, H), ValueError,
              "g must be [B, T, H] = %s" % ((B, T, H),))
    _need(beta.dtype in (torch.bfloat16, torch.float32), TypeError,
          "beta must be bf16 or fp32, got %s" % beta.dtype)
    _need(tuple(beta.shape) == (B, T, H), ValueError,
          "beta must be [B, T, H] = %s" % ((B, T, H),))
    N = B
    if cu_seqlens is not None:
        _need(str(cu_seqlens.dtype) in _INT_DTYPES, TypeError, "cu_seqlens must be integer")
        _need(cu_seqlens.dim() == 1 and cu_seqlens.numel() >= 1, ValueError,
              "cu_seqlens must be 1-D [N + 1]")
        _need(B == 1, ValueError, "a packed batch (cu_seqlens) needs B == 1")
        N = cu_seqlens.numel() - 1
    if initial_state is not None:
        _need(initial_state.is_floating_point(), TypeError, "initial_state must be floating")
        _need(tuple(initial_state.shape) == (N, H, Dk, Dv), ValueError,
              "initial_state must be [N, H, Dk, Dv] = %s" % ((N, H, Dk, Dv),))
    if workspace is not None:
        _need(workspace.dtype == torch.uint8 and workspace.is_contiguous(), TypeError,
              "workspace must be a contiguous uint8 tensor")
    if devices:
        _check_devices(named, q.device)


def _validate_conv(x, weight, bias, conv_state, cache_indices, has_initial_state,
                   cu_seqlens):
    """Shapes, dtypes and devices of causal_conv1d's tensors (see _validate_gdn)."""
    import torch
    named = dict(x=x, weight=weight, bias=bias, conv_state=conv_state,
                 cache_indices=cache_indices, has_initial_state=has_initial_state,
                 cu_seqlens=cu_seqlens)
    for name, t in named.items():
        _need(t is None or isinstance(t, torch.Tensor), TypeError,
              "%s must be a torch tensor" % name)
    _need(x.dim() == 3, ValueError, "x must be 3-D [B, T, C]")
    _need(x.dtype in (torch.bfloat16, torch.float32), TypeError, "x must be bf16 or fp32")
    _need(x.is_contiguous(), ValueError, "x must be contiguous")
    B, T, C = x.shape
    _need(weight.dtype == torch.float32, TypeError, "weight must be fp32")
    _need(weight.dim() == 2 and weight.shape[0] == C, ValueError, "weight must be [C, W]")
    W = weight.shape[1]
    if bias is not None:
        _need(bias.dtype == torch.float32, TypeError, "bias must be fp32")
        _need(tuple(bias.shape) == (C,), ValueError, "bias must be [C]")
    N = B
    if cu_seqlens is not None:
        _need(str(cu_seqlens.dtype) in _INT_DTYPES, TypeError, "cu_seqlens must be integer")
        _need(cu_seqlens.dim() == 1 and cu_seqlens.numel() >= 1, ValueError,
              "cu_seqlens must be 1-D [N + 1]")
        _need(B == 1, ValueError, "a packed batch (cu_seqlens) needs B == 1")
        N = cu_seqlens.numel() - 1
    if conv_state is not None:
        _need(conv_state.dtype == x.dtype, TypeError, "conv_state must have x's dtype")
        _need(conv_state.dim() == 3 and tuple(conv_state.shape[1:]) == (W - 1, C), ValueError,
              "conv_state must be [lines, W - 1, C] = [lines, %d, %d]" % (W - 1, C))
        _need(conv_state.is_contiguous(), ValueError,
              "conv_state must be contiguous (it is updated in place)")
    for name in ("cache_indices", "has_initial_state"):
        t = named[name]
        if t is not None:
            _need(str(t.dtype) in _INT_DTYPES or t.dtype == torch.bool, TypeError,
                  "%s must be integer" % name)
            _need(tuple(t.shape) == (N,), ValueError, "%s must be [N] = [%d]" % (name, N))
    _check_devices(named, x.device)


def chunk_gated_delta_rule(q, k, v, g, beta, scale=None, initial_state=None,
                           output_final_state=True, cu_seqlens=None, chunk_size=128,
                           variant="auto", workspace=None, stop_after=0):
    """Chunked Gated DeltaNet forward on the current CUDA (HIP) stream.

    q, k: [B, T, Hg, Dk]; v: [B, T, H, Dv]; g: [B, T, H] fp32 log-decay; beta: [B, T, H];
    initial_state: [N, H, Dk, Dv] fp32 or None; cu_seqlens: int32 [N + 1] (B == 1) or None.
    Returns (o [B, T, H, Dv] in q's dtype, final state [N, H, Dk, Dv] fp32 or None).
    ``workspace``: optional uint8 device tensor for the staged variant (allocated here when
    needed and not given).
    """
    import torch
    _validate_gdn(q, k, v, g, beta, initial_state, cu_seqlens, workspace)
    q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
    g, beta = g.contiguous(), beta.contiguous()
    if cu_seqlens is not None:
        cu_seqlens = cu_seqlens.to(torch.int32).contiguous()
    desc = make_desc(q, v, beta, cu_seqlens, chunk_size, variant, stop_after)
    if scale is None:
        scale = q.shape[-1] ** -0.5
    if initial_state is not None:
        initial_state = initial_state.to(torch.float32).contiguous()
    o = torch.empty_like(v)
    ht = None
    if output_final_state:
        ht = torch.empty((desc.N, desc.H, desc.Dk, desc.Dv), device=q.device,
                         dtype=torch.float32)
    ws_bytes = gdn_chunk_fwd_workspace_size(desc)
    if ws_bytes:
        if workspace is None or workspace.numel() < ws_bytes:
            workspace = torch.empty(ws_bytes, device=q.device, dtype=torch.uint8)
        desc.workspace = workspace.data_ptr()
        desc.workspace_bytes = workspace.numel()
    st = gdn_chunk_fwd(desc, q, k, v, g, beta, initial_state, cu_seqlens, scale, o, ht)
    if st != 0:
        raise GdnError(st, "gdn_chunk_fwd")
    return o, ht


def chunk_gated_delta_rule_bwd(q, k, v, g, beta, do, dht=None, scale=None,
                               initial_state=None, cu_seqlens=None, workspace=None,
                               variant="auto", grad_dtype=None):
    """Gradients of chunk_gated_delta_rule's inputs on the current stream, given the
    gradient ``do`` of o [B, T, H, Dv] (q's dtype) and ``dht`` of the final state
    [N, H, Dk, Dv] (or None: zero).  Forward inputs as for chunk_gated_delta_rule.
    Returns (dq, dk [B, T, Hg, Dk], dv [B, T, H, Dv] in ``grad_dtype``: torch.float32 by
    default, or torch.bfloat16 with bf16 inputs; dg, dbeta [B, T, H] and dh0 [N, H, Dk, Dv]
    in fp32, dh0 None when initial_state is None).  ``variant``: "auto" (long sequences run
    per segment when that pays), "segmented" (always) or any other name (one pass per
    sequence)."""
    import torch
    gdt = torch.float32 if grad_dtype is None else grad_dtype
    _need(gdt in (torch.float32, torch.bfloat16), TypeError,
          "grad_dtype must be torch.float32 or torch.bfloat16")
    _need(gdt == torch.float32 or q.dtype == torch.bfloat16, TypeError,
          "bf16 gradients need bf16 inputs")
    _validate_gdn(q, k, v, g, beta, initial_state, cu_seqlens, workspace, devices=False)
    _need(isinstance(do, torch.Tensor) and do.dtype == q.dtype, TypeError,
          "do must be a tensor of q's dtype")
    _need(do.shape == v.shape, ValueError, "do must have v's shape [B, T, H, Dv]")
    B, T, Hg, Dk = q.shape
    H, Dv = v.shape[2], v.shape[3]
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    if dht is not None:
        _need(isinstance(dht, torch.Tensor) and dht.is_floating_point(), TypeError,
              "dht must be a floating tensor")
        _need(tuple(dht.shape) == (N, H, Dk, Dv), ValueError,
              "dht must be [N, H, Dk, Dv] = %s" % ((N, H, Dk, Dv),))
    _check_devices(dict(q=q, k=k, v=v, g=g, beta=beta, do=do, dht=dht,
                        initial_state=initial_state, cu_seqlens=cu_seqlens,
                        workspace=workspace), q.device)
    q, k, v, do = q.contiguous(), k.contiguous(), v.contiguous(), do.contiguous()
    g, beta = g.contiguous(), beta.contiguous()
    if cu_seqlens is not None:
        cu_seqlens = cu_seqlens.to(torch.int32).contiguous()
    if initial_state is not None:
        initial_state = initial_state.to(torch.float32).contiguous()
    if dht is not None:
        dht = dht.to(torch.float32).contiguous()
    desc = make_desc(q, v, beta, cu_seqlens, 64, variant)
    if scale is None:
        scale = Dk ** -0.5
    f = dict(device=q.device, dtype=torch.float32)
    fg = dict(device=q.device, dtype=gdt)
    desc.grad_dtype = 1 if gdt == torch.bfloat16 else 0
    dq, dk = torch.empty(q.shape, **fg), torch.empty(k.shape, **fg)
    dv = torch.empty(v.shape, **fg)
    dg, dbeta = torch.empty(B, T, H, **f), torch.empty(B, T, H, **f)
    dh0 = torch.empty(N, H, Dk, Dv, **f) if initial_state is not None else None
    ws_bytes = gdn_chunk_bwd_workspace_size(desc)
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(max(ws_bytes, 1), device=q.device, dtype=torch.uint8)
    desc.workspace = workspace.data_ptr()
    desc.workspace_bytes = workspace.numel()
    st = gdn_chunk_bwd(desc, q, k, v, g, beta, initial_state, cu_seqlens, scale, do, dht, dq,
                       dk, dv, dg, dbeta, dh0)
    if st != 0:
        raise GdnError(st, "gdn_chunk_bwd")
    return dq, dk, dv, dg, dbeta, dh0


def fused_sigmoid_gating_delta_rule(q, k, v, a, b, A_log, dt_bias=None, scale=None,
                                    initial_state=None, output_final_state=True,
                                    cu_seqlens=None, inplace_final_state=False):
    """The decode operator (token by token, gates made in the kernel) on the current stream:
    g = -exp(A_log) softplus(a + dt_bias) and beta = sigmoid(b), then the gated delta rule.

    q, k: [B, T, Hg, Dk]; v: [B, T, H, Dv]; a, b: [B, T, H] (bf16 or fp32, one dtype);
    A_log, dt_bias: [H] fp32 (dt_bias may be None); initial_state [N, H, Dk, Dv] or None.
    ``inplace_final_state``: write the final state into ``initial_state`` (fp32, contiguous)
    instead of a new tensor, as a decode loop does.  Returns (o, final state or None)."""
    import torch
    _validate_gdn(q, k, v, None, b, initial_state, cu_seqlens, None, devices=False)
    _need(isinstance(a, torch.Tensor) and a.dtype == b.dtype, TypeError,
          "a must be a tensor of b's dtype")
    _need(a.shape == b.shape, ValueError, "a must have b's shape [B, T, H]")
    H = v.shape[2]
    _need(isinstance(A_log, torch.Tensor) and A_log.dtype == torch.float32, TypeError,
          "A_log must be an fp32 tensor")
    _need(tuple(A_log.shape) == (H,), ValueError, "A_log must be [H] = [%d]" % H)
    if dt_bias is not None:
        _need(isinstance(dt_bias, torch.Tensor) and dt_bias.dtype == torch.float32, TypeError,
              "dt_bias must be an fp32 tensor")
        _need(tuple(dt_bias.shape) == (H,), ValueError, "dt_bias must be [H] = [%d]" % H)
    if inplace_final_state:
        _need(initial_state is not None and initial_state.dtype == torch.float32 and
              initial_state.is_contiguous(), ValueError,
              "inplace_final_state needs a contiguous fp32 initial_state")
    _check_devices(dict(q=q, k=k, v=v, a=a, b=b, A_log=A_log, dt_bias=dt_bias,
                        initial_state=initial_state, cu_seqlens=cu_seqlens), q.device)
    q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
    a, b, A_log = a.contiguous(), b.contiguous(), A_log.contiguous()
    if dt_bias is not None:
        dt_bias = dt_bias.contiguous()
    if cu_seqlens is not None:
        cu_seqlens = cu_seqlens.to(torch.int32).contiguous()
    desc = make_desc(q, v, b, cu_seqlens, 0, "recurrent")
    if scale is None:
        scale = q.shape[-1] ** -0.5
    if initial_state is not None and not inplace_final_state:
        initial_state = initial_state.to(torch.float32).contiguous()
    o = torch.empty_like(v)
    ht = None
    if inplace_final_state:
        ht = initial_state
    elif output_final_state:
        ht = torch.empty((desc.N, desc.H, desc.Dk, desc.Dv), device=q.device,
                         dtype=torch.float32)
    st = gdn_fused_sigmoid_gating_delta_rule(desc, q, k, v, a, b, A_log, dt_bias,
                                             initial_state, cu_seqlens, scale, o, ht)
    if st != 0:
        raise GdnError(st, "gdn_fused_sigmoid_gating_delta_rule")
    return o, ht


def gdn_causal_conv1d_fwd(desc: GdnConvDesc, x, weight, bias, conv_state, cache_indices,
                          has_initial_state, cu_seqlens, y, stream=None) -> int:
    """Raw call (tensors, integer device addresses or None); returns the status code."""
    import torch
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    return int(load().gdn_causal_conv1d_fwd(
        ctypes.byref(desc), _ptr(x), _ptr(weight), _ptr(bias), _ptr(conv_state),
        _ptr(cache_indices), _ptr(has_initial_state), _ptr(cu_seqlens), _ptr(y), stream))


def causal_conv1d(x, weight, bias=None, conv_state=None, cache_indices=None,
                  has_initial_state=None, cu_seqlens=None, activation=None):
    """Causal depthwise conv1d on the current stream; returns y and updates conv_state in
    place.  x: [B, T, C] (packed: B = 1 with cu_seqlens int32 [N + 1]); weight [C, W] fp32;
    bias [C] fp32; conv_state [lines, W - 1, C] in x's dtype; cache_indices and
    has_initial_state int32 [N]; activation None or "silu"."""
    import torch
    _validate_conv(x, weight, bias, conv_state, cache_indices, has_initial_state, cu_seqlens)
    B, T, C = x.shape
    weight = weight.contiguous()
    if bias is not None:
        bias = bias.contiguous()
    i32 = lambda t: None if t is None else t.to(torch.int32).contiguous()
    cu, idx, init = i32(cu_seqlens), i32(cache_indices), i32(has_initial_state)
    N = B if cu is None else cu.numel() - 1
    desc = GdnConvDesc(B=B, T=T, N=N, channels=C, width=weight.shape[1], dtype=_dtype_code(x),
                       activation=ACTIVATIONS[activation],
                       state_lines=0 if conv_state is None else conv_state.shape[0])
    y = torch.empty_like(x)
    st = gdn_causal_conv1d_fwd(desc, x, weight, bias, conv_state, idx, init, cu, y)
    if st != 0:
        raise GdnError(st, "gdn_causal_conv1d_fwd")
    return y
