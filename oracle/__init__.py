"""Oracle for the chunked Gated DeltaNet forward — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import this package.  The product path (``gated_deltanet_chunked_02_amd`` and its
HIP library) never imports, links or calls anything here, and shares no code with it.

Contents
--------
* ``recurrence`` — the plain definition: the gated delta rule evaluated token by token in
  fp64 (C, ``gdn_oracle.c``, OpenMP over (sequence, head) pairs).  This is the oracle the
  GPU path is compared with.
* ``dense_form`` — the same result as one triangular solve over a whole sequence (numpy /
  scipy fp64); used only to pin ``recurrence`` on tiny inputs.
* ``chunked`` — the seven chunk stages of the MegaGDN-PTO page (section 1.1: cumsum,
  transpose, scaled_dot_kkt, solve_tril, wy_fast, chunk_h, chunk_o), in fp64 numpy, in the
  page's order; it yields every stage intermediate for per-stage parity of the staged GPU
  variant and is itself pinned to ``recurrence``.
* ``conv1d`` — the causal depthwise convolution with its decode state that precedes the
  gated delta rule (the TileLang × xLLM page's causal_conv1d operator), in fp64 numpy.
* ``backward`` — gradients of the forward recurrence (reverse pass through the token
  steps, fp64 numpy), pinned by finite differences of ``recurrence``.

Every function here follows its cited passage; none is blocked, fused or reordered beyond
what that passage states.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "libgdn_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (plain -O2, OpenMP).  Returns the library path."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-Wall",
             "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def use_native() -> str:
    """Switch this process to a copy of the same C source built with -O3 -march=native for
    the host it runs on (the CPU-baseline timing; the tests use the portable -O2 build,
    which can travel between machines).  Built in a temporary directory, never shipped.
    Returns the library path."""
    global _lib
    import tempfile
    path = os.path.join(tempfile.gettempdir(), "libgdn_oracle_native_%d.so" % os.getpid())
    subprocess.check_call(
        ["gcc", "-O3", "-march=native", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-Wall",
         "-o", path, _SRC, "-lm"])
    _lib = None
    _load(path)
    return path


def cpu_model() -> str:
    """The host CPU's model name as lscpu reports it (from /proc/cpuinfo), with its x86
    family and model numbers, which identify the generation when the name is generic."""
    info = {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if ":" in line:
                    key, val = line.split(":", 1)
                    info.setdefault(key.strip().lower(), val.strip())
                if line.strip() == "":
                    break
    except OSError:
        return "unknown"
    name = info.get("model name", "unknown")
    if "cpu family" in info and "model" in info:
        name += " (x86 family %s, model %s)" % (info["cpu family"], info["model"])
    return name


def _load(path=None):
    global _lib
    if _lib is None:
        if path is None:
            path = _LIB
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build(force=False)
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        lib.gdn_oracle_fwd.restype = ctypes.c_int
        lib.gdn_oracle_fwd.argtypes = [
            ctypes.c_int32, P, P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
            ctypes.c_int32, P, P, P, P, P, P, ctypes.c_double, P, P, P, ctypes.c_int64,
            ctypes.c_int32]
        lib.gdn_oracle_max_threads.restype = ctypes.c_int
        lib.gdn_oracle_max_threads.argtypes = [ctypes.c_int32]
        _lib = lib
    return _lib


def _f64(x):
    """Widen any array-like (numpy, or a CPU torch tensor of any float dtype) to a
    contiguous float64 numpy array without changing its values."""
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor: bf16 has no numpy dtype, widen in torch
        import torch
        x = x.detach().to("cpu", torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def sequences(B: int, T: int, cu_seqlens=None):
    """(start, length) of every sequence: the rows of a dense [B, T] batch, or the packed
    spans of cu_seqlens (packed varlen, MegaGDN-PTO page section 5.3)."""
    if cu_seqlens is None:
        starts = np.arange(B, dtype=np.int64) * T
        lens = np.full(B, T, dtype=np.int64)
    else:
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        starts, lens = cu[:-1].copy(), np.diff(cu)
    return starts, lens


def max_threads(nthreads: int = 0) -> int:
    return int(_load().gdn_oracle_max_threads(nthreads))


def recurrence(q, k, v, g, beta, h0=None, scale=None, cu_seqlens=None, pairs=None,
               nthreads: int = 0):
    """Token-by-token fp64 gated delta rule (see gdn_oracle.c for the definition).

    q, k: [B, T, Hg, Dk]; v: [B, T, H, Dv]; g, beta: [B, T, H]; h0: [N, H, Dk, Dv] or None.
    cu_seqlens (packed varlen) requires B == 1.  ``pairs``: optional iterable of
    n * H + h to evaluate; other outputs stay zero.
    Returns (o [B, T, H, Dv] float64, ht [N, H, Dk, Dv] float64).
    """
    q, k, v, g, beta, h0 = (_f64(x) for x in (q, k, v, g, beta, h0))
    B, T, Hg, Dk = q.shape
    H, Dv = v.shape[2], v.shape[3]
    assert k.shape == q.shape and v.shape[:2] == (B, T) and g.shape == (B, T, H)
    assert beta.shape == (B, T, H) and H % Hg == 0
    if cu_seqlens is not None:
        assert B == 1
    starts, lens = sequences(B, T, cu_seqlens)
    N = len(starts)
    assert h0 is None or h0.shape == (N, H, Dk, Dv)
    if scale is None:
        scale = Dk ** -0.5
    o = np.zeros((B, T, H, Dv), dtype=np.float64)
    ht = np.zeros((N, H, Dk, Dv), dtype=np.float64)
    pl = None if pairs is None else np.ascontiguousarray(np.asarray(list(pairs), np.int64))
    ptr = lambda a: None if a is None else a.ctypes.data_as(ctypes.c_void_p)
    rc = _load().gdn_oracle_fwd(
        N, ptr(starts), ptr(lens), H, Hg, Dk, Dv, ptr(q), ptr(k), ptr(v), ptr(g),
        ptr(beta), ptr(h0), float(scale), ptr(o), ptr(ht), ptr(pl),
        0 if pl is None else len(pl), nthreads)
    if rc != 0:
        raise RuntimeError("gdn_oracle_fwd failed with %d" % rc)
    return o, ht
