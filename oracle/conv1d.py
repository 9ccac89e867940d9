"""Oracle for the causal 1-D convolution that precedes the gated delta rule — TEST
INFRASTRUCTURE ONLY (the same import rules as the rest of ``oracle/``).

The TileLang × xLLM page (the section on its three operators, "causal_conv1d") describes
a causal convolution over the sequence: each output depends only on the current and the
earlier tokens; a convolution state carries the last inputs from one call to the next for
incremental decode; per-sequence cache indices select which state line a sequence uses;
a mode says whether a sequence starts from its cached state.  The page prints no formula.
The reading taken here (plain depthwise causal convolution):

  for every sequence n, channel c and token position t of that sequence, with width W,
  x~ = (the W - 1 inputs before the sequence, then the sequence's inputs),
  the W - 1 leading entries being the cached state line when the sequence starts from it
  and zeros otherwise,

      z[t, c] = bias[c] + sum_{i=0..W-1} weight[c, i] * x~[t + i, c]
      y[t, c] = z                      (no activation)
              = z * sigmoid(z)         (SiLU activation)

  so weight[c, W - 1] multiplies the current token (the cross-correlation convention of a
  left-padded conv1d), and after the call the state line holds the last W - 1 entries of
  x~ (which reach back into the old state when the sequence is shorter than W - 1).

fp64 throughout; parity unpinned by any value printed on the page (it prints none): pinned
instead by numpy's convolution, an impulse response, continuation across calls and the
SiLU identity silu(z) - silu(-z) = z (tests/test_oracle.py).
"""
from __future__ import annotations

import numpy as np


def silu(z):
    """z * sigmoid(z), written as z / (1 + exp(-z)) (fp64)."""
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def causal_conv1d(x, weight, bias=None, conv_state=None, cache_indices=None,
                  has_initial_state=None, cu_seqlens=None, activation="none"):
    """The convolution above for a dense batch or a packed one.

    x: [B, T, C] (packed: B = 1 and cu_seqlens [N + 1]); weight [C, W]; bias [C] or None;
    conv_state [lines, W - 1, C] or None (zeros in, nothing out); cache_indices [N] or None
    (sequence n uses line n); has_initial_state [N] or None (every sequence reads its line).
    Returns (y [B, T, C] fp64, the new conv_state as a copy, or None)."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    B, T, C = x.shape
    W = w.shape[1]
    b = np.zeros(C) if bias is None else np.asarray(bias, dtype=np.float64)
    if cu_seqlens is None:
        seqs = [(n, 0, T) for n in range(B)]
        rows = lambda n, s, e: x[n, s:e]
    else:
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        seqs = [(n, int(cu[n]), int(cu[n + 1])) for n in range(len(cu) - 1)]
        rows = lambda n, s, e: x[0, s:e]
    state_in = None if conv_state is None else np.asarray(conv_state, dtype=np.float64)
    state_out = None if state_in is None else state_in.copy()
    y = np.zeros_like(x)
    for idx, (n, s, e) in enumerate(seqs):
        line = idx if cache_indices is None else int(cache_indices[idx])
        start_from_state = state_in is not None and (
            has_initial_state is None or bool(has_initial_state[idx]))
        head = state_in[line] if start_from_state else np.zeros((W - 1, C))
        xt = np.concatenate([head, rows(n, s, e)], axis=0)  # [W - 1 + len, C]
        L = e - s
        out = np.empty((L, C))
        for t in range(L):
            z = b.copy()
            for i in range(W):
                z += w[:, i] * xt[t + i]
            out[t] = silu(z) if activation == "silu" else z
        if cu_seqlens is None:
            y[n] = out
        else:
            y[0, s:e] = out
        if state_out is not None:
            state_out[line] = xt[L:]  # the last W - 1 entries of x~
    return y, state_out
