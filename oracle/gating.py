"""Gate parametrisation of the per-token decode operator — TEST INFRASTRUCTURE ONLY (the
same import rules as the rest of ``oracle/``).

The TileLang × xLLM page (its section on the three core operators,
``fused_sigmoid_gating_delta_rule``) describes a decode-time kernel that fuses a sigmoid
activation and the gate computation, from A_log (named there as the decay rate) and the
query, key, value and beta inputs, with the delta-rule state update.  It prints no formula.
The reading taken here, written out in fp64:

    g_t    = -exp(A_log[h]) * softplus(a_t + dt_bias[h])     (the log-decay, always <= 0)
    beta_t = sigmoid(b_t)                                     (the sigmoid activation)

A_log is the logarithm of a per-head decay rate (so exp(A_log) > 0); a_t is the per-token,
per-head gate input and softplus(a_t + dt_bias) > 0 its step size, so the decay e^{g_t} lies
in (0, 1); b_t is the raw beta input.  dt_bias may be absent (zero).  The state update and
the output are then exactly the gated delta rule of ``recurrence`` with these g and beta.

softplus(x) = log(1 + e^x) and sigmoid(x) = 1 / (1 + e^-x) are evaluated in forms that do
not overflow: max(x, 0) + log1p(e^-|x|), and e^x / (1 + e^x) for x < 0.
"""
from __future__ import annotations

import numpy as np


def softplus(x):
    x = np.asarray(x, dtype=np.float64)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def sigmoid(x):
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(-np.abs(x))  # <= 1, never overflows
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def gates(a, b, A_log, dt_bias=None):
    """(g, beta) from the raw gate inputs.  a, b: [B, T, H]; A_log, dt_bias: [H] (dt_bias may
    be None).  Returns fp64 arrays of a's shape."""
    from . import _f64
    a, b, A_log = _f64(a), _f64(b), _f64(A_log)
    x = a if dt_bias is None else a + _f64(dt_bias)
    g = -np.exp(A_log) * softplus(x)
    return g, sigmoid(b)


def gated_recurrence(q, k, v, a, b, A_log, dt_bias=None, h0=None, scale=None,
                     cu_seqlens=None, nthreads: int = 0):
    """The decode operator: gates from (a, b, A_log, dt_bias), then the token recurrence.
    Returns (o, ht) as ``recurrence`` does."""
    from . import recurrence
    g, beta = gates(a, b, A_log, dt_bias)
    return recurrence(q, k, v, g, beta, h0, scale=scale, cu_seqlens=cu_seqlens,
                      nthreads=nthreads)
