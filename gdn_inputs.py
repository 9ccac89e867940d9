"""Seeded synthetic inputs for the chunked Gated DeltaNet forward.

This module holds no arithmetic of the method itself: it only draws the operands
(q, k, v, g, beta, h0, cu_seqlens) with the shapes and value distributions of the
workloads on the MegaGDN-PTO page (16 sequences x 8192 tokens, head sweeps, packed
variable-length batches; "quick start" and section 5.3) and the FlashQLA how-to (long
prompts, GQA head groups).  Both the oracle-side tests and the HIP-side tests / bench use
it, so the two sides see the same bytes.

Recipe (fixed draw order: lengths -> q -> k -> v -> g_pre -> beta_pre -> h0):
  * q, k ~ N(0, 1), L2-normalised per head vector in fp32, then cast (bf16 round-to-nearest-even);
  * v ~ N(0, 1), cast;
  * g = logsigmoid(x), x ~ N(3, 1), kept fp32 (the log-decay, always <= 0);
  * beta = sigmoid(N(0, 1)), cast to the beta dtype;
  * h0 ~ N(0, std^2) fp32 when the workload has an initial state;
  * packed varlen: lengths ~ U{1 .. max_len}, B = 1, cu_seqlens int32 on the same device.
The causal conv1d workloads (``draw_conv``) draw, in order: x ~ N(0, 1) cast to the dtype,
weight ~ N(0, 1 / W), bias ~ N(0, 0.1^2), state lines ~ N(0, 1) cast; sequence n uses state
line (7 n + 3) mod lines when that is a permutation.
"N(mu, s)" is read as mean mu and standard deviation s.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch

DTYPES = {"bf16": torch.bfloat16, "f32": torch.float32}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    H: int
    Hg: int
    Dk: int
    Dv: int
    C: int
    dtype: str              # q, k, v (and o) dtype: "bf16" or "f32"
    seed: int
    B: int = 1
    T: int = 0
    n_varlen: int = 0       # > 0: packed batch of this many sequences
    max_len: int = 0        # varlen lengths ~ U{1 .. max_len}
    h0_std: Optional[float] = None
    beta_dtype: str = ""    # default: same as dtype

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    # Tiny fp32 case (the oracle finishes in well under a second).
    "tiny_f32": Workload("tiny_f32_1x256_h2_d64", H=2, Hg=2, Dk=64, Dv=64, C=64, dtype="f32",
                         seed=0, B=1, T=256, h0_std=0.1),
    # Kernel bench shaped like the page's stage-latency chart: 16 x 8192, H=32, D=128.
    "headline": Workload("bf16_16x8192_h32_d128_c128", H=32, Hg=32, Dk=128, Dv=128, C=128,
                         dtype="bf16", seed=1, B=16, T=8192),
    # GQA wide heads: 32 value heads over 8 q/k groups, D=256, nonzero initial state.
    "gqa": Workload("bf16_gqa_4x8192_h32_hg8_d256_c128", H=32, Hg=8, Dk=256, Dv=256, C=128,
                    dtype="bf16", seed=2, B=4, T=8192, h0_std=0.05),
    # Packed varlen batch: 64 sequences, lengths U{1..8192}, H=64.
    "varlen": Workload("bf16_varlen_64seq_u1_8192_h64_d128_c128", H=64, Hg=64, Dk=128,
                       Dv=128, C=128, dtype="bf16", seed=3, n_varlen=64, max_len=8192,
                       h0_std=0.05),
    # Long-prompt prefill: one 65536-token sequence, 32 value heads over 16 q/k groups.
    "long": Workload("bf16_long_1x65536_h32_hg16_d128_c128", H=32, Hg=16, Dk=128, Dv=128,
                     C=128, dtype="bf16", seed=4, B=1, T=65536),
    # Decode: one new token for each of 256 sequences, each with a carried state
    # (the per-token delta-rule kernel of the TileLang × xLLM page), same head layout.
    "decode": Workload("bf16_decode_256x1_h32_hg16_d128", H=32, Hg=16, Dk=128, Dv=128,
                       C=128, dtype="bf16", seed=5, B=256, T=1, h0_std=0.05),
}


def draw(w: Workload, device="cpu"):
    """Return a dict of tensors on ``device``: q, k, v, g, beta, h0 (or None),
    cu_seqlens (or None), plus scale = Dk^-0.5, C, and the workload."""
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed)
    dt = DTYPES[w.dtype]
    bdt = DTYPES[w.beta_dtype or w.dtype]
    cu = None
    if w.n_varlen > 0:
        lens = torch.randint(1, w.max_len + 1, (w.n_varlen,), generator=gen, device=dev)
        cu = torch.zeros(w.n_varlen + 1, dtype=torch.int64, device=dev)
        cu[1:] = torch.cumsum(lens, 0)
        B, T, N = 1, int(cu[-1].item()), w.n_varlen
        cu = cu.to(torch.int32)
    else:
        B, T, N = w.B, w.T, w.B

    def unit(shape):
        x = torch.randn(shape, generator=gen, device=dev, dtype=torch.float32)
        x = x / x.norm(dim=-1, keepdim=True).clamp_min(1e-12)
        return x.to(dt)

    q = unit((B, T, w.Hg, w.Dk))
    k = unit((B, T, w.Hg, w.Dk))
    v = torch.randn((B, T, w.H, w.Dv), generator=gen, device=dev, dtype=torch.float32).to(dt)
    g = torch.nn.functional.logsigmoid(
        torch.randn((B, T, w.H), generator=gen, device=dev, dtype=torch.float32) + 3.0)
    beta = torch.sigmoid(
        torch.randn((B, T, w.H), generator=gen, device=dev, dtype=torch.float32)).to(bdt)
    h0 = None
    if w.h0_std is not None:
        h0 = torch.randn((N, w.H, w.Dk, w.Dv), generator=gen, device=dev,
                         dtype=torch.float32) * w.h0_std
    return dict(q=q, k=k, v=v, g=g, beta=beta, h0=h0, cu_seqlens=cu,
                scale=w.Dk ** -0.5, C=w.C, workload=w)


def small(name="small", *, B=1, T=256, H=2, Hg=None, Dk=64, Dv=None, C=64, dtype="bf16",
          seed=0, h0_std=0.05, n_varlen=0, max_len=0, beta_dtype=""):
    """A reduced workload with the same recipe (for parity tests at oracle-friendly sizes)."""
    return Workload(name, H=H, Hg=Hg or H, Dk=Dk, Dv=Dv or Dk, C=C, dtype=dtype, seed=seed,
                    B=B, T=T, n_varlen=n_varlen, max_len=max_len, h0_std=h0_std,
                    beta_dtype=beta_dtype)


# ---------------------------------------------------------------- causal conv1d inputs
@dataclasses.dataclass(frozen=True)
class ConvWorkload:
    name: str
    channels: int
    width: int
    dtype: str
    seed: int
    B: int = 1
    T: int = 0
    lines: int = 0          # state lines (0: no state)
    activation: str = "silu"

    def with_(self, **kw) -> "ConvWorkload":
        return dataclasses.replace(self, **kw)


# The convolution runs over the concatenated q, k, v projections of a layer, so its channel
# count is 2 Hg Dk + H Dv: 12288 for the 32-head, D = 128 shape of the prefill workload.
CONV_WORKLOADS = {
    "conv_prefill": ConvWorkload("conv_bf16_16x8192_c12288_w4_silu", channels=12288, width=4,
                                 dtype="bf16", seed=6, B=16, T=8192, lines=16),
    "conv_decode": ConvWorkload("conv_bf16_decode_256x1_c12288_w4_silu", channels=12288,
                                width=4, dtype="bf16", seed=7, B=256, T=1, lines=256),
}


def draw_conv(w: ConvWorkload, device="cpu"):
    """x ~ N(0, 1), weight ~ N(0, 1 / W), bias ~ N(0, 0.1^2), state lines ~ N(0, 1) cast to
    the dtype; sequence n uses line (n * 7 + 3) mod lines when that is a permutation, else n;
    every sequence starts from its line.  Draw order: x, weight, bias, state."""
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed)
    dt = DTYPES[w.dtype]
    x = torch.randn((w.B, w.T, w.channels), generator=gen, device=dev).to(dt)
    weight = torch.randn((w.channels, w.width), generator=gen, device=dev) / w.width ** 0.5
    bias = torch.randn((w.channels,), generator=gen, device=dev) * 0.1
    state = idx = None
    if w.lines:
        state = torch.randn((w.lines, w.width - 1, w.channels), generator=gen,
                            device=dev).to(dt)
        import math
        perm = math.gcd(7, w.lines) == 1 and w.lines >= w.B
        idx = torch.tensor([(n * 7 + 3) % w.lines if perm else n for n in range(w.B)],
                           dtype=torch.int32, device=dev)
    return dict(x=x, weight=weight, bias=bias, conv_state=state, cache_indices=idx,
                has_initial_state=None, cu_seqlens=None, activation=w.activation,
                workload=w)


# ---------------------------------------------------------------- decode gate inputs
def draw_gating(w: Workload, B: int, T: int, device="cpu"):
    """Raw gate inputs of the decode operator with the sigmoid-gate parametrisation, for a
    [B, T] token layout (that of ``draw(w)``'s g: a packed batch has B = 1 and T = its total)
    and the heads of workload ``w``.  Own generator (seed + 1000), draw order a, b, A_log,
    dt_bias:
      * a ~ N(0, 1) and b ~ N(0, 1) per token and value head, cast to the beta dtype;
      * A_log = log(U(1, 16)) per value head (decay rates spread over a decade), fp32;
      * dt_bias ~ N(-4, 0.5^2) per value head, fp32 (small step sizes, so the per-token
        decay is mild, like the log-decays of the chunked workloads)."""
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed + 1000)
    bdt = DTYPES[w.beta_dtype or w.dtype]
    a = torch.randn((B, T, w.H), generator=gen, device=dev).to(bdt)
    b = torch.randn((B, T, w.H), generator=gen, device=dev).to(bdt)
    A_log = torch.log(torch.rand((w.H,), generator=gen, device=dev) * 15.0 + 1.0)
    dt_bias = torch.randn((w.H,), generator=gen, device=dev) * 0.5 - 4.0
    return dict(a=a, b=b, A_log=A_log, dt_bias=dt_bias)


# ---------------------------------------------------------------- backward inputs
def draw_grads(w: Workload, B: int, T: int, N: int, device="cpu", dht_std=0.1):
    """Upstream gradients for the backward pass, for a [B, T] token layout and N sequences
    (those of ``draw(w)``).  Own generator (seed + 2000), draw order do, dht:
      * do ~ N(0, 1) per output element, cast to the q/k/v dtype;
      * dht ~ N(0, dht_std^2) fp32 [N, H, Dk, Dv] (None when dht_std is None)."""
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed + 2000)
    do = torch.randn((B, T, w.H, w.Dv), generator=gen, device=dev).to(DTYPES[w.dtype])
    dht = None
    if dht_std is not None:
        dht = torch.randn((N, w.H, w.Dk, w.Dv), generator=gen, device=dev) * dht_std
    return dict(do=do, dht=dht)
