"""Benchmark of the chunked Gated DeltaNet forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload headline] [--variant auto]

One step = one gdn_chunk_fwd call over the whole workload (all stages), inputs already
resident in HBM.  Prints ONE JSON line: whole-job tokens/s, the roofline of the dominant
kernel (algorithmic bytes per launch / measured launch time, against MI355X's 8 TB/s), and
the fp64 oracle timed on a bounded sample of the same workload on the host cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import gdn_inputs  # noqa: E402

METRIC = "GDN chunk-fwd tokens/s at 1 MI355X (16×8192, H=32, D=128, bf16); % roofline"


def metric_for(w) -> str:
    """The metric's name for workload ``w``: the headline's own string for the 16 x 8192
    workload, the same form with the workload's shape otherwise."""
    if w == gdn_inputs.WORKLOADS["headline"]:
        return METRIC
    heads = "H=%d" % w.H if w.Hg == w.H else "H=%d, Hg=%d" % (w.H, w.Hg)
    if w.n_varlen:
        shape = "varlen %d seqs U{1..%d}" % (w.n_varlen, w.max_len)
    else:
        shape = "%d×%d" % (w.B, w.T)
    return "GDN chunk-fwd tokens/s at 1 MI355X (%s, %s, D=%d, %s); %% roofline" % (
        shape, heads, w.Dk, w.dtype)


HBM_PEAK_GBS = 8000.0       # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
F32_PEAK_TFLOPS = 157.3

# HBM bytes of the fused kernel on the 16x8192, H=32, D=128, C=128 workload, from two
# rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE; KiB per dispatch), each scaled by what the
# same counter reads for a plain 1 GiB device copy (FETCH_SIZE reads 0.5 GiB there, so x2;
# WRITE_SIZE reads 1 GiB, so x1).  The figures hold only for the kernel sources they were
# taken on: SOURCES_SHA256 is checked against the current files and traffic reports null
# once they differ.
PMC_TRAFFIC = {
    "workload": "bf16_16x8192_h32_d128_c128",
    "fetch_kib": 1674309.08, "write_kib": 1081386.26,
    "fetch_scale": 2.0, "write_scale": 1.0,
    "sources_sha256": "673222c874991f11d0fc932cf4041011c23f5b85bbbc8bd19474f11eb246b52b",
}
FUSED_SOURCES = ("fused.hip", "gdn_device.h", "gdn_internal.h")


def fused_sources_sha256() -> str:
    """sha256 over the sha256sum-style listing of the fused kernel's sources (the same
    digest as `sha256sum fused.hip gdn_device.h gdn_internal.h | sha256sum` run from the
    repository root with the package-relative paths)."""
    import hashlib
    lines = []
    for fn in FUSED_SOURCES:
        rel = "gated_deltanet_chunked_02_amd/csrc/" + fn
        with open(os.path.join(ROOT, rel), "rb") as f:
            lines.append("%s  %s\n" % (hashlib.sha256(f.read()).hexdigest(), rel))
    return hashlib.sha256("".join(lines).encode()).hexdigest()


def pmc_traffic(workload: str, variant: str):
    """Scaled HBM bytes per launch, or None when no counters match this kernel build."""
    t = PMC_TRAFFIC
    if t is None or variant != "fused" or workload != t["workload"]:
        return None
    if fused_sources_sha256() != t["sources_sha256"]:
        return None
    return 1024.0 * (t["fetch_kib"] * t["fetch_scale"] + t["write_kib"] * t["write_scale"])


def algorithmic_work(inp, variant="fused", C=None):
    """Bytes moved and flops a perfect implementation needs (per call).

    Bytes: q and k once per q/k head, v, g, beta and h0 (if given) read once, o and ht
    written once.  Flops (triangle-aware, per token and value head, at the chunk length C
    the kernel runs): 2 (3 C Dk / 2 + 2 C Dv / 2 + 3 Dk Dv) + C^2 / 3 — K K^T and Q K^T
    (half), T K and T V (half), P v_new (half), W h, K^T v_new and Q h (full), plus the
    triangular inverse.  The recurrent variant does 6 Dk Dv per token and value head instead
    (k.H, q.H and the rank-one update of the state)."""
    q, v = inp["q"], inp["v"]
    B, T, Hg, Dk = q.shape
    H, Dv = v.shape[2], v.shape[3]
    C = inp["C"] if C is None else C
    el = q.element_size()
    toks = B * T
    nseq = B if inp["cu_seqlens"] is None else inp["cu_seqlens"].numel() - 1
    by = toks * Hg * Dk * el * 2 + toks * H * Dv * el * 2 + toks * H * 4 + \
        toks * H * inp["beta"].element_size() + nseq * H * Dk * Dv * 4
    if inp["h0"] is not None:
        by += nseq * H * Dk * Dv * 4
    fl = toks * H * (2 * (3 * C * Dk / 2 + 2 * C * Dv / 2 + 3 * Dk * Dv) + C * C / 3)
    if variant == "recurrent":
        fl = toks * H * 6 * Dk * Dv
    return float(by), float(fl)


def cpu_baseline(inp, o_gpu, ht_gpu, budget_s: float):
    """Time the fp64 oracle (as it stands) on a bounded sample of (sequence, head) pairs of
    the same workload, scale to whole-job tokens/s, and check the sampled GPU outputs."""
    import oracle
    from tests.gdn_testlib import oracle_pairs, rel_l2
    B, T = inp["q"].shape[:2]
    H = inp["v"].shape[2]
    nseq = B if inp["cu_seqlens"] is None else inp["cu_seqlens"].numel() - 1
    cores = len(os.sched_getaffinity(0))
    oracle.use_native()  # the same C source, -O3 -march=native for this host
    threads = oracle.max_threads(cores)
    rng = np.random.default_rng(12345)
    all_pairs = [(n, h) for n in range(nseq) for h in range(H)]
    order = rng.permutation(len(all_pairs))
    # calibrate on one pair per thread, then size the sample to the budget
    t0 = time.perf_counter()
    first = [all_pairs[i] for i in order[:threads]]
    oracle_pairs(inp, first, nthreads=threads)
    t_first = time.perf_counter() - t0
    n_more = int(max(0, budget_s / max(t_first, 1e-3) - 1)) * threads
    more = [all_pairs[i] for i in order[threads:threads + n_more]]
    t0 = time.perf_counter()
    res = oracle_pairs(inp, first + more, nthreads=threads)
    t_sample = time.perf_counter() - t0
    npairs = len(res)
    # whole-job estimate: the oracle's time scales with the token-heads it steps through
    # (the pairs of a packed batch differ in length)
    sampled_th = sum(o_ref.shape[0] for o_ref, _ in res.values())
    t_job = t_sample * (B * T * H) / max(sampled_th, 1)
    value = B * T / t_job
    errs_o, errs_h = [], []
    o64 = None
    for (n, h), (o_ref, ht_ref) in res.items():
        from tests.gdn_testlib import pair_slices
        ts, b, _ = pair_slices(inp, n, h)
        o64 = o_gpu[b, ts, h].double().cpu().numpy()
        errs_o.append(rel_l2(o64, o_ref))
        errs_h.append(rel_l2(ht_gpu[n, h].double().cpu().numpy(), ht_ref))
    return {
        # the oracle's parallel loop runs over the sampled pairs
        "value": value, "unit": "tokens/s", "cores": min(threads, npairs), "kind": "oracle",
        "sample": "%d of %d (sequence, head) pairs at full length, fp64 token recurrence "
                  "(C, gcc -O3 -march=native, OpenMP), %.1f s; scaled by token-heads to the "
                  "whole job" % (npairs, len(all_pairs), t_sample),
        "cpu_model": oracle.cpu_model(), "host_threads_available": cores,
        "sample_seconds": t_sample,
        "parity_sampled": {"pairs": npairs, "o_rel_l2_max": max(errs_o),
                           "ht_rel_l2_max": max(errs_h)},
    }


def copy_rate(dev, warmup=10, launches=30):
    """GB/s of a plain 1 GiB device copy (bf16; 1 GiB read + 1 GiB written per launch) on
    the current stream: the bandwidth a streaming kernel can reach on this machine, measured in
    the same process after the timed region."""
    n = 1 << 29
    a = torch.ones(n, device=dev, dtype=torch.bfloat16)
    b = torch.empty_like(a)
    for _ in range(warmup):
        b.copy_(a)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(launches):
        b.copy_(a)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / launches
    del a, b
    return 4 * n / (ms * 1e-3) / 1e9


def copy_reference(args, dev):
    """A plain copy of 1 GiB (bf16): 1 GiB read + 1 GiB written per launch."""
    n = 1 << 29
    a = torch.ones(n, device=dev, dtype=torch.bfloat16)
    b = torch.empty_like(a)
    for _ in range(args.warmup):
        b.copy_(a)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(args.steps):
        b.copy_(a)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / args.steps
    print(json.dumps({"mode": "copy", "bytes_read": 2 * n, "bytes_written": 2 * n,
                      "ms_per_copy": ms, "GBps": 4 * n / (ms * 1e-3) / 1e9}), flush=True)


def conv_bench(args, dev, gdn):
    """Time gdn_causal_conv1d_fwd (both of its launches) on a conv workload.  Algorithmic
    bytes: x read and y written once, weight and bias, and each sequence's state line read
    and written once."""
    w = gdn_inputs.CONV_WORKLOADS[args.workload]
    print("[bench] drawing %s on %s" % (w.name, dev), file=sys.stderr, flush=True)
    inp = gdn_inputs.draw_conv(w, device=dev)
    x, wt, b, st, idx = (inp[n] for n in ("x", "weight", "bias", "conv_state", "cache_indices"))
    y = torch.empty_like(x)
    desc = gdn.GdnConvDesc(B=w.B, T=w.T, N=w.B, channels=w.channels, width=w.width,
                           dtype=gdn._dtype_code(x), activation=gdn.ACTIVATIONS[w.activation],
                           state_lines=w.lines)
    stream = torch.cuda.current_stream()
    st0 = None if st is None else st.clone()  # the drawn state lines, for the parity sample

    def step():
        rc = gdn.gdn_causal_conv1d_fwd(desc, x, wt, b, st, idx, None, None, y, stream)
        if rc != 0:
            raise gdn.GdnError(rc, "gdn_causal_conv1d_fwd")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    t_wall = time.perf_counter()
    for s, e in ev:
        s.record(stream)
        step()
        e.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    avg_ms = float(np.mean([s.elapsed_time(e) for s, e in ev]))
    ms_per_step = 1e3 * t_wall / args.steps
    el = x.element_size()
    toks = w.B * w.T
    by = 2.0 * toks * w.channels * el + w.channels * (w.width + 1) * 4 + \
        2.0 * w.B * (w.width - 1) * w.channels * el
    gbs = by / (avg_ms * 1e-3) / 1e9
    out = {
        "metric": "causal conv1d tokens/s at 1 MI355X", "value": toks / (ms_per_step * 1e-3),
        "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if x.dtype == torch.bfloat16 else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "T": w.T, "channels": w.channels,
                   "width": w.width, "activation": w.activation, "state_lines": w.lines,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "k_conv1d + k_conv_state (W=%d)" % w.width,
                     "launch_ms": avg_ms, "algorithmic_bytes": by},
        "cpu_baseline": None,
    }
    if args.cpu_budget > 0:
        # one more call from the drawn state lines, whose y the sample is checked against
        if st is not None:
            st.copy_(st0)
        step()
        torch.cuda.synchronize()
        out["cpu_baseline"] = conv_cpu_baseline(w, inp, st0, y, args.cpu_budget)
    print(json.dumps(out), flush=True)


def conv_cpu_baseline(w, inp, st0, y_gpu, budget_s: float):
    """The conv oracle (numpy, fp64, one thread) on a bounded sample: every sequence at full
    length over a slice of the channels (the convolution is depthwise, so channels are
    independent), doubled until it takes about a third of the budget; scaled by
    channel-tokens to the whole job.  The sample doubles as a parity check of y."""
    import oracle
    from oracle import conv1d
    C = w.channels
    x = inp["x"]
    wt, bias, idx = inp["weight"].cpu().double().numpy(), inp["bias"].cpu().double().numpy(), \
        (None if inp["cache_indices"] is None else inp["cache_indices"].cpu().numpy())
    st = None if st0 is None else st0.cpu().double().numpy()
    nc, took, errs = 8, 0.0, []
    while True:
        sl = slice(0, nc)
        xs = x[:, :, sl].float().cpu().double().numpy()
        t0 = time.perf_counter()
        ys, _ = conv1d.causal_conv1d(xs, wt[sl], bias[sl],
                                     None if st is None else st[:, :, sl], idx,
                                     activation=w.activation)
        took = time.perf_counter() - t0
        yg = y_gpu[:, :, sl].float().cpu().double().numpy()
        errs = [float(np.linalg.norm(yg - ys) / max(np.linalg.norm(ys), 1e-30))]
        if took >= budget_s / 3 or nc >= C:
            break
        nc = min(C, nc * 2)
    scale = C / nc
    return {"value": w.B * w.T / (took * scale), "unit": "tokens/s", "cores": 1,
            "kind": "oracle",
            "sample": "all %d sequences at full length over %d of %d channels, fp64 numpy "
                      "(one thread), %.1f s; scaled by channel-tokens to the whole job"
                      % (w.B, nc, C, took),
            "cpu_model": oracle.cpu_model(), "sample_seconds": took,
            "parity_sampled": {"channels": nc, "y_rel_l2": errs[0]}}


def bwd_algorithmic_bytes(inp, grad_bytes=4):
    """Bytes a perfect backward moves: the forward's inputs (q, k, v, g, beta, h0) and the
    upstream gradients (do, dht) read once; dq, dk, dv (grad_bytes each: fp32 or bf16), dg,
    dbeta (fp32) and dh0 written once."""
    q, v = inp["q"], inp["v"]
    B, T, Hg, Dk = q.shape
    H, Dv = v.shape[2], v.shape[3]
    el = q.element_size()
    toks = B * T
    nseq = B if inp["cu_seqlens"] is None else inp["cu_seqlens"].numel() - 1
    state = nseq * H * Dk * Dv * 4
    rd = toks * (2 * Hg * Dk + 2 * H * Dv) * el + toks * H * (4 + inp["beta"].element_size())
    wr = toks * (2 * Hg * Dk + H * Dv) * grad_bytes + toks * H * 8
    if inp["h0"] is not None:
        rd += state
        wr += state
    if inp.get("dht") is not None:
        rd += state
    return float(rd + wr)


def bwd_cpu_baseline(inp, grads_gpu, budget_s: float):
    """Time the fp64 oracle's backward (reverse-mode through the token recurrence, numpy) on
    a bounded sample of (sequence, head) pairs, scale to whole-job tokens/s, and check the
    sampled GPU gradients: dv, dg and dbeta of the pair, and dq, dk too when no other value
    head shares the pair's q/k head (else those are sums over the group)."""
    import oracle
    from oracle import backward
    from tests.gdn_testlib import pair_slices, rel_l2
    B, T = inp["q"].shape[:2]
    H = inp["v"].shape[2]
    nseq = B if inp["cu_seqlens"] is None else inp["cu_seqlens"].numel() - 1
    rng = np.random.default_rng(12345)
    pairs = [(n, h) for n in range(nseq) for h in range(H)]
    order = rng.permutation(len(pairs))
    f = lambda x: x.double().cpu().numpy()
    t_sample, th, errs, used = 0.0, 0, [], 0
    for i in order:
        if t_sample >= budget_s:
            break
        n, h = pairs[i]
        ts, b, hk = pair_slices(inp, n, h)
        sl = lambda x, j: f(x[b:b + 1, ts, j:j + 1])
        args = [sl(inp["q"], hk), sl(inp["k"], hk), sl(inp["v"], h), sl(inp["g"], h),
                sl(inp["beta"], h)]
        h0 = None if inp["h0"] is None else f(inp["h0"][n:n + 1, h:h + 1])
        dht = None if inp.get("dht") is None else f(inp["dht"][n:n + 1, h:h + 1])
        do = sl(inp["do"], h)
        t0 = time.perf_counter()
        ref = backward.recurrence_backward(*args, h0, inp["scale"], do, dht)
        t_sample += time.perf_counter() - t0
        th += args[0].shape[1]
        used += 1
        shared = inp["v"].shape[2] != inp["q"].shape[2]
        for j, idx in enumerate((hk, hk, h, h, h)):
            if j < 2 and shared:
                continue
            x = grads_gpu[j][b:b + 1, ts, idx:idx + 1]
            errs.append(rel_l2(f(x), ref[j]))
    t_job = t_sample * (B * T * H) / max(th, 1)
    return {
        "value": B * T / t_job, "unit": "tokens/s", "cores": 1, "kind": "oracle",
        "sample": "%d of %d (sequence, head) pairs at full length, fp64 reverse-mode "
                  "through the token recurrence (numpy, one thread), %.1f s; scaled by "
                  "token-heads to the whole job" % (used, len(pairs), t_sample),
        "cpu_model": oracle.cpu_model(), "sample_seconds": t_sample,
        "parity_sampled": {"pairs": used, "grad_rel_l2_max": max(errs) if errs else None,
                           "compared": "dv, dg, dbeta" if inp["v"].shape[2] !=
                           inp["q"].shape[2] else "dq, dk, dv, dg, dbeta"},
    }


def bwd_bench(args, dev, gdn, w, inp):
    """Time gdn_chunk_bwd: the staged recompute of the forward's chunk quantities (C = 64)
    and the two backward kernels, one call per step."""
    q, k, v, g, beta = (inp[n] for n in ("q", "k", "v", "g", "beta"))
    h0, cu = inp["h0"], inp["cu_seqlens"]
    N = q.shape[0] if cu is None else cu.numel() - 1
    inp.update(gdn_inputs.draw_grads(w, q.shape[0], q.shape[1], N, device=dev,
                                     dht_std=None if h0 is None else 0.1))
    do, dht = inp["do"], inp["dht"]
    desc = gdn.make_desc(q, v, beta, cu, 64, args.variant)
    how = gdn.gdn_chunk_bwd_resolved_variant(desc, cu)
    ws = torch.empty(gdn.gdn_chunk_bwd_workspace_size(desc), device=dev, dtype=torch.uint8)
    desc.workspace, desc.workspace_bytes = ws.data_ptr(), ws.numel()
    f = dict(device=dev, dtype=torch.float32)
    gbf = args.grad_dtype == "bf16"
    if gbf and q.dtype != torch.bfloat16:
        raise SystemExit("--grad-dtype bf16 needs bf16 inputs")
    desc.grad_dtype = 1 if gbf else 0
    fg = dict(device=dev, dtype=torch.bfloat16 if gbf else torch.float32)
    dq, dk, dv = torch.empty(q.shape, **fg), torch.empty(k.shape, **fg), torch.empty(v.shape, **fg)
    dg, dbeta = torch.empty(g.shape, **f), torch.empty(g.shape, **f)
    dh0 = None if h0 is None else torch.empty(h0.shape, **f)
    stream = torch.cuda.current_stream()

    def step():
        st = gdn.gdn_chunk_bwd(desc, q, k, v, g, beta, h0, cu, inp["scale"], do, dht, dq, dk,
                               dv, dg, dbeta, dh0, stream)
        if st != 0:
            raise gdn.GdnError(st, "gdn_chunk_bwd")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print("[bench] warmup done; timing %d backward steps" % args.steps, file=sys.stderr,
          flush=True)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    t_wall = time.perf_counter()
    for s, e in ev:
        s.record(stream)
        step()
        e.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    avg_ms = float(np.mean([s.elapsed_time(e) for s, e in ev]))
    ms_per_step = 1e3 * t_wall / args.steps
    tokens = q.shape[0] * q.shape[1]
    by = bwd_algorithmic_bytes(inp, 2 if gbf else 4)
    gbs = by / (avg_ms * 1e-3) / 1e9
    copy_gbs = copy_rate(dev)
    cpu = None
    if args.cpu_budget > 0:
        print("[bench] timing the oracle's backward on the host", file=sys.stderr, flush=True)
        cpu = bwd_cpu_baseline(inp, (dq, dk, dv, dg, dbeta), args.cpu_budget)
    heads = "H=%d" % w.H if w.Hg == w.H else "H=%d, Hg=%d" % (w.H, w.Hg)
    shape = ("varlen %d seqs U{1..%d}" % (w.n_varlen, w.max_len) if w.n_varlen
             else "%d×%d" % (w.B, w.T))
    out = {
        "metric": "GDN chunk-bwd tokens/s at 1 MI355X (%s, %s, D=%d, %s); %% roofline" % (
            shape, heads, w.Dk, w.dtype),
        "value": tokens / (ms_per_step * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if q.dtype == torch.bfloat16 else "f32", "data": "synthetic",
        "config": {"workload": w.name, "pass": "backward", "B": int(q.shape[0]),
                   "T": int(q.shape[1]), "H": w.H, "Hg": w.Hg, "Dk": w.Dk, "Dv": w.Dv,
                   "C": 64, "h0": h0 is not None, "variant": how,
                   "grad_dtype": "bf16" if gbf else "f32", "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": None,
                     "copy_GBps": copy_gbs, "frac_of_copy": gbs / copy_gbs,
                     "kernel": "gdn_chunk_bwd whole call (%s, k_bwd_chunk%s)" % (
                         {"segmented": "staged stages 0-4; per segment: the k_fused maps and "
                                       "segment scan, k_fused store mode, k_bwd_dh from zero, "
                                       "the reverse segment scan, k_bwd_dh",
                          "fused": "staged stages 0-4, k_fused store mode, k_bwd_dh",
                          "staged": "staged stages 0-6, k_bwd_dh"}[how],
                         " over each q/k head's value heads" if w.H != w.Hg else ""),
                     "launch_ms": avg_ms, "algorithmic_bytes": by},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # The GPU's clocks settle over the first tens of milliseconds of sustained work (about
    # 9 % slower launches before); 100 warm-up launches reach the steady state, and 200
    # timed launches (about 0.25 s) average over it.
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="headline",
                    choices=sorted(gdn_inputs.WORKLOADS) + sorted(gdn_inputs.CONV_WORKLOADS),
                    help="conv_*: the causal conv1d before the delta rule")
    ap.add_argument("--variant", default="auto", choices=["auto", "fused", "staged", "segmented", "recurrent"])
    ap.add_argument("--chunk", type=int, default=0,
                    help="override the workload's chunk size C (64 or 128)")
    ap.add_argument("--set", action="append", default=[], metavar="FIELD=INT",
                    help="override an integer field of the workload (e.g. H=16, T=4096)")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle work for the CPU baseline (0 = skip)")
    ap.add_argument("--gated", action="store_true",
                    help="time the decode operator with in-kernel gates "
                         "(gdn_fused_sigmoid_gating_delta_rule) on the workload's tokens")
    ap.add_argument("--bwd", action="store_true",
                    help="time the backward pass (gdn_chunk_bwd) on the workload")
    ap.add_argument("--grad-dtype", default="f32", choices=["f32", "bf16"],
                    help="--bwd: dtype of dq, dk, dv (bf16 needs bf16 inputs)")
    ap.add_argument("--mode", default="gdn", choices=["gdn", "copy"],
                    help="copy: time a plain 1 GiB device-to-device copy (the reference "
                         "kernel for scaling HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on one GPU only; multi-GPU runs are not part of it "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(2)

    import gated_deltanet_chunked_02_amd as gdn
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.mode == "copy":
        copy_reference(args, dev)
        return
    if args.workload in gdn_inputs.CONV_WORKLOADS:
        conv_bench(args, dev, gdn)
        return
    w = gdn_inputs.WORKLOADS[args.workload]
    if args.chunk:
        w = w.with_(C=args.chunk)
    for kv in args.set:
        field, val = kv.split("=", 1)
        w = w.with_(**{field: int(val)})
    print("[bench] drawing %s on %s" % (w.name, dev), file=sys.stderr, flush=True)
    inp = gdn_inputs.draw(w, device=dev)
    if args.bwd:
        bwd_bench(args, dev, gdn, w, inp)
        return
    q, k, v, g, beta = (inp[n] for n in ("q", "k", "v", "g", "beta"))
    h0, cu = inp["h0"], inp["cu_seqlens"]
    gate_in = None
    if args.gated:
        gate_in = gdn_inputs.draw_gating(w, g.shape[0], g.shape[1], device=dev)
        args.variant = "recurrent"
    desc = gdn.make_desc(q, v, beta, cu, w.C, args.variant)
    o = torch.empty_like(v)
    ht = torch.empty((desc.N, desc.H, desc.Dk, desc.Dv), device=dev, dtype=torch.float32)
    ws_bytes = gdn.gdn_chunk_fwd_workspace_size(desc)
    ws = None
    if ws_bytes:
        ws = torch.empty(ws_bytes, device=dev, dtype=torch.uint8)
        desc.workspace, desc.workspace_bytes = ws.data_ptr(), ws.numel()
    variant = gdn.gdn_resolved_variant(desc, cu)
    c_run = gdn.gdn_resolved_chunk(desc, cu)
    stream = torch.cuda.current_stream()

    def step():
        if gate_in is not None:
            st = gdn.gdn_fused_sigmoid_gating_delta_rule(
                desc, q, k, v, gate_in["a"], gate_in["b"], gate_in["A_log"],
                gate_in["dt_bias"], h0, cu, inp["scale"], o, ht, stream)
        else:
            st = gdn.gdn_chunk_fwd(desc, q, k, v, g, beta, h0, cu, inp["scale"], o, ht, stream)
        if st != 0:
            raise gdn.GdnError(st, "gdn_chunk_fwd")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print("[bench] warmup done; timing %d steps" % args.steps, file=sys.stderr, flush=True)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for s, e in ev:
        s.record(stream)
        step()
        e.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    launch_ms = [s.elapsed_time(e) for s, e in ev]
    ms_per_step = 1e3 * t_wall / args.steps
    tokens = q.shape[0] * q.shape[1]
    value = tokens / (ms_per_step * 1e-3)

    by, fl = algorithmic_work(inp, variant, c_run)
    if gate_in is not None:  # a and b replace g and beta; A_log and dt_bias per head
        by += (gate_in["a"].element_size() - 4) * gate_in["a"].numel() + 8 * w.H
    avg_ms = float(np.mean(launch_ms))
    gbs = by / (avg_ms * 1e-3) / 1e9
    tfl = fl / (avg_ms * 1e-3) / 1e12
    peak_tf = F32_PEAK_TFLOPS if q.dtype == torch.float32 else BF16_PEAK_TFLOPS
    bound = "hbm" if by / HBM_PEAK_GBS >= fl / (peak_tf * 1e3) else "mfma"
    if variant == "staged":
        kernel = "staged pipeline (8 launches; per-kernel split in profiles/)"
    elif variant == "segmented":
        kernel = "segmented: three k_fused passes over the segments and the segment scan"
    elif variant == "recurrent":
        kernel = "k_recurrent%s (D=%d, one wave per 32 state columns)" % (
            "<gated>" if gate_in is not None else "", w.Dk)
    else:
        kernel = "k_fused (D=%d, %d-token chunks)" % (w.Dk, c_run)
    if bound == "hbm":
        roof = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": gbs / HBM_PEAK_GBS}
    else:
        roof = {"bound": "mfma", "achieved": tfl, "peak": peak_tf, "unit": "TFLOP/s",
                "frac": tfl / peak_tf}
    roof["traffic"] = pmc_traffic(w.name, variant)
    if bound == "hbm":
        roof["copy_GBps"] = copy_rate(dev)
        roof["frac_of_copy"] = gbs / roof["copy_GBps"]
    roof["kernel"] = kernel
    roof["launch_ms"] = avg_ms
    roof["algorithmic_bytes"] = by
    roof["algorithmic_flops"] = fl
    roof["mfma_tflops"] = tfl

    cpu = None
    if args.cpu_budget > 0:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        if gate_in is not None:
            # the oracle's gate map first (fp64), then the same timed token recurrence
            from oracle import gating
            gg, bb = gating.gates(gate_in["a"].cpu(), gate_in["b"].cpu(),
                                  gate_in["A_log"].cpu(), gate_in["dt_bias"].cpu())
            inp = dict(inp, g=torch.from_numpy(gg), beta=torch.from_numpy(bb))
        cpu = cpu_baseline(inp, o, ht, args.cpu_budget)

    out = {
        "metric": ("GDN gated decode (sigmoid gating in the kernel) tokens/s at 1 MI355X "
                   "(%d×%d, H=%d, Hg=%d, D=%d, %s)" % (w.B, w.T, w.H, w.Hg, w.Dk, w.dtype)
                   if gate_in is not None else metric_for(w)), "value": value, "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if q.dtype == torch.bfloat16 else "f32", "data": "synthetic",
        "config": {"workload": w.name, "B": int(q.shape[0]), "T": int(q.shape[1]),
                   "H": w.H, "Hg": w.Hg, "Dk": w.Dk, "Dv": w.Dv, "C": c_run,
                   "C_requested": w.C,
                   "variant": variant, "h0": inp["h0"] is not None,
                   "parallelism": "single GPU"},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
