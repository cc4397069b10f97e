#!/usr/bin/env python3
"""Attention TFLOP/s for causal bf16 fwd+bwd at S=32768, D=128 on one MI355X.

One step is the whole hot path on one batch of synthetic input that already
sits in HBM: attn_fwd, then the three backward kernels (Delta, dK/dV, dQ)
through attn_bwd_phases. That is the same work attn_bwd does, split so each
kernel can be bracketed with HIP events on the stream it runs on (the
binding launches on torch's current stream, which the events record on).

Headline workload (one GPU's Ulysses head share of a Qwen2.5-7B-shaped layer):
B=1, Hq=28, Hkv=4, S=32768, D=128, causal, bf16 inputs drawn N(0, 1) from
seed 3.

FLOPs are algorithmic: only visible (i, j) pairs count, 4*D per pair for the
forward (QK^T and PV) and 10*D per pair for the backward (QK^T, dO V^T,
P^T dO, dS K, dS^T Q). The dQ kernel's second recompute of QK^T and dO V^T is
not counted. Per kernel: fwd 4*D, dK/dV 8*D, dQ 2*D per pair.

Prints one JSON line. The roofline object describes the kernel with the
largest share of the step time. ``cpu_baseline`` times the fp64 oracle on a
bounded sample of the same workload on the host cores. ``workloads`` holds
the other configurations measured the same way (mid: bf16 forward; packed32k:
packed fwd+bwd; fp8_64k: fp8 forward against the fp8 dense peak; ring4_gqa32k:
the gqa32k forward as a 4-chunk Ring-Attention pass with attn_fwd_merge, the
same with attn_fwd + attn_merge, the ring's forward + backward (attn_bwd_accumulate
per chunk pair), and the merge kernel's HBM rate; key_split_1h32k: a small-grid forward with and
without the key split; fp8_64k_fwd_bwd: the fp8 forward and its backward).
``mfma_ceiling`` is the rate a register-only MFMA loop sustains on the same
GPU and its clock, the practical ceiling the kernels' fractions compare with.

    python bench.py [--steps 20] [--warmup 3] [--gpus 1] [--no-secondary]
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA peak
SECONDARY_WARM_MS = 200.0  # least warmup before a secondary workload's timed steps
PEAK_FP8_TFLOPS = 5000.0   # MI355X dense fp8 MFMA peak
PEAK_HBM_GBS = 8000.0


def _pairs(seqlen: int, causal: bool, cu=None) -> float:
    """Visible (query, key) pairs of one (batch, head)."""
    if cu is not None:
        lens = [int(b) - int(a) for a, b in zip(cu[:-1], cu[1:])]
        return float(sum(L * (L + 1) // 2 if causal else L * L for L in lens))
    return seqlen * (seqlen + 1) / 2.0 if causal else float(seqlen) * seqlen


KERNEL_SOURCES = {
    "attn_fwd_bf16_kernel": ("attn_fwd.hip", "attn_device.h", "attn_internal.h", "attn_index.h"),
    "attn_fwd_combine_kernel": ("attn_fwd.hip", "attn_device.h", "attn_internal.h", "attn_index.h"),
    "attn_fwd_fewkeys_kernel": ("attn_fwd.hip", "attn_device.h", "attn_internal.h", "attn_index.h"),
    "attn_bwd_dkdv_kernel": ("attn_bwd.hip", "attn_device.h", "attn_internal.h", "attn_index.h"),
    "attn_bwd_dq_kernel": ("attn_bwd.hip", "attn_device.h", "attn_internal.h", "attn_index.h"),
    "attn_bwd_delta_kernel": ("attn_bwd.hip", "attn_device.h", "attn_internal.h", "attn_index.h"),
    "attn_fwd_fp8_kernel": ("attn_fwd_fp8.hip", "attn_device.h", "attn_internal.h", "attn_index.h"),
    "attn_merge_kernel": ("attn_merge.hip", "attn_device.h", "attn_internal.h", "attn_index.h"),
    "attn_widen_fp8_kernel": ("attn_bwd.hip", "attn_device.h", "attn_internal.h", "attn_index.h"),
    "attn_bwd_dkdv_reduce_kernel": ("attn_bwd.hip", "attn_device.h", "attn_internal.h", "attn_index.h"),
    "attn_bwd_dq_reduce_kernel": ("attn_bwd.hip", "attn_device.h", "attn_internal.h", "attn_index.h"),
}
KERNEL_OF_PHASE = {"attn_fwd": "attn_fwd_bf16_kernel", "bwd_delta": "attn_bwd_delta_kernel",
                   "bwd_dkdv": "attn_bwd_dkdv_kernel", "bwd_dq": "attn_bwd_dq_kernel"}


def code_text(source: str) -> str:
    """C++/HIP source with comments removed and blank space collapsed."""
    source = re.sub(r"/\*.*?\*/", " ", source, flags=re.S)
    source = re.sub(r"//[^\n]*", " ", source)
    return " ".join(source.split())


def kernel_source_hash(kernel: str) -> str:
    """Hash of the code of the source files a kernel is built from (counter records go stale when the code
    changes, not when its comments do)."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "long_context_exact_fwd_amd", "csrc", name), encoding="utf-8") as f:
            h.update(name.encode())
            h.update(code_text(f.read()).encode())
    return h.hexdigest()[:16]


def _traffic(kernel: str):
    """HBM bytes per launch from the committed counter record, if the kernel's sources are unchanged."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path, encoding="utf-8") as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    k = rec.get("kernels", {}).get(kernel)
    if not k or k.get("source_hash") != kernel_source_hash(kernel):
        return None
    return k.get("bytes_per_launch")


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, x, sample_len: int, single_len: int = 8192):
    """Oracle (fp64, numpy) fwd+bwd of one kv group over a causal prefix of the same inputs.

    Two timings: the group's G query heads over the first ``sample_len`` tokens with one worker thread
    per core share (numpy's own BLAS threading pinned to 1 inside each worker), and one query head over
    the first ``single_len`` tokens on a single thread. The oracle runs six contractions per visible
    pair (scores, PV, dO V^T, dS K, dS^T Q, P^T dO), so its rate counts 12 D flops per pair; the GPU
    metric's convention (14 D, which also counts the backward's recomputed scores) is given beside it.
    The whole workload's time is extrapolated from each sample: cost is linear in (query head, visible
    pair) at fixed D.
    """
    import oracle
    affinity = len(os.sched_getaffinity(0))
    workers = min(16, affinity)
    L = min(sample_len, w.seqlen)
    g = w.hq // w.hkv
    vals = {n: x.values(n) for n in ("q", "k", "v", "do")}

    def run(nheads, length, nthreads):
        q = vals["q"][:, :length, :nheads]
        k = vals["k"][:, :length, :1]
        v = vals["v"][:, :length, :1]
        do = vals["do"][:, :length, :nheads]
        t0 = time.perf_counter()
        oracle.attention_bwd_group(q, k, v, do, b=0, kv_head=0, causal=w.causal, scale=w.scale, workers=nthreads)
        return time.perf_counter() - t0

    full_pairs = _pairs(w.seqlen, w.causal, x.cu_seqlens) * w.batch * w.hq
    dt = run(g, L, workers)
    pairs = _pairs(L, w.causal) * g
    L1 = min(single_len, w.seqlen)
    dt1 = run(1, L1, 1)
    pairs1 = _pairs(L1, w.causal)
    D = w.head_dim
    return {
        "value": 12.0 * D * pairs / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": workers,
        "kind": "oracle",
        "sample": (f"fp64 numpy oracle fwd+bwd (attention_bwd_group) of one kv group ({g} query heads) over the "
                   f"first {L} tokens of the same seeded inputs, causal; {dt:.1f} s on {workers} threads; "
                   f"flops counted as the oracle executes them (12*D per visible pair)"),
        "seconds": round(dt, 6),
        "threads": workers,
        "host_cores": os.cpu_count(),
        "affinity_cores": affinity,
        "cpu_model": _cpu_model(),
        "value_14d_convention": 14.0 * D * pairs / dt / 1e12,
        "single_thread": {
            "seconds": round(dt1, 6),
            "value": 12.0 * D * pairs1 / dt1 / 1e12,
            "unit": "TFLOP/s",
            "sample": f"one query head over the first {L1} tokens, causal, 1 thread",
        },
        "extrapolated_full_workload_s": {
            "note": "extrapolated, not measured: sample time x (visible pairs x query heads of the whole "
                    "workload) / (those of the sample)",
            "threads": round(dt * full_pairs / pairs, 2),
            "single_thread": round(dt1 * full_pairs / pairs1, 1),
        },
    }


class Timer:
    """HIP events around each named phase of a step, on torch's current stream."""

    def __init__(self, names, steps):
        import torch
        self.names = names
        self.ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(steps)]

    def mark(self, step, j):
        self.ev[step][j].record()

    def per_phase_ms(self):
        n = len(self.ev)
        return {name: sum(e[j].elapsed_time(e[j + 1]) for e in self.ev) / n for j, name in enumerate(self.names)}

    def step_stats_ms(self):
        """Median, min and max over the timed steps of each phase and of the whole step (first to last event)."""
        def stats(vals):
            v = sorted(vals)
            mid = len(v) // 2
            med = v[mid] if len(v) % 2 else 0.5 * (v[mid - 1] + v[mid])
            return {"median": round(med, 4), "min": round(v[0], 4), "max": round(v[-1], 4)}
        out = {name: stats([e[j].elapsed_time(e[j + 1]) for e in self.ev]) for j, name in enumerate(self.names)}
        out["step"] = stats([e[0].elapsed_time(e[-1]) for e in self.ev])
        return out


def run_steps(step, names, steps, warmup, min_warm_ms=0.0):
    """Warm up, then time exactly `steps` steps between two synchronisations; returns (ms/step, per-phase ms).

    ``min_warm_ms`` > 0 adds warmup steps until the warmup has taken that long
    (the secondary workloads: after seconds of host-side input generation the
    GPU's power management needs tens of milliseconds of load to settle, and
    a 1 ms kernel timed inside that transient reads up to 25 % slow). The
    number of warmup steps run is left in ``run_steps.last_warmup``.
    """
    import torch
    n_warm = 0
    t0 = time.perf_counter()
    for _ in range(warmup):
        step(None, 0)
        n_warm += 1
    torch.cuda.synchronize()
    while min_warm_ms > 0 and (time.perf_counter() - t0) * 1e3 < min_warm_ms:
        for _ in range(max(1, n_warm)):
            step(None, 0)
            n_warm += 1
        torch.cuda.synchronize()
    run_steps.last_warmup = n_warm
    tm = Timer(names, steps)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(steps):
        step(tm, i)
    end.record()
    torch.cuda.synchronize()
    run_steps.last_stats = tm.step_stats_ms()
    return start.elapsed_time(end) / steps, tm.per_phase_ms()


def bf16_case(w, x, dev):
    """Device buffers and a step function (fwd, then Delta, dK/dV, dQ if the workload has a backward)."""
    import torch
    import long_context_exact_fwd_amd as lca
    up = lca.bf16_from_bits
    q, k, v = up(x.q_bits, dev), up(x.k_bits, dev), up(x.v_bits, dev)
    cu = torch.from_numpy(x.cu_seqlens).to(dev) if x.cu_seqlens is not None else None
    B, S, Hq = w.batch, w.seqlen, w.hq
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device=dev)
    kw = dict(causal=w.causal, cu_seqlens=cu, scale=w.scale)
    nf = lca.fwd_workspace_bytes(B, Hq, w.hkv, S, w.head_dim)
    fws = torch.empty((nf + 3) // 4, dtype=torch.float32, device=dev) if nf > 0 else None
    names = ["attn_fwd"]
    if w.backward:
        do = up(x.do_bits, dev)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws = torch.empty(lca.bwd_workspace_bytes(B, Hq, w.hkv, S, w.head_dim) // 4, dtype=torch.float32, device=dev)
        names += ["bwd_delta", "bwd_dkdv", "bwd_dq"]

    def step(tm, i):
        if tm is not None:
            tm.mark(i, 0)
        lca.fwd(q, k, v, out=o, lse=lse, workspace=fws, **kw)
        if tm is not None:
            tm.mark(i, 1)
        if w.backward:
            for j, ph in enumerate((lca.BWD_DELTA, lca.BWD_DKDV, lca.BWD_DQ)):
                lca.bwd(q, k, v, o, lse, do, dq=dq, dk=dk, dv=dv, workspace=ws, phases=ph, **kw)
                if tm is not None:
                    tm.mark(i, j + 2)

    return step, names


def fp8_case(w, x, dev):
    import torch
    import long_context_exact_fwd_amd as lca
    q8, k8, v8 = (torch.from_numpy(b).to(dev) for b in (x.q_bits, x.k_bits, x.v_bits))
    ds = [torch.tensor([float(d)], dtype=torch.float32, device=dev) for d in x.descale]
    o = torch.empty((w.batch, w.seqlen, w.hq, w.head_dim), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.batch, w.hq, w.seqlen), dtype=torch.float32, device=dev)

    def step(tm, i):
        if tm is not None:
            tm.mark(i, 0)
        lca.fwd_fp8(q8, k8, v8, *ds, causal=w.causal, scale=w.scale, out=o, lse=lse)
        if tm is not None:
            tm.mark(i, 1)

    return step, ["attn_fwd_fp8"]


def fp8_train_case(steps, warmup, dev):
    """fp8_64k's inputs (B=1, Hq=8, Hkv=1, S=65536, D=128 causal, E4M3 with per-tensor scales) through
    attn_fwd_fp8 and then attn_bwd_fp8 (widening of the codes to bf16 + the bf16 backward kernels with
    the scales folded in), with a seeded bf16 dO."""
    import torch
    import seeded_inputs as si
    import long_context_exact_fwd_amd as lca
    w = si.WORKLOADS["fp8_64k"]
    x = si.workload_inputs(w, with_do=True)
    q8, k8, v8 = (torch.from_numpy(b).to(dev) for b in (x.q_bits, x.k_bits, x.v_bits))
    ds = [torch.tensor([float(d)], dtype=torch.float32, device=dev) for d in x.descale]
    do = lca.bf16_from_bits(x.do_bits, dev)
    B, S, Hq, D = q8.shape
    Hkv = k8.shape[2]
    o = torch.empty((B, S, Hq, D), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(o), torch.empty((B, S, Hkv, D), dtype=torch.bfloat16, device=dev), None
    dv = torch.empty_like(dk)
    ws = torch.empty((lca.bwd_fp8_workspace_bytes(B, Hq, Hkv, S, D) + 3) // 4, dtype=torch.float32, device=dev)

    def step(tm, i):
        if tm is not None:
            tm.mark(i, 0)
        lca.fwd_fp8(q8, k8, v8, *ds, causal=w.causal, scale=w.scale, out=o, lse=lse)
        if tm is not None:
            tm.mark(i, 1)
        lca.bwd_fp8(q8, k8, v8, *ds, o, lse, do, causal=w.causal, scale=w.scale, workspace=ws, dq=dq, dk=dk, dv=dv)
        if tm is not None:
            tm.mark(i, 2)

    ms, per = run_steps(step, ["attn_fwd_fp8", "attn_bwd_fp8"], steps, warmup, SECONDARY_WARM_MS)
    pairs = _pairs(S, True) * B * Hq
    tf_f = 4.0 * D * pairs / (per["attn_fwd_fp8"] * 1e-3) / 1e12
    tf_b = 10.0 * D * pairs / (per["attn_bwd_fp8"] * 1e-3) / 1e12
    return {
        "config": f"fp8_64k inputs (B={B} Hq={Hq} Hkv={Hkv} S={S} D={D} causal, E4M3 per-tensor scales) fwd_fp8 + "
                  f"bwd_fp8, bf16 dO, N(0,1) seed {w.seed}",
        "tflops": round(14.0 * D * pairs / (ms * 1e-3) / 1e12, 2), "ms_per_step": round(ms, 4), "steps": steps,
        "phases_ms": {n: round(t, 4) for n, t in per.items()},
        "fwd_fp8": {"tflops": round(tf_f, 2), "pct_of_peak": round(100.0 * tf_f / PEAK_FP8_TFLOPS, 2),
                    "peak_tflops": PEAK_FP8_TFLOPS},
        "bwd_fp8": {"tflops": round(tf_b, 2), "pct_of_peak": round(100.0 * tf_b / PEAK_BF16_TFLOPS, 2),
                    "peak_tflops": PEAK_BF16_TFLOPS, "note": "bf16 MFMAs on the widened codes"},
    }


def secondary(name, steps, warmup, dev):
    """Time one of the other workloads the same way; returns a dict for the `workloads` object."""
    import seeded_inputs as si
    w = si.WORKLOADS[name]
    x = si.workload_inputs(w)
    step, names = (fp8_case if w.fp8 else bf16_case)(w, x, dev)
    ms, per = run_steps(step, names, steps, warmup, SECONDARY_WARM_MS)
    pairs = _pairs(w.seqlen, w.causal, x.cu_seqlens) * w.batch * w.hq
    flops = (14.0 if w.backward else 4.0) * w.head_dim * pairs
    peak = PEAK_FP8_TFLOPS if w.fp8 else PEAK_BF16_TFLOPS
    tf = flops / (ms * 1e-3) / 1e12
    return {
        "config": f"B={w.batch} Hq={w.hq} Hkv={w.hkv} S={w.seqlen} D={w.head_dim} causal={w.causal} "
                  f"packed={w.packed} {'fp8 e4m3' if w.fp8 else 'bf16'} {'fwd+bwd' if w.backward else 'fwd'}, "
                  f"N(0,1) seed {w.seed}",
        "tflops": round(tf, 2), "pct_of_peak": round(100.0 * tf / peak, 2), "peak_tflops": peak,
        "ms_per_step": round(ms, 4), "steps": steps, "phases_ms": {n: round(t, 4) for n, t in per.items()},
    }


def key_split_case(steps, warmup, dev):
    """Forward of a grid too small to fill the GPU (B=1, Hq=1, Hkv=1, S=32768, D=128, causal: 256
    query-block units), with the key split chosen from the sizes and with it turned off."""
    import torch
    import seeded_inputs as si
    import long_context_exact_fwd_amd as lca
    B, Hq, Hkv, S, D, seed = 1, 1, 1, 32768, 128, 6
    x = si.make_inputs(B, Hq, Hkv, S, D, seed, with_do=False)
    up = lca.bf16_from_bits
    q, k, v = up(x.q_bits, dev), up(x.k_bits, dev), up(x.v_bits, dev)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device=dev)
    nf = lca.fwd_workspace_bytes(B, Hq, Hkv, S, D)
    fws = torch.empty((nf + 3) // 4, dtype=torch.float32, device=dev)
    scale = 1.0 / math.sqrt(D)
    flops = 4.0 * D * _pairs(S, True) * B * Hq
    out = {"config": f"B={B} Hq={Hq} Hkv={Hkv} S={S} D={D} causal bf16 fwd, N(0,1) seed {seed}; "
                     f"{B * Hq * (S // 128)} query-block units",
           "workspace_bytes": nf}
    for label, split in (("split", True), ("unsplit", False)):
        def step(tm, i, split=split):
            if tm is not None:
                tm.mark(i, 0)
            lca.fwd(q, k, v, causal=True, scale=scale, out=o, lse=lse, workspace=fws if split else None,
                    split=split)
            if tm is not None:
                tm.mark(i, 1)
        ms, _ = run_steps(step, ["attn_fwd"], steps, warmup, SECONDARY_WARM_MS)
        tf = flops / (ms * 1e-3) / 1e12
        out[label] = {"ms": round(ms, 4), "tflops": round(tf, 2), "pct_of_peak": round(100.0 * tf / PEAK_BF16_TFLOPS, 2)}
    out["key_split"] = nf // (4 * B * Hq * S * (D + 1))  # workspace = ks partial O planes + ks row-stat planes
    return out


def ring_case(nchunk, steps, warmup, dev):
    """Ring-Attention forward of the gqa32k shape on one GPU, plus the merge kernel on its own.

    Query chunk r attends to key chunks 0..r (non-causal for c < r, causal for
    c = r), and each key chunk's result is folded into the query chunk's
    running fp32 result, in ring order: by attn_fwd_merge itself (the headline
    figure), and for comparison by attn_fwd followed by attn_merge. All
    chunks' work runs on this GPU, so the visible pairs are those of the full
    causal sequence. ``fwd_bwd`` adds the ring's backward: attn_bwd_accumulate
    on every (query chunk, key chunk) pair with the query chunk's final O and
    LSE, summing the gradients in fp32.
    """
    import torch
    import seeded_inputs as si
    import long_context_exact_fwd_amd as lca
    w = si.WORKLOADS["gqa32k"]
    x = si.workload_inputs(w, with_do=True)
    up = lca.bf16_from_bits
    q, k, v, do = up(x.q_bits, dev), up(x.k_bits, dev), up(x.v_bits, dev), up(x.do_bits, dev)
    B, S, Hq, D = q.shape
    L = S // nchunk
    qs = [q[:, r * L:(r + 1) * L].contiguous() for r in range(nchunk)]
    ks = [k[:, c * L:(c + 1) * L].contiguous() for c in range(nchunk)]
    vs = [v[:, c * L:(c + 1) * L].contiguous() for c in range(nchunk)]
    dos = [do[:, r * L:(r + 1) * L].contiguous() for r in range(nchunk)]
    del q, k, v, do
    po = torch.empty((B, L, Hq, D), dtype=torch.bfloat16, device=dev)
    pl = torch.empty((B, Hq, L), dtype=torch.float32, device=dev)
    o_acc = [torch.empty((B, L, Hq, D), dtype=torch.float32, device=dev) for _ in range(nchunk)]
    l_acc = [torch.empty((B, Hq, L), dtype=torch.float32, device=dev) for _ in range(nchunk)]
    o_out = [torch.empty((B, L, Hq, D), dtype=torch.bfloat16, device=dev) for _ in range(nchunk)]

    def step_fused(tm, i):
        if tm is not None:
            tm.mark(i, 0)
        for r in range(nchunk):
            for c in range(r + 1):
                lca.fwd_merge(qs[r], ks[c], vs[c], o_acc[r], l_acc[r], causal=(c == r), scale=w.scale,
                              accumulate=(c > 0), o_out=o_out[r] if c == r else None)
        if tm is not None:
            tm.mark(i, 1)

    def step(tm, i):
        if tm is not None:
            tm.mark(i, 0)
        for r in range(nchunk):
            for c in range(r + 1):
                lca.fwd(qs[r], ks[c], vs[c], causal=(c == r), scale=w.scale, out=po, lse=pl)
                lca.merge(o_acc[r], l_acc[r], po, pl, accumulate=(c > 0), o_out=o_out[r] if c == r else None)
        if tm is not None:
            tm.mark(i, 1)

    pairs = _pairs(S, True) * B * Hq
    # the ring's backward: fp32 gradient sums per chunk, the final O (bf16) and LSE of each query chunk
    dq_acc = [torch.empty((B, L, Hq, D), dtype=torch.float32, device=dev) for _ in range(nchunk)]
    dk_acc = [torch.empty(tuple(ks[0].shape), dtype=torch.float32, device=dev) for _ in range(nchunk)]
    dv_acc = [torch.empty(tuple(vs[0].shape), dtype=torch.float32, device=dev) for _ in range(nchunk)]
    bws = torch.empty((lca.bwd_workspace_bytes(B, Hq, w.hkv, L, D) + 3) // 4, dtype=torch.float32, device=dev)

    def step_fwd_bwd(tm, i):
        if tm is not None:
            tm.mark(i, 0)
        step_fused(None, i)
        if tm is not None:
            tm.mark(i, 1)
        for r in range(nchunk):
            # diagonal pair first: it is the first pair of query chunk r and (rows in order) of key chunk r,
            # so it writes the three sums and every other pair adds to them
            for c in range(r, -1, -1):
                lca.bwd_accumulate(qs[r], ks[c], vs[c], o_out[r], l_acc[r], dos[r], dq_acc[r], dk_acc[c], dv_acc[c],
                                   causal=(c == r), accumulate=(c != r), scale=w.scale, workspace=bws)
        if tm is not None:
            tm.mark(i, 2)

    ms_f, _ = run_steps(step_fused, ["ring_fwd_merge"], steps, warmup, SECONDARY_WARM_MS)
    tf_f = 4.0 * D * pairs / (ms_f * 1e-3) / 1e12
    ms_fb, per_fb = run_steps(step_fwd_bwd, ["ring_fwd_merge", "ring_bwd_accumulate"], steps, warmup,
                              SECONDARY_WARM_MS)
    tf_fb = 14.0 * D * pairs / (ms_fb * 1e-3) / 1e12
    del dq_acc, dk_acc, dv_acc, bws
    ms, _ = run_steps(step, ["ring_fwd"], steps, warmup, SECONDARY_WARM_MS)
    tf = 4.0 * D * pairs / (ms * 1e-3) / 1e12

    # the merge kernel alone: accumulate into chunk 0's running result, no bf16 copy
    reps = 50
    for _ in range(3):
        lca.merge(o_acc[0], l_acc[0], po, pl, accumulate=True)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        lca.merge(o_acc[0], l_acc[0], po, pl, accumulate=True)
    e1.record()
    torch.cuda.synchronize()
    m_ms = e0.elapsed_time(e1) / reps
    elems, rows = B * L * Hq * D, B * L * Hq
    m_bytes = elems * (4 + 2 + 4) + rows * (4 + 4 + 4)  # O_acc read + O_part read + O_acc write; 3 LSEs
    gbs = m_bytes / (m_ms * 1e-3) / 1e9
    return {
        "config": f"ring forward of gqa32k (B={B} Hq={Hq} Hkv={w.hkv} S={S} D={D} causal bf16) in {nchunk} chunks "
                  f"of {L}: attn_fwd_merge per (query chunk, key chunk <= it), all on one GPU, "
                  f"N(0,1) seed {w.seed}",
        "tflops": round(tf_f, 2), "pct_of_peak": round(100.0 * tf_f / PEAK_BF16_TFLOPS, 2),
        "peak_tflops": PEAK_BF16_TFLOPS, "ms_per_step": round(ms_f, 4), "steps": steps,
        "fwd_bwd": {"what": "the fused ring forward, then attn_bwd_accumulate per chunk pair (fp32 gradient sums)",
                    "tflops": round(tf_fb, 2), "pct_of_peak": round(100.0 * tf_fb / PEAK_BF16_TFLOPS, 2),
                    "ms_per_step": round(ms_fb, 4), "phases_ms": {n: round(t, 4) for n, t in per_fb.items()},
                    "flops": "14 D per visible pair, as the gqa32k step"},
        "unfused": {"what": "attn_fwd (bf16 partial O) + attn_merge per chunk pair", "tflops": round(tf, 2),
                    "pct_of_peak": round(100.0 * tf / PEAK_BF16_TFLOPS, 2), "ms_per_step": round(ms, 4)},
        "merge": {"kernel": "attn_merge_kernel", "bound": "hbm", "avg_launch_ms": round(m_ms, 5),
                  "algorithmic_bytes_per_launch": m_bytes, "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                  "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                  "shape": f"O [{B},{L},{Hq},{D}] fp32 running + bf16 part, accumulate"},
    }


def mfma_ceiling_case(dev, iters=40000, reps=5):
    """The bf16 matrix pipe's sustained rate on this GPU under a pure MFMA load, and its clock.

    Runs the probe of csrc/probe/mfma_ceiling.hip (one 8-wave workgroup per
    CU, 8 independent register-only v_mfma_f32_32x32x16_bf16 chains per wave)
    and times it with HIP events on the launch stream, once with N(0, 1)-like
    operands that change from one MFMA to the next (the figure the kernels
    compare with: their operands are such data) and once with constant
    low-entropy operands. The clock is the ratio of the shader-clock counter
    to the 100 MHz counter around each wave's loop (median over workgroups).
    """
    import ctypes
    import numpy as np
    import torch
    from long_context_exact_fwd_amd import build as bld
    lib = ctypes.CDLL(bld.PROBE_LIB)
    lib.mfma_ceiling_launch.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_void_p]
    lib.mfma_ceiling_launch.restype = ctypes.c_int
    lib.mfma_ceiling_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.mfma_ceiling_flops.restype = ctypes.c_double
    groups = torch.cuda.get_device_properties(dev).multi_processor_count
    out = torch.empty(groups * 512, dtype=torch.float32, device=dev)
    clocks = torch.zeros(2 * groups, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream(dev)

    def run(random_operands):
        def launch():
            rc = lib.mfma_ceiling_launch(ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(clocks.data_ptr()), groups,
                                         iters, int(random_operands), ctypes.c_void_p(stream.cuda_stream))
            if rc != 0:
                raise RuntimeError(f"mfma_ceiling_launch returned {rc}")

        launch()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            launch()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        tf = lib.mfma_ceiling_flops(groups, iters) / (ms * 1e-3) / 1e12
        ck = clocks.view(groups, 2).cpu().numpy().astype(np.float64)
        ghz = float(np.median(ck[:, 0] / np.maximum(ck[:, 1], 1.0))) * 0.1
        return {"ms": round(ms, 4), "tflops": round(tf, 1), "pct_of_peak": round(100.0 * tf / PEAK_BF16_TFLOPS, 2),
                "clock_ghz": round(ghz, 3)}

    res = {"what": f"register-only v_mfma_f32_32x32x16_bf16 loop, {groups} workgroups x 8 waves (2 per SIMD), "
                   f"8 chains x {iters} per wave, operands N(0,1)-like and different for every MFMA"}
    res.update(run(True))
    res["low_entropy_operands"] = run(False)
    return res


def build_info() -> dict:
    """How libmi355attn.so was compiled (the flags long_context_exact_fwd_amd/build.py passes to hipcc)."""
    from long_context_exact_fwd_amd import build as b
    flags = [f for f in b.CFLAGS if not f.startswith("-I") and not os.path.isabs(f) and "include" not in f]
    return {"compiler": os.path.basename(b.HIPCC), "arch": b.ARCH, "flags": " ".join(flags),
            "library": os.path.basename(b.LIB)}


def device_info(dev) -> dict:
    """What the HIP runtime reports for the device; the clock under load is measured by mfma_ceiling."""
    import torch
    pr = torch.cuda.get_device_properties(dev)
    return {"name": pr.name, "arch": getattr(pr, "gcnArchName", ""), "compute_units": pr.multi_processor_count,
            "memory_gib": round(pr.total_memory / 2 ** 30, 1), "torch": torch.__version__,
            "hip": getattr(torch.version, "hip", None)}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-sample-len", type=int, default=32768)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true", help="skip the mid / packed32k / fp8_64k measurements")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after the timed region, run one plain device copy of this many MiB (counter calibration)")
    a = ap.parse_args(argv)
    if a.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {a.gpus}); the kernels run one GPU's "
              f"head share and no collectives are implemented", file=sys.stderr)
        return 2

    import torch
    import seeded_inputs as si
    import long_context_exact_fwd_amd as lca

    lca.load_library()
    w = si.WORKLOADS["gqa32k"]
    x = si.workload_inputs(w)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    step, names = bf16_case(w, x, dev)
    t0 = time.perf_counter()
    ms_per_step, per = run_steps(step, names, a.steps, a.warmup)
    step_stats = run_steps.last_stats
    wall = time.perf_counter() - t0
    print(f"bench: {a.steps} timed steps done", file=sys.stderr, flush=True)

    D, Hq = w.head_dim, w.hq
    pairs = _pairs(w.seqlen, w.causal, x.cu_seqlens) * w.batch * Hq
    flops_k = {"attn_fwd": 4.0 * D * pairs, "bwd_delta": 0.0, "bwd_dkdv": 8.0 * D * pairs, "bwd_dq": 2.0 * D * pairs}
    value = 14.0 * D * pairs / (ms_per_step * 1e-3) / 1e12

    dom = max(("attn_fwd", "bwd_dkdv", "bwd_dq"), key=lambda n: per[n])
    achieved = flops_k[dom] / (per[dom] * 1e-3) / 1e12
    roofline = {
        "bound": "mfma",
        "kernel": KERNEL_OF_PHASE[dom],
        "achieved": round(achieved, 2),
        "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
        "traffic": _traffic(KERNEL_OF_PHASE[dom]),
        "avg_launch_ms": round(per[dom], 4),
        "algorithmic_flops_per_launch": flops_k[dom],
    }
    # every kernel of the step against its own bound: the three contractions
    # against the bf16 MFMA peak (dQ also with the 6 D flops per pair it
    # executes), Delta against HBM (read O and dO, write Delta and LSE*log2 e)
    rows = w.batch * w.seqlen * Hq
    delta_bytes = 2.0 * rows * D * 2 + 8.0 * rows
    per_kernel = {}
    for ph in ("attn_fwd", "bwd_dkdv", "bwd_dq"):
        tf = flops_k[ph] / (per[ph] * 1e-3) / 1e12
        per_kernel[KERNEL_OF_PHASE[ph]] = {"bound": "mfma", "avg_launch_ms": round(per[ph], 4),
                                           "achieved": round(tf, 2), "unit": "TFLOP/s",
                                           "frac": round(tf / PEAK_BF16_TFLOPS, 4)}
    dq_exec = 6.0 * D * pairs / (per["bwd_dq"] * 1e-3) / 1e12
    per_kernel[KERNEL_OF_PHASE["bwd_dq"]]["executed_frac"] = round(dq_exec / PEAK_BF16_TFLOPS, 4)
    gbs = delta_bytes / (per["bwd_delta"] * 1e-3) / 1e9
    per_kernel[KERNEL_OF_PHASE["bwd_delta"]] = {"bound": "hbm", "avg_launch_ms": round(per["bwd_delta"], 4),
                                                "achieved": round(gbs, 1), "unit": "GB/s",
                                                "frac": round(gbs / PEAK_HBM_GBS, 4)}

    if a.calib_copy_mib > 0:
        n = a.calib_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    result = {
        "metric": "attention TFLOP/s fwd+bwd (causal bf16, S=32K, D=128) and % of MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"gqa32k: B={w.batch} Hq={Hq} Hkv={w.hkv} S={w.seqlen} D={D} causal={w.causal} "
                        f"packed={w.packed}, N(0,1) seed {w.seed}",
            "batch": w.batch, "hq": Hq, "hkv": w.hkv, "seq_len": w.seqlen, "head_dim": D, "causal": w.causal,
        },
        "pct_of_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "phases_ms": {n: round(t, 4) for n, t in per.items()},
        "per_step_ms": step_stats,
        "wall_s_timed": round(wall, 3),
        "roofline": roofline,
        "kernels": per_kernel,
        "cpu_baseline": None,
        "workloads": None,
        "build": build_info(),
        "device": device_info(dev),
    }
    if not a.no_secondary:
        del step
        torch.cuda.empty_cache()
        sec_steps = max(3, min(10, a.steps))
        result["workloads"] = {}
        for name in ("mid", "packed32k", "fp8_64k"):
            result["workloads"][name] = secondary(name, sec_steps, min(2, a.warmup), dev)
            print(f"bench: {name} done", file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
        result["workloads"]["ring4_gqa32k"] = ring_case(4, sec_steps, min(2, a.warmup), dev)
        print("bench: ring4_gqa32k done", file=sys.stderr, flush=True)
        result["workloads"]["key_split_1h32k"] = key_split_case(sec_steps, min(2, a.warmup), dev)
        print("bench: key_split_1h32k done", file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
        result["workloads"]["fp8_64k_fwd_bwd"] = fp8_train_case(sec_steps, min(2, a.warmup), dev)
        print("bench: fp8_64k_fwd_bwd done", file=sys.stderr, flush=True)
        try:
            ceil = mfma_ceiling_case(dev)
        except (OSError, RuntimeError) as e:  # probe library missing or launch refused: no ceiling figure
            ceil = {"error": str(e)}
        result["mfma_ceiling"] = ceil
        if "tflops" in ceil:
            result["roofline"]["frac_of_mfma_ceiling"] = round(roofline["achieved"] / ceil["tflops"], 4)
        print("bench: mfma ceiling done", file=sys.stderr, flush=True)
    if not a.no_cpu_baseline:
        print("bench: timing the CPU oracle sample", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(w, x, a.cpu_sample_len)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
