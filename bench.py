#!/usr/bin/env python3
"""Benchmark of the gated delta-rule path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step is one pass of the whole hot path over one batch of synthetic input:
the chunked prefill of the Gated DeltaNet bf16 workload (B=8, H=16, T=4096,
d_k=d_v=128, chunk 64, random fp32 S0) followed by the first decode token on
the state it returns.  ``value`` is prefill throughput in tokens/s (B*T per
step).  The decode step's own throughput (GB/s against HBM peak) is measured
on the batch-64 x 16-head decode workload, 1024 steps captured in a HIP graph,
both in place on one state (as the recurrence runs) and rotated over 16 state
buffers so the 67 MB state cannot stay in the 256 MB Infinity Cache.  The
packed variable-length prefill (the same 32768 tokens x 16 heads split into 16
rows of 593 to 5858 tokens) is timed alongside (``packed``), and so is the
prefill with the per-token prologue fused in (``fused_prologue``: raw q and k
normalised in the kernels, beta and alpha from logits), and Gated DeltaNet-2
(``gdn2``: erase and write gates, per-channel decay) at the B=4, H=16, T=8192
shape, and the prefill backward (``backward``: all input gradients).

Printed: one JSON line (the contract below), preceded by progress lines on
stderr.  Peaks are MI355X's published figures: HBM 8 TB/s, dense bf16 MFMA
2.5 PFLOP/s.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import gated_delta_rule_04_amd as gdn  # noqa: E402
import workloads as W  # noqa: E402

METRIC = "prefill tokens/s + % bf16 MFMA peak; decode step GB/s + % HBM peak (1 GPU)"
HBM_PEAK_GBPS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
CHUNK = 64
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefill_gdn_bf16_b8_h16_t4096_d128_traffic.json")
KERNEL_SOURCES = [os.path.join(ROOT, "gated_delta_rule_04_amd", "csrc", f)
                  for f in ("gdn_chunk.hip", "gdn_mfma.h", "gdn_internal.h", "gdn_solve.h")]


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


# ------------------------------------------------------------------------------
# algorithmic work (per launch), independent of how the kernels do it
# ------------------------------------------------------------------------------

def prefill_bytes(w: W.Prefill) -> int:
    """Every input read once and every output written once."""
    es = 2 if w.dtype == torch.bfloat16 else 4
    tok = w.B * w.T * w.H
    b = tok * (2 * w.dk + 2 * w.dv) * es          # q, k, v, o
    b += tok * 4                                   # beta
    if w.mode == W.MODE_SCALAR:
        b += tok * 4
    elif w.mode == W.MODE_CHANNEL:
        b += tok * w.dk * es
    state = w.B * w.H * w.dv * w.dk * 4
    b += state * (2 if w.s0_std > 0 else 1)        # S0 (if given) + S_final
    return b


def prefill_flops(w: W.Prefill, dense: bool) -> float:
    """Per token-head: the five C x C-sized products (A, W-or-X side, U, Q K^T,
    P U) at half size (causal) or full tile size (dense), the three state
    contractions and the triangular solve, FLOP = 2 MAC."""
    C, dk, dv = CHUNK, w.dk, w.dv
    tri = 1.0 if dense else 0.5
    per = 2.0 * (tri * C * (3 * dk + 2 * dv) + 3 * dk * dv + C * C / 6.0)
    return per * w.B * w.T * w.H


def decode_bytes(w: W.Decode) -> int:
    es = 2 if w.dtype == torch.bfloat16 else 4
    heads = w.B * w.H
    b = 2 * heads * w.dv * w.dk * 4                   # state read + write
    b += heads * (2 * w.dk + 2 * w.dv) * es           # q, k, v, o
    b += heads * 4 * (2 if w.mode == W.MODE_SCALAR else 1)
    if w.mode == W.MODE_CHANNEL:
        b += heads * w.dk * es
    return b


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per prefill launch from the committed rocprofv3 counter summary,
    or None when it is absent or was taken on a different kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


# ------------------------------------------------------------------------------
# GPU measurements
# ------------------------------------------------------------------------------

def bench_step(w: W.Prefill, steps: int, warmup: int):
    """Time exactly ``steps`` steps (prefill + first decode token), each prefill
    launch bracketed by HIP events on the stream it runs on.  Then the average
    duration of one prefill launch: ``steps`` launches back to back between one
    pair of events, queued behind a running launch (an event pair around every
    launch also counts the idle time of the marker packets, some 15-20 us)."""
    log("generating %s" % w.name)
    host = W.make_prefill(w)
    dev = {k: (None if v is None else v.cuda()) for k, v in host.items()}
    tok = W.make_decode(W.Decode("next_token", w.B, w.H, w.dk, w.dv, 1, w.dtype, w.gate, 0.0,
                                 seed=w.seed + 100))
    tdev = {k: (None if v is None else v.cuda()) for k, v in tok.items()}
    o = torch.empty((w.B, w.T, w.H, w.dv), dtype=w.dtype, device="cuda")
    S = torch.empty((w.B, w.H, w.dv, w.dk), dtype=torch.float32, device="cuda")
    o1 = torch.empty((w.B, w.H, w.dv), dtype=w.dtype, device="cuda")
    a1 = None if tdev["alpha"] is None else tdev["alpha"][0]

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        gdn.chunk_fwd(dev["q"], dev["k"], dev["v"], dev["alpha"], dev["beta"], dev["S0"],
                      mode=w.mode, o=o, S_final=S)
        if ev is not None:
            ev[1].record()
        gdn.decode_step(tdev["q"][0], tdev["k"][0], tdev["v"][0], a1, tdev["beta"][0], S, o=o1,
                        mode=w.mode)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = sorted(e0.elapsed_time(e1) for e0, e1 in evs)

    def prefill():
        gdn.chunk_fwd(dev["q"], dev["k"], dev["v"], dev["alpha"], dev["beta"], dev["S0"],
                      mode=w.mode, o=o, S_final=S)

    b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    prefill()                       # keeps the GPU busy while the timed launches are queued
    b0.record()
    for _ in range(steps):
        prefill()
    b1.record()
    torch.cuda.synchronize()
    launch_ms = b0.elapsed_time(b1) / steps

    # Cold last-level cache (256 MB on MI355X): before every launch a 512 MB
    # write and a read of the same 512 MB (so none of the write's dirty lines
    # drain during the launch), outside an event pair around the launch.  Its
    # median compares with the warm launches' median under the same kind of
    # event pair (step_events_us_median), which counts the marker packets too.
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    reps = max(5, steps // 2)
    cev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for i in range(reps):
        scratch.fill_(i & 255)
        scratch.sum(dtype=torch.int32)
        cev[i][0].record()
        prefill()
        cev[i][1].record()
    torch.cuda.synchronize()
    cold_ms = sorted(e0.elapsed_time(e1) for e0, e1 in cev)[reps // 2]
    del scratch
    # outputs of the last launch, for the parity spot check against the oracle
    return dict(wall_s=wall, kernel_ms=kern_ms, launch_ms=launch_ms, cold_ms=cold_ms, host=host, o=o,
                S=S)


def packed_bytes(w: W.Packed) -> int:
    """Algorithmic bytes of a packed prefill: the rows' tokens as one row, plus
    one initial (if given) and one final state per sequence."""
    rows = prefill_bytes(W.Prefill(w.name, 1, w.H, w.T, w.dk, w.dv, w.dtype, w.gate, 0.0, w.seed))
    rows -= w.H * w.dv * w.dk * 4                                   # the single row's S_final
    return rows + w.N * w.H * w.dv * w.dk * 4 * (2 if w.s0_std > 0 else 1) + (w.N + 1) * 4


def bench_packed(w: W.Packed, steps: int):
    """Average duration of one ``gdn_chunk_fwd_varlen`` launch: ``steps``
    launches back to back between one event pair, behind a running launch."""
    log("generating %s" % w.name)
    host = W.make_packed(w)
    d = {k: (None if v is None else v.cuda()) for k, v in host.items()}
    o = torch.empty((1, w.T, w.H, w.dv), dtype=w.dtype, device="cuda")
    S = torch.empty((w.N, w.H, w.dv, w.dk), dtype=torch.float32, device="cuda")

    def launch():
        gdn.chunk_fwd_varlen(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["cu_seqlens"],
                             d["S0"], mode=w.mode, o=o, S_final=S)

    for _ in range(3):
        launch()
    torch.cuda.synchronize()
    b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    launch()
    b0.record()
    for _ in range(steps):
        launch()
    b1.record()
    torch.cuda.synchronize()
    ms = b0.elapsed_time(b1) / steps
    nbytes = packed_bytes(w)
    lens = W.packed_lengths(w)
    return dict(workload=w.name, N=w.N, T=w.T, H=w.H, lengths_min=min(lens), lengths_max=max(lens),
                launch_us=ms * 1e3, tokens_per_s=w.T / (ms * 1e-3),
                hbm_gbps=nbytes / (ms * 1e-3) / 1e9, hbm_frac=nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                algorithmic_bytes=nbytes)


def bench_fused(w: W.Prefill, steps: int):
    """Average duration of one ``gdn_chunk_fwd_fused`` launch on raw inputs of
    the workload's shape (q, k not normalised, beta and alpha logits, per-head
    rates and biases), every part of the prologue on; timed in alternation
    with the plain call on the workload's own inputs (three rounds each, mean),
    so that both see the same clock."""
    log("generating raw inputs for the fused prologue (%s shape)" % w.name)
    d = {k: (None if v is None else v.cuda()) for k, v in
         W.make_prologue(w.B, w.T, w.H, w.dk, w.dv, w.dtype, w.mode, seed=w.seed + 200,
                         s0_std=w.s0_std).items()}
    p = {k: (None if v is None else v.cuda()) for k, v in W.make_prefill(w).items()}
    o = torch.empty((w.B, w.T, w.H, w.dv), dtype=w.dtype, device="cuda")
    S = torch.empty((w.B, w.H, w.dv, w.dk), dtype=torch.float32, device="cuda")

    def fused():
        gdn.chunk_fwd_fused(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], mode=w.mode,
                            l2norm_qk=True, beta_logits=True, alpha_logits=True, A=d["A"],
                            dt_bias=d["dt_bias"], o=o, S_final=S)

    def plain():
        gdn.chunk_fwd(p["q"], p["k"], p["v"], p["alpha"], p["beta"], p["S0"], mode=w.mode,
                      o=o, S_final=S)

    def timed(f):
        b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        f()
        b0.record()
        for _ in range(steps):
            f()
        b1.record()
        torch.cuda.synchronize()
        return b0.elapsed_time(b1) / steps

    for _ in range(3):
        fused()
        plain()
    torch.cuda.synchronize()
    tf, tp = [], []
    for r in range(6):
        order = (fused, plain) if r % 2 == 0 else (plain, fused)
        for f in order:
            (tf if f is fused else tp).append(timed(f))
    ms, ms_plain = sum(tf) / len(tf), sum(tp) / len(tp)
    nbytes = prefill_bytes(w) + w.H * 4 * (2 if w.mode == W.MODE_SCALAR else 1 + w.dk)
    return dict(workload=w.name + "_fused_prologue", launch_us=ms * 1e3,
                plain_launch_us_same_period=ms_plain * 1e3,
                tokens_per_s=w.B * w.T / (ms * 1e-3), hbm_gbps=nbytes / (ms * 1e-3) / 1e9,
                hbm_frac=nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, algorithmic_bytes=nbytes)


def bench_gdn2(w: W.Prefill, steps: int):
    """Average duration of one ``gdn2_chunk_fwd`` launch (erase and write gates)
    at the shape and per-channel decay of ``w``."""
    log("generating Gated DeltaNet-2 inputs (%s shape)" % w.name)
    d = {k: (None if v is None else v.cuda()) for k, v in W.make_gdn2(w.with_(seed=w.seed + 300)).items()}
    o = torch.empty((w.B, w.T, w.H, w.dv), dtype=w.dtype, device="cuda")
    S = torch.empty((w.B, w.H, w.dv, w.dk), dtype=torch.float32, device="cuda")

    def launch():
        gdn.gdn2_chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["erase"], d["write"], d["S0"],
                           o=o, S_final=S)

    for _ in range(3):
        launch()
    torch.cuda.synchronize()
    b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    launch()
    b0.record()
    for _ in range(steps):
        launch()
    b1.record()
    torch.cuda.synchronize()
    ms = b0.elapsed_time(b1) / steps
    es = 2 if w.dtype == torch.bfloat16 else 4
    tok = w.B * w.T * w.H
    nbytes = prefill_bytes(w) - tok * 4 + tok * (w.dk + w.dv) * es   # gates instead of beta
    del d
    return dict(workload="gdn2_" + w.name, launch_us=ms * 1e3, tokens_per_s=w.B * w.T / (ms * 1e-3),
                hbm_gbps=nbytes / (ms * 1e-3) / 1e9, hbm_frac=nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                algorithmic_bytes=nbytes)


def bench_backward(w: W.Prefill, steps: int):
    """Average duration of one ``gdn_chunk_bwd`` launch on the workload's inputs
    with a random output gradient (and final-state gradient)."""
    log("backward inputs (%s)" % w.name)
    d = {k: (None if v is None else v.cuda()) for k, v in W.make_prefill(w).items()}
    g = torch.Generator().manual_seed(w.seed + 400)
    do = torch.randn(w.B, w.T, w.H, w.dv, generator=g).to(w.dtype).cuda()
    dST = torch.randn(w.B, w.H, w.dv, w.dk, generator=g).cuda()

    def launch():
        gdn.chunk_bwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], do, dST, mode=w.mode)

    launch()
    torch.cuda.synchronize()
    n = max(2, steps // 4)
    b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    launch()
    b0.record()
    for _ in range(n):
        launch()
    b1.record()
    torch.cuda.synchronize()
    ms = b0.elapsed_time(b1) / n
    es = 2 if w.dtype == torch.bfloat16 else 4
    tok = w.B * w.T * w.H
    state = w.B * w.H * w.dv * w.dk * 4
    nbytes = 2 * prefill_bytes(w) + tok * w.dv * es + state   # inputs + dout, dS_final; the same again out
    return dict(workload=w.name + "_backward", launch_us=ms * 1e3, launches=n,
                tokens_per_s=w.B * w.T / (ms * 1e-3), hbm_gbps=nbytes / (ms * 1e-3) / 1e9,
                hbm_frac=nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, algorithmic_bytes=nbytes)


def bench_decode(w: W.Decode, reps: int = 3, rotate: int = 1):
    """``w.steps`` decode steps captured in one HIP graph; per-step time from
    the median replay.  ``rotate`` > 1 cycles the steps over that many state
    buffers (HBM-resident working set)."""
    inp = W.make_decode(w)
    d = {k: (None if v is None else v.cuda()) for k, v in inp.items() if k != "S"}
    states = [inp["S"].cuda() for _ in range(rotate)]
    o = torch.empty((w.steps, w.B, w.H, w.dv), dtype=w.dtype, device="cuda")

    def run_all():
        for t in range(w.steps):
            a = None if d["alpha"] is None else d["alpha"][t]
            gdn.decode_step(d["q"][t], d["k"][t], d["v"][t], a, d["beta"][t], states[t % rotate],
                            o=o[t], mode=w.mode)

    run_all()                                  # eager warm-up
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=side):
        run_all()
    g.replay()
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) / w.steps)
    del g
    ms = sorted(times)[len(times) // 2]
    gb = decode_bytes(w) / (ms * 1e-3) / 1e9
    return dict(us_per_step=ms * 1e3, gbps=gb, hbm_frac=gb / HBM_PEAK_GBPS)


def device_copy_gbps(nbytes=1 << 30):
    """Plain device-to-device copy of 1 GiB (read + write), five launches: the
    achievable-bandwidth reference, and the known-size kernel that scales the
    HBM byte counters (FETCH_SIZE / WRITE_SIZE) of a counter run."""
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").uniform_()
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 5
    return 2 * nbytes / (ms * 1e-3) / 1e9


# ------------------------------------------------------------------------------
# CPU baseline: the fp64 oracle on a bounded sample of the same workload
# ------------------------------------------------------------------------------

def cpu_baseline(w: W.Prefill, host, o_gpu, S_gpu, budget_s: float = 12.0):
    """The oracle over batch rows of the same input, as many rows as fit in about
    ``budget_s`` seconds; when the whole batch takes less, whole-batch passes are
    repeated until the budget is used (at least one pass), so the rate is a
    steady one.  Also checks the GPU's outputs of those rows against it."""
    import numpy as np
    import oracle  # test infrastructure: used only for this baseline leg
    threads = oracle.num_threads()

    def rows(lo, hi):
        return {k: (None if v is None else v[lo:hi]) for k, v in host.items()}

    t0 = time.perf_counter()
    ro, rS = oracle.gdn_fwd(**rows(0, 1), mode=w.mode)
    t1 = time.perf_counter() - t0
    n, secs, passes = 1, t1, 1
    extra = int(max(0, min(w.B - 1, budget_s / max(t1, 1e-3) - 1)))
    if extra > 0:
        t0 = time.perf_counter()
        ro2, rS2 = oracle.gdn_fwd(**rows(1, 1 + extra), mode=w.mode)
        secs += time.perf_counter() - t0
        ro, rS = np.concatenate([ro, ro2]), np.concatenate([rS, rS2])
        n = 1 + extra
    toks = n * w.T
    if n == w.B:
        while secs < budget_s:      # the whole batch is quick: repeat it
            t0 = time.perf_counter()
            oracle.gdn_fwd(**rows(0, n), mode=w.mode)
            secs += time.perf_counter() - t0
            toks += n * w.T
            passes += 1
    og = o_gpu[:n].float().cpu().numpy()
    Sg = S_gpu[:n].cpu().numpy()
    parity = dict(rel_err_o=W.per_head_rel_err(og, ro, (0, 2)),
                  rel_err_S=W.per_head_rel_err(Sg, rS, (0, 1)), rows_checked=n)
    what = ("%d pass(es) over all %d batch rows" % (passes, n) if n == w.B else
            "batch rows 0..%d (%d of %d)" % (n - 1, n, w.B))
    base = dict(value=toks / secs, unit="tokens/s", cores=threads, kind="oracle",
                sample="fp64 token loop, %s, all %d heads, T=%d: %d tokens in %.1f s on %d threads"
                       % (what, w.H, w.T, toks, secs, threads))
    return base, parity


# ------------------------------------------------------------------------------
# rocprofv3 output -> committed summaries (runs on any host, reads CSV files)
# ------------------------------------------------------------------------------

def _csv_rows(path):
    import csv
    import glob
    out = []
    for f in sorted(glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True)):
        with open(f) as fh:
            out += list(csv.DictReader(fh))
    return out


def _per_dispatch(rows, counter):
    per = {}
    for r in rows:
        if r["Counter_Name"] == counter:
            key = (int(r["Dispatch_Id"]), r["Kernel_Name"])
            per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    return per


def summarize_pmc(fetch_dir, write_dir, out_json):
    """HBM bytes per prefill launch from a FETCH_SIZE run and a WRITE_SIZE run of
    this script (KiB per dispatch), each scaled by what the counter reads for the
    1 GiB device copy that the same run performs."""
    fetch = _per_dispatch(_csv_rows(fetch_dir), "FETCH_SIZE")
    write = _per_dispatch(_csv_rows(write_dir), "WRITE_SIZE")
    copy_kib = (1 << 30) / 1024.0

    def copy_scale(per):
        vals = [v for (d, k), v in per.items() if "copyBuffer" in k and v > 0.25 * copy_kib]
        return copy_kib / (sum(vals) / len(vals))

    def kernel_kib(per, name):
        vals = [v for (d, k), v in per.items() if name in k]
        return sum(vals) / len(vals), len(vals)

    fs, ws = copy_scale(fetch), copy_scale(write)
    rec = dict(kernel_source_sha256=kernel_source_hash(), fetch_scale=fs, write_scale=ws,
               note="FETCH_SIZE / WRITE_SIZE KiB per dispatch, scaled so the 1 GiB device "
                    "copy reads 1 GiB and writes 1 GiB")
    total = 0.0
    # the two kernels of one gdn_chunk_fwd call on the bf16 d_k = 128 scalar-decay
    # workload (mangled names: bf16, d_k 128, scalar decay, no normalisation; the
    # state kernel with 64-row value slices)
    kernels = (("chunk_prep", "chunk_prep_kernelIDF16bLi128ELi1ELb0E"),
               ("chunk_state", "chunk_state_wsIDF16bLi128ELi64ELi1ELb0E"))
    for name, mangled in kernels:
        fk, nf = kernel_kib(fetch, mangled)
        wk, nw = kernel_kib(write, mangled)
        rec[name] = dict(fetch_kib=fk, write_kib=wk, dispatches=[nf, nw],
                         hbm_read_bytes=fk * 1024 * fs, hbm_write_bytes=wk * 1024 * ws)
        total += fk * 1024 * fs + wk * 1024 * ws
    rec["hbm_bytes_per_launch"] = total
    with open(out_json, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1))


# ------------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=W.GDN_BF16_PREFILL.name,
                    choices=[w.name for w in W.PREFILL_WORKLOADS])
    ap.add_argument("--no-decode", action="store_true", help="skip the decode workload")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle baseline")
    ap.add_argument("--no-packed", action="store_true",
                    help="skip the packed variable-length prefill workload")
    ap.add_argument("--no-fused", action="store_true",
                    help="skip the prefill with the fused per-token prologue")
    ap.add_argument("--no-gdn2", action="store_true",
                    help="skip the Gated DeltaNet-2 prefill")
    ap.add_argument("--no-backward", action="store_true", help="skip the prefill backward")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the HBM-traffic summary from two rocprofv3 --pmc runs and exit")
    args = ap.parse_args()
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], TRAFFIC_FILE)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build runs the path on a single MI355X "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    gdn.load()
    w = next(x for x in W.PREFILL_WORKLOADS if x.name == args.workload)

    r = bench_step(w, args.steps, args.warmup)
    ms_step = r["wall_s"] * 1e3 / args.steps
    ev_ms = r["kernel_ms"][len(r["kernel_ms"]) // 2]
    kern_ms = r["launch_ms"]
    tokens = w.B * w.T
    nbytes, f_c, f_d = prefill_bytes(w), prefill_flops(w, False), prefill_flops(w, True)
    log("prefill launch %.1f us (mean of %d back to back; %.1f us median with an event pair "
        "per step), step %.3f ms" % (kern_ms * 1e3, args.steps, ev_ms * 1e3, ms_step))

    log("prefill launch with an event pair: %.1f us (median) warm, %.1f us on a cold last-level cache"
        % (ev_ms * 1e3, r["cold_ms"] * 1e3))
    prefill = dict(launch_us=kern_ms * 1e3, step_events_us_median=ev_ms * 1e3,
                   cold_cache_events_us_median=r["cold_ms"] * 1e3,
                   tokens_per_s_kernel=tokens / (kern_ms * 1e-3),
                   tflops_causal=f_c / (kern_ms * 1e-3) / 1e12,
                   mfma_frac_causal=f_c / (kern_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                   tflops_dense=f_d / (kern_ms * 1e-3) / 1e12,
                   mfma_frac_dense=f_d / (kern_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                   hbm_gbps=nbytes / (kern_ms * 1e-3) / 1e9,
                   hbm_frac=nbytes / (kern_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                   algorithmic_bytes=nbytes, flops_causal=f_c, flops_dense=f_d)
    traffic = measured_traffic() if w.name == W.GDN_BF16_PREFILL.name else None
    prep = "chunk_prep_kda" if w.mode == W.MODE_CHANNEL else "chunk_prep_kernel"
    state = "chunk_state_ws" if w.dtype == torch.bfloat16 else "chunk_state_kernel"
    roofline = dict(bound="hbm", achieved=nbytes / (kern_ms * 1e-3) / 1e9,
                    peak=HBM_PEAK_GBPS, unit="GB/s",
                    frac=nbytes / (kern_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                    traffic=traffic,
                    kernel="gdn_chunk_fwd launch: %s + %s" % (prep, state),
                    launch_us=kern_ms * 1e3)

    decode = None
    if not args.no_decode:
        decode = {}
        for dw in W.DECODE_WORKLOADS:
            lit = bench_decode(dw, rotate=1)
            rot = bench_decode(dw, rotate=16)
            decode[dw.name] = dict(bytes_per_step=decode_bytes(dw),
                                   in_place=lit, rotated_16_states=rot)
            log("decode %s: in place %.2f us/step %.0f GB/s; rotated %.2f us/step %.0f GB/s" % (
                dw.name, lit["us_per_step"], lit["gbps"], rot["us_per_step"], rot["gbps"]))

    packed = None
    if not args.no_packed:
        packed = bench_packed(W.GDN_BF16_PACKED, args.steps)
        log("packed %s: %.1f us per launch, %.3g tokens/s (rows %d..%d tokens)" % (
            packed["workload"], packed["launch_us"], packed["tokens_per_s"], packed["lengths_min"],
            packed["lengths_max"]))

    fused = None
    if not args.no_fused and w.mode != W.MODE_NONE:
        fused = bench_fused(w, args.steps)
        log("fused prologue: %.1f us per launch (plain call in alternation: %.1f us)" % (
            fused["launch_us"], fused["plain_launch_us_same_period"]))

    gdn2 = None
    if not args.no_gdn2:
        gdn2 = bench_gdn2(W.KDA_BF16_PREFILL, args.steps)
        log("gated deltanet-2 %s: %.1f us per launch" % (gdn2["workload"], gdn2["launch_us"]))

    bwd = None
    if not args.no_backward:
        bwd = bench_backward(w, args.steps)
        log("backward: %.1f us per launch" % bwd["launch_us"])

    copy_gbps = device_copy_gbps()   # also the known-size reference for HBM byte counters
    log("device copy %.0f GB/s" % copy_gbps)

    base, parity = None, None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        base, parity = cpu_baseline(w, r["host"], r["o"], r["S"])
        prefill.update(parity)
        log("oracle %.0f tokens/s; parity o %.2e S %.2e" % (base["value"], parity["rel_err_o"],
                                                          parity["rel_err_S"]))

    out = dict(metric=METRIC, value=tokens / (ms_step * 1e-3), unit="tokens/s", n_gpus=1,
               steps=args.steps, warmup=args.warmup, ms_per_step=ms_step, higher_is_better=True,
               scaling="weak", vs_baseline=None,
               dtype="bf16" if w.dtype == torch.bfloat16 else "f32", data="synthetic",
               config=dict(workload=w.name, B=w.B, H=w.H, T=w.T, dk=w.dk, dv=w.dv, chunk=CHUNK,
                           decay={0: "none", 1: "scalar", 2: "channel"}[w.mode],
                           step="chunked prefill + first decode token",
                           state="fp32", parallelism="single GPU"),
               roofline=roofline, cpu_baseline=base, prefill=prefill, decode=decode, packed=packed,
               fused_prologue=fused, gdn2=gdn2, backward=bwd,
               device_copy_gbps=copy_gbps)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
