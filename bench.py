#!/usr/bin/env python3
"""Benchmark of the gated delta-rule path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step is one pass of the whole hot path over one batch of synthetic input:
the chunked prefill of the long-context Gated DeltaNet workload (B=1, H=32,
T=65536, d_k=d_v=128, bf16 inputs, fp32 state, chunk 64: the largest of the
workloads that fits one GPU) followed by the first decode token on the state
it returns.  ``value`` is prefill throughput in tokens/s (B*T per step, whole
step time), measured over exactly K steps after W warm-up steps.

Every prefill workload is also timed on its own (section ``prefill``) with
the protocol of the state-reduction notes' efficiency section: 10 warm-up
launches, 100 timed launches, 3 trials, median of the trial medians.  Two
figures per workload: ``cold`` (each launch preceded by a 512 MB write and a
read of the same 512 MB outside its HIP-event pair, so the 256 MB Infinity
Cache holds none of its inputs: the headline) and ``warm`` (100 launches back
to back between one event pair, queued behind a running launch).  Each
section carries tokens/s, % of HBM peak on the algorithmic bytes, % of bf16
MFMA peak under the causal and the dense-tile FLOP count, the
attainable-roofline fraction, the SHA-256 of every input buffer and a parity
check of all heads against the fp64 oracle.  The decode step (batch 64 x 16
heads, d_k 128 and 64) runs 1024 steps captured in one HIP graph, in place and
rotated over 16 state buffers (HBM-resident), 3 replays.  The packed
variable-length prefill, the fused prologue, Gated DeltaNet-2 and the
backward are timed alongside.

Printed: one JSON line (the contract below), preceded by progress lines on
stderr.  Peaks are MI355X's published figures: HBM 8 TB/s, dense bf16 MFMA
2.5 PFLOP/s.

Profiling helpers (no timing JSON):
    python bench.py --profile NAME [--reps N]     run one workload N times (for rocprofv3)
    python bench.py --summarize-pmc DIR NAME      counter summary of such a run -> JSON
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import platform
import statistics
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
NUM_SIMDS = 1024          # 256 compute units x 4 SIMDs
NUM_XCDS = 8
CHUNK = 64
COUNTER_FILE = os.path.join(ROOT, "profiles", "counters.json")
_CSRC = os.path.join(ROOT, "gated_delta_rule_04_amd", "csrc")
# The sources the kernels of a workload are compiled from: a workload's counters
# are valid while these files are unchanged.
PREFILL_SOURCES = [os.path.join(_CSRC, f) for f in ("gdn_chunk.hip", "gdn_mfma.h", "gdn_internal.h",
                                                     "gdn_solve.h")]
DECODE_SOURCES = [os.path.join(_CSRC, f) for f in ("gdn_decode.hip", "gdn_internal.h")]
# the backward also runs the prefill's prep kernel
BACKWARD_SOURCES = PREFILL_SOURCES + [os.path.join(_CSRC, f) for f in ("gdn_bwd_chunk.hip", "gdn_backward.h")]
EPILOGUE_SOURCES = [os.path.join(_CSRC, f) for f in ("gdn_epilogue.hip", "gdn_internal.h")]
HEADLINE = W.GDN_BF16_LONG
PROTOCOL = dict(trials=3, warmup=10, reps=100)


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
    """Per token-head: the five C x C-sized products (A, the write error's key
    side, U, Q K^T, P U) at half size (causal) or full tile size (dense), the
    three state contractions and the triangular solve, FLOP = 2 MAC."""
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


def kernel_source_hash(name: str) -> str:
    """SHA-256 of the kernel sources workload ``name`` runs (decode, prefill,
    backward or the output epilogue)."""
    h = hashlib.sha256()
    srcs = (DECODE_SOURCES if name.startswith("decode") else BACKWARD_SOURCES if name.endswith("_backward")
            else EPILOGUE_SOURCES if name.endswith("_gated_rmsnorm") else PREFILL_SOURCES)
    for p in srcs:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def committed_counters(name):
    """Counter summary of workload ``name`` from profiles/counters.json, or None
    when it is absent or was taken on a different kernel source."""
    try:
        with open(COUNTER_FILE) as f:
            rec = json.load(f).get(name)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("kernel_source_sha256") != kernel_source_hash(name):
        return None
    return rec


def host_info():
    model = platform.processor() or "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return dict(cpu_model=model, cpus_in_affinity=len(os.sched_getaffinity(0)))


def sha256_inputs(host):
    return {k: W.sha256(v) for k, v in host.items() if v is not None}


# ------------------------------------------------------------------------------
# GPU timing
# ------------------------------------------------------------------------------

def _events(n):
    return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(n)]


def timing_protocol(launch, scratch, trials=3, warmup=10, reps=100):
    """Per trial: ``warmup`` launches, then ``reps`` launches back to back
    between one event pair (warm, mean per launch), then ``reps`` launches each
    after a write and a read of the whole ``scratch`` buffer, each between its
    own event pair (cold, median).  Returns both figures as the median over the
    trials, with every trial's value."""
    warm, cold = [], []
    for _ in range(trials):
        for _ in range(warmup):
            launch()
        b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        launch()                       # keeps the GPU busy while the timed launches queue
        b0.record()
        for _ in range(reps):
            launch()
        b1.record()
        torch.cuda.synchronize()
        warm.append(b0.elapsed_time(b1) / reps * 1e3)
        ev = _events(reps)
        for i in range(reps):
            scratch.fill_(i & 255)
            scratch.view(torch.int64).sum()
            ev[i][0].record()
            launch()
            ev[i][1].record()
        torch.cuda.synchronize()
        cold.append(statistics.median(e0.elapsed_time(e1) * 1e3 for e0, e1 in ev))
    return dict(cold_us=statistics.median(cold), cold_trials_us=cold,
                warm_us=statistics.median(warm), warm_trials_us=warm,
                protocol="%d trials x (%d warm-up, %d timed launches); cold: event pair per "
                         "launch after a %d MB write + read, median; warm: back to back, mean"
                         % (trials, warmup, reps, scratch.numel() >> 20))


class PrefillRun:
    """Device copies of a prefill workload's inputs and its output buffers."""

    def __init__(self, w: W.Prefill, host):
        self.w = w
        self.dev = {k: (None if v is None else v.cuda()) for k, v in host.items()}
        self.o = torch.empty((w.B, w.T, w.H, w.dv), dtype=w.dtype, device="cuda")
        self.S = torch.empty((w.B, w.H, w.dv, w.dk), dtype=torch.float32, device="cuda")
        ws = gdn.workspace_bytes(w.B, w.T, w.H, w.dk, w.dv, w.dtype, w.mode)
        self.ws = torch.empty(ws, dtype=torch.uint8, device="cuda") if ws else None

    def __call__(self):
        d = self.dev
        gdn.chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], mode=self.w.mode,
                      o=self.o, S_final=self.S, workspace=self.ws)


def derived(w: W.Prefill, us: float):
    nbytes, f_c, f_d = prefill_bytes(w), prefill_flops(w, False), prefill_flops(w, True)
    s = us * 1e-6
    t_roof = max(f_c / (BF16_PEAK_TFLOPS * 1e12), nbytes / (HBM_PEAK_GBPS * 1e9))
    return dict(launch_us=us, tokens_per_s=w.B * w.T / s,
                hbm_gbps=nbytes / s / 1e9, hbm_frac=nbytes / s / 1e9 / HBM_PEAK_GBPS,
                tflops_causal=f_c / s / 1e12, mfma_frac_causal=f_c / s / 1e12 / BF16_PEAK_TFLOPS,
                tflops_dense=f_d / s / 1e12, mfma_frac_dense=f_d / s / 1e12 / BF16_PEAK_TFLOPS,
                attainable_frac=t_roof / s)


def parity(w: W.Prefill, host, o_gpu, S_gpu, ref=None):
    """All heads of o and S_final against the fp64 oracle (per-(b, h) slice
    max|x - r| / max|r|, worst slice)."""
    import oracle  # test infrastructure: the baseline and parity leg only
    if ref is None:
        ref = oracle.gdn_fwd(host["q"], host["k"], host["v"], host["alpha"], host["beta"],
                             host["S0"], mode=w.mode)
    ro, rS = ref
    tol = 1e-4 if w.dtype == torch.float32 else 2e-2
    e_o = W.per_head_rel_err(o_gpu.float().numpy(), ro, (0, 2))
    e_S = W.per_head_rel_err(S_gpu.numpy(), rS, (0, 1))
    return dict(rel_err_o=e_o, rel_err_S=e_S, tolerance=tol, heads_checked=w.B * w.H,
                ok=bool(e_o <= tol and e_S <= tol))


def bench_prefill(w: W.Prefill, scratch, with_parity=True, keep=False):
    log("prefill %s: generating inputs" % w.name)
    host = W.make_prefill(w)
    hashes = sha256_inputs(host)
    run = PrefillRun(w, host)
    log("prefill %s: timing (%s)" % (w.name, PROTOCOL))
    t = timing_protocol(run, scratch, **PROTOCOL)
    sec = dict(workload=w.name, B=w.B, H=w.H, T=w.T, dk=w.dk, dv=w.dv,
               dtype="bf16" if w.dtype == torch.bfloat16 else "f32",
               decay={0: "none", 1: "scalar", 2: "channel"}[w.mode],
               algorithmic_bytes=prefill_bytes(w), flops_causal=prefill_flops(w, False),
               flops_dense=prefill_flops(w, True), timing=t,
               cold=derived(w, t["cold_us"]), warm=derived(w, t["warm_us"]),
               input_sha256=hashes)
    c = committed_counters(w.name)
    if c:
        sec["counters"] = c
    log("prefill %s: cold %.1f us (trials %s), warm %.1f us; %.1f %% of HBM peak cold" % (
        w.name, t["cold_us"], ", ".join("%.1f" % x for x in t["cold_trials_us"]), t["warm_us"],
        100 * sec["cold"]["hbm_frac"]))
    o_cpu, S_cpu = run.o.cpu(), run.S.cpu()
    if with_parity:
        sec["parity"] = parity(w, host, o_cpu, S_cpu)
        log("prefill %s: parity o %.2e S %.2e over %d heads" % (
            w.name, sec["parity"]["rel_err_o"], sec["parity"]["rel_err_S"], w.B * w.H))
    if keep:
        return sec, host, run, (o_cpu, S_cpu)
    del run
    torch.cuda.empty_cache()
    return sec, None, None, (o_cpu, S_cpu)


def bench_step(w: W.Prefill, host, run: PrefillRun, steps: int, warmup: int):
    """The contract's step: the prefill plus the first decode token on the state
    it returns; exactly ``steps`` steps after ``warmup`` untimed ones, wall clock
    between two synchronisations."""
    tok = W.make_decode(W.Decode("next_token", w.B, w.H, w.dk, w.dv, 1, w.dtype, w.gate, 0.0,
                                 seed=w.seed + 100))
    td = {k: (None if v is None else v.cuda()) for k, v in tok.items()}
    o1 = torch.empty((w.B, w.H, w.dv), dtype=w.dtype, device="cuda")
    a1 = None if td["alpha"] is None else td["alpha"][0]

    def step():
        run()
        gdn.decode_step(td["q"][0], td["k"][0], td["v"][0], a1, td["beta"][0], run.S, o=o1,
                        mode=w.mode)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def bench_decode(w: W.Decode, reps: int = 3, rotate: int = 1):
    """``w.steps`` decode steps captured in one HIP graph; per-step time from
    the median of ``reps`` replays.  ``rotate`` > 1 cycles the steps over that
    many state buffers (HBM-resident working set)."""
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
        times.append(e0.elapsed_time(e1) * 1e3 / w.steps)
    del g
    us = statistics.median(times)
    gb = decode_bytes(w) / (us * 1e-6) / 1e9
    return dict(us_per_step=us, replays_us_per_step=times, gbps=gb, hbm_frac=gb / HBM_PEAK_GBPS)


def packed_bytes(w: W.Packed) -> int:
    """Algorithmic bytes of a packed prefill: the rows' tokens as one row, plus
    one initial (if given) and one final state per sequence."""
    rows = prefill_bytes(W.Prefill(w.name, 1, w.H, w.T, w.dk, w.dv, w.dtype, w.gate, 0.0, w.seed))
    rows -= w.H * w.dv * w.dk * 4                                   # the single row's S_final
    return rows + w.N * w.H * w.dv * w.dk * 4 * (2 if w.s0_std > 0 else 1) + (w.N + 1) * 4


def _mean_launch_us(launch, n):
    b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    launch()
    b0.record()
    for _ in range(n):
        launch()
    b1.record()
    torch.cuda.synchronize()
    return b0.elapsed_time(b1) * 1e3 / n


def bench_packed(w: W.Packed, reps: int):
    """Mean duration of one ``gdn_chunk_fwd_varlen`` launch (``reps`` back to
    back between one event pair, behind a running launch), median of 3 trials."""
    log("packed %s" % w.name)
    host = W.make_packed(w)
    d = {k: (None if v is None else v.cuda()) for k, v in host.items()}
    o = torch.empty((1, w.T, w.H, w.dv), dtype=w.dtype, device="cuda")
    S = torch.empty((w.N, w.H, w.dv, w.dk), dtype=torch.float32, device="cuda")

    def launch():
        gdn.chunk_fwd_varlen(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["cu_seqlens"],
                             d["S0"], mode=w.mode, o=o, S_final=S)

    for _ in range(3):
        launch()
    trials = [_mean_launch_us(launch, reps) for _ in range(3)]
    us = statistics.median(trials)
    nbytes = packed_bytes(w)
    lens = W.packed_lengths(w)
    return dict(workload=w.name, N=w.N, T=w.T, H=w.H, lengths_min=min(lens), lengths_max=max(lens),
                launch_us=us, trials_us=trials, tokens_per_s=w.T / (us * 1e-6),
                hbm_gbps=nbytes / (us * 1e-6) / 1e9, hbm_frac=nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS,
                algorithmic_bytes=nbytes, counters=committed_counters(w.name + "_gated_rmsnorm"))


def bench_fused(w: W.Prefill, reps: int):
    """Mean duration of one ``gdn_chunk_fwd_fused`` launch on raw inputs of the
    workload's shape (q, k not normalised, beta and alpha logits, per-head rates
    and biases), every part of the prologue on; timed in alternation with the
    plain call on the workload's own inputs (six rounds each, median), so that
    both see the same clock."""
    log("fused prologue (%s shape)" % w.name)
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

    for _ in range(3):
        fused()
        plain()
    tf, tp = [], []
    for r in range(6):
        order = (fused, plain) if r % 2 == 0 else (plain, fused)
        for f in order:
            (tf if f is fused else tp).append(_mean_launch_us(f, reps))
    us, us_plain = statistics.median(tf), statistics.median(tp)
    nbytes = prefill_bytes(w) + w.H * 4 * (2 if w.mode == W.MODE_SCALAR else 1 + w.dk)
    return dict(workload=w.name + "_fused_prologue", launch_us=us, plain_launch_us_same_period=us_plain,
                overhead_frac=us / us_plain - 1.0,
                tokens_per_s=w.B * w.T / (us * 1e-6), hbm_gbps=nbytes / (us * 1e-6) / 1e9,
                hbm_frac=nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, algorithmic_bytes=nbytes)


def bench_gdn2(w: W.Prefill, reps: int):
    """Mean duration of one ``gdn2_chunk_fwd`` launch (erase and write gates) at
    the shape and per-channel decay of ``w``, median of 3 trials."""
    log("gated deltanet-2 (%s shape)" % w.name)
    d = {k: (None if v is None else v.cuda()) for k, v in W.make_gdn2(w.with_(seed=w.seed + 300)).items()}
    o = torch.empty((w.B, w.T, w.H, w.dv), dtype=w.dtype, device="cuda")
    S = torch.empty((w.B, w.H, w.dv, w.dk), dtype=torch.float32, device="cuda")

    def launch():
        gdn.gdn2_chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["erase"], d["write"], d["S0"],
                           o=o, S_final=S)

    for _ in range(3):
        launch()
    trials = [_mean_launch_us(launch, reps) for _ in range(3)]
    us = statistics.median(trials)
    es = 2 if w.dtype == torch.bfloat16 else 4
    tok = w.B * w.T * w.H
    nbytes = prefill_bytes(w) - tok * 4 + tok * (w.dk + w.dv) * es   # gates instead of beta
    del d
    return dict(workload="gdn2_" + w.name, launch_us=us, trials_us=trials,
                tokens_per_s=w.B * w.T / (us * 1e-6),
                hbm_gbps=nbytes / (us * 1e-6) / 1e9, hbm_frac=nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS,
                algorithmic_bytes=nbytes, counters=committed_counters(w.name + "_gated_rmsnorm"))


def bench_backward(w: W.Prefill, reps: int):
    """Mean duration of one ``gdn_chunk_bwd`` launch on the workload's inputs with
    a random output gradient (and final-state gradient), median of 3 trials."""
    log("backward (%s)" % w.name)
    d = {k: (None if v is None else v.cuda()) for k, v in W.make_prefill(w).items()}
    g = torch.Generator().manual_seed(w.seed + 400)
    do = torch.randn(w.B, w.T, w.H, w.dv, generator=g).to(w.dtype).cuda()
    dST = torch.randn(w.B, w.H, w.dv, w.dk, generator=g).cuda()

    def launch():
        gdn.chunk_bwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], do, dST, mode=w.mode)

    launch()
    trials = [_mean_launch_us(launch, reps) for _ in range(3)]
    us = statistics.median(trials)
    es = 2 if w.dtype == torch.bfloat16 else 4
    tok = w.B * w.T * w.H
    state = w.B * w.H * w.dv * w.dk * 4
    nbytes = 2 * prefill_bytes(w) + tok * w.dv * es + state   # inputs + dout, dS_final; the same again out
    return dict(workload=w.name + "_backward", launch_us=us, trials_us=trials,
                tokens_per_s=w.B * w.T / (us * 1e-6), hbm_gbps=nbytes / (us * 1e-6) / 1e9,
                hbm_frac=nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, algorithmic_bytes=nbytes,
                counters=committed_counters(w.name + "_backward"))


def bench_epilogue(w: W.Prefill, reps: int):
    """Mean duration of one ``gdn_gated_rmsnorm`` launch on an output of the
    workload's shape [B, T, H, d_v] (bf16), median of 3 trials."""
    log("output epilogue (%s shape)" % w.name)
    g = torch.Generator().manual_seed(w.seed + 500)
    shape = (w.B, w.T, w.H, w.dv)
    o = torch.randn(*shape, generator=g).to(w.dtype).cuda()
    gate = torch.randn(*shape, generator=g).to(w.dtype).cuda()
    wt = (1.0 + 0.5 * torch.randn(w.dv, generator=g)).cuda()
    out = torch.empty_like(o)

    def launch():
        gdn.gated_rmsnorm(o, gate, wt, eps=1e-6, out=out)

    launch()
    trials = [_mean_launch_us(launch, reps) for _ in range(3)]
    us = statistics.median(trials)
    nbytes = 3 * o.numel() * o.element_size() + w.dv * 4   # o, gate read; out written; the gain
    return dict(workload=w.name + "_gated_rmsnorm", launch_us=us, trials_us=trials,
                hbm_gbps=nbytes / (us * 1e-6) / 1e9, hbm_frac=nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS,
                algorithmic_bytes=nbytes, counters=committed_counters(w.name + "_gated_rmsnorm"))


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
# CPU baseline: the fp64 oracle on the headline workload
# ------------------------------------------------------------------------------

def cpu_baseline(w: W.Prefill, host, budget_s: float = 10.0):
    """The oracle over the whole workload, one pass, repeated until about
    ``budget_s`` seconds are used (at least one pass).  Returns the baseline and
    the first pass's outputs (the parity reference)."""
    import oracle  # test infrastructure: used only for this baseline leg
    threads = oracle.num_threads()
    secs, passes, ref = 0.0, 0, None
    while passes == 0 or secs < budget_s:
        t0 = time.perf_counter()
        r = oracle.gdn_fwd(host["q"], host["k"], host["v"], host["alpha"], host["beta"], host["S0"],
                           mode=w.mode)
        secs += time.perf_counter() - t0
        passes += 1
        if ref is None:
            ref = r
    toks = passes * w.B * w.T
    base = dict(value=toks / secs, unit="tokens/s", cores=threads, kind="oracle",
                sample="fp64 token loop over the whole workload (all %d heads, T=%d), %d pass(es): "
                       "%d tokens in %.1f s on %d threads (OpenMP over heads)"
                       % (w.B * w.H, w.T, passes, toks, secs, threads))
    return base, ref


# ------------------------------------------------------------------------------
# rocprofv3 output -> committed summaries (runs on any host, reads CSV files)
# ------------------------------------------------------------------------------

def _csv_rows(path, pattern):
    out = []
    for f in sorted(glob.glob(os.path.join(path, "**", pattern), recursive=True)):
        with open(f) as fh:
            out += list(csv.DictReader(fh))
    return out


def short_kernel_name(name: str) -> str:
    """Readable kernel name: a mangled gdn kernel becomes name<template args>."""
    import re
    m = re.match(r"_ZN3gdn12_GLOBAL__N_1(\d+)(.*)", name)
    if not m:
        return name.replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "").strip()
    n = int(m.group(1))
    base, rest = m.group(2)[:n], m.group(2)[n:]
    args = []
    if rest.startswith("I"):
        rest = rest[1:]
        while rest and not rest.startswith("E"):
            t = re.match(r"DF16b|f|Li(\d+)E|Lb([01])E", rest)
            if not t:
                break
            g = t.group(0)
            args.append("bf16" if g == "DF16b" else "f32" if g == "f" else
                        t.group(1) if t.group(1) is not None else ("true" if t.group(2) == "1" else "false"))
            rest = rest[len(g):]
    return "%s<%s>" % (base, ", ".join(args)) if args else base


def summarize_pmc(dirs, name, out_json=COUNTER_FILE):
    """Per-kernel counter averages of a ``--profile NAME`` run under one or
    more ``rocprofv3 --pmc`` runs (one directory each).  HBM bytes: FETCH_SIZE
    and WRITE_SIZE (KiB per dispatch) scaled by what the same counter reads for
    the 1 GiB device copy that the profile run performs.  MFMA utilisation:
    SQ_VALU_MFMA_BUSY_CYCLES over (GRBM_GUI_ACTIVE / 8) x 1024 SIMDs; the clock:
    GRBM_GUI_ACTIVE / 8 over the dispatch's duration (the collected
    GRBM_GUI_ACTIVE is the sum of the 8 XCDs' copies, each of which counts the
    GPU's active cycles: a 1 GiB copy reads 19.1 G cycles/s, 2.39 GHz per XCD)."""
    per = {}   # (kernel, counter) -> list of per-dispatch values
    durs = {}
    for d in dirs:
        for r in _csv_rows(d, "*counter_collection.csv"):
            key = (r["Kernel_Name"], int(r["Dispatch_Id"]))
            per.setdefault((r["Kernel_Name"], r["Counter_Name"]), {}).setdefault(key, 0.0)
            per[(r["Kernel_Name"], r["Counter_Name"])][key] += float(r["Counter_Value"])
            durs[key] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    copy_kib = (1 << 30) / 1024.0
    scale = {}
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        vals = [v for (k, c), dd in per.items() if c == ctr and "copyBuffer" in k
                for v in dd.values() if v > 0.25 * copy_kib]
        if vals:
            scale[ctr] = copy_kib / (sum(vals) / len(vals))
    kernels = sorted({k for (k, c) in per if "gdn" in k})
    rec = dict(kernel_source_sha256=kernel_source_hash(name), workload=name, counter_scale=scale,
               note="per dispatch averages; HBM bytes = FETCH_SIZE / WRITE_SIZE KiB scaled so the "
                    "1 GiB device copy reads and writes 1 GiB; mfma_util = SQ_VALU_MFMA_BUSY_CYCLES "
                    "/ (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs); clock = GRBM_GUI_ACTIVE / 8 / duration "
                    "(the collected GRBM_GUI_ACTIVE sums the 8 XCDs' copies); bf16_mfma_flop = "
                    "SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512",
               kernels={})
    total_bytes = 0.0
    for k in kernels:
        ent = {}
        n = 0
        for (kk, c), dd in per.items():
            if kk != k:
                continue
            ent[c] = sum(dd.values()) / len(dd)
            n = max(n, len(dd))
        ent["dispatches"] = n
        if "FETCH_SIZE" in ent and "FETCH_SIZE" in scale:
            ent["hbm_read_bytes"] = ent["FETCH_SIZE"] * 1024 * scale["FETCH_SIZE"]
        if "WRITE_SIZE" in ent and "WRITE_SIZE" in scale:
            ent["hbm_write_bytes"] = ent["WRITE_SIZE"] * 1024 * scale["WRITE_SIZE"]
        if "hbm_read_bytes" in ent and "hbm_write_bytes" in ent:
            total_bytes += ent["hbm_read_bytes"] + ent["hbm_write_bytes"]
        # GRBM_GUI_ACTIVE as collected is the sum over the 8 XCDs' copies of
        # the counter; each XCD counts the GPU's active cycles
        if "SQ_VALU_MFMA_BUSY_CYCLES" in ent and ent.get("GRBM_GUI_ACTIVE"):
            ent["mfma_util"] = ent["SQ_VALU_MFMA_BUSY_CYCLES"] / (ent["GRBM_GUI_ACTIVE"] / NUM_XCDS * NUM_SIMDS)
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in ent:
            ent["bf16_mfma_flop"] = ent["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512
        gui = [v for (kk, c), dd in per.items() if kk == k and c == "GRBM_GUI_ACTIVE"
               for key, v in dd.items() if durs.get(key)]
        dd_ = [durs[key] for (kk, c), dd in per.items() if kk == k and c == "GRBM_GUI_ACTIVE"
               for key in dd if durs.get(key)]
        if gui and dd_:
            ent["clock_mhz"] = sum(gui) / NUM_XCDS / sum(dd_) / 1e6
            ent["duration_us"] = sum(dd_) / len(dd_) * 1e6
        rec["kernels"][short_kernel_name(k)] = ent
    if total_bytes:
        rec["hbm_bytes_per_launch"] = total_bytes
    try:
        with open(out_json) as f:
            allrec = json.load(f)
    except (OSError, ValueError):
        allrec = {}
    old = allrec.get(name, {})
    if old.get("kernel_source_sha256") == rec["kernel_source_sha256"]:
        # a second counter pass over the same source adds its counters
        for k, ent in old.get("kernels", {}).items():
            for c, v in ent.items():
                rec["kernels"].setdefault(k, {}).setdefault(c, v)
        if "hbm_bytes_per_launch" not in rec and "hbm_bytes_per_launch" in old:
            rec["hbm_bytes_per_launch"] = old["hbm_bytes_per_launch"]
        rec["counter_scale"] = {**old.get("counter_scale", {}), **scale}
    allrec[name] = rec
    with open(out_json, "w") as f:
        json.dump(allrec, f, indent=1, sort_keys=True)
    print(json.dumps(rec, indent=1, sort_keys=True))


def summarize_trace(path):
    """Markdown table of per-kernel durations from a ``--kernel-trace`` run."""
    rows = _csv_rows(path, "*kernel_trace.csv")
    per = {}
    for r in rows:
        n = short_kernel_name(r["Kernel_Name"])
        per.setdefault(n, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3)
    print("| kernel | calls | avg us | median us | min us | max us |")
    print("|---|---|---|---|---|---|")
    for n, v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        print("| `%s` | %d | %.1f | %.1f | %.1f | %.1f |" % (n, len(v), sum(v) / len(v),
                                                          statistics.median(v), min(v), max(v)))


def profile_run(name, reps):
    """Run one workload ``reps`` times and nothing else (plus the 1 GiB device
    copy that scales the byte counters): the program rocprofv3 observes."""
    device_copy_gbps()
    pw = {w.name: w for w in W.PREFILL_WORKLOADS}
    dw = {w.name: w for w in W.DECODE_WORKLOADS}
    if name in pw:
        run = PrefillRun(pw[name], W.make_prefill(pw[name]))
        for _ in range(reps):
            run()
    elif name.endswith("_backward") and name[:-len("_backward")] in pw:
        w = pw[name[:-len("_backward")]]
        d = {k: (None if v is None else v.cuda()) for k, v in W.make_prefill(w).items()}
        g = torch.Generator().manual_seed(w.seed + 400)
        do = torch.randn(w.B, w.T, w.H, w.dv, generator=g).to(w.dtype).cuda()
        dST = torch.randn(w.B, w.H, w.dv, w.dk, generator=g).cuda()
        for _ in range(reps):
            gdn.chunk_bwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], do, dST, mode=w.mode)
    elif name.endswith("_gated_rmsnorm") and name[:-len("_gated_rmsnorm")] in pw:
        w = pw[name[:-len("_gated_rmsnorm")]]
        g = torch.Generator().manual_seed(w.seed + 500)
        shape = (w.B, w.T, w.H, w.dv)
        o = torch.randn(*shape, generator=g).to(w.dtype).cuda()
        gate = torch.randn(*shape, generator=g).to(w.dtype).cuda()
        wt = (1.0 + 0.5 * torch.randn(w.dv, generator=g)).cuda()
        out = torch.empty_like(o)
        for _ in range(reps):
            gdn.gated_rmsnorm(o, gate, wt, eps=1e-6, out=out)
    elif name in dw:
        w = dw[name].with_(steps=min(dw[name].steps, reps))
        bench_decode(w, reps=1, rotate=16)
    else:
        raise SystemExit("unknown workload %s" % name)
    torch.cuda.synchronize()
    log("profiled %s x %d" % (name, reps))


# ------------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--only", nargs="*", default=None,
                    help="prefill workloads to time (default: all)")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle baseline")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the packed, fused-prologue, Gated DeltaNet-2 and backward timings")
    ap.add_argument("--profile", metavar="NAME", help="run one workload for a profiler and exit")
    ap.add_argument("--reps", type=int, default=20)
    ap.add_argument("--summarize-pmc", nargs="+", metavar="ARG",
                    help="DIR [DIR ...] NAME: counter summary of --profile NAME runs -> profiles/counters.json")
    ap.add_argument("--summarize-trace", metavar="DIR", help="per-kernel duration table of a kernel trace")
    args = ap.parse_args()
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[:-1], args.summarize_pmc[-1])
        return
    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build runs the path on a single MI355X "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    gdn.load()
    if args.profile:
        profile_run(args.profile, args.reps)
        return

    copy_gbps = device_copy_gbps()
    log("device copy %.0f GB/s" % copy_gbps)
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    wl = [w for w in W.PREFILL_WORKLOADS if args.only is None or w.name in args.only]
    if HEADLINE not in wl:
        wl.append(HEADLINE)
    prefill, head = {}, None
    for w in wl:
        is_head = w is HEADLINE
        sec, host, run, outs = bench_prefill(w, scratch, with_parity=not is_head, keep=is_head)
        prefill[w.name] = sec
        if is_head:
            wall = bench_step(w, host, run, args.steps, args.warmup)
            head = (sec, host, outs)
            del run
            torch.cuda.empty_cache()
            log("step (prefill + first decode token) x %d: %.3f ms per step" % (
                args.steps, wall * 1e3 / args.steps))
            ms_step = wall * 1e3 / args.steps
    del scratch
    torch.cuda.empty_cache()

    decode = None
    if not args.no_decode:
        decode = {}
        for dw in W.DECODE_WORKLOADS:
            lit = bench_decode(dw, rotate=1)
            rot = bench_decode(dw, rotate=16)
            decode[dw.name] = dict(bytes_per_step=decode_bytes(dw), in_place=lit, rotated_16_states=rot,
                                   counters=committed_counters(dw.name))
            log("decode %s: in place %.2f us/step %.0f GB/s; rotated %.2f us/step %.0f GB/s (%.1f %%)" % (
                dw.name, lit["us_per_step"], lit["gbps"], rot["us_per_step"], rot["gbps"],
                100 * rot["hbm_frac"]))

    packed = fused = gdn2 = bwd = epi = None
    if not args.no_variants:
        packed = bench_packed(W.GDN_BF16_PACKED, args.steps)
        log("packed: %.1f us per launch" % packed["launch_us"])
        fused = bench_fused(W.GDN_BF16_PREFILL, args.steps)
        log("fused prologue: %.1f us per launch (plain call in alternation: %.1f us)" % (
            fused["launch_us"], fused["plain_launch_us_same_period"]))
        gdn2 = bench_gdn2(W.KDA_BF16_PREFILL, args.steps)
        log("gated deltanet-2: %.1f us per launch" % gdn2["launch_us"])
        epi = bench_epilogue(W.GDN_BF16_PREFILL, args.steps)
        log("output epilogue: %.1f us per launch (%.0f GB/s)" % (epi["launch_us"], epi["hbm_gbps"]))
        bwd = [bench_backward(w, max(2, args.steps // 4)) for w in (W.GDN_BF16_PREFILL, W.KDA_BF16_PREFILL)]
        for x in bwd:
            log("backward %s: %.1f us per launch" % (x["workload"], x["launch_us"]))
    torch.cuda.empty_cache()

    sec, host, outs = head
    w = HEADLINE
    base = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) on %s" % w.name)
        base, ref = cpu_baseline(w, host)
        sec["parity"] = parity(w, host, outs[0], outs[1], ref=ref)
        log("oracle %.0f tokens/s; parity o %.2e S %.2e over all %d heads" % (
            base["value"], sec["parity"]["rel_err_o"], sec["parity"]["rel_err_S"], w.B * w.H))

    c = sec.get("counters") or {}
    traffic = c.get("hbm_bytes_per_launch")
    cold = sec["cold"]
    roofline = dict(bound="hbm", achieved=cold["hbm_gbps"], peak=HBM_PEAK_GBPS, unit="GB/s",
                    frac=cold["hbm_frac"], traffic=traffic,
                    kernel="gdn_chunk_fwd launch (%s)" % ", ".join(sorted(c.get("kernels", {})) or ["-"]),
                    launch_us=cold["launch_us"], launch_us_warm=sec["warm"]["launch_us"],
                    mfma_frac_causal=cold["mfma_frac_causal"], mfma_frac_dense=cold["mfma_frac_dense"])
    out = dict(metric=METRIC, value=w.B * w.T / (ms_step * 1e-3), unit="tokens/s", n_gpus=1,
               steps=args.steps, warmup=args.warmup, ms_per_step=ms_step, higher_is_better=True,
               scaling="weak", vs_baseline=None,
               dtype="bf16" if w.dtype == torch.bfloat16 else "f32", data="synthetic",
               config=dict(workload=w.name, B=w.B, H=w.H, T=w.T, dk=w.dk, dv=w.dv, chunk=CHUNK,
                           decay={0: "none", 1: "scalar", 2: "channel"}[w.mode],
                           step="chunked prefill + first decode token",
                           state="fp32", parallelism="single GPU"),
               roofline=roofline, cpu_baseline=base, prefill=prefill, decode=decode, packed=packed,
               fused_prologue=fused, gdn2=gdn2, output_epilogue=epi, backward=bwd, device_copy_gbps=copy_gbps,
               host=host_info(), peaks=dict(hbm_gbps=HBM_PEAK_GBPS, bf16_tflops=BF16_PEAK_TFLOPS))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
