#!/usr/bin/env python3
"""Benchmark of tiled causal linear attention (forward + backward) on one MI355X.

Workload: the sequence-length sweep at a fixed 131072 tokens per head,
n in {1024, 4096, 16384, 65536} with batch 131072 / n, 16 heads, head dim 128,
block 64, per-head decay lambda_h = exp(-2^(-8(h+1)/16)), bf16 storage, inputs
N(0,1)/sqrt(128) from the seeded generator, resident in HBM.  One step runs, for
each of the four shapes, la_fwd (output and final state) then la_bwd (dQ, dK,
dV) through the C ABI.  ``value`` is forward+backward tokens per second over
the whole step (4 x 131072 tokens).

The JSON line also carries, per sequence length, forward-only and backward-only
tokens/s with algorithmic TFLOP/s (% of the 2.5 PFLOP/s bf16 dense peak) and
GB/s; the recurrent decode step at 256 sequences x 64 heads (GB/s against
8 TB/s); the roofline of the kernel that takes the most time (its average
launch duration measured with HIP events on its own stream during a second
pass over the same steps); and the fp64 oracle timed on a bounded sample on the
host cores.

Subcommand ``summarize`` turns rocprofv3 outputs into the text summaries kept
under profiles/ (see --help).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import math
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

D, BK, H = 128, 64, 16
SWEEP_N = (1024, 4096, 16384, 65536)
TOKENS_PER_POINT = 131072
HBM_PEAK_GBS = 8000.0      # MI355X published HBM3E bandwidth
BF16_PEAK_TFLOPS = 2500.0  # MI355X published dense bf16 MFMA rate
PROFILES = os.path.join(ROOT, "profiles")
CALIB_BYTES = 1 << 30      # bytes read and written by the calibration copy
# library kernel name (as the library's profiler reports it) -> the device function it
# launches; several library names can share one device function (the forward sweep
# serves both la_fwd and the dQ pass of la_bwd)
DEVICE_FN = {
    "fwd_dma": "k_fwd_dma", "dq_dma": "k_fwd_dma", "fwd_mfma": "k_fwd_mfma", "dq_mfma": "k_fwd_mfma",
    "dkdv_dma": "k_rev_dma_split", "dkdv_mfma": "k_rev_mfma", "dkdv_generic": "k_rev_generic",
    "fwd_dma_fused": "k_fwd_dma_fused", "dq_dma_fused": "k_fwd_dma_fused",
    # the chunk aggregates' default form (two loader waves); LA_STATE=dma2 runs k_chunk_state_dma
    "chunk_state_dma": "k_chunk_state_ld", "chunk_state_rev_dma": "k_chunk_state_ld",
    "chunk_state_mfma": "k_chunk_state_mfma", "chunk_state_rev_mfma": "k_chunk_state_mfma",
    "state_scan": "k_scan", "state_scan_rev": "k_scan", "decode": "k_decode",
}
KERNEL_SOURCES = {         # device function -> source file its code lives in
    "k_fwd_dma": "k_fwd_dma.hip", "k_fwd_dma_fused": "k_fwd_dma.hip", "k_fwd_mfma": "k_fwd_mfma.hip",
    "k_rev_dma": "k_bwd_dma.hip", "k_chunk_state_ld": "k_state_dma.hip",
    "k_rev_dma_split": "k_bwd_dma.hip",
    "k_rev_mfma": "k_bwd_mfma.hip", "k_rev_generic": "k_generic.hip", "k_chunk_state_dma": "k_state_dma.hip",
    "k_chunk_state_mfma": "k_fwd_mfma.hip", "k_scan": "k_generic.hip", "k_decode": "k_generic.hip",
    "k_fwd_dma128": "k_fwd_dma128.hip", "k_fwd_dma_varlen": "k_fwd_dma.hip", "k_dlam_dma": "k_dlam_dma.hip",
    "k_dlam_state_dma": "k_state_dma.hip", "k_dlam_scan": "k_dlam.hip", "k_dlam_reduce": "k_dlam.hip",
    "k_chunk_state_dma_varlen": "k_state_dma.hip", "k_scan_varlen": "k_generic.hip",
}


# ----------------------------------------------------------------------------- algorithmic counts
def fwd_flops_per_token_head(d=D, bk=BK):
    # intra: causal Q K^T and A V over (Bk+1)/2 keys on average; inter: Q S and the state update
    return 2 * d * (bk + 1) + 4 * d * d


def bwd_flops_per_token_head(d=D, bk=BK):
    # the algorithmic count of the backward: intra G = dO V^T, P = Q K^T and the dQ, dK, dV
    # products over (Bk+1)/2 keys on average; inter dO S^T, V dS^T, K dS and the dS update
    return 5 * d * (bk + 1) + 8 * d * d


def bwd_flops_executed_per_token_head(d=D, bk=BK):
    # as executed: the dQ sweep also carries the state S over its blocks (+2 d^2), since only
    # chunk-start states are kept from the forward
    return bwd_flops_per_token_head(d, bk) + 2 * d * d


def kernel_bytes(name, B, Hh, N, d, chunks, agg=1, with_state=True):
    """Algorithmic HBM bytes one launch of library kernel `name` must move (bf16 tensors);
    `agg`: parts per chunk of the chunk aggregates (the scans run over them)."""
    th = B * Hh * N                    # token-heads
    t = 2 * d * th                     # one bf16 [B, H, N, D] tensor
    st = B * Hh * d * d * 4            # one float32 state per sequence
    frac = (chunks - 1) / chunks if chunks > 1 else 0.0
    return {
        "fwd_mfma": 4 * t + (st if with_state else 0), "fwd_dma": 4 * t + (st if with_state else 0),
        "dq_mfma": 4 * t, "dq_dma": 4 * t,
        "dkdv_mfma": 6 * t, "dkdv_generic": 6 * t, "dkdv_dma": 6 * t,
        "chunk_state_mfma": 2 * t * frac,
        "chunk_state_rev_mfma": 2 * t * frac,
        "chunk_state_dma": 2 * t * frac, "chunk_state_rev_dma": 2 * t * frac,
        "state_scan": 2 * st * (chunks - 1) * agg, "state_scan_rev": 2 * st * (chunks - 1) * agg,
    }.get(name)


def source_digest(kernel):
    """Digest of the source of a device function: its .hip file and every csrc header."""
    src = KERNEL_SOURCES.get(kernel)
    if not src:
        return None
    csrc = os.path.join(ROOT, "causal_linear_attention_tiled_amd", "csrc")
    p = os.path.join(csrc, src)
    if not os.path.exists(p):
        return None
    h = hashlib.sha256(open(p, "rb").read())
    for hdr in sorted(glob.glob(os.path.join(csrc, "*.h"))):
        h.update(open(hdr, "rb").read())
    return h.hexdigest()[:16]


def read_traffic(kernel):
    """Measured HBM bytes per launch of `kernel` from profiles/, or None when absent or stale."""
    path = os.path.join(PROFILES, f"{kernel}_sweep_traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("source_sha256_16") != source_digest(kernel):
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def read_mfma(kernel, tag="sweep"):
    """Matrix-core figures of device function `kernel` from profiles/mfma_<tag>.txt (its totals
    row), or None when absent or when the kernel's source has changed since."""
    path = os.path.join(PROFILES, f"mfma_{tag}.txt")
    if not os.path.exists(path):
        return None
    for line in open(path):
        cols = [c.strip() for c in line.split("|")]
        if len(cols) == 11 and cols[0] == kernel and cols[1] == "all":
            if cols[10] != source_digest(kernel):
                return None
            return {"mfma_tflops_executed": float(cols[5]), "pct_bf16_peak_executed": float(cols[6]),
                    "MfmaUtil": float(cols[7]), "VALUBusy": float(cols[8]), "LdsUtil": float(cols[9]),
                    "source": f"profiles/mfma_{tag}.txt"}
    return None


# ----------------------------------------------------------------------------- inputs
def device_normal(torch, sid, shape, seed=0):
    import numpy as np
    import synth
    total = int(np.prod(shape))
    out = torch.empty(total, dtype=torch.bfloat16, device="cuda")
    flat = out.view(torch.int16)
    step = 1 << 27
    for s0 in range(0, total, step):
        n = min(step, total - s0)
        host = synth.normal(seed, sid, (n,), 1.0 / math.sqrt(shape[-1]), "bf16", start=s0)
        flat[s0:s0 + n].copy_(torch.from_numpy(host.view(np.int16)))
    return out.view(*shape)


# ----------------------------------------------------------------------------- HBM probe
def hbm_rates(torch, timed):
    """What this GPU's HBM delivers to plain streaming kernels (torch's own), in GB/s: a 4 GiB
    read (row sums of a [2^20, 1024] float32 tensor, the fastest read-only torch kernel measured
    here: a full reduction or a bf16 sum runs at 1-4 TB/s), a 4 GiB write (fill) and a
    2 + 2 GiB copy (reads and writes mixed 1:1)."""
    x = torch.empty(1 << 30, dtype=torch.float32, device="cuda")
    x.fill_(1.0)
    nbytes = x.numel() * 4
    rows = x.view(1 << 20, 1 << 10)
    half = x.numel() // 2
    a, b = x[:half], x[half:]
    for fn in (lambda: rows.sum(dim=1), lambda: x.fill_(0.5), lambda: b.copy_(a)):
        fn()  # the first call of each loads its kernel
    r_ms = timed(lambda: rows.sum(dim=1), 10)
    w_ms = timed(lambda: x.fill_(0.5), 10)
    c_ms = timed(lambda: b.copy_(a), 10)
    del x, rows, a, b
    return {"read_gbs": round(nbytes / (r_ms * 1e-3) / 1e9, 1), "write_gbs": round(nbytes / (w_ms * 1e-3) / 1e9, 1),
            "copy_gbs": round(2 * half * 4 / (c_ms * 1e-3) / 1e9, 1),
            "note": "torch row-sum / fill / copy kernels over 4 GiB; context for the roofline, not the peak"}


def flatness_floor(sweep, rates):
    """The sweep's forward flatness if every point ran at the probe's read and write rates:
    a point reads Q, K, V and writes O (reads and writes do not overlap on this HBM), and a
    point split into C chunks reads K and V of C - 1 chunks once more for the chunk
    aggregates.  Returns (floor flatness, per-point floor ms)."""
    r, w = rates["read_gbs"] * 1e9, rates["write_gbs"] * 1e9
    ms = []
    for x in sweep:
        tensor = 2 * D * x["batch"] * H * x["n"]
        state = x["batch"] * H * D * D * 4
        extra = 2 * tensor * (x["chunks"] - 1) / x["chunks"] if x["chunks"] > 1 else 0.0
        ms.append(1e3 * ((3 * tensor + extra) / r + (tensor + state) / w))
    return max(ms) / min(ms), ms


# ----------------------------------------------------------------------------- CPU baseline
def cpu_baseline(seconds_target):
    """The fp64 oracle (recurrent form, fwd + bwd) on a bounded sample of the sweep workload."""
    import numpy as np
    import oracle
    import synth
    n = 4096
    B = TOKENS_PER_POINT // n
    lam = synth.decay_schedule(H).astype(np.float64)
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))

    def run(pairs, reps=1):
        qs, ks, vs, gs, ls = [], [], [], [], []
        for p in range(pairs):
            b, h = p // H, p % H
            q, k, v, g = (synth.bf16_bits_to_f64(synth.pair_slice(0, i, B, H, n, D, b, h, "bf16"))
                          for i in (1, 2, 3, 4))
            qs.append(q); ks.append(k); vs.append(v); gs.append(g); ls.append(lam[h])
        q, k, v, g = (np.stack(x) for x in (qs, ks, vs, gs))
        t0 = time.perf_counter()
        for _ in range(reps):
            oracle.fwd_recurrent(q, k, v, np.array(ls))
            oracle.bwd_recurrent(q, k, v, g, np.array(ls))
        return time.perf_counter() - t0

    pairs, reps = threads, 1
    dt = run(pairs)
    if dt < seconds_target / 4:
        # more sequences (up to all of this sweep point), then repeated passes over them
        scale = seconds_target / max(dt, 1e-3)
        pairs = min(B * H, max(threads, int(pairs * scale) // threads * threads))
        reps = max(1, int(round(scale * threads / pairs)))
        dt = run(pairs, reps)
    tokens = reps * pairs * n / H   # tokens of the metric carry all H heads
    return {"value": tokens / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{pairs} of the {B * H} (batch, head) sequences of the n={n} sweep point "
                      f"(d={D}, per-head decay), {reps} pass(es), fwd+bwd, recurrent form in fp64, "
                      f"{dt:.1f} s",
            "cpu_model": cpu_model(), "one_thread": one_thread_oracle(n)}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def one_thread_oracle(n):
    """The oracle on one thread (its OpenMP loop over sequences pinned to one thread, in a
    child process): fwd+bwd of one (batch, head) sequence of the sweep point."""
    code = ("import sys, time, numpy as np; sys.path.insert(0, %r); import oracle, synth; "
            "q, k, v, g = (synth.bf16_bits_to_f64(synth.pair_slice(0, i, %d, %d, %d, %d, 0, 0, 'bf16'))[None] "
            "for i in (1, 2, 3, 4)); lam = synth.decay_schedule(%d)[:1].astype(np.float64); "
            "oracle.fwd_recurrent(q[:, :8], k[:, :8], v[:, :8], lam); t0 = time.perf_counter(); "
            "oracle.fwd_recurrent(q, k, v, lam); oracle.bwd_recurrent(q, k, v, g, lam); "
            "print(time.perf_counter() - t0)" % (ROOT, TOKENS_PER_POINT // n, H, n, D, H))
    env = dict(os.environ, OMP_NUM_THREADS="1")
    try:
        out = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                             timeout=120, check=True).stdout.split()
        dt = float(out[-1])
    except (subprocess.SubprocessError, ValueError, IndexError):
        return None
    return {"value": n / H / dt, "unit": "tokens/s", "seconds": round(dt, 3),
            "sample": f"one (batch, head) sequence of n={n}, fwd+bwd, 1 thread"}


# ----------------------------------------------------------------------------- serving
def serving_workload(torch, la, lam, timed):
    """Ragged prefill of 64 sequences (lengths log-uniform in [128, 8192], seeded), 16 heads,
    packed token-major in one la_fwd_varlen launch; then a paged decode step of those 64
    sequences, whose states sit at seeded slots of a 256-slot pool."""
    import numpy as np
    rng = np.random.default_rng(2024)
    lens = np.exp(rng.uniform(np.log(128), np.log(8192), 64)).astype(np.int64)
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T, Bv = int(offs[-1]), len(lens)
    qv, kv_, vv = (device_normal(torch, sid, (T, H, D)) for sid in (1, 2, 3))
    ov = torch.empty_like(qv)
    sv = torch.empty((Bv, H, D, D), dtype=torch.float32, device="cuda")
    nb = la.la_fwd_varlen_workspace_bytes(offs, H, D, BK, la.LA_BF16)
    wsv = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
    pre = lambda: la.la_fwd_varlen(qv, kv_, vv, lam, offs, BK, out=ov, kv_out=sv, ws=wsv)
    for _ in range(3):
        pre()
    pre_ms = timed(pre, 20)
    pre_bytes = T * H * 8 * D + Bv * H * D * D * 4
    pool = torch.zeros((256, H, D, D), dtype=torch.float32, device="cuda")
    slots = rng.permutation(256)[:Bv]
    pool[torch.from_numpy(slots).cuda()] = sv
    slot_of = torch.from_numpy(slots.astype(np.int32)).cuda()
    dq_, dk_, dv_ = (device_normal(torch, 16 + i, (Bv, H, D)) for i in range(3))
    od = torch.empty_like(dq_)
    dec = lambda: la.la_decode_step_paged(pool, slot_of, dq_, dk_, dv_, lam, out=od)
    for _ in range(3):
        dec()
    dec_ms = timed(dec, 50)
    dec_bytes = Bv * H * (8 * D * D + 8 * D)
    return {"workload": f"ragged prefill of {Bv} sequences (lengths log-uniform in [128, 8192], "
                        f"{T} tokens), 16 heads, d=128, one launch; then paged decode of the {Bv} "
                        f"sequences in a 256-slot state pool",
            "prefill_ms": round(pre_ms, 4), "prefill_tokens_per_s": round(T / (pre_ms * 1e-3)),
            "prefill_gbs": round(pre_bytes / (pre_ms * 1e-3) / 1e9, 1),
            "decode_step_ms": round(dec_ms, 4), "decode_tokens_per_s": round(Bv / (dec_ms * 1e-3)),
            "decode_gbs": round(dec_bytes / (dec_ms * 1e-3) / 1e9, 1),
            "note": "the 64 decode states (64 MB) fit the 256 MB infinity cache, so the decode "
                    "rate is not an HBM figure"}


# ----------------------------------------------------------------------------- breakdowns
def kernel_breakdown(torch, la, fn, reps):
    """Per library kernel of one call of fn: launches and average microseconds, from HIP events
    the library records around each launch on its stream."""
    torch.cuda.synchronize()
    la.la_prof_collect()
    la.la_prof_enable(True)
    for _ in range(reps):
        fn()
    torch.cuda.synchronize()
    prof = la.la_prof_collect()
    la.la_prof_enable(False)
    out = {nm: {"launches_per_call": launches / reps, "avg_us": round(1e3 * total / launches, 2)}
           for nm, (launches, total) in prof.items()}
    out["sum_us_per_call"] = round(sum(1e3 * total / reps for _, total in prof.values()), 2)
    return out


# untimed calls before every named workload is timed (first calls pay code-object loading,
# TLB warm-up of fresh allocations and clock ramp-up)
WARMUP_CALLS = 20


def median_ms(torch, fn, reps):
    """Milliseconds per call as the median over reps calls, each bracketed by its own pair of
    HIP events on the current stream (so launch gaps between calls are left out)."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in ev)
    return t[len(t) // 2]


GRAPH_WARM_REPLAYS = 5


def graph_ms(torch, fn, reps):
    """fn captured once in a HIP graph (torch.cuda.CUDAGraph) and replayed: milliseconds per
    replay, which leaves out the host side of every launch.  The first replays of a new graph
    run slower (the training step: 0.509 ms per replay timed after one untimed replay, 0.468
    after three), so a few untimed replays come first, as the eager timings have their untimed
    calls."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for _ in range(GRAPH_WARM_REPLAYS):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del g
    return ms


# ----------------------------------------------------------------------------- other workloads
def other_workloads(torch, la, timed):
    """The remaining named workloads, each timed on its own (inputs resident, HIP events):
    bf16 forward B4 H16 N2048; the training step B2 H32 N8192 (fwd, then bwd with the
    forward's chunk states); the long-context prefill B1 H64 N262144 at block 128."""
    import synth
    out = {}

    def fwd_case(name, B, Hh, N, bk, reps):
        lam_h = synth.decay_schedule(Hh)
        q, k, v = (device_normal(torch, sid, (B, Hh, N, D)) for sid in (1, 2, 3))
        o = torch.empty_like(q)
        s = torch.empty((B, Hh, D, D), dtype=torch.float32, device="cuda")
        ws = torch.empty(max(la.la_fwd_workspace_bytes(B, Hh, N, D, bk, la.LA_BF16), 1), dtype=torch.uint8,
                         device="cuda")
        fn = lambda: la.la_fwd(q, k, v, lam_h, bk, out=o, kv_out=s, ws=ws)
        for _ in range(WARMUP_CALLS):
            fn()
        ms = timed(fn, reps)
        byts = 8 * D * B * Hh * N + B * Hh * D * D * 4
        plan = la.la_plan(B, Hh, N, D, bk, la.LA_BF16)
        stepped = 64 if bk >= 64 and D == 128 and os.environ.get("LA_FWD128") != "1" else bk
        out[name] = {"workload": f"bf16 forward B{B} H{Hh} N{N} d{D} block {bk}, per-head decay, final state"
                                 + (f" (chunk boundaries on multiples of {bk}; the kernel steps {stepped}-token "
                                    "blocks, the same function)" if stepped != bk else ""),
                     "kernel_block": stepped,
                     "plan": plan, "ms": round(ms, 4), "median_ms": round(median_ms(torch, fn, reps), 4),
                     "graph_ms": round(graph_ms(torch, fn, reps), 4),
                     "tokens_per_s": round(B * N / (ms * 1e-3)),
                     "gbs": round(byts / (ms * 1e-3) / 1e9, 1),
                     "frac_of_8tbs": round(byts / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "kernels": kernel_breakdown(torch, la, fn, max(3, reps // 4))}
        del q, k, v, o, s, ws

    fwd_case("fwd_b4_h16_n2048", 4, 16, 2048, BK, 200)

    # the float32 correctness shape: latency-bound, its time only (no roofline)
    Hh, N1, D1 = 2, 256, 16
    q, k, v = (torch.randn(1, Hh, N1, D1, device="cuda", generator=torch.Generator(device="cuda").manual_seed(sid))
               .div(math.sqrt(D1)) for sid in (1, 2, 3))
    o = torch.empty_like(q)
    s = torch.empty((1, Hh, D1, D1), dtype=torch.float32, device="cuda")
    fn = lambda: la.la_fwd(q, k, v, [1.0] * Hh, BK, out=o, kv_out=s)
    for _ in range(WARMUP_CALLS):
        fn()
    out["fwd_fp32_b1_h2_n256_d16"] = {
        "workload": f"float32 forward B1 H{Hh} N{N1} d{D1} block {BK}, no decay (lambda = 1), final state; "
                    "generic kernels, latency-bound (time only)",
        "plan": la.la_plan(1, Hh, N1, D1, BK, la.LA_F32), "median_ms": round(median_ms(torch, fn, 200), 4),
        "ms": round(timed(fn, 200), 4), "kernels": kernel_breakdown(torch, la, fn, 20)}
    del q, k, v, o, s

    B, Hh, N = 2, 32, 8192
    lam_h = synth.decay_schedule(Hh)
    q, k, v, g = (device_normal(torch, sid, (B, Hh, N, D)) for sid in (1, 2, 3, 4))
    o, dq, dk, dv = (torch.empty_like(q) for _ in range(4))
    s = torch.empty((B, Hh, D, D), dtype=torch.float32, device="cuda")
    wf = la.la_fwd_workspace_bytes(B, Hh, N, D, BK, la.LA_BF16)
    ws_f = torch.empty(max(wf, 1), dtype=torch.uint8, device="cuda")
    ws_b = torch.empty(max(la.la_bwd_workspace_bytes(B, Hh, N, D, BK, la.LA_BF16), 1), dtype=torch.uint8,
                       device="cuda")

    def train():
        la.la_fwd(q, k, v, lam_h, BK, out=o, kv_out=s, ws=ws_f)
        la.la_bwd(q, k, v, g, lam_h, BK, dq=dq, dk=dk, dv=dv, ws=ws_b, fwd_ws=ws_f if wf else None)
    for _ in range(WARMUP_CALLS):
        train()
    ms = timed(train, 50)
    byts = (8 + 14) * D * B * Hh * N
    out["train_b2_h32_n8192"] = {"workload": "bf16 fwd+bwd B2 H32 N8192 d128 block 64, per-head decay",
                                 "plan": la.la_plan(B, Hh, N, D, BK, la.LA_BF16),
                                 "ms": round(ms, 4), "median_ms": round(median_ms(torch, train, 50), 4),
                                 "graph_ms": round(graph_ms(torch, train, 50), 4),
                                 "tokens_per_s": round(B * N / (ms * 1e-3)),
                                 "gbs": round(byts / (ms * 1e-3) / 1e9, 1),
                                 "frac_of_8tbs": round(byts / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                 "kernels": kernel_breakdown(torch, la, train, 5)}
    del q, k, v, g, o, dq, dk, dv, s, ws_f, ws_b

    fwd_case("prefill_b1_h64_n262144_block128", 1, 64, 262144, 128, 50)
    return out


# ----------------------------------------------------------------------------- counter runs
def profile_all(args):
    """One call of every workload, for rocprofv3 counter runs (no timing loops): the sweep step
    (la_fwd + la_bwd at every n), la_dlam at every n, the bf16 forward B4 H16 N2048, the
    training step B2 H32 N8192, the long-context prefill B1 H64 N262144 at block 128, the
    decode step (256 sequences x 64 heads), the ragged prefill and paged decode, and a 1 GiB
    device copy (the byte counters' calibration).  Prints one line per workload."""
    import numpy as np
    import torch
    import causal_linear_attention_tiled_amd as la
    import synth

    def say(msg):
        print(f"[profile-all] {msg}", flush=True)

    lam = synth.decay_schedule(H)
    only = set(args.only.split(",")) if args.only else None
    want = lambda name: only is None or name in only
    for n in SWEEP_N if (want("sweep") or want("dlam")) else ():
        B = TOKENS_PER_POINT // n
        q, k, v, g = (device_normal(torch, sid, (B, H, n, D)) for sid in (1, 2, 3, 4))
        ws_f = torch.empty(max(la.la_fwd_workspace_bytes(B, H, n, D, BK, la.LA_BF16), 1), dtype=torch.uint8,
                           device="cuda")
        if want("sweep"):
            o, s = la.la_fwd(q, k, v, lam, BK, ws=ws_f)
            la.la_bwd(q, k, v, g, lam, BK, fwd_ws=ws_f if la.la_fwd_workspace_bytes(B, H, n, D, BK, la.LA_BF16)
                      else None)
            torch.cuda.synchronize()
            say(f"sweep n={n}")
        if want("dlam"):
            la.la_dlam(q, k, v, g, lam, BK)
            torch.cuda.synchronize()
            say(f"dlam n={n}")
        del q, k, v, g, ws_f
    if want("fwd2048"):
        q, k, v = (device_normal(torch, sid, (4, 16, 2048, D)) for sid in (1, 2, 3))
        la.la_fwd(q, k, v, lam, BK)
        torch.cuda.synchronize()
        say("forward B4 H16 N2048")
        del q, k, v
    if want("train"):
        lam32 = synth.decay_schedule(32)
        q, k, v, g = (device_normal(torch, sid, (2, 32, 8192, D)) for sid in (1, 2, 3, 4))
        ws_f = torch.empty(max(la.la_fwd_workspace_bytes(2, 32, 8192, D, BK, la.LA_BF16), 1), dtype=torch.uint8,
                           device="cuda")
        la.la_fwd(q, k, v, lam32, BK, ws=ws_f)
        la.la_bwd(q, k, v, g, lam32, BK, fwd_ws=ws_f)
        torch.cuda.synchronize()
        say("training step B2 H32 N8192")
        del q, k, v, g, ws_f
    if want("prefill"):
        lam64 = synth.decay_schedule(64)
        q, k, v = (device_normal(torch, sid, (1, 64, 262144, D)) for sid in (1, 2, 3))
        la.la_fwd(q, k, v, lam64, 128)
        torch.cuda.synchronize()
        say("long-context prefill B1 H64 N262144 block 128")
        del q, k, v
    if want("decode"):
        lam64 = synth.decay_schedule(64)
        state = torch.zeros((256, 64, D, D), dtype=torch.float32, device="cuda")
        dq_, dk_, dv_ = (device_normal(torch, 16 + i, (256, 64, D)) for i in range(3))
        la.la_decode_step(state, dq_, dk_, dv_, lam64)
        torch.cuda.synchronize()
        say("decode step 256 x 64")
        del state, dq_, dk_, dv_
    if want("serving"):
        rng = np.random.default_rng(2024)
        lens = np.exp(rng.uniform(np.log(128), np.log(8192), 64)).astype(np.int64)
        offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
        T = int(offs[-1])
        qv, kv_, vv = (device_normal(torch, sid, (T, H, D)) for sid in (1, 2, 3))
        _, sv = la.la_fwd_varlen(qv, kv_, vv, lam, offs, BK)
        pool = torch.zeros((256, H, D, D), dtype=torch.float32, device="cuda")
        slots = rng.permutation(256)[:len(lens)]
        pool[torch.from_numpy(slots).cuda()] = sv
        slot_of = torch.from_numpy(slots.astype(np.int32)).cuda()
        d3 = [device_normal(torch, 16 + i, (len(lens), H, D)) for i in range(3)]
        la.la_decode_step_paged(pool, slot_of, *d3, lam)
        torch.cuda.synchronize()
        say(f"ragged prefill ({T} tokens) and paged decode")
        del qv, kv_, vv, pool, d3
    if args.calib_copy:
        src = torch.empty(CALIB_BYTES // 2, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        say("calibration copy 1 GiB")


# ----------------------------------------------------------------------------- main bench
def bench(args):
    import numpy as np
    import torch

    so = os.path.join(ROOT, "causal_linear_attention_tiled_amd", "liblinattn.so")
    if not os.path.exists(so):
        import __graft_entry__
        __graft_entry__.build()
    import causal_linear_attention_tiled_amd as la
    import synth

    torch.cuda.init()
    lam = synth.decay_schedule(H)
    shapes = []
    for n in SWEEP_N:
        B = TOKENS_PER_POINT // n
        q, k, v, g = (device_normal(torch, sid, (B, H, n, D)) for sid in (1, 2, 3, 4))
        o, dq, dk, dv = (torch.empty_like(q) for _ in range(4))
        s = torch.empty((B, H, D, D), dtype=torch.float32, device="cuda")
        wf = la.la_fwd_workspace_bytes(B, H, n, D, BK, la.LA_BF16)
        wb = la.la_bwd_workspace_bytes(B, H, n, D, BK, la.LA_BF16)
        ws_f = torch.empty(max(wf, 1), dtype=torch.uint8, device="cuda")
        ws_b = torch.empty(max(wb, 1), dtype=torch.uint8, device="cuda")
        plan = la.la_plan(B, H, n, D, BK, la.LA_BF16)
        chunks, agg = plan["chunks"], plan["agg_parts"]
        shapes.append(dict(n=n, B=B, q=q, k=k, v=v, g=g, o=o, s=s, dq=dq, dk=dk, dv=dv, ws_f=ws_f,
                           ws_b=ws_b, chunks=chunks, agg=agg))
    torch.cuda.synchronize()

    def fwd(sh):
        la.la_fwd(sh["q"], sh["k"], sh["v"], lam, BK, out=sh["o"], kv_out=sh["s"], ws=sh["ws_f"])

    def bwd(sh):
        # the forward of the same step left its chunk states in ws_f
        la.la_bwd(sh["q"], sh["k"], sh["v"], sh["g"], lam, BK, dq=sh["dq"], dk=sh["dk"], dv=sh["dv"],
                  ws=sh["ws_b"], fwd_ws=sh["ws_f"] if sh["chunks"] > 1 else None)

    def step():
        for sh in shapes:
            fwd(sh)
            bwd(sh)

    def timed(fn, reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ms_per_step = timed(step, args.steps)
    wall = time.perf_counter() - t0
    tokens_per_step = TOKENS_PER_POINT * len(SWEEP_N)
    value = tokens_per_step / (ms_per_step * 1e-3)
    if args.calib_copy:
        # a plain device copy of known size, for calibrating the HBM byte counters
        src = torch.empty(CALIB_BYTES // 2, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
    if args.quick:
        print(json.dumps({"ms_per_step": round(ms_per_step, 4), "value": round(value, 1)}), flush=True)
        return

    # second pass over the same steps with per-kernel HIP events (on the launch stream)
    la.la_prof_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    prof = la.la_prof_collect()
    la.la_prof_enable(False)

    # algorithmic bytes per launch for every kernel (same launches, same order every step)
    bytes_by_kernel = {}
    for sh in shapes:
        names = ["fwd_mfma", "dq_mfma", "fwd_dma", "dq_dma", "dkdv_mfma", "dkdv_generic", "dkdv_dma"]
        if sh["chunks"] > 1:
            names += ["chunk_state_mfma", "chunk_state_rev_mfma", "chunk_state_dma", "chunk_state_rev_dma",
                      "state_scan", "state_scan_rev"]
        for nm in names:
            b = kernel_bytes(nm, sh["B"], H, sh["n"], D, sh["chunks"], sh["agg"])
            bytes_by_kernel.setdefault(nm, []).append(b)
    kernels = {}
    for nm, (launches, total_ms) in prof.items():
        avg_ms = total_ms / launches
        per_step_bytes = sum(bytes_by_kernel.get(nm, [])) or None
        launches_per_step = launches / args.steps
        avg_bytes = per_step_bytes / launches_per_step if per_step_bytes else None
        kernels[nm] = {"device_function": DEVICE_FN.get(nm, nm), "launches_per_step": launches_per_step,
                       "avg_ms": round(avg_ms, 5), "share": None, "alg_bytes_per_launch": avg_bytes,
                       "gbs": (avg_bytes / (avg_ms * 1e-3) / 1e9) if avg_bytes else None,
                       "counters": read_mfma(DEVICE_FN.get(nm, nm))}
    total_prof = sum(v[1] for v in prof.values())
    for nm in kernels:
        kernels[nm]["share"] = round(prof[nm][1] / total_prof, 4)
    # the same per device function: the dominant kernel is the device function that takes
    # the most time (launches of one function by several library calls pooled)
    by_fn = {}
    for nm, (launches, total_ms) in prof.items():
        f = by_fn.setdefault(DEVICE_FN.get(nm, nm), {"launches": 0, "total_ms": 0.0, "bytes": 0.0,
                                                     "calls": [], "known": True})
        f["launches"] += launches
        f["total_ms"] += total_ms
        f["calls"].append(nm)
        b = sum(bytes_by_kernel.get(nm, [])) * args.steps
        f["bytes"] += b
        f["known"] &= b > 0
    dom = max(by_fn, key=lambda k_: by_fn[k_]["total_ms"])
    df = by_fn[dom]
    avg_ms = df["total_ms"] / df["launches"]
    avg_bytes = df["bytes"] / df["launches"] if df["known"] else None
    achieved = avg_bytes / (avg_ms * 1e-3) / 1e9 if avg_bytes else None
    roofline = {"bound": "hbm", "kernel": dom, "library_calls": df["calls"],
                "achieved": round(achieved, 1) if achieved else None,
                "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4) if achieved else None,
                "traffic": read_traffic(dom), "avg_launch_ms": round(avg_ms, 5),
                "launches_per_step": df["launches"] / args.steps, "alg_bytes_per_launch": avg_bytes,
                "share": round(df["total_ms"] / total_prof, 4),
                "counters": read_mfma(dom)}

    # per sequence length breakdown
    sweep = []
    for sh in shapes:
        reps = max(3, args.steps)
        f_ms = timed(lambda: fwd(sh), reps)
        b_ms = timed(lambda: bwd(sh), reps)
        th = sh["B"] * H * sh["n"]
        ff, bf = fwd_flops_per_token_head() * th, bwd_flops_per_token_head() * th
        fbytes = 8 * D * th + sh["B"] * H * D * D * 4
        bbytes = 14 * D * th
        sweep.append({
            "n": sh["n"], "batch": sh["B"], "chunks": sh["chunks"], "agg_parts": sh["agg"],
            "fwd_ms": round(f_ms, 4), "fwd_tokens_per_s": round(TOKENS_PER_POINT / (f_ms * 1e-3)),
            "fwd_tflops": round(ff / (f_ms * 1e-3) / 1e12, 1),
            "fwd_pct_bf16_peak": round(100 * ff / (f_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 2),
            "fwd_gbs": round(fbytes / (f_ms * 1e-3) / 1e9, 1),
            "bwd_ms": round(b_ms, 4), "bwd_tokens_per_s": round(TOKENS_PER_POINT / (b_ms * 1e-3)),
            "bwd_tflops": round(bf / (b_ms * 1e-3) / 1e12, 1),
            "bwd_gbs": round(bbytes / (b_ms * 1e-3) / 1e9, 1),
            "fwd_bwd_tokens_per_s": round(TOKENS_PER_POINT / ((f_ms + b_ms) * 1e-3)),
        })
    fwd_tps = [x["fwd_tokens_per_s"] for x in sweep]

    # derivative with respect to the decay (la_dlam) over the same inputs, per sequence length
    dlam = []
    for sh in shapes:
        wsd = torch.empty(la.la_dlam_workspace_bytes(sh["B"], H, sh["n"], D, BK, la.LA_BF16), dtype=torch.uint8,
                          device="cuda")
        outd = torch.empty(H, dtype=torch.float32, device="cuda")
        run_dlam = lambda: la.la_dlam(sh["q"], sh["k"], sh["v"], sh["g"], lam, BK, out=outd, ws=wsd)
        run_dlam()
        d_ms = timed(run_dlam, max(3, args.steps))
        th = sh["B"] * H * sh["n"]
        # Q, K, V, dO read by the sweep, and K, V once more by the chunk aggregates
        dbytes = 8 * D * th + (4 * D * th * (sh["chunks"] - 1) / sh["chunks"] if sh["chunks"] > 1 else 0)
        dlam.append({"n": sh["n"], "batch": sh["B"], "chunks": sh["chunks"], "ms": round(d_ms, 4),
                     "tokens_per_s": round(TOKENS_PER_POINT / (d_ms * 1e-3)),
                     "gbs": round(dbytes / (d_ms * 1e-3) / 1e9, 1)})

    # recurrent decode step: 256 sequences x 64 heads, float32 state 1 GiB
    Bs, Hd = 256, 64
    lam_d = synth.decay_schedule(Hd)
    state = torch.zeros((Bs, Hd, D, D), dtype=torch.float32, device="cuda")
    dq_, dk2, dv2 = (device_normal(torch, 16 + i, (Bs, Hd, D)) for i in range(3))
    od = torch.empty_like(dq_)
    dec = lambda: la.la_decode_step(state, dq_, dk2, dv2, lam_d, out=od)
    for _ in range(3):
        dec()
    dec_ms = timed(dec, 50)
    dec_bytes = Bs * Hd * (8 * D * D + 8 * D)
    decode = {"workload": "recurrent decode step, 256 sequences x 64 heads, d=128, float32 state",
              "ms": round(dec_ms, 4), "gbs": round(dec_bytes / (dec_ms * 1e-3) / 1e9, 1),
              "frac_of_8tbs": round(dec_bytes / (dec_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
              "tokens_per_s": round(Bs / (dec_ms * 1e-3))}

    serving = serving_workload(torch, la, lam, timed)
    workloads = other_workloads(torch, la, timed)

    tflops_step = sum((fwd_flops_per_token_head() + bwd_flops_per_token_head()) * TOKENS_PER_POINT * H
                      for _ in SWEEP_N) / (ms_per_step * 1e-3) / 1e12
    tflops_exec = sum((fwd_flops_per_token_head() + bwd_flops_executed_per_token_head()) * TOKENS_PER_POINT * H
                      for _ in SWEEP_N) / (ms_per_step * 1e-3) / 1e12
    rates = hbm_rates(torch, timed)
    floor, floor_ms = flatness_floor(sweep, rates)
    for x, f in zip(sweep, floor_ms):
        x["fwd_floor_ms"] = round(f, 4)
    out = {
        # value: fwd+bwd tokens/s over the whole sweep (131072 tokens per point); the per-point
        # tokens/s, TFLOP/s and % of bf16 peak are under "sweep", the step's under "tflops_alg"
        "metric": "fwd/bwd tokens/s + TFLOP/s (% bf16 MFMA peak) vs seq len 1K\u201364K, 1 GPU",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: seeded N(0,1)/sqrt(d) inputs, resident in HBM",
        "config": {"workload": "causal linear attention fwd+bwd, seq-length sweep n in {1024,4096,16384,65536}, "
                               "batch 131072/n, heads 16, d 128, block 64, per-head decay",
                   "tokens_per_step": tokens_per_step, "heads": H, "head_dim": D, "block": BK},
        "tflops_alg": round(tflops_step, 1),
        "pct_bf16_peak": round(100 * tflops_step / BF16_PEAK_TFLOPS, 2),
        "tflops_alg_counts": "forward 2d(Bk+1)+4d^2, backward 5d(Bk+1)+8d^2 flop per token-head",
        "tflops_executed_count": round(tflops_exec, 1),
        "tflops_executed_note": "backward counted with the dQ sweep's own state carry (+2d^2)",
        "roofline": roofline,
        "sweep": sweep,
        "fwd_flatness": round(max(fwd_tps) / min(fwd_tps), 3),
        "fwd_flatness_floor": round(floor, 3),
        "fwd_flatness_floor_note": "the forward's flatness if every sweep point ran at hbm_rates (reads and "
                                   "writes not overlapping), with the chunk aggregates' extra reads of K, V",
        "hbm_rates": rates,
        "kernels": kernels,
        "decode": decode,
        "serving": serving,
        "decay_gradient": dlam,
        "workloads": workloads,
        "wall_s_timed": round(wall, 3),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(out), flush=True)


# ----------------------------------------------------------------------------- rocprofv3 summaries


def _csv(dirname, suffix):
    files = glob.glob(os.path.join(dirname, "**", f"*{suffix}"), recursive=True)
    if not files:
        raise SystemExit(f"no *{suffix} under {dirname}")
    return list(csv.DictReader(open(files[0])))


def _counter_means(dirname, counter):
    """{kernel name: (dispatches, mean counter value per dispatch)} from a --pmc run."""
    by = {}
    for r in _csv(dirname, "counter_collection.csv"):
        if r["Counter_Name"] == counter:
            by.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return {k: (len(v), sum(v) / len(v)) for k, v in by.items()}


def _fn(kernel_name):
    """Device function of a demangled kernel name ('k_fwd_dma' from '... ::k_fwd_dma<4, false>(...)'),
    else the name up to its argument list."""
    import re
    m = re.search(r"(k_[A-Za-z0-9_]+)\s*[<(]", kernel_name)
    return m.group(1) if m else kernel_name.split("(")[0][-60:]


def _dispatch_table(dirname):
    """{dispatch id: {"fn", "name", "grid", counters...}} from a --pmc run (with or without a
    kernel trace in the same directory; durations in ns when one is there)."""
    rows = _csv(dirname, "counter_collection.csv")
    disp = {}
    for r in rows:
        did = r.get("Dispatch_Id") or r.get("Correlation_Id")
        d = disp.setdefault(did, {"fn": _fn(r["Kernel_Name"]), "name": r["Kernel_Name"],
                                  "grid": int(float(r.get("Grid_Size", 0) or 0))})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        if r.get("Start_Timestamp") and r.get("End_Timestamp"):
            d["ns"] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
    try:
        trace = _csv(dirname, "kernel_trace.csv")
    except SystemExit:
        trace = []
    for r in trace:
        did = r.get("Dispatch_Id") or r.get("Correlation_Id")
        if did in disp:
            disp[did]["ns"] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
    return disp


def _groups(disp, key):
    by = {}
    for d in disp.values():
        by.setdefault(key(d), []).append(d)
    return by


def summarize(args):
    """Summarize rocprofv3 output into short text files (see --help).

    stats:   kernel table from --kernel-trace --stats
    fetch / write: per-kernel FETCH_SIZE / WRITE_SIZE means from a --pmc run
    traffic: HBM bytes per launch of --kernel from the FETCH_SIZE and WRITE_SIZE runs,
             each scaled by what the same counter reads for the 1 GiB calibration copy."""
    os.makedirs(args.out, exist_ok=True)
    lines = [f"# command: {args.command}"]
    if args.kind == "stats":
        rows = _csv(args.dir, "kernel_stats.csv")
        lines.append("kernel | calls | avg_us | total_ms | pct")
        for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
            lines.append(f"{r['Name'][:110]} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                         f"{float(r['TotalDurationNs']) / 1e6:.3f} | {float(r['Percentage']):.2f}")
        out = os.path.join(args.out, f"kernels_{args.tag}_stats.txt")
    elif args.kind in ("fetch", "write"):
        counter = "FETCH_SIZE" if args.kind == "fetch" else "WRITE_SIZE"
        lines.append(f"kernel | dispatches | mean {counter} (KiB per dispatch)")
        for k, (n, mean) in sorted(_counter_means(args.dir, counter).items()):
            lines.append(f"{k[:110]} | {n} | {mean:.1f}")
        out = os.path.join(args.out, f"counters_{args.tag}_{args.kind}.txt")
    elif args.kind == "pmc":
        # every counter of the run, mean per dispatch, per (device function, grid size)
        disp = _dispatch_table(args.dir)
        names = sorted({k for d in disp.values() for k in d if k not in ("fn", "name", "grid", "ns")})
        lines.append("function | grid | dispatches | " + " | ".join(f"mean {n}" for n in names))
        for (fn, grid), ds in sorted(_groups(disp, lambda d: (d["fn"], d["grid"])).items()):
            means = [sum(d.get(n, 0.0) for d in ds) / len(ds) for n in names]
            lines.append(f"{fn} | {grid} | {len(ds)} | " + " | ".join(f"{m:.4g}" for m in means))
        out = os.path.join(args.out, f"counters_{args.tag}_{args.name}.txt")
    elif args.kind == "mfma":
        # matrix-core work against the bf16 dense peak: rocprof's MfmaFlopsBF16 (MOPS x 512),
        # MfmaUtil, VALUBusy and LdsUtil per dispatch, with the dispatch durations of the same run
        disp = _dispatch_table(args.dir)
        lines.append(f"peak: {BF16_PEAK_TFLOPS} TFLOP/s bf16 dense (MI355X published)")
        lines.append("function | grid | dispatches | avg_us | mfma_gflop_per_dispatch | mfma_tflops | "
                     "pct_bf16_peak | MfmaUtil | VALUBusy | LdsUtil | source_sha256_16")

        def row(label, grid, ds):
            ns = sum(d.get("ns", 0.0) for d in ds)
            fl = sum(d.get("MfmaFlopsBF16", 0.0) for d in ds)
            w = lambda key: (sum(d.get(key, 0.0) * d.get("ns", 0.0) for d in ds) / ns) if ns else float("nan")
            tf = fl / ns / 1e3 if ns else float("nan")
            return (f"{label} | {grid} | {len(ds)} | {ns / len(ds) / 1e3:.2f} | {fl / len(ds) / 1e9:.3f} | "
                    f"{tf:.1f} | {100 * tf / BF16_PEAK_TFLOPS:.2f} | {w('MfmaUtil'):.2f} | {w('VALUBusy'):.2f} | "
                    f"{w('LdsUtil'):.2f} | {source_digest(label)}")
        for (fn, grid), ds in sorted(_groups(disp, lambda d: (d["fn"], d["grid"])).items()):
            lines.append(row(fn, grid, ds))
        lines.append("# totals per device function (durations summed, utilisations duration-weighted)")
        for fn, ds in sorted(_groups(disp, lambda d: d["fn"]).items()):
            lines.append(row(fn, "all", ds))
        out = os.path.join(args.out, f"mfma_{args.tag}.txt")
    else:
        fetch = _dispatch_table(args.fetch)
        write = _dispatch_table(args.write)
        sym = args.kernel

        def pick(disp, counter, match):
            ds = [d for d in disp.values() if match(d) and counter in d]
            return (len(ds), sum(d[counter] for d in ds) / len(ds)) if ds else None
        is_copy = lambda d: "copy" in d["name"] or "elementwise" in d["name"]
        is_k = lambda d: d["fn"] == sym and (not args.grid or d["grid"] == args.grid)
        copy_f = [d["FETCH_SIZE"] for d in fetch.values() if is_copy(d) and "FETCH_SIZE" in d]
        copy_w = [d["WRITE_SIZE"] for d in write.values() if is_copy(d) and "WRITE_SIZE" in d]
        kf, kw = pick(fetch, "FETCH_SIZE", is_k), pick(write, "WRITE_SIZE", is_k)
        if not (copy_f and copy_w and kf and kw):
            raise SystemExit("kernel or calibration copy missing from the counter runs")
        calib_kib = CALIB_BYTES / 1024
        f_fetch = calib_kib / max(copy_f)
        f_write = calib_kib / max(copy_w)
        fetch_b = kf[1] * f_fetch * 1024
        write_b = kw[1] * f_write * 1024
        lines += [f"kernel: {args.kernel} (dispatches of that device function"
                  + (f" with grid size {args.grid})" if args.grid else ")"),
                  f"dispatches: {kf[0]}",
                  f"fetch_kib_per_dispatch_raw: {kf[1]:.1f}",
                  f"write_kib_per_dispatch_raw: {kw[1]:.1f}",
                  f"calibration: 1 GiB device copy; FETCH_SIZE scale {f_fetch:.4f}, WRITE_SIZE scale {f_write:.4f}",
                  f"hbm_fetch_bytes_per_launch: {fetch_b:.0f}",
                  f"hbm_write_bytes_per_launch: {write_b:.0f}",
                  f"hbm_bytes_per_launch: {fetch_b + write_b:.0f}",
                  f"source_sha256_16: {source_digest(args.kernel)}"]
        if args.alg_bytes:
            lines.append(f"algorithmic_bytes_per_launch: {args.alg_bytes:.0f}")
            lines.append(f"measured_over_algorithmic: {(fetch_b + write_b) / args.alg_bytes:.4f}")
        out = os.path.join(args.out, f"{args.kernel}_{args.tag}_traffic.txt")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("wrote", out)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--quick", action="store_true", help="timed steps only (for profiled runs)")
    ap.add_argument("--calib-copy", action="store_true", help="also run a 1 GiB device copy")
    ap.add_argument("--profile-all", action="store_true",
                    help="one call of every workload and nothing timed (for rocprofv3 counter runs)")
    ap.add_argument("--only", default="", help="--profile-all: comma-separated subset of "
                    "sweep,dlam,fwd2048,train,prefill,decode,serving")
    ap.add_argument("--out", default=PROFILES, help="summarize: output directory")
    ap.add_argument("--fetch", default="", help="summarize --kind traffic: FETCH_SIZE run dir")
    ap.add_argument("--write", default="", help="summarize --kind traffic: WRITE_SIZE run dir")
    ap.add_argument("--kernel", default="k_fwd_dma", help="summarize --kind traffic: device function")
    ap.add_argument("summarize", nargs="?", help=argparse.SUPPRESS)
    ap.add_argument("--kind", choices=["stats", "fetch", "write", "traffic", "pmc", "mfma"], default="stats")
    ap.add_argument("--name", default="pmc", help="summarize --kind pmc: file name part")
    ap.add_argument("--grid", type=int, default=0, help="summarize --kind traffic: only dispatches of this grid size")
    ap.add_argument("--alg-bytes", type=float, default=0.0,
                    help="summarize --kind traffic: algorithmic bytes per launch, for the ratio")
    ap.add_argument("--dir", default="")
    ap.add_argument("--tag", default="sweep")
    ap.add_argument("--command", default="")
    args = ap.parse_args()
    if args.summarize == "summarize":
        return summarize(args)
    if args.profile_all:
        return profile_all(args)
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; the library has no multi-GPU "
                                   "path (sequences would shard by batch and head, or by sequence "
                                   "segments with one D x D state exchange)", "n_gpus": args.gpus}))
        sys.exit(2)
    bench(args)


if __name__ == "__main__":
    main()
