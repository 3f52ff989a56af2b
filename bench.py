"""Benchmark of the Wall Attention forward hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload long_bf16] [--gpus 1]

A step is one pass of the whole hot path over one batch of synthetic inputs
already resident in HBM: the log2 prefix scan of g (and of g_scalar when the
workload has one), the key-cache preparation and the fused forward kernel.
The default workload is the long-context causal case (B=1, T=8192, HQ=16,
H=4, K=V=128, bf16, bimodal gate), on which the headline metric is quoted.

Prints one JSON line.  ``value`` is whole-step throughput in counted TFLOP/s
(4*K per visible query/key pair and query head: 2K for QK^T and 2V for PV,
K = V), timed over K back-to-back steps after W untimed ones (the defaults
keep the timed steps in the steady state of the part's clocks, which the
first ~40 ms of work after idle do not reach); ``roofline`` prices the fused
forward kernel alone, timed with HIP events on the stream it is launched on
over a second pass of the same K steps (an event record leaves a gap on the
stream, so none sits in the timed region), against the dense bf16 MFMA peak;
``cpu_baseline`` times the fp64 oracle on a bounded row sample of the same
workload on this host.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "wall_attn_fwd causal TFLOP/s and % of bf16 MFMA peak, T=8192 HQ=16 K=128"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0
FWD_KERNEL_SOURCES = ["channel_decay_softmax_amd/csrc/wall_fwd_bf16.hip",
                      "channel_decay_softmax_amd/csrc/wall_common.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fwd_bf16_long_bf16_traffic.json")


def visible_pairs(lens, W):
    """Sum over query rows of the number of visible keys (causal, optional window)."""
    tot = 0
    for L in lens:
        if W and W > 0:
            w = min(W, L)
            tot += w * (w + 1) // 2 + (L - w) * w
        else:
            tot += L * (L + 1) // 2
    return tot


def seq_lengths(inp):
    if inp.cu_seqlens is not None:
        cu = inp.cu_seqlens.tolist()
        return [cu[i + 1] - cu[i] for i in range(len(cu) - 1)]
    return [inp.q.shape[1]] * inp.q.shape[0]


def source_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(workload):
    """Per-launch HBM bytes of the fused kernel, measured with rocprofv3 counters
    (see profiles/), or None when absent or taken on an older kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        rec = json.load(f)
    if rec.get("workload") != workload or rec.get("source_hash") != source_hash(FWD_KERNEL_SOURCES):
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(inp, flop_per_pair, target_s):
    """Time the fp64 oracle (as it stands) on a bounded sample of query rows."""
    import numpy as np

    import oracle

    oracle.build(force=False)
    lens = seq_lengths(inp)
    B, T = inp.q.shape[:2]
    HQ = inp.q.shape[2]
    W = inp.window_size
    # row r of a sequence starting at s sees min(r - s + 1, W) keys
    starts = []
    if inp.cu_seqlens is not None:
        cu = inp.cu_seqlens.tolist()
        for i, L in enumerate(lens):
            starts += [cu[i]] * L
    else:
        for b in range(B):
            starts += [b * T] * T
    starts = np.asarray(starts)
    keys = np.arange(B * T) - starts + 1
    if W:
        keys = np.minimum(keys, W)
    rng = np.random.default_rng(0)
    order = rng.permutation(B * T)

    def run(rows):
        t0 = time.perf_counter()
        oracle.wall_attn_oracle(inp.q, inp.k, inp.v, inp.g, scale=inp.scale, g_scalar=inp.g_scalar,
                                sink_bias=inp.sink_bias, window_size=W,
                                cu_seqlens=inp.cu_seqlens, rows=rows)
        return time.perf_counter() - t0

    # calibrate on a small sample, then size the timed sample to about target_s
    cal = order[:64]
    t_cal = run(cal)
    pairs_cal = int(keys[cal].sum()) * HQ
    rate = pairs_cal / max(t_cal, 1e-6)
    want_pairs = rate * target_s
    csum = np.cumsum(keys[order]) * HQ
    n = int(min(B * T, max(64, np.searchsorted(csum, want_pairs) + 1)))
    rows = np.sort(order[:n])
    t = run(rows)
    pairs = int(keys[rows].sum()) * HQ
    return {
        "value": pairs * flop_per_pair / t / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": f"{n} of {B * T} query rows (all {HQ} heads), {pairs} visible pairs, "
                  f"{t:.1f} s fp64 product form",
        "seconds": t,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=int(os.environ.get("WORLD_SIZE", "1")))
    # the part's clocks settle after about 40 ms of back-to-back steps (the
    # first steps after idle run up to 20% slower): the defaults warm up for
    # about 60 ms and time about 60 ms of steady state
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="long_bf16")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="run a plain device copy of this many MiB (read + write) before the "
                         "timed region, as the reference kernel for HBM byte counters")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus}): the Wall Attention forward "
              "is built and measured for a single GPU; see DESIGN.md for how it would shard.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import channel_decay_softmax_amd as wall
    from wall_inputs import make_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda", 0)
    inp = make_inputs(args.workload)
    d = inp.to(dev)
    B, T, HQ, K = d.q.shape
    H, V = d.k.shape[2], d.v.shape[3]
    lens = seq_lengths(inp)
    pairs = visible_pairs(lens, inp.window_size) * HQ
    flop_per_pair = 2 * K + 2 * V
    flop = pairs * flop_per_pair
    cu = d.cu_seqlens
    nseq = 0 if cu is None else cu.numel() - 1
    max_seqlen = max(lens)

    # every buffer is allocated before the timed region
    P = torch.empty((B, T, HQ, K), dtype=torch.float32, device=dev)
    G = None if d.g_scalar is None else torch.empty((B, T, HQ), dtype=torch.float32, device=dev)
    ws_scan = torch.empty(wall.prefix_scan_workspace_size(B, T, HQ * K), dtype=torch.uint8, device=dev)
    ws_fwd = torch.empty(wall.attn_fwd_workspace_size(d.q.dtype, B, T, HQ, H, K, V, nseq),
                         dtype=torch.uint8, device=dev)
    o = torch.empty((B, T, HQ, V), dtype=d.q.dtype, device=dev)
    lse = torch.empty((B, T, HQ), dtype=torch.float32, device=dev)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]

    def step(marks=None):
        if marks:
            marks[0].record()
        wall.wall_prefix_scan(d.g, cu, out=P, workspace=ws_scan)
        if G is not None:
            wall.wall_prefix_scan(d.g_scalar, cu, out=G, workspace=ws_scan)
        if marks:
            marks[1].record()
        wall.wall_attn_fwd_prepare(d.k, d.v, P, HQ, ws_fwd, cu)
        if marks:
            marks[2].record()
        wall.wall_attn_fwd_run(d.q, P, H, V, ws_fwd, o, lse, G=G, sink_bias=d.sink_bias,
                               scale=d.scale, window_size=inp.window_size, cu_seqlens=cu,
                               max_seqlen=max_seqlen)
        if marks:
            marks[3].record()

    if args.copy_mb:
        n = args.copy_mb * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)  # reads and writes copy_mb MiB each
        torch.cuda.synchronize()
        del src, dst
    print(f"[bench] {args.workload}: B={B} T={T} HQ={HQ} H={H} K={K} V={V} {d.q.dtype} "
          f"pairs={pairs} flop={flop:.4e}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print("[bench] warmup done", file=sys.stderr, flush=True)
    # the timed region: K whole steps back to back, nothing else on the stream
    t0 = time.perf_counter()
    for i in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    # then the same K steps with HIP events between the phases (an event record
    # leaves a gap of a few microseconds on the stream, so these are kept out
    # of the timed region): the per-phase split and the fused kernel's average
    # duration that prices it against the roofline
    for i in range(args.steps):
        step(ev[i])
    torch.cuda.synchronize()
    scan_ms = [e[0].elapsed_time(e[1]) for e in ev]
    prep_ms = [e[1].elapsed_time(e[2]) for e in ev]
    run_ms = [e[2].elapsed_time(e[3]) for e in ev]
    run_avg = statistics.fmean(run_ms)
    achieved = flop / (run_avg * 1e-3) / 1e12
    value = flop / (ms_step * 1e-3) / 1e12
    traffic = load_traffic(args.workload)
    print(f"[bench] step {ms_step:.3f} ms: scan {statistics.fmean(scan_ms)*1e3:.1f} us, "
          f"prepare {statistics.fmean(prep_ms)*1e3:.1f} us, fused {run_avg*1e3:.1f} us "
          f"(min {min(run_ms)*1e3:.1f}) -> fused {achieved:.1f} TFLOP/s", file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the fp64 oracle on the host", file=sys.stderr, flush=True)
        cpu = cpu_baseline(inp, flop_per_pair, args.cpu_seconds)

    dtype = {torch.bfloat16: "bf16", torch.float32: "f32"}[d.q.dtype]
    rec = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": args.workload, "B": B, "T": T, "HQ": HQ, "H": H, "K": K, "V": V,
                   "causal": True, "window_size": inp.window_size,
                   "g_scalar": inp.g_scalar is not None, "sink": inp.sink_bias is not None,
                   "num_seqs": nseq or None, "visible_pairs": pairs, "counted_flop": flop},
        "pct_of_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "stages_us": {"prefix_scan": round(statistics.fmean(scan_ms) * 1e3, 2),
                      "prepare": round(statistics.fmean(prep_ms) * 1e3, 2),
                      "fused_fwd": round(run_avg * 1e3, 2)},
        "roofline": {"kernel": "fwd_bf16_kernel<128,128>" if K == 128 else "fwd_bf16_kernel",
                     "bound": "mfma", "achieved": round(achieved, 3),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic},
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
