"""Benchmark of the Wall Attention forward hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload long_bf16] [--gpus 1]

A step is one pass of the whole hot path over one batch of synthetic inputs
already resident in HBM: the log2 prefix of g with the key-cache preparation
(wall_attn_fwd_prepare_gate, one combined pass on the long-context workload),
the prefix scan of g_scalar when the workload has one, and the fused forward
kernel.
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
``call`` beside it prices the forward's C-ABI calls (prefix and preparation,
fused kernel) the same way, and ``executed`` gives the matrix-core flops the
kernel really issues (from the rocprofv3 counters under profiles/): keys
whose scores are exactly -m in float32 are summed in closed form, so on a
decaying gate it issues fewer than the counted ones; float32 workloads are
priced against the vector fp32 peak (``bound: "alu"``).  ``cpu_baseline`` times the fp64 oracle on this
host on every row of the workload when that takes at most about a minute
(the long-context workload), else on a fixed row sample.
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
PEAK_F32_VALU_TFLOPS = 157.3  # MI355X vector fp32, published
PEAK_HBM_GBS = 8000.0
FWD_KERNEL_SOURCES = ["channel_decay_softmax_amd/csrc/wall_fwd_bf16.hip",
                      "channel_decay_softmax_amd/csrc/wall_common.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fwd_bf16_long_bf16_traffic.json")
MFMA_FILE = os.path.join(ROOT, "profiles", "fwd_bf16_long_bf16_mfma.json")
BWD_METRIC = "wall_attn_bwd causal TFLOP/s (dq, dk, dv, dg), T=8192 HQ=16 K=128"
DECODE_METRIC = "wall_attn_decode streaming step HBM GB/s (prefix and cache append of one token, split-KV decode), B=16 T=8192 HQ=16 K=128"
DECODE_KERNEL_SOURCES = ["channel_decay_softmax_amd/csrc/wall_decode.hip",
                         "channel_decay_softmax_amd/csrc/wall_common.h"]
DECODE_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_decode_bf16_traffic.json")
BWD_KERNEL_SOURCES = ["channel_decay_softmax_amd/csrc/wall_bwd_mfma.hip", "channel_decay_softmax_amd/csrc/wall_bwd.hip",
                      "channel_decay_softmax_amd/csrc/wall_scan.hip", "channel_decay_softmax_amd/csrc/wall_common.h"]
BWD_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "bwd_long_bf16_traffic.json")


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


def load_traffic(workload, path=TRAFFIC_FILE, sources=FWD_KERNEL_SOURCES):
    """Per-launch HBM bytes of the timed kernel, measured with rocprofv3 counters
    (see profiles/), or None when absent or taken on an older kernel source."""
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("workload") != workload or rec.get("source_hash") != source_hash(sources):
        return None
    return rec.get("bytes_per_launch")


def load_executed(workload):
    """Matrix-core flops the fused kernel executes per launch and its MFMA busy
    fraction, from rocprofv3 counters (see profiles/), or None when absent or
    taken on an older kernel source."""
    if not os.path.exists(MFMA_FILE):
        return None
    with open(MFMA_FILE) as f:
        rec = json.load(f)
    if rec.get("workload") != workload or rec.get("source_hash") != source_hash(FWD_KERNEL_SOURCES):
        return None
    return rec


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(inp, flop_per_pair, full_limit_s):
    """Time the fp64 oracle (as it stands) on every query row of the workload
    when a calibration predicts at most ``full_limit_s`` seconds for that,
    else on the first rows of a fixed seeded permutation sized to that time
    (the same rows on every run of one host).  Timed with time.perf_counter,
    the monotonic high-resolution clock."""
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
    order = np.random.default_rng(0).permutation(B * T)

    def run(rows):
        t0 = time.perf_counter()
        oracle.wall_attn_oracle(inp.q, inp.k, inp.v, inp.g, scale=inp.scale, g_scalar=inp.g_scalar,
                                sink_bias=inp.sink_bias, window_size=W,
                                cu_seqlens=inp.cu_seqlens, rows=rows)
        return time.perf_counter() - t0

    # calibrate on the last rows (the most keys), then run every row if it fits
    cal = np.arange(B * T - 64, B * T)
    rate = int(keys[cal].sum()) * HQ / max(run(cal), 1e-6)
    total_pairs = int(keys.sum()) * HQ
    if total_pairs / rate <= full_limit_s:
        rows = None
        n = B * T
        pairs = total_pairs
    else:
        csum = np.cumsum(keys[order]) * HQ
        n = int(min(B * T, max(64, np.searchsorted(csum, rate * full_limit_s) + 1)))
        rows = np.sort(order[:n])
        pairs = int(keys[rows].sum()) * HQ
    t = run(rows)
    return {
        "value": pairs * flop_per_pair / t / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": f"{n} of {B * T} query rows (all {HQ} heads), {pairs} visible pairs, "
                  f"{t:.1f} s fp64 product form, time.perf_counter",
        "seconds": t,
        "cpu": cpu_model(),
    }


def decode_bytes(B, T, HQ, H, K, V, C, es):
    """Algorithmic HBM bytes of one decode call and of one row's append (prefix
    row and cache row in one pass)."""
    nc = -(-T // C)
    dec = (B * T * HQ * K * es + B * T * H * V * es + B * nc * HQ * K * 4   # k_tilde, v, anchors
           + B * HQ * K * es + B * HQ * K * 4 + B * HQ * V * es + B * HQ * 4)  # q, p_curr, o, lse
    opens = (T - 1) % C == 0
    # one row through wall_stream_append: g and the previous P row in, the new P
    # row out; k in, the k_tilde row out; the chunk anchor read (or written)
    app = B * HQ * K * es + 2 * B * HQ * K * 4 + B * H * K * es + B * HQ * K * es + B * HQ * K * 4
    return dec, app, opens


def decode_cpu_baseline(inp, nseq, es):
    """Time the fp64 decode oracle (as it stands) on the first nseq sequences;
    the oracle's cache is built beforehand, outside the timing."""
    import numpy as np

    import oracle

    oracle.build(force=False)
    B, T, HQ, K = inp.q.shape[0], inp.k.shape[1], inp.q.shape[2], inp.q.shape[3]
    H, V, C = inp.k.shape[2], inp.v.shape[3], inp.chunk_size
    sel = slice(0, nseq)
    g = inp.g[sel].double().numpy()
    P = oracle.prefix_scan_oracle(g)
    kt, r = oracle.kv_cache_oracle(inp.k[sel], P, C)
    q, v = inp.q[sel].double().numpy(), inp.v[sel].double().numpy()
    pc = np.ascontiguousarray(P[:, T - 1:T])
    t0 = time.perf_counter()
    oracle.decode_oracle(q, v, pc, kt, r, C, sink_bias=inp.sink_bias, scale=inp.scale)
    t = time.perf_counter() - t0
    dec, _, _ = decode_bytes(nseq, T, HQ, H, K, V, C, es)
    return {
        "value": dec / t / 1e9,
        "unit": "GB/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": f"{nseq} of {B} sequences (all {HQ} heads, {T} cached rows), {t:.2f} s fp64 cached decode",
        "seconds": t,
    }


def bench_decode(args):
    """One step of the streaming decode loop: the newest token's log2 prefix from
    the previous row's and its row of the anchored key cache (one pass), then the
    split-KV decode of every sequence's newest query."""
    import torch

    import channel_decay_softmax_amd as wall
    from wall_inputs import make_decode_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda", 0)
    inp = make_decode_inputs(args.workload)
    d = inp.to(dev)
    B, _, HQ, K = d.q.shape
    T, H, V, C = d.k.shape[1], d.k.shape[2], d.v.shape[3], inp.chunk_size
    es = 2 if d.q.dtype == torch.bfloat16 else 4
    # the prefill state: the log2 prefix and the cache of the first T-1 rows
    P = torch.empty((B, T, HQ, K), dtype=torch.float32, device=dev)
    P[:, :T - 1] = wall.wall_prefix_scan(d.g[:, :T - 1].contiguous())
    kt = torch.empty((B, T, HQ, K), dtype=d.q.dtype, device=dev)
    r = torch.empty((B, -(-T // C), HQ, K), dtype=torch.float32, device=dev)
    wall.build_wall_kv_cache(d.k, P, C, k_tilde=kt, r_cache=r, t0=0, t1=T - 1)
    pc = P[:, T - 1:T]
    o = torch.empty((B, 1, HQ, V), dtype=d.q.dtype, device=dev)
    lse = torch.empty((B, 1, HQ), dtype=torch.float32, device=dev)
    ws = torch.empty(wall.decode_workspace_size(B, T, HQ, V), dtype=torch.uint8, device=dev)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]

    def step(marks=None):
        if marks:
            marks[0].record()
        wall.wall_stream_append(d.g, d.k, P, kt, r, C, T - 1, T)
        if marks:
            marks[1].record()
        wall.wall_attn_decode(d.q, d.v, pc, kt, r, sink_bias=d.sink_bias, scale=inp.scale,
                              cache_chunk_size=C, out=o, lse=lse, workspace=ws)
        if marks:
            marks[2].record()

    if args.copy_mb:
        n = args.copy_mb * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)  # reads and writes copy_mb MiB each
        torch.cuda.synchronize()
        del src, dst
    dec, app, _ = decode_bytes(B, T, HQ, H, K, V, C, es)
    print(f"[bench] {args.workload}: B={B} T={T} HQ={HQ} H={H} K={K} V={V} C={C} {d.q.dtype} "
          f"decode bytes={dec} append bytes={app}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    for i in range(args.steps):
        step(ev[i])
    torch.cuda.synchronize()
    app_ms = [e[0].elapsed_time(e[1]) for e in ev]
    dec_ms = [e[1].elapsed_time(e[2]) for e in ev]
    dec_avg = statistics.fmean(dec_ms)
    achieved = dec / (dec_avg * 1e-3) / 1e9
    value = (dec + app) / (ms_step * 1e-3) / 1e9
    print(f"[bench] step {ms_step * 1e3:.1f} us: append {statistics.fmean(app_ms) * 1e3:.1f} us, "
          f"decode {dec_avg * 1e3:.1f} us -> decode {achieved:.0f} GB/s", file=sys.stderr, flush=True)
    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the fp64 decode oracle on the host", file=sys.stderr, flush=True)
        cpu = decode_cpu_baseline(inp, B, es)
    rec = {
        "metric": DECODE_METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {torch.bfloat16: "bf16", torch.float32: "f32"}[d.q.dtype],
        "data": "synthetic",
        "config": {"workload": args.workload, "B": B, "T": T, "HQ": HQ, "H": H, "K": K, "V": V,
                   "chunk_size": C, "sink": inp.sink_bias is not None, "decode_bytes": dec,
                   "append_bytes": app},
        "tokens_per_s": round(B / (ms_step * 1e-3), 1),
        "stages_us": {"append": round(statistics.fmean(app_ms) * 1e3, 2), "decode": round(dec_avg * 1e3, 2)},
        "roofline": {"kernel": "decode_split + decode_merge", "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": load_traffic(args.workload, DECODE_TRAFFIC_FILE, DECODE_KERNEL_SOURCES)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


def bwd_cpu_baseline(inp, rows, flop_per_pair):
    """Time the fp64 backward oracle (as it stands) on the first ``rows`` tokens of
    the workload taken as sequences of their own (every head)."""
    import numpy as np

    import oracle

    oracle.build(force=False)
    sl = slice(0, rows)
    rng = np.random.default_rng(5)
    do = rng.standard_normal((inp.q.shape[0], rows, inp.q.shape[2], inp.v.shape[3]))
    t0 = time.perf_counter()
    oracle.wall_attn_bwd_oracle(inp.q[:, sl], inp.k[:, sl], inp.v[:, sl], inp.g[:, sl], do, scale=inp.scale)
    t = time.perf_counter() - t0
    pairs = inp.q.shape[0] * inp.q.shape[2] * rows * (rows + 1) // 2
    return {
        "value": pairs * flop_per_pair / t / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": f"the first {rows} of {inp.q.shape[1]} rows as a sequence of their own (all "
                  f"{inp.q.shape[2]} heads), {pairs} visible pairs, {t:.1f} s fp64 backward",
        "seconds": t,
    }


def bench_backward(args):
    """The backward of the fused forward on the workload: given q, k, v, the
    prefixes, o and lse, one step computes dq, dk, dv, dg (and dg_scalar, dsink)."""
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
    flop_per_pair = 6 * K + 4 * V  # QK^T again, dO V^T, dS K, dS^T Q, P^T dO
    flop = pairs * flop_per_pair
    cu = d.cu_seqlens
    maxlen = max(lens)
    P = wall.wall_prefix_scan(d.g, cu)
    G = None if d.g_scalar is None else wall.wall_prefix_scan(d.g_scalar, cu)
    o, lse = wall.wall_attn_fwd(d.q, d.k, d.v, P, G, d.sink_bias, d.scale, inp.window_size, cu, maxlen)
    rng = __import__("numpy").random.default_rng(9)
    do = torch.from_numpy(rng.standard_normal((B, T, HQ, V))).to(d.q.dtype).to(dev)
    nseq = 0 if cu is None else cu.numel() - 1
    ws = torch.empty(wall.lib().wall_attn_bwd_workspace_size(B, T, HQ, K, nseq), dtype=torch.uint8, device=dev)

    def step():
        wall.wall_attn_bwd(d.q, d.k, d.v, P, o, lse, do, G, d.sink_bias, d.scale, inp.window_size, cu, maxlen,
                           g_dtype=d.g.dtype, workspace=ws)

    if args.copy_mb:
        n = args.copy_mb * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)  # reads and writes copy_mb MiB each
        torch.cuda.synchronize()
        del src, dst
    print(f"[bench] backward {args.workload}: B={B} T={T} HQ={HQ} H={H} K={K} V={V} {d.q.dtype} "
          f"pairs={pairs} flop={flop:.4e}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    value = flop / (ms_step * 1e-3) / 1e12
    print(f"[bench] backward step {ms_step:.3f} ms -> {value:.1f} TFLOP/s", file=sys.stderr, flush=True)
    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the fp64 backward oracle on the host", file=sys.stderr, flush=True)
        cpu = bwd_cpu_baseline(inp, 2048, flop_per_pair)
    # bf16 inputs run the products on bf16 MFMA (float32 accumulation), float32
    # inputs on the float32 vector ALUs
    if d.q.dtype == torch.bfloat16:
        dt, bound, peak = "bf16", "mfma", PEAK_BF16_TFLOPS
    else:
        dt, bound, peak = "f32", "alu", PEAK_F32_VALU_TFLOPS
    rec = {
        "metric": BWD_METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dt,
        "data": "synthetic",
        "config": {"workload": args.workload, "B": B, "T": T, "HQ": HQ, "H": H, "K": K, "V": V,
                   "visible_pairs": pairs, "counted_flop": flop},
        "roofline": {"kernel": "the whole backward step (dq and dk/dv products, group sum, D, scans)",
                     "bound": bound, "achieved": round(value, 3), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(value / peak, 4),
                     "traffic": (load_traffic(args.workload, BWD_TRAFFIC_FILE, BWD_KERNEL_SOURCES)
                                 if d.q.dtype == torch.bfloat16 else None)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=int(os.environ.get("WORLD_SIZE", "1")))
    # the part's clocks settle after about 40 ms of back-to-back steps (the
    # first steps after idle run up to 20% slower): the defaults warm up for
    # about 60 ms and time about 60 ms of steady state
    # (the decode step is about a third as long: it defaults to 600 and 600)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="long_bf16")
    ap.add_argument("--cpu-seconds", type=float, default=60.0,
                    help="the oracle runs every row of the workload when predicted to take at most this long, "
                         "else a fixed sample sized to it")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward (wall_attn_bwd) of the workload instead of the forward hot path")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="run a plain device copy of this many MiB (read + write) before the "
                         "timed region, as the reference kernel for HBM byte counters")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus}): the Wall Attention forward "
              "is built and measured for a single GPU.  Across GPUs it would shard by key/value-head "
              "group (each GPU runs the same kernels on its heads, with no communication).",
              file=sys.stderr)
        sys.exit(2)
    from wall_inputs import DECODE_WORKLOADS
    decode = args.workload in DECODE_WORKLOADS
    if args.backward and not decode:
        args.steps = 50 if args.steps is None else args.steps
        args.warmup = 30 if args.warmup is None else args.warmup
        return bench_backward(args)
    if args.steps is None:
        args.steps = 600 if decode else 200
    if args.warmup is None:
        args.warmup = 600 if decode else 200
    if decode:
        return bench_decode(args)

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
        if G is not None:
            wall.wall_prefix_scan(d.g_scalar, cu, out=G, workspace=ws_scan)
        if marks:
            marks[1].record()
        # the prefix of g and the preparation (one combined pass where the layout allows)
        wall.wall_attn_fwd_prepare_gate(d.q, d.k, d.v, d.g, P, ws_fwd, scale=d.scale, cu_seqlens=cu)
        if marks:
            marks[2].record()
        wall.wall_attn_fwd_run(d.q, d.k, d.v, P, ws_fwd, o, lse, G=G, sink_bias=d.sink_bias,
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
    print(f"[bench] step {ms_step:.3f} ms: scalar-gate scan {statistics.fmean(scan_ms)*1e3:.1f} us, "
          f"prefix + prepare {statistics.fmean(prep_ms)*1e3:.1f} us, fused {run_avg*1e3:.1f} us "
          f"(min {min(run_ms)*1e3:.1f}) -> fused {achieved:.1f} TFLOP/s", file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the fp64 oracle on the host", file=sys.stderr, flush=True)
        cpu = cpu_baseline(inp, flop_per_pair, args.cpu_seconds)

    dtype = {torch.bfloat16: "bf16", torch.float32: "f32"}[d.q.dtype]
    # bf16 runs on the matrix cores; float32 runs on the vector ALUs
    if dtype == "bf16":
        kname, bound, peak = ("fwd_bf16_kernel<128,128>" if K == 128 else "fwd_bf16_kernel"), "mfma", PEAK_BF16_TFLOPS
    else:
        kname, bound, peak = "fwd_f32_kernel", "alu", PEAK_F32_VALU_TFLOPS
    prep_avg = statistics.fmean(prep_ms)
    call_tflops = flop / ((prep_avg + run_avg) * 1e-3) / 1e12
    # The fused kernel forms the keys whose scores are exactly -m in closed form
    # and skips score products of channel steps whose q~ is 0: on a decaying
    # gate it executes fewer matrix-core flops than the counted 4K per pair.
    # The counters' figure (same kernel source) is reported beside the counted one.
    ex = load_executed(args.workload) if dtype == "bf16" else None
    executed = None
    if ex:
        ex_tflops = ex["executed_mfma_flop_per_launch"] / (run_avg * 1e-3) / 1e12
        executed = {"flop_per_launch": ex["executed_mfma_flop_per_launch"],
                    "of_counted": round(ex["executed_mfma_flop_per_launch"] / flop, 4),
                    "tflops": round(ex_tflops, 3), "frac": round(ex_tflops / peak, 4),
                    "mfma_busy": ex["mfma_busy"], "source": "profiles/fwd_bf16_long_bf16_mfma.json"}
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
        "pct_of_peak": round(100.0 * value / peak, 2),
        "stages_us": {"scalar_gate_scan": round(statistics.fmean(scan_ms) * 1e3, 2),
                      "prefix_and_prepare": round(prep_avg * 1e3, 2),
                      "fused_fwd": round(run_avg * 1e3, 2)},
        "roofline": {"kernel": kname, "bound": bound, "achieved": round(achieved, 3),
                     "peak": peak, "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": traffic if dtype == "bf16" else None,
                     # matrix-core flops the kernel executes (rocprofv3 counters)
                     "executed": executed,
                     # the C-ABI calls of the forward from the gate: prefix and preparation, fused kernel
                     "call": {"what": "wall_attn_fwd_prepare_gate + wall_attn_fwd_run",
                              "us": round((prep_avg + run_avg) * 1e3, 2),
                              "achieved": round(call_tflops, 3), "frac": round(call_tflops / peak, 4)}},
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
