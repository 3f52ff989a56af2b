"""GPU parity of the backward (wall_attn_bwd through the C ABI, and the
autograd path of wall_attn) against the fp64 oracle's backward.

Each gradient is compared as a whole tensor, relative to its own size:
max |d| <= tol_max * max|ref| and RMS(d) <= tol_rms * RMS(ref).  bf16 inputs
are widened to float32 in the kernels; the gradients are rounded once to
bf16 (relative 2^-9) and the products carry the forward's bf16-rounded o
and the float32 lse, so bf16 is held to 3e-2 / 1e-2 and float32 to 1e-4 /
1e-5.
"""

import math

import numpy as np
import pytest
import torch

import channel_decay_softmax_amd as wall
import oracle
from wall_inputs import make_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = {"bfloat16": (3e-2, 1e-2), "float32": (1e-4, 1e-5)}


def say(msg):
    print(f"[gpu] {msg}", flush=True)


def f64(t):
    return None if t is None else t.detach().float().cpu().double().numpy()


CASES = [
    dict(wl="long_bf16", T=300, HQ=4, H=2, K=128, V=128),
    dict(wl="tiny_fp32", B=2, T=200, HQ=2, H=1, K=64, V=64),
    dict(wl="options_bf16", B=2, T=257, HQ=4, H=2, K=128, V=64, window=50),
    dict(wl="varlen_bf16", T=250, HQ=2, H=1, K=64, V=128, nseq=None, cu=[0, 100, 100, 101, 250]),
    dict(wl="gqa_bf16", B=1, T=190, HQ=4, H=2, K=64, V=64, dtype="float32"),
    dict(wl="gqa_bf16", B=2, T=333, HQ=8, H=4, K=64, V=64),
    dict(wl="long_bf16", B=1, T=700, HQ=2, H=1, K=128, V=128),
    dict(wl="options_bf16", B=1, T=520, HQ=2, H=2, K=64, V=64, window=130),
    dict(wl="options_bf16", B=3, T=97, HQ=4, H=1, K=128, V=128, window=40),
    dict(wl="varlen_bf16", T=400, HQ=4, H=2, K=128, V=64, nseq=None, cu=[0, 1, 33, 160, 161, 300, 400]),
    dict(wl="long_bf16", B=2, T=130, HQ=2, H=1, K=128, V=128),
]


def case_id(c):
    return "-".join(f"{k}{v}" for k, v in c.items() if k != "cu")


@pytest.mark.parametrize("c", CASES, ids=case_id)
def test_backward_parity(c):
    over = {k: v for k, v in c.items() if k not in ("wl", "cu")}
    inp = make_inputs(c["wl"], **over)
    if c.get("cu") is not None:
        inp.cu_seqlens = torch.tensor(c["cu"], dtype=torch.int32)
    B, T, HQ, K = inp.q.shape
    V = inp.v.shape[3]
    say(f"backward {case_id(c)} {inp.q.dtype} W={inp.window_size} gs={inp.g_scalar is not None} "
        f"sink={inp.sink_bias is not None} varlen={inp.cu_seqlens is not None}")
    rng = np.random.default_rng(17)
    do = torch.from_numpy(rng.standard_normal((B, T, HQ, V))).to(inp.q.dtype)
    d = inp.to(DEV)
    cu = d.cu_seqlens
    maxlen = None if cu is None else int((cu[1:] - cu[:-1]).max().item())
    P = wall.wall_prefix_scan(d.g, cu)
    G = None if d.g_scalar is None else wall.wall_prefix_scan(d.g_scalar, cu)
    o, lse = wall.wall_attn_fwd(d.q, d.k, d.v, P, G, d.sink_bias, d.scale, d.window_size, cu, maxlen)
    grads = wall.wall_attn_bwd(d.q, d.k, d.v, P, o, lse, do.to(DEV), G, d.sink_bias, d.scale, d.window_size,
                               cu, maxlen, g_dtype=d.g.dtype)
    torch.cuda.synchronize()
    ref = oracle.wall_attn_bwd_oracle(inp.q, inp.k, inp.v, inp.g, do, scale=inp.scale, g_scalar=inp.g_scalar,
                                      sink_bias=inp.sink_bias, window_size=inp.window_size,
                                      cu_seqlens=inp.cu_seqlens)
    tmax, trms = TOL[str(inp.q.dtype).split(".")[1]]
    for name, gg, rr in zip(["dq", "dk", "dv", "dg", "dg_scalar", "dsink"], grads, ref):
        if rr is None:
            assert gg is None
            continue
        x = f64(gg)
        dd = np.abs(x - rr)
        mx, rms = dd.max(), math.sqrt((dd ** 2).mean())
        rmax, rrms = np.abs(rr).max(), math.sqrt((rr ** 2).mean())
        say(f"  {name}: max|d|={mx:.3e} (ref max {rmax:.3e})  rms={rms:.3e} (ref rms {rrms:.3e})")
        assert mx <= tmax * max(rmax, 1e-30) and rms <= trms * max(rrms, 1e-30), name
    # a decay-gate entry at a sequence's first token has gradient 0
    starts = [0] if inp.cu_seqlens is None else sorted(set(x for x in c["cu"][:-1] if x < T))
    dg = f64(grads[3])
    for s in starts:
        assert not dg[:, s].any()


def test_autograd_matches_direct_backward():
    inp = make_inputs("options_bf16", B=1, T=160, HQ=4, H=2, K=64, V=64, window=40)
    say("autograd wall_attn vs wall_attn_bwd")
    d = inp.to(DEV)
    leaves = [t.clone().requires_grad_() for t in (d.q, d.k, d.v, d.g, d.g_scalar, d.sink_bias)]
    q, k, v, g, gs, sk = leaves
    o = wall.wall_attn(q, k, v, g, scale=d.scale, g_scalar=gs, sink_bias=sk, window_size=d.window_size)
    rng = np.random.default_rng(3)
    do = torch.from_numpy(rng.standard_normal(o.shape)).to(o.dtype).to(DEV)
    o.backward(do)
    P = wall.wall_prefix_scan(d.g)
    G = wall.wall_prefix_scan(d.g_scalar)
    o2, lse2 = wall.wall_attn_fwd(d.q, d.k, d.v, P, G, d.sink_bias, d.scale, d.window_size)
    direct = wall.wall_attn_bwd(d.q, d.k, d.v, P, o2, lse2, do, G, d.sink_bias, d.scale, d.window_size,
                                g_dtype=d.g.dtype)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), o2)
    for leaf, gd in zip(leaves, direct):
        assert torch.equal(leaf.grad, gd)


def test_backward_deterministic():
    """No atomics: two calls give the same bits."""
    inp = make_inputs("options_bf16", B=1, T=300, HQ=4, H=2, K=128, V=128, window=100)
    say("backward twice, same bits")
    d = inp.to(DEV)
    P = wall.wall_prefix_scan(d.g)
    G = wall.wall_prefix_scan(d.g_scalar)
    o, lse = wall.wall_attn_fwd(d.q, d.k, d.v, P, G, d.sink_bias, d.scale, d.window_size)
    do = torch.from_numpy(np.random.default_rng(4).standard_normal(o.shape)).to(o.dtype).to(DEV)
    a = wall.wall_attn_bwd(d.q, d.k, d.v, P, o, lse, do, G, d.sink_bias, d.scale, d.window_size)
    b = wall.wall_attn_bwd(d.q, d.k, d.v, P, o, lse, do, G, d.sink_bias, d.scale, d.window_size)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_backward_full_size_sampled():
    """The long-context workload at its full size (B=1, T=8192, HQ=16, H=4,
    K=V=128) in the launch configuration the benchmark times, with the
    upstream gradient zero after the first R0 rows.  Causality makes every
    gradient of rows < R0 equal to the backward of the first R0 rows alone
    (later queries then add nothing to dk, dv or the gate sums), which the
    oracle computes; dq, dk and dv of rows >= R0 must be zero, and dg there
    zero up to rounding."""
    R0 = 768
    inp = make_inputs("long_bf16")
    B, T, HQ, K = inp.q.shape
    V = inp.v.shape[3]
    say(f"backward full size T={T} HQ={HQ} K={K}, upstream gradient on rows < {R0}")
    rng = np.random.default_rng(21)
    do = torch.zeros((B, T, HQ, V), dtype=inp.q.dtype)
    do[:, :R0] = torch.from_numpy(rng.standard_normal((B, R0, HQ, V))).to(inp.q.dtype)
    d = inp.to(DEV)
    P = wall.wall_prefix_scan(d.g)
    o, lse = wall.wall_attn_fwd(d.q, d.k, d.v, P, None, None, d.scale)
    grads = wall.wall_attn_bwd(d.q, d.k, d.v, P, o, lse, do.to(DEV), scale=d.scale, g_dtype=d.g.dtype)
    torch.cuda.synchronize()
    sl = slice(0, R0)
    ref = oracle.wall_attn_bwd_oracle(inp.q[:, sl], inp.k[:, sl], inp.v[:, sl], inp.g[:, sl], do[:, sl],
                                      scale=inp.scale)
    tmax, trms = TOL["bfloat16"]
    for name, gg, rr in zip(["dq", "dk", "dv", "dg"], grads[:4], ref[:4]):
        x = f64(gg)
        rmax, rrms = np.abs(rr).max(), math.sqrt((rr ** 2).mean())
        if name == "dg":
            # dg after R0 is minus the whole sum of the X terms: zero up to rounding
            assert np.abs(x[:, R0:]).max() <= tmax * rmax, "dg after the last row with a gradient"
        else:
            assert not x[:, R0:].any(), f"{name}: nonzero gradient after row {R0}"
        dd = np.abs(x[:, :R0] - rr)
        mx, rms = dd.max(), math.sqrt((dd ** 2).mean())
        say(f"  {name}: max|d|={mx:.3e} (ref max {rmax:.3e})  rms={rms:.3e} (ref rms {rrms:.3e})")
        assert mx <= tmax * rmax and rms <= trms * rrms, name


def test_backward_full_size_every_row():
    """The long-context workload at its full size with an upstream gradient on
    every row, in the benchmark's launch path: the dq and dk/dv walks leave
    out the far pairs (some 800 rows back on the slow channels) for
    every key and query tile, and the dv of the rows past each walk comes
    from the per-block suffix sums.  Every gradient of every row and head
    against the oracle's full backward (about a minute on the host)."""
    inp = make_inputs("long_bf16")
    B, T, HQ, K = inp.q.shape
    say(f"backward full size T={T} HQ={HQ} K={K}, upstream gradient on every row")
    do = _do(inp, 43)
    grads = _bwd_gpu(inp, do)
    ref = oracle.wall_attn_bwd_oracle(inp.q, inp.k, inp.v, inp.g, do, scale=inp.scale)
    _compare(grads, ref, "bfloat16", q=f64(inp.q))


def test_backward_options_full_size_sampled():
    """options_bf16 at its full size (B=4, T=4096, HQ=32, H=8, window 1024,
    g_scalar, sink), upstream gradient zero after row R0 = 1536 (past the
    window, so it takes effect).  Batch element 0 is checked against the
    oracle's backward of its first R0 rows; the other elements only for
    their zero tails."""
    R0 = 1536
    inp = make_inputs("options_bf16")
    B, T, HQ, K = inp.q.shape
    V = inp.v.shape[3]
    say(f"backward options full size B={B} T={T} HQ={HQ} W={inp.window_size}, upstream gradient on rows < {R0}")
    rng = np.random.default_rng(23)
    do = torch.zeros((B, T, HQ, V), dtype=inp.q.dtype)
    do[:, :R0] = torch.from_numpy(rng.standard_normal((B, R0, HQ, V))).to(inp.q.dtype)
    d = inp.to(DEV)
    P = wall.wall_prefix_scan(d.g)
    G = wall.wall_prefix_scan(d.g_scalar)
    o, lse = wall.wall_attn_fwd(d.q, d.k, d.v, P, G, d.sink_bias, d.scale, d.window_size)
    grads = wall.wall_attn_bwd(d.q, d.k, d.v, P, o, lse, do.to(DEV), G, d.sink_bias, d.scale, d.window_size,
                               g_dtype=d.g.dtype)
    torch.cuda.synchronize()
    s = (slice(0, 1), slice(0, R0))
    ref = oracle.wall_attn_bwd_oracle(inp.q[s], inp.k[s], inp.v[s], inp.g[s], do[s], scale=inp.scale,
                                      g_scalar=inp.g_scalar[s], sink_bias=inp.sink_bias,
                                      window_size=inp.window_size)
    tmax, trms = TOL["bfloat16"]
    for name, gg, rr in zip(["dq", "dk", "dv", "dg", "dg_scalar"], grads[:5], ref[:5]):
        x = f64(gg)
        rmax = np.abs(rr).max()
        if name in ("dg", "dg_scalar"):
            assert np.abs(x[:, R0:]).max() <= tmax * rmax, f"{name} after the last row with a gradient"
        else:
            assert not x[:, R0:].any(), f"{name}: nonzero gradient after row {R0}"
        dd = np.abs(x[:1, :R0] - rr)
        mx, rms = dd.max(), math.sqrt((dd ** 2).mean())
        rrms = math.sqrt((rr ** 2).mean())
        say(f"  {name}: max|d|={mx:.3e} (ref max {rmax:.3e})  rms={rms:.3e} (ref rms {rrms:.3e})")
        assert mx <= tmax * rmax and rms <= trms * rrms, name


# --------------------------------------------------------------------------- strong decay
def _bwd_gpu(inp, do):
    d = inp.to(DEV)
    cu = d.cu_seqlens
    maxlen = None if cu is None else int((cu[1:] - cu[:-1]).max().item())
    P = wall.wall_prefix_scan(d.g, cu)
    G = None if d.g_scalar is None else wall.wall_prefix_scan(d.g_scalar, cu)
    o, lse = wall.wall_attn_fwd(d.q, d.k, d.v, P, G, d.sink_bias, d.scale, d.window_size, cu, maxlen)
    grads = wall.wall_attn_bwd(d.q, d.k, d.v, P, o, lse, do.to(DEV), G, d.sink_bias, d.scale, d.window_size,
                               cu, maxlen, g_dtype=d.g.dtype)
    torch.cuda.synchronize()
    return grads


def _compare(grads, ref, dtype, names=("dq", "dk", "dv", "dg", "dg_scalar", "dsink"), q=None):
    """Each gradient against the reference at the module's bars.  With q given,
    dg is measured against the larger of its own size and that of the terms
    q (.) dq it sums: under strong decay those terms cancel (dg shrinks with
    the decay's derivative) while the rounding of their sum stays that of the
    terms."""
    tmax, trms = TOL[dtype]
    for name, gg, rr in zip(names, grads, ref):
        if rr is None:
            assert gg is None
            continue
        x = f64(gg)
        dd = np.abs(x - rr)
        mx, rms = dd.max(), math.sqrt((dd ** 2).mean())
        rmax, rrms = np.abs(rr).max(), math.sqrt((rr ** 2).mean())
        if name == "dg" and q is not None:
            terms = q * ref[0]
            rmax, rrms = max(rmax, np.abs(terms).max()), max(rrms, math.sqrt((terms ** 2).mean()))
        say(f"  {name}: max|d|={mx:.3e} (ref max {rmax:.3e})  rms={rms:.3e} (ref rms {rrms:.3e})")
        assert mx <= tmax * max(rmax, 1e-30) and rms <= trms * max(rrms, 1e-30), name


def _strong(gate, dtype, K, T=420, window=None):
    """A strong uniform gate on every channel, two query heads of one kv head,
    and a packed sequence start inside the first tile."""
    inp = make_inputs("long_bf16", dtype=dtype, B=1, T=T, HQ=2, H=1, K=K, V=K)
    inp.g = torch.full_like(inp.g, gate)
    inp.cu_seqlens = torch.tensor([0, 37, T], dtype=torch.int32)
    inp.window_size = window
    return inp


def _do(inp, seed):
    B, T, HQ, _ = inp.q.shape
    rng = np.random.default_rng(seed)
    return torch.from_numpy(rng.standard_normal((B, T, HQ, inp.v.shape[3]))).to(inp.q.dtype)


@pytest.mark.parametrize("K", [64, 128])
@pytest.mark.parametrize("dtype", ["bfloat16", "float32"])
@pytest.mark.parametrize("gate", [-1.5, -2.0, -5.0])
def test_backward_strong_uniform_decay(gate, dtype, K):
    """Gates past the reach of one anchor per 128-row tile (the prefix falls 2.2
    to 7.2 log2 units per token, 69 to 231 per 32-row block): boundary anchors
    for pairs in different blocks, the block's own anchor for unflagged
    blocks, and the pair-by-pair kernel for spread ones keep every gradient
    at the bar."""
    inp = _strong(gate, dtype, K)
    say(f"backward uniform g={gate} {dtype} K=V={K}")
    do = _do(inp, 31)
    grads = _bwd_gpu(inp, do)
    ref = oracle.wall_attn_bwd_oracle(inp.q, inp.k, inp.v, inp.g, do, scale=inp.scale, cu_seqlens=inp.cu_seqlens)
    _compare(grads, ref, dtype, q=f64(inp.q))


@pytest.mark.parametrize("kv", [(64, 128), (128, 64), (128, 128)])
@pytest.mark.parametrize("packed", [False, True])
def test_backward_far_tiles(kv, packed):
    """A uniform gate of -0.1 nats per token over 2048 rows: past a few hundred
    rows the bound on a pair's score (q~ and k~ moved to an anchor between the
    rows) falls below 2^-26 of L_i = lse_i log2e, and past about 930 rows the
    moved values round to 0 in bf16, so the dq kernel starts its walk late, the
    dk/dv kernel stops early and the rows it leaves reach dv through the suffix
    sums of bf16(2^-L_i) do_i.  Each value channel has a mean of its own, so
    those sums carry much of dv and a mix-up of channels or blocks would show;
    packed: two sequences (the sums restart at the second).  Every gradient
    against the oracle."""
    K, V = kv
    T = 2048
    inp = make_inputs("long_bf16", B=1, T=T, HQ=2, H=1, K=K, V=V)
    inp.g = torch.full_like(inp.g, -0.1)
    ramp = torch.linspace(-0.4, 0.4, V, dtype=torch.float64)
    inp.v = (inp.v.double() * 0.5 + ramp).to(inp.v.dtype)
    if packed:
        inp.cu_seqlens = torch.tensor([0, 700, T], dtype=torch.int32)
    say(f"backward far tiles K={K} V={V} packed={packed}")
    do = _do(inp, 37)
    grads = _bwd_gpu(inp, do)
    ref = oracle.wall_attn_bwd_oracle(inp.q, inp.k, inp.v, inp.g, do, scale=inp.scale, cu_seqlens=inp.cu_seqlens)
    _compare(grads, ref, "bfloat16", q=f64(inp.q))


@pytest.mark.parametrize("sink", [False, True])
def test_backward_bimodal_far_pairs(sink):
    """The long-context gate (slow channels near -0.03 nats per token, fast
    ones near -0.8) over 4096 rows with an upstream gradient on every row: the
    dq and dk/dv walks leave out the far pairs whose score bound lies below
    2^-26 of L_i (some 850 rows back on the slow channels), with and
    without a sink (which moves every L_i).  Every gradient against the
    oracle."""
    T = 4096
    inp = make_inputs("long_bf16", B=1, T=T, HQ=2, H=1, K=128, V=128)
    if sink:
        inp.sink_bias = torch.tensor([0.75, -1.5], dtype=torch.float32)
    say(f"backward bimodal gate T={T} sink={sink}")
    do = _do(inp, 41)
    grads = _bwd_gpu(inp, do)
    ref = oracle.wall_attn_bwd_oracle(inp.q, inp.k, inp.v, inp.g, do, scale=inp.scale, sink_bias=inp.sink_bias)
    _compare(grads, ref, "bfloat16", q=f64(inp.q))


@pytest.mark.parametrize("dtype", ["bfloat16", "float32"])
def test_backward_strong_decay_window(dtype):
    """g = -2 with a 50-token window and a packed start."""
    inp = _strong(-2.0, dtype, 128, T=360, window=50)
    say(f"backward uniform g=-2 window 50 {dtype}")
    do = _do(inp, 33)
    grads = _bwd_gpu(inp, do)
    ref = oracle.wall_attn_bwd_oracle(inp.q, inp.k, inp.v, inp.g, do, scale=inp.scale, window_size=50,
                                      cu_seqlens=inp.cu_seqlens)
    _compare(grads, ref, dtype, q=f64(inp.q))


def test_backward_strong_and_slow_channels():
    """Half the channels forget at -3 nats per token, half at -0.01: every block
    is spread, while the slow channels carry the gradients across tiles."""
    inp = make_inputs("long_bf16", B=1, T=700, HQ=4, H=2)
    g = torch.full(inp.g.shape, -0.01, dtype=torch.float64)
    g[..., 64:] = -3.0
    inp.g = g.to(inp.g.dtype)
    say("backward channels at -3 and -0.01")
    do = _do(inp, 35)
    grads = _bwd_gpu(inp, do)
    ref = oracle.wall_attn_bwd_oracle(inp.q, inp.k, inp.v, inp.g, do, scale=inp.scale)
    _compare(grads, ref, "bfloat16", q=f64(inp.q))


def test_backward_one_spread_block():
    """Ordinary gates except one strong step inside a single 32-row block of one
    query head's channels: only that block takes the pair-by-pair path, next to
    anchored blocks in the same tile."""
    inp = make_inputs("long_bf16", B=1, T=300, HQ=2, H=1)
    g = inp.g.double().clone()
    g[0, 150, 1, :] = -200.0
    inp.g = g.to(inp.g.dtype)
    say("backward one spread block")
    do = _do(inp, 37)
    grads = _bwd_gpu(inp, do)
    ref = oracle.wall_attn_bwd_oracle(inp.q, inp.k, inp.v, inp.g, do, scale=inp.scale)
    _compare(grads, ref, "bfloat16")


@pytest.mark.parametrize("dtype", ["bfloat16", "float32"])
def test_backward_all_gates_closed(dtype):
    """g = -800 per token: every earlier key's decay and its derivative are 0,
    so with s_ii = scale q_i.k_i, Z_i = n_i + e^{s_ii} (n_i earlier tokens of i's
    sequence), A_ij = 1/Z_i (j < i) and e^{s_ii}/Z_i (j = i),
    dS_ij = A_ij (do_i.v_j - do_i.o_i):
        dq_i = scale dS_ii k_i,  dk_j = scale sum_hq dS_jj q_j,
        dv_j = sum_hq sum_{i >= j} A_ij do_i,  dg = 0."""
    inp = _strong(-800.0, dtype, 128, T=300)
    say(f"backward g=-800 closed form {dtype}")
    do = _do(inp, 39)
    grads = _bwd_gpu(inp, do)
    q = inp.q.double().numpy()[0]
    k = inp.k.double().numpy()[0]
    v = inp.v.double().numpy()[0]
    dd = do.double().numpy()[0]
    T, HQ = q.shape[0], q.shape[1]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for a, b in ((0, 37), (37, T)):
        for hq in range(HQ):
            vs = v[a:b, 0]
            s = inp.scale * np.einsum("ik,ik->i", q[a:b, hq], k[a:b, 0])
            n = np.arange(b - a)
            Z = n + np.exp(s)
            A = np.tril(np.ones((b - a, b - a)), -1) / Z[:, None]
            A[n, n] = np.exp(s) / Z
            o = A @ vs
            D = np.einsum("iv,iv->i", dd[a:b, hq], o)
            dS = A * (dd[a:b, hq] @ vs.T - D[:, None])
            diag = dS[n, n]
            dq[a:b, hq] = inp.scale * diag[:, None] * k[a:b, 0]
            dk[a:b, 0] += inp.scale * diag[:, None] * q[a:b, hq]
            dv[a:b, 0] += A.T @ dd[a:b, hq]
    _compare(grads[:3], [dq[None], dk[None], dv[None]], dtype, names=("dq", "dk", "dv"))
    # dg: every X term cancels; what is left is rounding of the pairs i = j
    dg = f64(grads[3])
    bound = 1e-5 * np.abs(q * dq).sum(axis=0).max()
    say(f"  dg: max|dg|={np.abs(dg).max():.3e} (bound {bound:.3e})")
    assert np.abs(dg).max() <= bound
