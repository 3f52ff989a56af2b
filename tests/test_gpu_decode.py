"""GPU parity of the decode path (cache build, split-KV decode), called through
the C ABI, against the fp64 oracle.

Cache: the anchors are floors of the same float32 P on both sides, taken by
the same rule (a chunk's anchor moves to a later row's floored P once that
row lies more than 64 log2 units below it), so they must match bit for bit;
k_tilde is the oracle's value rounded to the cache dtype (within 2^-8
relative for bf16, 4e-6 for float32, which covers the rounding and exp2f),
or below 2^-120 where the oracle's is (a lowered row may flush there).
Building the cache in several appends gives the same bits as one build.

Decode: the forward's tolerances (bf16 max|do| <= 2e-2, RMS <= 2e-3, lse
<= 2e-2; float32 1e-4), against (a) the oracle's cached decode on the same
float32 P and (b) the product-form forward oracle at the query's row, and
the GPU decode equals the GPU prefill's row within the same bounds.
"""

import math

import numpy as np
import pytest
import torch

import channel_decay_softmax_amd as wall
import oracle
from wall_inputs import make_decode_inputs

pytestmark = pytest.mark.gpu

TOL = {
    "bfloat16": dict(max=2e-2, rms=2e-3, lse=2e-2, kt=2.0 ** -8),
    "float32": dict(max=1e-4, rms=1e-4, lse=1e-4, kt=4e-6),
}
DEV = "cuda:0"


def say(msg):
    print(f"[gpu] {msg}", flush=True)


def f64(t):
    return t.detach().float().cpu().double().numpy()


def check_o(o, lse, o_ref, lse_ref, dtype, what):
    tol = TOL[dtype]
    d = np.abs(o - o_ref)
    mx, rms, ml = d.max(), math.sqrt((d ** 2).mean()), np.abs(lse - lse_ref).max()
    say(f"{what}: max|do|={mx:.3e} rms={rms:.3e} max|dlse|={ml:.3e}")
    assert mx <= tol["max"] and rms <= tol["rms"] and ml <= tol["lse"], what


CASES = [
    dict(dtype="bfloat16", B=2, T=300, Tcap=320, HQ=8, H=2, K=128, V=128, C=64, sink=True, gate="bimodal"),
    dict(dtype="float32", B=2, T=1000, Tcap=1000, HQ=4, H=4, K=64, V=64, C=128, sink=False, gate="small"),
    dict(dtype="bfloat16", B=1, T=5000, Tcap=5100, HQ=2, H=1, K=64, V=128, C=64, sink=True, gate="logsig4"),
    dict(dtype="bfloat16", B=3, T=1, Tcap=64, HQ=2, H=1, K=128, V=64, C=64, sink=True, gate="bimodal"),
    dict(dtype="float32", B=2, T=129, Tcap=129, HQ=4, H=2, K=128, V=128, C=64, sink=True, gate="bimodal"),
    # uniform gates strong enough to move the chunk anchors (g per token, natural log)
    dict(dtype="bfloat16", B=2, T=300, Tcap=300, HQ=4, H=2, K=128, V=128, C=64, sink=True, gate=-1.5),
    dict(dtype="bfloat16", B=2, T=300, Tcap=320, HQ=2, H=1, K=64, V=64, C=64, sink=False, gate=-5.0),
    dict(dtype="float32", B=2, T=300, Tcap=300, HQ=2, H=2, K=128, V=64, C=128, sink=True, gate=-2.0),
    dict(dtype="float32", B=1, T=200, Tcap=200, HQ=2, H=1, K=64, V=128, C=64, sink=True, gate=-5.0),
    dict(dtype="bfloat16", B=2, T=150, Tcap=150, HQ=2, H=1, K=128, V=128, C=64, sink=True, gate=-800.0),
]


def case_id(c):
    return (f"{c['dtype']}-B{c['B']}-T{c['T']}-cap{c['Tcap']}-HQ{c['HQ']}-H{c['H']}-K{c['K']}-V{c['V']}-C{c['C']}"
            f"-g{c['gate']}")


def check_kt(kt, kt_ref, dtype):
    dk = np.abs(kt - kt_ref)
    ok = dk <= TOL[dtype]["kt"] * np.abs(kt_ref) + 2.0 ** -120
    assert ok.all(), f"k_tilde: max {dk.max():.3e}"


@pytest.mark.parametrize("c", CASES, ids=case_id)
def test_cache_and_decode_parity(c):
    say(f"decode {case_id(c)} sink={c['sink']}")
    gate = c["gate"] if isinstance(c["gate"], str) else "small"
    inp = make_decode_inputs("decode_bf16", chunk_size=c["C"], B=c["B"], T=c["Tcap"], HQ=c["HQ"], H=c["H"],
                             K=c["K"], V=c["V"], dtype=c["dtype"], gate=gate, sink=c["sink"])
    if not isinstance(c["gate"], str):
        inp.g = torch.full_like(inp.g, c["gate"])
    d = inp.to(DEV)
    T, C = c["T"], c["C"]
    NC = -(-T // C)
    P = wall.wall_prefix_scan(d.g)
    # the cache of the T tokens so far, in buffers of T_cap rows (rows T.. not yet appended)
    kt, r = wall.build_wall_kv_cache(d.k, P, C, t1=T)
    o, lse = wall.wall_attn_decode(d.q, d.v, P[:, T - 1:T], kt, r, sink_bias=d.sink_bias, scale=inp.scale,
                                   cache_chunk_size=C, seq_len=T)
    # the same cache appended in pieces: rows on, next to and inside chunk boundaries
    kt2 = torch.full_like(kt, float("nan"))
    r2 = torch.full_like(r, float("nan"))
    cuts = sorted({0, 1, 63, 64, 65, C + 1, T // 2, T - 1, T} & set(range(T + 1)))
    for t0, t1 in zip(cuts[:-1], cuts[1:]):
        wall.build_wall_kv_cache(d.k, P, C, k_tilde=kt2, r_cache=r2, t0=t0, t1=t1)
    torch.cuda.synchronize()
    assert torch.equal(kt2[:, :T], kt[:, :T]) and torch.equal(r2[:, :NC], r[:, :NC]), \
        "appended cache differs from one build"

    # cache against the oracle on the same float32 P
    Ph = f64(P)
    kt_ref, r_ref = oracle.kv_cache_oracle(inp.k[:, :T], Ph[:, :T], C)
    assert np.array_equal(f64(r[:, :NC]), r_ref), "anchors differ"
    check_kt(f64(kt[:, :T]), kt_ref, c["dtype"])

    # decode against the cached-decode oracle and the forward oracle's row T-1
    og, lg = f64(o)[:, 0], f64(lse)[:, 0]
    o_ref, l_ref = oracle.decode_oracle(inp.q, inp.v[:, :T], Ph[:, T - 1:T], kt_ref, r_ref, C,
                                        sink_bias=inp.sink_bias, scale=inp.scale)
    check_o(og, lg, o_ref[:, 0], l_ref[:, 0], c["dtype"], "decode vs cached-decode oracle")
    B, HQ, K = c["B"], c["HQ"], c["K"]
    qf = torch.zeros((B, T, HQ, K), dtype=inp.q.dtype)
    qf[:, T - 1] = inp.q[:, 0]
    rows = [b * T + T - 1 for b in range(B)]
    o_f, l_f = oracle.wall_attn_oracle(qf, inp.k[:, :T], inp.v[:, :T], inp.g[:, :T], scale=inp.scale,
                                       sink_bias=inp.sink_bias, rows=rows)
    check_o(og, lg, o_f[:, T - 1], l_f[:, T - 1], c["dtype"], "decode vs forward oracle row")
    # the GPU prefill's row T-1
    of, lf = wall.wall_attn(qf.to(DEV), d.k[:, :T].contiguous(), d.v[:, :T].contiguous(),
                            d.g[:, :T].contiguous(), scale=inp.scale, sink_bias=d.sink_bias, return_lse=True)
    torch.cuda.synchronize()
    check_o(og, lg, f64(of)[:, T - 1], f64(lf)[:, T - 1], c["dtype"], "decode vs GPU prefill row")


def test_streaming_decode_matches_forward_rows():
    """Append-as-you-go: the cache is built for the first rows, then every step
    appends one token and decodes it; each step must give the forward's row."""
    B, Tcap, HQ, H, K, V, C = 2, 160, 4, 2, 128, 128, 64
    say(f"streaming decode B={B} rows 120..{Tcap - 1} HQ={HQ} H={H} K={K} V={V} C={C}")
    inp = make_decode_inputs("decode_bf16", chunk_size=C, B=B, T=Tcap, HQ=HQ, H=H, K=K, V=V, sink=True)
    rng = np.random.default_rng(8)
    qall = torch.from_numpy(rng.standard_normal((B, Tcap, HQ, K))).to(torch.bfloat16)
    d = inp.to(DEV)
    P = wall.wall_prefix_scan(d.g)
    kt = torch.empty((B, Tcap, HQ, K), dtype=torch.bfloat16, device=DEV)
    r = torch.empty((B, -(-Tcap // C), HQ, K), dtype=torch.float32, device=DEV)
    t_first = 120
    wall.build_wall_kv_cache(d.k, P, C, k_tilde=kt, r_cache=r, t0=0, t1=t_first)
    outs = []
    for t in range(t_first, Tcap):
        wall.build_wall_kv_cache(d.k, P, C, k_tilde=kt, r_cache=r, t0=t, t1=t + 1)
        o, lse = wall.wall_attn_decode(qall[:, t:t + 1].to(DEV), d.v, P[:, t:t + 1], kt, r,
                                       sink_bias=d.sink_bias, scale=inp.scale, cache_chunk_size=C,
                                       seq_len=t + 1)
        outs.append((f64(o)[:, 0], f64(lse)[:, 0]))
    torch.cuda.synchronize()
    rows = [b * Tcap + t for b in range(B) for t in range(t_first, Tcap)]
    o_f, l_f = oracle.wall_attn_oracle(qall, inp.k, inp.v, inp.g, scale=inp.scale, sink_bias=inp.sink_bias,
                                       rows=rows)
    og = np.stack([x[0] for x in outs], axis=1)
    lg = np.stack([x[1] for x in outs], axis=1)
    check_o(og, lg, o_f[:, t_first:], l_f[:, t_first:], "bfloat16", "streaming decode vs forward rows")


def test_decode_full_size_sampled():
    """The decode workload at its full size, in the launch configuration the
    benchmark times; the oracle checks three of the sixteen sequences."""
    inp = make_decode_inputs("decode_bf16")
    B, T, HQ, H, K = inp.q.shape[0], inp.k.shape[1], inp.q.shape[2], inp.k.shape[2], inp.q.shape[3]
    say(f"decode full size B={B} T={T} HQ={HQ} H={H} K={K} bf16 C=64")
    d = inp.to(DEV)
    P = wall.wall_prefix_scan(d.g)
    kt, r = wall.build_wall_kv_cache(d.k, P, 64)
    o, lse = wall.wall_attn_decode(d.q, d.v, P[:, T - 1:T], kt, r, scale=inp.scale)
    torch.cuda.synchronize()
    sel = [0, 7, 15]
    Ph = f64(P[sel])
    kt_ref, r_ref = oracle.kv_cache_oracle(inp.k[sel], Ph, 64)
    assert np.array_equal(f64(r[sel]), r_ref)
    o_ref, l_ref = oracle.decode_oracle(inp.q[sel], inp.v[sel], Ph[:, T - 1:T], kt_ref, r_ref, 64,
                                        scale=inp.scale)
    check_o(f64(o[sel])[:, 0], f64(lse[sel])[:, 0], o_ref[:, 0], l_ref[:, 0], "bfloat16",
            "full-size decode vs cached-decode oracle (3 sequences)")


@pytest.mark.parametrize("dtype", ["bfloat16", "float32"])
def test_prefix_append_matches_full_prefix(dtype):
    """P built by appends of 1..100 rows (the first without a previous row)
    equals the fp64 prefix of g / ln 2 within the float32 bound of a
    sequential sum, (rows + 2) * 2^-24 * sum |g| / ln 2, and the scan's P
    within twice that."""
    B, T, HQ, K = 3, 300, 2, 64
    say(f"prefix append {dtype} B={B} T={T} C={HQ * K}")
    inp = make_decode_inputs("decode_bf16", B=B, T=T, HQ=HQ, H=1, K=K, V=64, dtype=dtype)
    d = inp.to(DEV)
    P = torch.full((B, T, HQ, K), float("nan"), dtype=torch.float32, device=DEV)
    cuts = [0, 1, 2, 9, 64, 65, 164, 165, 299, 300]
    for t0, t1 in zip(cuts[:-1], cuts[1:]):
        wall.wall_prefix_append(d.g[:, t0:t1], prev=None if t0 == 0 else P[:, t0 - 1], out=P[:, t0:t1])
    Ps = wall.wall_prefix_scan(d.g)
    torch.cuda.synchronize()
    g = f64(inp.g)
    ref = oracle.prefix_scan_oracle(inp.g)
    bound = (np.arange(T)[None, :, None, None] + 2) * 2.0 ** -24 * np.cumsum(np.abs(g), axis=1) / math.log(2.0)
    got = f64(P)
    assert np.isfinite(got).all()
    assert (np.abs(got - ref) <= bound + 1e-30).all(), f"max excess {(np.abs(got - ref) - bound).max():.3e}"
    assert (np.abs(got - f64(Ps)) <= 2 * bound + 1e-30).all()


def test_streaming_loop_with_incremental_prefix():
    """The README's streaming loop end to end on the GPU: a prefill of the
    first rows (prefix by append, cache build), then per token the prefix
    append, the cache append and the decode.  Every decoded row matches the
    product-form forward oracle's row; each chunk's anchor is its first row's
    floored P until a row lies more than 64 log2 units below it (the fast
    channels of this gate cross that inside a chunk), and the cache equals
    the oracle's for the appended prefix; the last chunk is partial (200
    rows, C = 64)."""
    B, Tcap, HQ, H, K, V, C = 2, 200, 4, 2, 128, 128, 64
    t_first = 60
    say(f"streaming loop B={B} rows {t_first}..{Tcap - 1} HQ={HQ} H={H} K={K} V={V} C={C}")
    inp = make_decode_inputs("decode_bf16", chunk_size=C, B=B, T=Tcap, HQ=HQ, H=H, K=K, V=V, sink=True)
    rng = np.random.default_rng(12)
    qall = torch.from_numpy(rng.standard_normal((B, Tcap, HQ, K))).to(torch.bfloat16)
    d = inp.to(DEV)
    P = torch.empty((B, Tcap, HQ, K), dtype=torch.float32, device=DEV)
    kt = torch.empty((B, Tcap, HQ, K), dtype=torch.bfloat16, device=DEV)
    r = torch.empty((B, -(-Tcap // C), HQ, K), dtype=torch.float32, device=DEV)
    wall.wall_prefix_append(d.g[:, :t_first], out=P[:, :t_first])
    wall.build_wall_kv_cache(d.k, P, C, k_tilde=kt, r_cache=r, t0=0, t1=t_first)
    outs, moved = [], 0
    for t in range(t_first, Tcap):
        wall.wall_prefix_append(d.g[:, t:t + 1], prev=P[:, t - 1], out=P[:, t:t + 1])
        before = r[:, t // C].clone()
        wall.build_wall_kv_cache(d.k, P, C, k_tilde=kt, r_cache=r, t0=t, t1=t + 1)
        if t % C != 0:
            moved += int((r[:, t // C] != before).any())
        o, lse = wall.wall_attn_decode(qall[:, t:t + 1].to(DEV), d.v, P[:, t:t + 1], kt, r,
                                       sink_bias=d.sink_bias, scale=inp.scale, cache_chunk_size=C,
                                       seq_len=t + 1)
        outs.append((f64(o)[:, 0], f64(lse)[:, 0]))
    torch.cuda.synchronize()
    Pg = f64(P)
    kt_ref, r_ref = oracle.kv_cache_oracle(inp.k, Pg, C)
    assert np.array_equal(f64(r), r_ref), "anchors differ from the oracle's"
    check_kt(f64(kt), kt_ref, "bfloat16")
    assert moved > 0  # some anchor moved inside a chunk during the loop
    rows = [b * Tcap + t for b in range(B) for t in range(t_first, Tcap)]
    o_f, l_f = oracle.wall_attn_oracle(qall, inp.k, inp.v, inp.g, scale=inp.scale, sink_bias=inp.sink_bias,
                                       rows=rows)
    og = np.stack([x[0] for x in outs], axis=1)
    lg = np.stack([x[1] for x in outs], axis=1)
    check_o(og, lg, o_f[:, t_first:], l_f[:, t_first:], "bfloat16", "streaming loop vs forward rows")


@pytest.mark.parametrize("dtype", ["bfloat16", "float32"])
def test_stream_append_equals_separate_calls(dtype):
    """wall_stream_append gives the bits of wall_prefix_append followed by
    build_wall_kv_cache, for a prefill, single rows and a multi-row append
    that opens a chunk, with a partial last chunk."""
    B, Tcap, HQ, H, K, C = 2, 200, 4, 2, 64, 64
    say(f"stream append vs separate calls {dtype} B={B} T_cap={Tcap} HQ={HQ} H={H} K={K} C={C}")
    inp = make_decode_inputs("decode_bf16", chunk_size=C, B=B, T=Tcap, HQ=HQ, H=H, K=K, V=64, dtype=dtype)
    d = inp.to(DEV)
    NC = -(-Tcap // C)

    def bufs():
        return (torch.full((B, Tcap, HQ, K), float("nan"), dtype=torch.float32, device=DEV),
                torch.zeros((B, Tcap, HQ, K), dtype=d.k.dtype, device=DEV),
                torch.full((B, NC, HQ, K), float("nan"), dtype=torch.float32, device=DEV))

    Pa, kta, ra = bufs()
    Pb, ktb, rb = bufs()
    for t0, t1 in [(0, 60), (60, 61), (61, 62), (62, 140), (140, 141), (141, 199), (199, 200)]:
        wall.wall_prefix_append(d.g[:, t0:t1], prev=None if t0 == 0 else Pa[:, t0 - 1], out=Pa[:, t0:t1])
        wall.build_wall_kv_cache(d.k, Pa, C, k_tilde=kta, r_cache=ra, t0=t0, t1=t1)
        wall.wall_stream_append(d.g, d.k, Pb, ktb, rb, C, t0, t1)
    torch.cuda.synchronize()
    assert torch.equal(Pa, Pb), "P differs"
    assert torch.equal(kta, ktb), "k_tilde differs"
    assert torch.equal(ra, rb), "anchors differ"
