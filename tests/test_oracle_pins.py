"""Pins for the fp64 oracle: it is checked against what the pages and the
mathematics fix, never against itself.

* hand-derived worked examples (tests/golden/worked_examples.json);
* the factored form of the Wall Attention blog ("Definition: Wall Attention":
  q~ = exp(P) q, k~ = exp(-P) k, o = Attn(q~, k~, v)), an independent formula;
* special cases that reduce to torch's scaled_dot_product_attention: g = 0 is
  vanilla softmax attention (README introduction), g_scalar alone is FoX's
  additive bias (blog FoX formula), the window is a band mask;
* closed forms: all gates closed, channel-uniform gate, T = 1, the sink;
* invariants: causality, GQA == explicit repetition, varlen == per-sequence.
"""

import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def rnd(rng, *shape):
    return rng.standard_normal(size=shape)


def sdpa(q, k, v, scale, mask=None, causal=False):
    """torch SDPA in fp64 on the CPU, [B,T,H,D] layout, GQA by repeat_interleave."""
    qt = torch.from_numpy(q).permute(0, 2, 1, 3)
    kt = torch.from_numpy(k).permute(0, 2, 1, 3)
    vt = torch.from_numpy(v).permute(0, 2, 1, 3)
    grp = qt.shape[1] // kt.shape[1]
    kt = kt.repeat_interleave(grp, dim=1)
    vt = vt.repeat_interleave(grp, dim=1)
    m = None if mask is None else torch.from_numpy(mask)
    o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, is_causal=causal, scale=scale)
    return o.permute(0, 2, 1, 3).numpy()


# --------------------------------------------------------------------------- golden


def test_worked_examples(oracle_mod):
    cases = json.load(open(GOLDEN))["cases"]
    env = {"exp": math.exp, "log": math.log}
    for c in cases:
        a = lambda key: None if key not in c else np.array(c[key], dtype=np.float64)
        g = np.log(np.array(c["g_gates"], dtype=np.float64))
        o, lse = oracle_mod.wall_attn_oracle(
            a("q"), a("k"), a("v"), g, scale=c["scale"], g_scalar=a("g_scalar"),
            sink_bias=a("sink_bias"), window_size=c.get("window_size"),
            cu_seqlens=c.get("cu_seqlens"))
        exp_o = np.array([[eval(e, env) for e in row] for row in c["expected"]["o"]])
        exp_l = np.array([[eval(e, env) for e in row] for row in c["expected"]["lse"]])
        np.testing.assert_allclose(o[..., 0, 0], exp_o, rtol=1e-14, atol=1e-14, err_msg=c["name"])
        np.testing.assert_allclose(lse[..., 0], exp_l, rtol=1e-14, atol=1e-14, err_msg=c["name"])


# --------------------------------------------------------------------------- factored form


def factored_form(q, k, v, g, scale, g_scalar=None, sink=None, window=None, cu=None):
    """The blog's factored form: P = cumsum(log gate) per sequence,
    q~ = exp(P) * q, k~ = exp(-P) * k, o = causal softmax attention of (q~, k~, v).
    Options enter as an additive bias G_i - G_j (cumsum of g_scalar), a band
    mask, a block-diagonal sequence mask and an extra logit."""
    B, T, HQ, K = q.shape
    H = k.shape[2]
    grp = HQ // H
    starts = np.zeros(T, dtype=np.int64)
    if cu is not None:
        for s in range(len(cu) - 1):
            starts[cu[s]:cu[s + 1]] = cu[s]
    P = np.zeros_like(g)
    Gs = None if g_scalar is None else np.zeros_like(g_scalar)
    for t in range(T):
        first = starts[t] == t
        P[:, t] = g[:, t] + (0 if first else P[:, t - 1])
        if Gs is not None:
            Gs[:, t] = g_scalar[:, t] + (0 if first else Gs[:, t - 1])
    o = np.zeros((B, T, HQ, v.shape[3]))
    lse = np.zeros((B, T, HQ))
    ii, jj = np.meshgrid(np.arange(T), np.arange(T), indexing="ij")
    vis = (jj <= ii) & (starts[jj] == starts[ii])
    if window:
        vis &= (ii - jj) < window
    for b in range(B):
        for hq in range(HQ):
            h = hq // grp
            qt = np.exp(P[b, :, hq]) * q[b, :, hq]
            kt = np.exp(-P[b, :, hq]) * k[b, :, h]
            s = scale * qt @ kt.T
            if Gs is not None:
                s = s + Gs[b, :, hq][:, None] - Gs[b, :, hq][None, :]
            s = np.where(vis, s, -np.inf)
            cols = [s]
            if sink is not None:
                cols.append(np.full((T, 1), sink[hq]))
            full = np.concatenate(cols, axis=1)
            m = full.max(axis=1, keepdims=True)
            e = np.exp(full - m)
            Z = e.sum(axis=1, keepdims=True)
            o[b, :, hq] = (e[:, :T] @ v[b, :, h]) / Z
            lse[b, :, hq] = (m + np.log(Z))[:, 0]
    return o, lse


@pytest.mark.parametrize("opts", ["plain", "fox", "window", "sink", "varlen", "all"])
def test_product_equals_factored(oracle_mod, opts):
    rng = np.random.default_rng(11)
    B, T, HQ, H, K, V = (1 if opts in ("varlen", "all") else 2), 29, 4, 2, 8, 5
    q, k, v = rnd(rng, B, T, HQ, K), rnd(rng, B, T, H, K), rnd(rng, B, T, H, V)
    g = 0.3 * rnd(rng, B, T, HQ, K)  # mixed signs, |P| small enough for exp(+-P)
    kw = {}
    if opts in ("fox", "all"):
        kw["g_scalar"] = -np.abs(rnd(rng, B, T, HQ))
    if opts in ("window", "all"):
        kw["window"] = 7
    if opts in ("sink", "all"):
        kw["sink"] = rnd(rng, HQ)
    if opts in ("varlen", "all"):
        kw["cu"] = [0, 5, 5, 17, 29]  # includes an empty sequence
    o_f, l_f = factored_form(q, k, v, g, 0.37, **kw)
    o, l = oracle_mod.wall_attn_oracle(
        q, k, v, g, scale=0.37, g_scalar=kw.get("g_scalar"), sink_bias=kw.get("sink"),
        window_size=kw.get("window"), cu_seqlens=kw.get("cu"))
    np.testing.assert_allclose(o, o_f, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l, l_f, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------- library special cases


def test_g_zero_is_vanilla_softmax_attention(oracle_mod):
    rng = np.random.default_rng(12)
    B, T, HQ, H, K, V = 2, 37, 6, 3, 16, 8
    q, k, v = rnd(rng, B, T, HQ, K), rnd(rng, B, T, H, K), rnd(rng, B, T, H, V)
    o, _ = oracle_mod.wall_attn_oracle(q, k, v, np.zeros((B, T, HQ, K)), scale=0.3)
    np.testing.assert_allclose(o, sdpa(q, k, v, 0.3, causal=True), rtol=0, atol=1e-13)


def test_gscalar_alone_is_fox_additive_bias(oracle_mod):
    rng = np.random.default_rng(13)
    B, T, HQ, H, K, V = 2, 33, 4, 2, 8, 8
    q, k, v = rnd(rng, B, T, HQ, K), rnd(rng, B, T, H, K), rnd(rng, B, T, H, V)
    gs = -np.abs(rnd(rng, B, T, HQ))
    G = np.cumsum(gs, axis=1)  # [B,T,HQ]
    ii, jj = np.meshgrid(np.arange(T), np.arange(T), indexing="ij")
    D = G.transpose(0, 2, 1)[:, :, :, None] - G.transpose(0, 2, 1)[:, :, None, :]  # [B,HQ,T,T]
    mask = np.where(jj <= ii, D, -np.inf)
    o, _ = oracle_mod.wall_attn_oracle(q, k, v, np.zeros((B, T, HQ, K)), scale=0.6, g_scalar=gs)
    np.testing.assert_allclose(o, sdpa(q, k, v, 0.6, mask=mask), rtol=0, atol=1e-13)


@pytest.mark.parametrize("W", [1, 4, 40])
def test_window_is_band_mask(oracle_mod, W):
    rng = np.random.default_rng(14)
    B, T, HQ, H, K, V = 1, 31, 2, 1, 8, 4
    q, k, v = rnd(rng, B, T, HQ, K), rnd(rng, B, T, H, K), rnd(rng, B, T, H, V)
    ii, jj = np.meshgrid(np.arange(T), np.arange(T), indexing="ij")
    band = (jj <= ii) & (ii - jj < W)
    o, _ = oracle_mod.wall_attn_oracle(q, k, v, np.zeros((B, T, HQ, K)), scale=0.5, window_size=W)
    np.testing.assert_allclose(o, sdpa(q, k, v, 0.5, mask=band), rtol=0, atol=1e-13)
    if W == 1:  # each query sees only itself
        np.testing.assert_allclose(o, np.repeat(v, HQ // H, axis=2), rtol=0, atol=1e-15)
    # with gates as well: W >= T is the same as no window
    g = -np.abs(rnd(rng, B, T, HQ, K))
    o1, l1 = oracle_mod.wall_attn_oracle(q, k, v, g, window_size=T)
    o2, l2 = oracle_mod.wall_attn_oracle(q, k, v, g)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


# --------------------------------------------------------------------------- closed forms


def test_sink_closed_form(oracle_mod):
    rng = np.random.default_rng(15)
    B, T, HQ, H, K, V = 1, 23, 3, 3, 8, 6
    q, k, v = rnd(rng, B, T, HQ, K), rnd(rng, B, T, H, K), rnd(rng, B, T, H, V)
    g = -np.abs(rnd(rng, B, T, HQ, K))
    sink = 2.0 * rnd(rng, HQ)
    o, l = oracle_mod.wall_attn_oracle(q, k, v, g)
    o_s, l_s = oracle_mod.wall_attn_oracle(q, k, v, g, sink_bias=sink)
    exp_l = np.logaddexp(l, sink[None, None, :])
    np.testing.assert_allclose(l_s, exp_l, rtol=0, atol=1e-13)
    np.testing.assert_allclose(o_s, o * np.exp(l - exp_l)[..., None], rtol=0, atol=1e-13)


def test_all_gates_closed(oracle_mod):
    """gate -> 0 on every channel: past logits become 0 (not -inf), so
    o_i = (sum_{j<i} v_j + e^{s_ii} v_i) / (i + e^{s_ii}), s_ii = scale q_i.k_i."""
    rng = np.random.default_rng(16)
    B, T, HQ, H, K, V = 1, 19, 2, 1, 8, 3
    q, k, v = rnd(rng, B, T, HQ, K), rnd(rng, B, T, H, K), rnd(rng, B, T, H, V)
    g = np.full((B, T, HQ, K), -800.0)  # exp(-800) underflows to exactly 0 in fp64
    o, _ = oracle_mod.wall_attn_oracle(q, k, v, g, scale=0.4)
    for hq in range(HQ):
        for i in range(T):
            s = 0.4 * q[0, i, hq] @ k[0, i, 0]
            exp_o = (v[0, :i, 0].sum(axis=0) + math.exp(s) * v[0, i, 0]) / (i + math.exp(s))
            np.testing.assert_allclose(o[0, i, hq], exp_o, rtol=0, atol=1e-13)


def test_channel_uniform_gate_is_scalar_decay(oracle_mod):
    """g_{t,n} = a_t on every channel: s_ij = scale * exp(A_i - A_j) * q_i.k_j."""
    rng = np.random.default_rng(17)
    B, T, HQ, H, K, V = 1, 27, 2, 2, 8, 4
    q, k, v = rnd(rng, B, T, HQ, K), rnd(rng, B, T, H, K), rnd(rng, B, T, H, V)
    a = -0.2 * np.abs(rnd(rng, B, T, HQ))
    g = np.repeat(a[..., None], K, axis=3)
    o, _ = oracle_mod.wall_attn_oracle(q, k, v, g, scale=0.5)
    A = np.cumsum(a, axis=1)
    ii, jj = np.meshgrid(np.arange(T), np.arange(T), indexing="ij")
    for hq in range(HQ):
        s = 0.5 * np.exp(A[0, :, hq][:, None] - A[0, :, hq][None, :]) * (q[0, :, hq] @ k[0, :, hq].T)
        s = np.where(jj <= ii, s, -np.inf)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        exp_o = (p @ v[0, :, hq]) / p.sum(axis=1, keepdims=True)
        np.testing.assert_allclose(o[0, :, hq], exp_o, rtol=0, atol=1e-13)


def test_single_token(oracle_mod):
    rng = np.random.default_rng(18)
    q, k, v, g = rnd(rng, 1, 1, 2, 4), rnd(rng, 1, 1, 1, 4), rnd(rng, 1, 1, 1, 3), rnd(rng, 1, 1, 2, 4)
    o, l = oracle_mod.wall_attn_oracle(q, k, v, g, scale=0.7)
    np.testing.assert_allclose(o[0, 0], np.repeat(v[0, 0], 2, axis=0), rtol=0, atol=1e-15)
    sink = np.array([0.3, -1.1])
    o, l = oracle_mod.wall_attn_oracle(q, k, v, g, scale=0.7, sink_bias=sink)
    s = 0.7 * (q[0, 0] @ k[0, 0, 0])  # [HQ]
    sig = 1.0 / (1.0 + np.exp(-(s - sink)))
    np.testing.assert_allclose(o[0, 0], v[0, 0, 0][None, :] * sig[:, None], rtol=0, atol=1e-15)
    np.testing.assert_allclose(l[0, 0], np.logaddexp(s, sink), rtol=0, atol=1e-15)


# --------------------------------------------------------------------------- invariants


def test_causality_and_first_gate(oracle_mod):
    rng = np.random.default_rng(19)
    B, T, HQ, H, K, V = 1, 24, 2, 1, 8, 4
    q, k, v = rnd(rng, B, T, HQ, K), rnd(rng, B, T, H, K), rnd(rng, B, T, H, V)
    g, gs = -np.abs(rnd(rng, B, T, HQ, K)), -np.abs(rnd(rng, B, T, HQ))
    cu = [0, 10, 24]
    base = oracle_mod.wall_attn_oracle(q, k, v, g, g_scalar=gs, cu_seqlens=cu)
    cut = 13
    pert = [x.copy() for x in (q, k, v, g, gs)]
    for x in pert:
        x[:, cut + 1:] += 5.0 * rng.standard_normal(size=x[:, cut + 1:].shape)
    alt = oracle_mod.wall_attn_oracle(*pert[:4], g_scalar=pert[4], cu_seqlens=cu)
    np.testing.assert_array_equal(alt[0][:, :cut + 1], base[0][:, :cut + 1])
    np.testing.assert_array_equal(alt[1][:, :cut + 1], base[1][:, :cut + 1])
    # the gate (and the scalar gate) at each sequence's first token never enters
    g2, gs2 = g.copy(), gs.copy()
    g2[:, [0, 10]] = 123.0
    gs2[:, [0, 10]] = -77.0
    alt = oracle_mod.wall_attn_oracle(q, k, v, g2, g_scalar=gs2, cu_seqlens=cu)
    np.testing.assert_array_equal(alt[0], base[0])


def test_gqa_equals_explicit_repeat(oracle_mod):
    rng = np.random.default_rng(20)
    B, T, HQ, H, K, V = 2, 21, 6, 2, 8, 5
    q, k, v = rnd(rng, B, T, HQ, K), rnd(rng, B, T, H, K), rnd(rng, B, T, H, V)
    g = -np.abs(rnd(rng, B, T, HQ, K))
    o1, l1 = oracle_mod.wall_attn_oracle(q, k, v, g)
    o2, l2 = oracle_mod.wall_attn_oracle(q, np.repeat(k, 3, axis=2), np.repeat(v, 3, axis=2), g)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_varlen_equals_per_sequence(oracle_mod):
    rng = np.random.default_rng(21)
    T, HQ, H, K, V = 40, 4, 2, 8, 6
    q, k, v = rnd(rng, 1, T, HQ, K), rnd(rng, 1, T, H, K), rnd(rng, 1, T, H, V)
    g, gs = -np.abs(rnd(rng, 1, T, HQ, K)), -np.abs(rnd(rng, 1, T, HQ))
    sink = rnd(rng, HQ)
    cu = [0, 7, 7, 25, 40]
    o, l = oracle_mod.wall_attn_oracle(q, k, v, g, g_scalar=gs, sink_bias=sink, window_size=9, cu_seqlens=cu)
    for s in range(len(cu) - 1):
        a, b = cu[s], cu[s + 1]
        if a == b:
            continue
        os_, ls_ = oracle_mod.wall_attn_oracle(q[:, a:b], k[:, a:b], v[:, a:b], g[:, a:b],
                                               g_scalar=gs[:, a:b], sink_bias=sink, window_size=9)
        np.testing.assert_array_equal(o[:, a:b], os_)
        np.testing.assert_array_equal(l[:, a:b], ls_)


def test_row_subset_matches_full(oracle_mod):
    rng = np.random.default_rng(22)
    B, T, HQ, H, K, V = 2, 30, 2, 1, 8, 4
    q, k, v = rnd(rng, B, T, HQ, K), rnd(rng, B, T, H, K), rnd(rng, B, T, H, V)
    g = -np.abs(rnd(rng, B, T, HQ, K))
    o, l = oracle_mod.wall_attn_oracle(q, k, v, g)
    rows = [0, 17, 29, 30, 59]
    o2, l2 = oracle_mod.wall_attn_oracle(q, k, v, g, rows=rows)
    of, lf = o.reshape(B * T, HQ, V), l.reshape(B * T, HQ)
    np.testing.assert_array_equal(o2.reshape(B * T, HQ, V)[rows], of[rows])
    np.testing.assert_array_equal(l2.reshape(B * T, HQ)[rows], lf[rows])
    assert np.isnan(o2.reshape(B * T, HQ, V)[1]).all()


# --------------------------------------------------------------------------- prefix scan


def test_prefix_scan_closed_form(oracle_mod):
    """Constant gate c: P_t = (t - s + 1) c / ln 2 inside each sequence."""
    T, C = 50, 3
    x = np.full((1, T, C), -0.7)
    cu = [0, 12, 12, 50]
    P = oracle_mod.prefix_scan_oracle(x, cu_seqlens=cu)
    pos = np.concatenate([np.arange(12), np.arange(38)])
    np.testing.assert_allclose(P[0, :, 0], (pos + 1) * -0.7 / math.log(2.0), rtol=1e-14)
    xb = np.full((3, 9, 2, 2), 0.25)
    Pb = oracle_mod.prefix_scan_oracle(xb, scale=2.0)
    np.testing.assert_allclose(Pb[:, :, 1, 1], np.tile((np.arange(9) + 1) * 0.5, (3, 1)), rtol=1e-15)


def test_prefix_scan_matches_numpy_cumsum(oracle_mod):
    rng = np.random.default_rng(23)
    x = rnd(rng, 2, 77, 3, 5)
    P = oracle_mod.prefix_scan_oracle(x, scale=1.0 / math.log(2.0))
    np.testing.assert_allclose(P, np.cumsum(x, axis=1) / math.log(2.0), rtol=1e-13, atol=1e-13)


# --------------------------------------------------------------------------- decode cache and decode


@pytest.mark.parametrize("case", [
    # strong decay, sink, GQA, a partial last chunk
    dict(B=2, T=150, HQ=4, H=2, K=8, V=6, C=64, g=-0.3, sink=True, scale=0.35),
    # gates of both signs, one row per chunk
    dict(B=1, T=40, HQ=2, H=1, K=5, V=3, C=1, g=0.05, sink=False, scale=0.8),
    # one chunk longer than the sequence, odd chunk size
    dict(B=1, T=23, HQ=3, H=3, K=4, V=4, C=7, g=-1.0, sink=True, scale=0.5),
    dict(B=3, T=23, HQ=2, H=1, K=4, V=2, C=64, g=-0.1, sink=False, scale=0.5),
    # a single cached token
    dict(B=2, T=1, HQ=2, H=2, K=3, V=5, C=64, g=-0.5, sink=True, scale=0.9),
    # gates strong enough to move the chunk anchors many times
    dict(B=2, T=140, HQ=2, H=1, K=6, V=4, C=64, g=-5.0, sink=True, scale=0.4),
    dict(B=1, T=70, HQ=2, H=2, K=4, V=3, C=64, g=-800.0, sink=False, scale=0.6),
])
def test_decode_equals_forward_last_row(oracle_mod, case):
    """README: the decode kernel reproduces the training forward token for
    token.  The cached decode (anchored keys, query factor exp2(p - R)) must
    give the product-form forward's last row, for any anchors."""
    rng = np.random.default_rng(31)
    B, T, HQ, H, K, V, C = (case[x] for x in ("B", "T", "HQ", "H", "K", "V", "C"))
    q, k, v = rnd(rng, B, T, HQ, K), rnd(rng, B, T, H, K), rnd(rng, B, T, H, V)
    if case["g"] < 0:
        g = case["g"] * np.abs(rnd(rng, B, T, HQ, K))
    else:
        g = case["g"] * rnd(rng, B, T, HQ, K)
    sink = rnd(rng, HQ) if case["sink"] else None
    P = oracle_mod.prefix_scan_oracle(g)
    kt, r = oracle_mod.kv_cache_oracle(k, P, C)
    assert r.shape == (B, -(-T // C), HQ, K)
    assert np.array_equal(r, np.round(r))  # integer anchors: exact powers of two
    o, l = oracle_mod.decode_oracle(q[:, -1:], v, P[:, -1:], kt, r, C, sink_bias=sink, scale=case["scale"])
    of, lf = oracle_mod.wall_attn_oracle(q, k, v, g, scale=case["scale"], sink_bias=sink)
    np.testing.assert_allclose(o[:, 0], of[:, -1], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(l[:, 0], lf[:, -1], rtol=1e-12, atol=1e-12)


def test_kv_cache_zero_gate_and_reconstruction(oracle_mod):
    """g = 0: every anchor is 0 and k_tilde is k repeated over the query
    heads of its group.  Any gate: the anchored keys carry exactly the
    factor exp2(R - P_j), so k_tilde * exp2(P_j - R) gives k back."""
    rng = np.random.default_rng(37)
    B, T, HQ, H, K, C = 2, 70, 4, 2, 6, 16
    k = rnd(rng, B, T, H, K)
    kt, r = oracle_mod.kv_cache_oracle(k, np.zeros((B, T, HQ, K)), C)
    assert not r.any()
    np.testing.assert_array_equal(kt, np.repeat(k, HQ // H, axis=2))
    P = oracle_mod.prefix_scan_oracle(-np.abs(rnd(rng, B, T, HQ, K)))
    kt, r = oracle_mod.kv_cache_oracle(k, P, C)
    Rj = np.repeat(r, C, axis=1)[:, :T]
    np.testing.assert_allclose(kt * np.exp2(P - Rj), np.repeat(k, HQ // H, axis=2), rtol=1e-13, atol=1e-14)
    # every key factor exp2(R - P_j) of a chunk stays at most 2^64, and the
    # anchor is the floored prefix of one of the chunk's own rows
    assert (Rj - P <= 64.0).all()
    for c in range(-(-T // C)):
        rows = np.floor(P[:, c * C:(c + 1) * C])
        assert np.all(np.any(rows == r[:, c:c + 1], axis=1))


def test_kv_cache_anchor_moves_worked_example(oracle_mod):
    """One chunk of four rows whose prefix falls 0, -10, -70.5, -100 (log2
    units): the anchor starts at 0, stays while the rows lie at most 64 below
    it, moves to floor(-70.5) = -71 at the third row, and stays (the fourth row
    is 29 below).  Worked by hand."""
    P = np.array([0.0, -10.0, -70.5, -100.0]).reshape(1, 4, 1, 1)
    k = np.array([1.0, 2.0, 3.0, 4.0]).reshape(1, 4, 1, 1)
    kt, r = oracle_mod.kv_cache_oracle(k, P, 4)
    assert r.reshape(-1).tolist() == [-71.0]
    np.testing.assert_allclose(kt.reshape(-1), [2.0 ** -71, 2.0 * 2.0 ** -61, 3.0 * 2.0 ** -0.5, 4.0 * 2.0 ** 29],
                               rtol=1e-15)


# --------------------------------------------------------------------------- backward


def _fd_check(oracle_mod, args, kw, grads, rng, eps=1e-6, rtol=1e-6):
    """Central differences of sum(o * do) in a random direction per input."""
    q, k, v, g, gs, sink, do = args

    def loss(q, k, v, g, gs, sink):
        o, _ = oracle_mod.wall_attn_oracle(q, k, v, g, g_scalar=gs, sink_bias=sink, **kw)
        return float((o * do).sum())

    base = [q, k, v, g, gs, sink]
    for idx, name in enumerate(["q", "k", "v", "g", "g_scalar", "sink"]):
        if base[idx] is None:
            assert grads[idx] is None
            continue
        d = rng.standard_normal(base[idx].shape)
        up, dn = list(base), list(base)
        up[idx] = base[idx] + eps * d
        dn[idx] = base[idx] - eps * d
        fd = (loss(*up) - loss(*dn)) / (2 * eps)
        an = float((grads[idx] * d).sum())
        assert abs(fd - an) <= rtol * max(1.0, abs(fd)), (name, fd, an)


@pytest.mark.parametrize("case", ["plain", "gqa_window_fox_sink", "varlen", "positive_gate", "single_token"])
def test_backward_matches_central_differences(oracle_mod, case):
    """The README checks its gate gradients with finite differences; here every
    gradient of the oracle's backward is held to central differences of the
    forward oracle."""
    rng = np.random.default_rng(41)
    B, T, HQ, H, K, V = 2, 29, 4, 2, 5, 3
    kw = dict(scale=0.45)
    gs = sink = None
    cu = None
    if case == "single_token":
        T = 1
    if case == "varlen":
        B, cu = 1, [0, 7, 7, 8, 29]
        kw["cu_seqlens"] = cu
    q, k, v = rnd(rng, B, T, HQ, K), rnd(rng, B, T, H, K), rnd(rng, B, T, H, V)
    g = (0.2 if case == "positive_gate" else -0.3) * np.abs(rnd(rng, B, T, HQ, K))
    if case == "gqa_window_fox_sink":
        gs = -0.2 * np.abs(rnd(rng, B, T, HQ))
        sink = rnd(rng, HQ)
        kw["window_size"] = 11
    do = rnd(rng, B, T, HQ, V)
    grads = oracle_mod.wall_attn_bwd_oracle(q, k, v, g, do, g_scalar=gs, sink_bias=sink, **kw)
    _fd_check(oracle_mod, (q, k, v, g, gs, sink, do), kw, grads, rng)
    # a decay-gate entry at a sequence's first token moves nothing: its gradient is 0
    starts = [0] if cu is None else sorted(set(x for x in cu[:-1] if x < T))
    for s in starts:
        np.testing.assert_allclose(grads[3][:, s], 0.0, atol=1e-10)
        if gs is not None:
            np.testing.assert_allclose(grads[4][:, s], 0.0, atol=1e-10)


def test_backward_g_zero_is_sdpa_autograd(oracle_mod):
    """g = 0: dq, dk, dv are softmax attention's, from torch autograd of
    scaled_dot_product_attention in fp64 (GQA by explicit repetition)."""
    rng = np.random.default_rng(43)
    B, T, HQ, H, K, V = 2, 33, 4, 2, 6, 5
    q, k, v, do = rnd(rng, B, T, HQ, K), rnd(rng, B, T, H, K), rnd(rng, B, T, H, V), rnd(rng, B, T, HQ, V)
    dq, dk, dv, _, _, _ = oracle_mod.wall_attn_bwd_oracle(q, k, v, np.zeros((B, T, HQ, K)), do, scale=0.3)
    qt = torch.tensor(q).transpose(1, 2).requires_grad_()
    kt = torch.tensor(k).transpose(1, 2).requires_grad_()
    vt = torch.tensor(v).transpose(1, 2).requires_grad_()
    o = F.scaled_dot_product_attention(qt, kt.repeat_interleave(HQ // H, 1), vt.repeat_interleave(HQ // H, 1),
                                       is_causal=True, scale=0.3)
    o.backward(torch.tensor(do).transpose(1, 2))
    np.testing.assert_allclose(dq, qt.grad.transpose(1, 2).numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dk, kt.grad.transpose(1, 2).numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dv, vt.grad.transpose(1, 2).numpy(), rtol=1e-10, atol=1e-12)
