"""The float range of the anchored factors, shown on the CPU.

A host model of the bf16 forward's logits (tests/anchor_model.py) against
the fp64 product form of the oracle.  With one middle-row anchor per
128-row tile the diagonal terms are lost once the prefix falls by more than
about 126 log2 units over half a tile (a gate below about exp(-1.3) per
token, held over 64 tokens): q~ flushes to 0 while k~ saturates.  With the
split rule the kernels use (last-row anchors for key tiles before the
query's tile, per-wave anchors inside it, pair-by-pair float32 terms when
even a wave's rows span more than 100 log2 units) every case stays at the
bf16 parity bar, up to a gate of -800 per token where only each token's own
key is left (the all-gates-closed closed form of the oracle pins).
"""

import math

import numpy as np
import pytest
import torch

import oracle
from tests.anchor_model import attend, logits
from wall_inputs import make_inputs

LN2 = math.log(2.0)


def _case(gate, K, T=300, seed=3):
    inp = make_inputs("long_bf16", B=1, T=T, HQ=1, H=1, K=K, V=K, seed=seed)
    if isinstance(gate, float):
        inp.g = torch.full_like(inp.g, gate)
    elif gate == "mixed_small":
        gen = torch.Generator().manual_seed(seed)
        inp.g = (0.02 * torch.randn(inp.g.shape, generator=gen, dtype=torch.float64)).to(inp.g.dtype)
    q = inp.q[0, :, 0].double().numpy()
    k = inp.k[0, :, 0].double().numpy()
    v = inp.v[0, :, 0].double().numpy()
    P = (np.cumsum(inp.g[0, :, 0].double().numpy(), axis=0) / LN2).astype(np.float32)
    o_ref, _ = oracle.wall_attn_oracle(inp.q, inp.k, inp.v, inp.g, scale=inp.scale)
    return q, k, v, P, inp.scale / LN2, o_ref[0, :, 0]


def _err(rule, gate, K, T=300):
    q, k, v, P, qscale, o_ref = _case(gate, K, T)
    o = attend(logits(q, k, P, qscale, rule), v)
    if not np.isfinite(o).all():  # inf * 0 in a saturated pair
        return math.inf, math.inf
    d = o - o_ref
    return float(np.abs(d).max()), float(np.sqrt(np.mean(d * d)))


@pytest.mark.parametrize("K", [64, 128])
@pytest.mark.parametrize("gate", [-1.5, -2.0, -5.0, -30.0, -800.0])
def test_split_anchors_exact_under_strong_decay(gate, K):
    mx, rms = _err("split", gate, K)
    assert mx <= 2e-2 and rms <= 2e-3, (gate, K, mx, rms)


@pytest.mark.parametrize("gate", ["bimodal", "mixed_small", -1.0])
def test_split_anchors_exact_on_ordinary_gates(gate):
    mx, rms = _err("split", gate, 128, T=333)
    assert mx <= 2e-2 and rms <= 2e-3, (gate, mx, rms)


@pytest.mark.parametrize("gate", [-1.5, -2.0, -5.0])
def test_middle_row_anchors_lose_the_diagonal(gate):
    """The rule the kernels used before: the error is of the order of o itself
    (or the output is not finite, where a saturated k~ meets a flushed q~)."""
    mx, _ = _err("mid", gate, 128)
    assert mx > 0.3, (gate, mx)


def test_middle_row_anchors_hold_inside_their_envelope():
    mx, rms = _err("mid", -1.0, 128)
    assert mx <= 2e-2 and rms <= 2e-3


def test_all_gates_closed_keeps_only_the_own_key():
    """g = -800 per token: every earlier key's decay is 0, the own key's is 1."""
    q, k, v, P, qscale, o_ref = _case(-800.0, 128)
    S = logits(q, k, P, qscale, "split")
    T = q.shape[0]
    own = np.einsum("tk,tk->t", q, k) * qscale
    np.testing.assert_allclose(np.diag(S), own, rtol=1e-6, atol=1e-9)
    off = S[np.tril_indices(T, -1)]
    assert np.all(off == 0.0)
