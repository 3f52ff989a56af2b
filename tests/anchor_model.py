"""Host model of the float range of the forward's anchored factors.

Test infrastructure only.  It emulates, in numpy, how the bf16 forward forms
each logit ``scale * sum_n exp2(P_in - P_jn) q_in k_jn`` from two anchored
factors, ``q_i exp2(P_i - R)`` and ``k_j exp2(R - P_j)`` (the per-tile anchor
identity of the Wall Attention blog, section "Fast training and
inference"), each rounded to bf16 and each clamped to the exponent range
the kernels clamp to.  A value below the float32 normal range is taken as
0, the most pessimistic reading of how the matrix cores treat denormal
operands.  The model shows on the CPU which anchor rules keep every term of
the product form that matters and which lose terms, for any gate strength.

It shares nothing with the HIP sources or with the oracle; the tests
compare what it predicts with the fp64 product form.

Two rules are modelled:

``mid``    one anchor per 128-row tile at the floored prefix of the tile's
           middle row, for every query that reads the tile (the rule the
           library used first).  Both factors of a pair stay within 2^(+-D),
           D the change of P over half a tile; once D passes ~126 the
           diagonal terms are lost.
``split``  the rule the kernels use now:
           * a key tile that lies wholly before the query's own 128-row
             tile is anchored at its own last row, so for a prefix that
             falls both factors are at most about 1 and a factor that
             underflows belongs to a term that is itself negligible;
           * the keys of the query's own tile are read against anchors the
             query's 32-row wave chooses for itself: the floored prefix at
             the middle of the wave's rows, unless some row of the wave is
             more than ``THR`` log2 units from it; then the keys before the
             wave use the row just before the wave, and the keys among the
             wave's own rows are formed pair by pair in float32 without
             anchors.
"""

from __future__ import annotations

import numpy as np
import torch

TILE = 128
WAVE = 32
EXP_LO, EXP_HI = -160.0, 126.0
THR = 100.0
FLT_MIN = 2.0 ** -126


def bf16(x):
    """Round to bf16 (nearest even) and flush magnitudes below 2^-126 to 0."""
    y = torch.from_numpy(np.asarray(x, dtype=np.float64)).to(torch.bfloat16).to(torch.float64).numpy()
    return np.where(np.abs(y) < FLT_MIN, 0.0, y)


def exp2c(e):
    return np.exp2(np.clip(e, EXP_LO, EXP_HI))


def shift(x, d):
    """x * 2^-d for integer d >= 0 as an exponent-field decrement: exact or 0."""
    y = x * np.exp2(-np.asarray(d, dtype=np.float64))
    return np.where(np.abs(y) < FLT_MIN, 0.0, y)


def _last_row_anchor(P, c, T):
    return np.floor(P[min(TILE * c + TILE - 1, T - 1)])


def logits(q, k, P, qscale, rule):
    """Scores S[i, j] (log2 units) for j <= i, -inf above the diagonal.

    q, k: [T, K] float64 (already dtype-rounded); P: [T, K] float32 prefix.
    """
    T, K = q.shape
    P = P.astype(np.float64)
    S = np.full((T, T), -np.inf)
    ntiles = (T + TILE - 1) // TILE
    if rule == "mid":
        R = [np.floor(P[min(TILE * c + TILE // 2, T - 1)]) for c in range(ntiles)]
        kt = np.zeros_like(k)
        for c in range(ntiles):
            r0, r1 = TILE * c, min(TILE * c + TILE, T)
            kt[r0:r1] = bf16(k[r0:r1] * exp2c(R[c] - P[r0:r1]))
        for i in range(T):
            qt = i // TILE
            a0 = bf16(q[i] * qscale * exp2c(P[i] - R[qt]))
            for c in range(qt + 1):
                a = shift(a0, np.maximum(R[c] - R[qt], 0.0)) if c < qt else a0
                r0, r1 = TILE * c, min(TILE * c + TILE, i + 1)
                S[i, r0:r1] = kt[r0:r1] @ a
        return S
    if rule != "split":
        raise ValueError(rule)
    L = [_last_row_anchor(P, c, T) for c in range(ntiles)]
    kt = np.zeros_like(k)
    for c in range(ntiles):
        r0, r1 = TILE * c, min(TILE * c + TILE, T)
        kt[r0:r1] = bf16(k[r0:r1] * exp2c(L[c] - P[r0:r1]))
    for q0 in range(0, T, WAVE):
        q1 = min(q0 + WAVE, T)
        qt = q0 // TILE
        t0 = TILE * qt
        M = np.floor(P[(q0 + q1 - 1) // 2])
        flagged = bool(np.abs(P[q0:q1] - M).max() > THR)
        for i in range(q0, q1):
            # key tiles before the query's own tile: last-row anchors, q~ carried
            if qt > 0:
                aL = bf16(q[i] * qscale * exp2c(P[i] - L[qt - 1]))
                for c in range(qt):
                    a = shift(aL, L[c] - L[qt - 1])
                    S[i, TILE * c:TILE * c + TILE] = kt[TILE * c:TILE * c + TILE] @ a
            if not flagged:
                a = bf16(q[i] * qscale * exp2c(P[i] - M))
                b = bf16(k[t0:i + 1] * exp2c(M - P[t0:i + 1]))
                S[i, t0:i + 1] = b @ a
            else:
                if q0 > t0:
                    A = np.floor(P[q0 - 1])
                    a = bf16(q[i] * qscale * exp2c(P[i] - A))
                    b = bf16(k[t0:q0] * exp2c(A - P[t0:q0]))
                    S[i, t0:q0] = b @ a
                f = np.exp2(np.clip(P[i] - P[q0:i + 1], EXP_LO, EXP_HI))
                f = np.where(f < FLT_MIN, 0.0, f)
                S[i, q0:i + 1] = (k[q0:i + 1] * f) @ (q[i] * qscale)
    return S


def attend(S, v):
    m = S.max(axis=1, keepdims=True)
    p = np.exp2(S - m)
    return (p @ v) / p.sum(axis=1, keepdims=True)
