"""Exact output distribution of the verify step for tiny vocabularies.

TEST INFRASTRUCTURE ONLY (checks the oracle; never used by the product path).

Given one draft position (k = 1) with target rows p_0, p_1 and draft row q_0,
the verify step is a deterministic function of (x~, u00, u01, u11): the draft
token and three uniforms. For V <= 8 this module partitions each uniform's
range [0,1) at every point where the rule can change its answer (r = p/q for
the acceptance test, the normalized CDF breakpoints C_j/Z for the two
inverse-CDF draws), evaluates the oracle once inside every cell of the
partition, and weights each answer by q(x~) times the cell's length. The
result is the oracle's exact output distribution.

"Speculative Decoding: The Physics of Stolen Time", section 2, proves that the
first emitted token is distributed as p_0; given acceptance, the bonus token is
distributed as p_1 and acceptance happens with probability sum_x min(p_0, q_0).
``closed_form`` evaluates that statement with exact rational arithmetic
(fractions.Fraction) on the same double-precision p and q, independently of
the oracle's code.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
from scipy.special import softmax

import oracle


def _cells(breaks):
    """Sorted cells of [0,1) cut at `breaks`, each with a float32 probe inside."""
    pts = sorted(set([0.0, 1.0] + [float(b) for b in breaks if 0.0 < b < 1.0]))
    cells = []
    for lo, hi in zip(pts[:-1], pts[1:]):
        mid = np.float32((lo + hi) / 2)
        if not (lo < float(mid) < hi):
            raise ValueError(f"cell [{lo}, {hi}) holds no float32 probe")
        cells.append((lo, hi, mid))
    return cells


def _cdf_breaks(w):
    c = np.cumsum(w)
    return list(c / c[-1]) if c[-1] > 0 else []


def cells_k1(target, draft, T):
    """The enumeration's inputs for k = 1: one batch row per cell.

    target: float32 [2, V] logits; draft: float32 [1, V]. Returns (target
    [n,2,V], draft [n,1,V], tokens [n,1] int32, uniforms [n,2,2] float32,
    weights [n] float64): every draft token x~ with q(x~) > 0 times every cell
    of the uniforms' partition that matters on its branch, each probed at its
    float32 midpoint and weighted by q(x~) times the cell lengths.
    """
    target = np.asarray(target, np.float32)
    draft = np.asarray(draft, np.float32)
    V = target.shape[1]
    p0 = softmax(target[0].astype(np.float64) / np.float64(np.float32(T)))
    p1 = softmax(target[1].astype(np.float64) / np.float64(np.float32(T)))
    q0 = softmax(draft[0].astype(np.float64) / np.float64(np.float32(T)))
    resid = np.maximum(0.0, p0 - q0)

    rows, weights = [], []
    for x in range(V):
        if q0[x] == 0.0:
            continue
        r = p0[x] / q0[x]
        for lo0, hi0, u00 in _cells([r]):
            accepted = float(u00) < r
            if accepted:
                for lo1, hi1, u11 in _cells(_cdf_breaks(p1)):
                    rows.append((x, u00, np.float32(0.5), u11))
                    weights.append(q0[x] * (hi0 - lo0) * (hi1 - lo1))
            else:
                w = resid if resid.sum() > 0 else p0
                for lo1, hi1, u01 in _cells(_cdf_breaks(w)):
                    rows.append((x, u00, u01, np.float32(0.5)))
                    weights.append(q0[x] * (hi0 - lo0) * (hi1 - lo1))

    n = len(rows)
    tgt = np.broadcast_to(target, (n, 2, V)).copy()
    dft = np.broadcast_to(draft, (n, 1, V)).copy()
    tok = np.array([[r[0]] for r in rows], np.int32)
    uni = np.zeros((n, 2, 2), np.float32)
    for j, (_, u00, u01, u11) in enumerate(rows):
        uni[j, 0, 0], uni[j, 0, 1], uni[j, 1, 1] = u00, u01, u11
    return tgt, dft, tok, uni, np.array(weights, np.float64)


def distribution(out_tokens, accepted_len, weights, V):
    """(dist0, dist1_accepted, accept_prob) of weighted outcomes of cells_k1 rows."""
    dist0 = np.zeros(V)
    dist1 = np.zeros(V)
    acc = 0.0
    for j in range(len(weights)):
        dist0[out_tokens[j, 0]] += weights[j]
        if accepted_len[j] == 1:
            dist1[out_tokens[j, 1]] += weights[j]
            acc += weights[j]
    return dist0, dist1, acc


def enumerate_k1(target, draft, T):
    """Exact distribution of (out0, out1) of the oracle for k = 1.

    target: float32 [2, V] logits; draft: float32 [1, V]. Returns
    (dist0 [V], dist1_accepted [V], accept_prob) as float64 arrays.
    """
    tgt, dft, tok, uni, weights = cells_k1(target, draft, T)
    res = oracle.spec_verify_ref(tgt, dft, tok, uni, T, oracle.SAMPLE, dtype=oracle.F32)
    return distribution(res.out_tokens, res.accepted_len, weights, tgt.shape[2])


def closed_form(target, draft, T):
    """Exact rationals: P(out0 = x) from the rule, sum_x min(p,q), p_0, p_1."""
    target = np.asarray(target, np.float32)
    draft = np.asarray(draft, np.float32)
    p0 = softmax(target[0].astype(np.float64) / np.float64(np.float32(T)))
    p1 = softmax(target[1].astype(np.float64) / np.float64(np.float32(T)))
    q0 = softmax(draft[0].astype(np.float64) / np.float64(np.float32(T)))
    P = [Fraction(float(v)) for v in p0]
    Q = [Fraction(float(v)) for v in q0]
    acc = sum(min(a, b) for a, b in zip(P, Q))
    W = [max(Fraction(0), a - b) for a, b in zip(P, Q)]
    Z = sum(W)
    rej = sum(Q) - acc
    out0 = [min(a, b) + (rej * w / Z if Z > 0 else Fraction(0)) for a, b, w in zip(P, Q, W)]
    return out0, acc, p0, p1
