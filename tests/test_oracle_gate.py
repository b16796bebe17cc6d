"""Pins of the oracle's confidence gate (oracle.spec_gate_ref), CPU only.

The gate is defined by "Speculative Pre-Positioning", section 2.4 (Eqs. 11-13)
and Algorithm 2, and, for the certified rule, by the speculative-decoding
design note's argmax-stability bound (2*tau <= gap). Pinned by hand-worked
examples, by numpy's argmax/partition on random rows, by the monotonicity of
the coverage c(tau) that the pages state, and by the argmax-stability property
itself under worst-case perturbations (which fixes the factor 2 exactly).
"""
import numpy as np
import pytest

import oracle

M, C = oracle.MARGIN, oracle.CERTIFIED


def gate(rows, rule, tau, admit=None):
    return oracle.spec_gate_ref(np.asarray(rows, np.float32), rule, tau, admit)


def test_worked_examples():
    r = gate([[1, 3, 2.5]], M, 0.4)
    assert r.argmax[0] == 1 and r.gap[0] == 0.5 and r.fire[0]
    assert not gate([[1, 3, 2.5]], M, 0.5).fire[0]             # strict: gap > tau
    assert gate([[1, 3, 2.5]], C, 0.25).fire[0]                # 2 * 0.25 <= 0.5
    assert not gate([[1, 3, 2.5]], C, 0.2500001).fire[0]
    # a tie at the top: gap 0, lowest index; the certified rule needs a strict argmax
    r = gate([[2, 5, 5, 1]], M, -1.0)
    assert r.argmax[0] == 1 and r.gap[0] == 0.0 and r.fire[0]
    assert not gate([[2, 5, 5, 1]], C, 0.0).fire[0]
    # one finite entry: gap +inf
    r = gate([[-np.inf, 4, -np.inf]], C, 1e30)
    assert r.argmax[0] == 1 and r.gap[0] == np.inf and r.fire[0]
    assert gate([[-np.inf, 4, -np.inf]], M, 3e38).fire[0]


def test_invalid_rows_never_fire():
    r = gate([[np.nan, 1, 0], [np.inf, 0, 1], [-np.inf, -np.inf, -np.inf], [0, 1, 2]], M, -10.0)
    assert list(r.argmax) == [-1, -1, -1, 2]
    assert np.isnan(r.gap[:3]).all() and r.gap[3] == 1.0
    assert list(r.fire) == [False, False, False, True]


def test_admissible_set():
    rows = [[0, 9, 1, 2], [7, 0, 1, 2], [0, 1, 2, 9]]
    A = oracle.admit_mask([1, 3], 4)
    r = gate(rows, M, 1.0, A)
    assert list(r.argmax) == [1, 0, 3]
    assert list(r.fire) == [True, False, True]
    # the mask's bit order across words: token 37 is bit 5 of word 1
    V = 40
    row = np.zeros((1, V), np.float32)
    row[0, 37] = 5.0
    assert gate(row, M, 1.0, oracle.admit_mask([37], V)).fire[0]
    assert not gate(row, M, 1.0, oracle.admit_mask([5, 36, 38], V)).fire[0]


def test_bf16_rows_read_as_bits():
    import torch
    t = torch.tensor([[0.5, 3.0, 2.75, -1.0]], dtype=torch.bfloat16)
    r = oracle.spec_gate_ref(t, M, 0.2)
    assert r.argmax[0] == 1 and r.gap[0] == 0.25 and r.fire[0]


def test_matches_numpy_on_random_rows():
    rng = np.random.default_rng(3)
    x = rng.normal(0, 2, (400, 257)).astype(np.float32)
    x[::7, 11] = x[::7].max(axis=1) + rng.uniform(0, 8, x[::7].shape[0]).astype(np.float32)
    A = oracle.admit_mask(rng.choice(257, 60, replace=False), 257)
    inA = np.array([(A[j >> 5] >> (j & 31)) & 1 for j in range(257)], bool)
    for tau in (0.0, 0.5, 2.0, 5.0):
        r = oracle.spec_gate_ref(x, M, tau, A)
        am = np.argmax(x, axis=1)
        part = np.partition(x, -2, axis=1)
        g32 = part[:, -1] - part[:, -2]                 # float32 subtraction
        assert (r.argmax == am).all()
        np.testing.assert_array_equal(r.gap, part[:, -1].astype(np.float64) - part[:, -2])
        assert (r.fire == ((g32 > np.float32(tau)) & inA[am])).all()


def test_coverage_is_monotone_in_tau():
    # c(tau) of Eq. 13 is non-increasing in tau
    rng = np.random.default_rng(4)
    x = rng.normal(0, 2, (300, 100)).astype(np.float32)
    x[np.arange(300), rng.integers(0, 100, 300)] += rng.uniform(0, 10, 300).astype(np.float32)
    taus = np.linspace(-1, 12, 40)
    for rule in (M, C):
        cov = [oracle.spec_gate_ref(x, rule, max(t, 0.0) if rule == C else t).fire.mean() for t in taus]
        assert all(a >= b for a, b in zip(cov, cov[1:]))
        assert cov[0] > 0.9 and cov[-1] < 0.2


def test_certified_rule_is_argmax_stability():
    # fires  => no perturbation with sup-norm < tau moves the argmax;
    # does not fire (strict argmax, admissible) => some perturbation with
    # sup-norm < tau makes another token at least tie the top (worst case:
    # lower the top by s, raise the runner-up by s, s just below tau)
    rng = np.random.default_rng(5)
    x = rng.normal(0, 1, (200, 50)).astype(np.float64)
    x[np.arange(200), rng.integers(0, 50, 200)] += rng.uniform(0, 4, 200)
    x32 = x.astype(np.float32)
    for tau in (0.05, 0.3, 1.0, 1.7):
        r = oracle.spec_gate_ref(x32, C, tau)
        xs = x32.astype(np.float64)
        a = np.argmax(xs, axis=1)
        second = np.argsort(xs, axis=1)[:, -2]
        for i in range(200):
            s = tau * (1 - 1e-6)
            y = xs[i].copy()
            y[a[i]] -= s
            y[second[i]] += s
            flipped = np.argmax(y) != a[i] or np.sum(y == y.max()) > 1
            gap = xs[i, a[i]] - xs[i, second[i]]
            if r.fire[i]:
                assert not flipped
            elif gap > 0 and abs(2 * tau - gap) > 1e-5:
                assert flipped


def test_rejects_bad_tau():
    with pytest.raises(ValueError):
        gate([[0, 1]], M, float("nan"))
    with pytest.raises(ValueError):
        gate([[0, 1]], C, -0.5)
