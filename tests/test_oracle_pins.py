"""Pins of the fp64 oracle against facts the pages and the mathematics fix.

Each test below ties the oracle to something other than its own code: a
closed form worked out by hand from exact rational probabilities, the pages'
printed number, exact enumeration, a textbook library routine, or a
statistical law. Together they are chosen so that a plausible mistake in the
oracle (p/q transposed, the residual sign flipped, temperature dropped on one
side, a non-strict comparison, the wrong uniform channel, an off-by-one in the
inverse CDF) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
from scipy import stats
from scipy.special import softmax

import oracle
from oracle import exact_enum

HERE = os.path.dirname(os.path.abspath(__file__))
NEG = -np.inf


def run(target, draft, tokens, uniforms, T=1.0, mode=oracle.SAMPLE):
    t = np.asarray(target, np.float32)
    d = None if draft is None else np.asarray(draft, np.float32)
    k = t.shape[1] - 1
    tok = np.asarray(tokens, np.int32).reshape(t.shape[0], k)
    u = None if uniforms is None else np.asarray(uniforms, np.float32)
    return oracle.spec_verify_ref(t, d, tok, u, T, mode, dtype=oracle.F32)


def logits_of(p, T=1.0):
    """Logits whose softmax at temperature T is p (zeros become -inf)."""
    p = np.asarray(p, np.float64)
    with np.errstate(divide="ignore"):
        return (T * np.log(p)).astype(np.float32)


# ---------------------------------------------------------------- hand-worked closed forms
# p = (0.1, 0.2, 0.3, 0.4), q = (0.4, 0.3, 0.2, 0.1); residual max(0, p - q) =
# (0, 0, 0.1, 0.3), Z = 0.4, normalized CDF (0, 0, 0.25, 1).

P4 = [0.1, 0.2, 0.3, 0.4]
Q4 = [0.4, 0.3, 0.2, 0.1]
UNIF4 = [0.25, 0.25, 0.25, 0.25]          # all-zero logits: exactly uniform


def test_hand_accept_when_ratio_above_one():
    # x = 3: r = 0.4 / 0.1 = 4 -> accepted for any u; bonus from the uniform
    # row with u = 0.6: CDF (0.25, 0.5, 0.75, 1) -> first C_j > 0.6 is j = 2.
    r = run([[logits_of(P4), np.zeros(4)]], [[logits_of(Q4)]], [[3]], [[[0.99, 0.01], [0.3, 0.6]]])
    assert r.accepted_len[0] == 1
    assert list(r.out_tokens[0]) == [3, 2]
    assert r.p_tok[0, 0] == pytest.approx(0.4, abs=1e-7)   # float32 logits
    assert r.q_tok[0, 0] == pytest.approx(0.1, abs=1e-7)


def test_hand_reject_and_residual():
    # x = 0: r = 0.1 / 0.4 = 0.25; u0 = 0.3 >= r -> reject. Residual draw with
    # u1 = 0.5: target 0.5 * 0.4 = 0.2 -> C = (0, 0, 0.1, 0.4) -> token 3.
    r = run([[logits_of(P4), np.zeros(4)]], [[logits_of(Q4)]], [[0]], [[[0.3, 0.5], [0.0, 0.0]]])
    assert r.accepted_len[0] == 0
    assert list(r.out_tokens[0]) == [3, -1]
    assert r.margin_acc[0] == pytest.approx(0.05, abs=1e-7)      # |0.3 - 0.25|
    assert r.margin_cdf[0] == pytest.approx(0.25, abs=1e-7)      # u=0.5 in [0.25, 1)


def test_hand_accept_below_ratio():
    # Same draft token, u0 = 0.2 < 0.25 -> accepted; bonus with u = 0.1 -> token 0.
    r = run([[logits_of(P4), np.zeros(4)]], [[logits_of(Q4)]], [[0]], [[[0.2, 0.9], [0.0, 0.1]]])
    assert r.accepted_len[0] == 1
    assert list(r.out_tokens[0]) == [0, 0]


def test_hand_residual_small_uniform():
    # x = 1: r = 0.2 / 0.3; u0 = 0.7 rejects; u1 = 0.1 -> 0.04 of Z = 0.4 -> token 2.
    r = run([[logits_of(P4), np.zeros(4)]], [[logits_of(Q4)]], [[1]], [[[0.7, 0.1], [0.0, 0.0]]])
    assert r.accepted_len[0] == 0
    assert list(r.out_tokens[0]) == [2, -1]


def test_hand_temperature_scales_both_rows():
    # Logits are T*ln(p) with T = 0.5, so softmax(logits / T) = p exactly:
    # p = (0.2, 0.8), q = (0.6, 0.4). x = 0: r = 1/3, u0 = 0.5 rejects; the
    # residual is (0, 0.4) so the token is 1. Ignoring T on either row would
    # give r = (1/3)/(0.55...) ~ 0.61 and accept instead.
    T = 0.5
    r = run([[logits_of([0.2, 0.8], T), np.zeros(2)]], [[logits_of([0.6, 0.4], T)]], [[0]],
            [[[0.5, 0.3], [0.0, 0.0]]], T=T)
    assert r.accepted_len[0] == 0
    assert list(r.out_tokens[0]) == [1, -1]
    assert r.p_tok[0, 0] == pytest.approx(0.2, abs=1e-7)
    assert r.q_tok[0, 0] == pytest.approx(0.6, abs=1e-7)
    # the gap is on raw logits: |0.5 ln 0.8 - 0.5 ln 0.2| = 0.5 ln 4
    assert r.gap[0, 0] == pytest.approx(0.5 * math.log(4.0), abs=1e-6)


def test_inverse_cdf_boundary_is_strict():
    # k = 0, uniform p over 4 tokens, u = 0.5 sits exactly on C_1 = 0.5.
    # "smallest j with C_j > u Z" gives j = 2 (a non-strict search would give 1).
    r = run([[np.zeros(4)]], [np.zeros((0, 4))], np.zeros((1, 0)), [[[0.0, 0.5]]])
    assert r.accepted_len[0] == 0
    assert r.out_tokens[0, 0] == 2
    r = run([[np.zeros(4)]], [np.zeros((0, 4))], np.zeros((1, 0)), [[[0.0, 0.0]]])
    assert r.out_tokens[0, 0] == 0


# ---------------------------------------------------------------- special cases of the rule


def test_q_equals_p_accepts_all(rng=np.random.default_rng(1)):
    # "Physics of Stolen Time", section 2: with q = p every ratio is 1 and
    # u < 1 always accepts; all k accepted then a bonus from p_k.
    B, k, V = 64, 5, 50
    t = rng.normal(0, 2, (B, k + 1, V)).astype(np.float32)
    d = t[:, :k].copy()
    tok = rng.integers(0, V, (B, k)).astype(np.int32)
    u = rng.random((B, k + 1, 2)).astype(np.float32)
    u[:, :, 0] = np.float32(1.0) - np.float32(2.0 ** -24)   # the largest u below 1
    r = run(t, d, tok, u)
    assert (r.accepted_len == k).all()
    assert (r.out_tokens[:, :k] == tok).all()
    # bonus = textbook inverse CDF of p_k
    for b in range(B):
        p = softmax(t[b, k].astype(np.float64))
        assert r.out_tokens[b, k] == np.searchsorted(np.cumsum(p), u[b, k, 1] * np.cumsum(p)[-1], "right")


def test_disjoint_supports_reject_first_and_resample_from_p(rng=np.random.default_rng(2)):
    # supp p and supp q disjoint: p(x) = 0 so r = 0 and even u = 0 rejects;
    # max(0, p - q) = p, so the token is the inverse-CDF draw from p.
    B, k, V = 40, 3, 16
    t = rng.normal(0, 1, (B, k + 1, V)).astype(np.float32)
    d = rng.normal(0, 1, (B, k, V)).astype(np.float32)
    t[:, :, V // 2:] = NEG
    d[:, :, : V // 2] = NEG
    tok = rng.integers(V // 2, V, (B, k)).astype(np.int32)
    u = rng.random((B, k + 1, 2)).astype(np.float32)
    u[:, 0, 0] = 0.0
    r = run(t, d, tok, u)
    assert (r.accepted_len == 0).all()
    for b in range(B):
        p = softmax(t[b, 0].astype(np.float64))
        c = np.cumsum(p)
        assert r.out_tokens[b, 0] == np.searchsorted(c, u[b, 0, 1] * c[-1], "right")
        assert (r.out_tokens[b, 1:] == -1).all()


def test_k0_is_categorical_sampling(rng=np.random.default_rng(3)):
    # With no drafts the step is one draw from p_0 = softmax(l / T).
    B, V = 200, 37
    for T in (0.3, 1.0, 2.5):
        t = rng.normal(0, 2, (B, 1, V)).astype(np.float32)
        u = rng.random((B, 1, 2)).astype(np.float32)
        r = run(t, np.zeros((B, 0, V), np.float32), np.zeros((B, 0)), u, T=T)
        for b in range(B):
            p = softmax(t[b, 0].astype(np.float64) / np.float64(np.float32(T)))
            c = np.cumsum(p)
            assert r.out_tokens[b, 0] == np.searchsorted(c, u[b, 0, 1] * c[-1], "right")
        assert (r.accepted_len == 0).all()


def test_gap_and_argmax_match_numpy(rng=np.random.default_rng(4)):
    # Gap = top-1 minus top-2 logit ("Speculative Pre-Positioning", Eq. 11);
    # argmax = first maximum. Rows are bf16-like (coarse) so ties occur.
    B, k, V = 100, 3, 64
    t = np.round(rng.normal(0, 2, (B, k + 1, V)) * 4) / 4
    t = t.astype(np.float32)
    tok = rng.integers(0, V, (B, k)).astype(np.int32)
    r = run(t, None, tok, None, mode=oracle.GREEDY)
    for b in range(B):
        for i in range(k + 1):
            top2 = np.partition(t[b, i].astype(np.float64), -2)[-2:]
            assert r.gap[b, i] == top2[1] - top2[0]
    ties = sum(r.gap[b, i] == 0 for b in range(B) for i in range(k + 1))
    assert ties > 0


def test_greedy_rule(rng=np.random.default_rng(5)):
    # "The Inference Wall" part 7: accept while the guess equals the target's
    # argmax; at the first mismatch emit the target's argmax; all matched -> k+1.
    B, k, V = 300, 4, 20
    t = np.round(rng.normal(0, 2, (B, k + 1, V)) * 2).astype(np.float32) / 2
    am = np.argmax(t, axis=2)
    tok = am[:, :k].copy().astype(np.int32)
    mism = rng.random((B, k)) < 0.3
    tok[mism] = rng.integers(0, V, mism.sum())
    r = run(t, None, tok, None, mode=oracle.GREEDY)
    for b in range(B):
        a = next((i for i in range(k) if tok[b, i] != am[b, i]), k)
        assert r.accepted_len[b] == a
        assert list(r.out_tokens[b, :a]) == list(tok[b, :a])
        assert r.out_tokens[b, a] == am[b, a]
        assert (r.out_tokens[b, a + 1:] == -1).all()


def test_greedy_equals_sampling_on_one_hot(rng=np.random.default_rng(6)):
    # Temperature 0 is the one-hot limit ("The Inference Wall" part 7, "Does it
    # make the answers worse?"): with p = onehot(argmax l) and q = onehot(x),
    # r is 1 or 0 and the residual is onehot(argmax), so the sampling rule
    # reproduces greedy verification for every uniform.
    B, k, V = 200, 4, 12
    t = np.round(rng.normal(0, 2, (B, k + 1, V)) * 2).astype(np.float32) / 2
    am = np.argmax(t, axis=2)
    tok = am[:, :k].copy().astype(np.int32)
    mism = rng.random((B, k)) < 0.35
    tok[mism] = rng.integers(0, V, mism.sum())
    g = run(t, None, tok, None, mode=oracle.GREEDY)
    oh_t = np.full_like(t, NEG)
    oh_d = np.full((B, k, V), NEG, np.float32)
    for b in range(B):
        for i in range(k + 1):
            oh_t[b, i, am[b, i]] = 0.0
        for i in range(k):
            oh_d[b, i, tok[b, i]] = 0.0
    u = rng.random((B, k + 1, 2)).astype(np.float32)
    s = run(oh_t, oh_d, tok, u)
    assert (s.accepted_len == g.accepted_len).all()
    assert (s.out_tokens == g.out_tokens).all()


def test_argmax_stable_under_small_perturbation(rng=np.random.default_rng(7)):
    # Design note, "Axis 1 reuses the gate": if every logit moves by less than
    # tau in sup-norm and 2 tau <= gap, the argmax cannot change.
    B, V = 500, 40
    t = rng.normal(0, 2, (B, 1, V)).astype(np.float32)
    base = run(t, None, np.zeros((B, 0)), None, mode=oracle.GREEDY)
    gap = base.gap[:, 0]
    tau = (gap / 2) * 0.999
    delta = (rng.random((B, 1, V)) * 2 - 1) * tau[:, None, None]
    pert = (t.astype(np.float64) + delta).astype(np.float32)
    # float32 rounding can move a value by half an ulp; keep |delta| < tau after it
    ok = np.abs(pert.astype(np.float64) - t.astype(np.float64)).max(axis=(1, 2)) < gap / 2
    moved = run(pert, None, np.zeros((B, 0)), None, mode=oracle.GREEDY)
    assert ok.mean() > 0.95
    assert (moved.out_tokens[ok, 0] == base.out_tokens[ok, 0]).all()


# ---------------------------------------------------------------- distribution-level pins


@pytest.mark.parametrize("seed", range(12))
def test_exact_enumeration_matches_p(seed):
    # Exact output distribution over (draft token, uniforms) for V <= 8 equals
    # p_0 within 1e-12; given acceptance, the bonus is distributed as p_1 and
    # acceptance has probability sum min(p, q) ("Physics of Stolen Time", section 2).
    rng = np.random.default_rng(100 + seed)
    V = int(rng.integers(2, 9))
    T = float(rng.choice([0.5, 1.0, 1.7]))
    t = rng.normal(0, 1.5, (2, V)).astype(np.float32)
    d = (t[:1] + rng.normal(0, 1.0, (1, V))).astype(np.float32)
    if seed % 4 == 3:
        d[0, : V // 2] = NEG          # draft misses part of the support
    dist0, dist1, acc = exact_enum.enumerate_k1(t, d, T)
    out0, acc_exact, p0, p1 = exact_enum.closed_form(t, d, T)
    assert np.abs(dist0 - p0).max() < 1e-12
    assert np.abs(dist0 - np.array([float(x) for x in out0])).max() < 1e-12
    assert abs(acc - float(acc_exact)) < 1e-12
    assert np.abs(dist1 - acc * p1).max() < 1e-12


def test_chi_square_one_million_trials():
    # 10^6 seeded trials: x ~ q, u ~ U(0,1); the first emitted token must be
    # indistinguishable from p_0 (losslessness, "Physics of Stolen Time", section 2).
    rng = np.random.default_rng(2024)
    V, n, T = 16, 1_000_000, 0.8
    t0 = rng.normal(0, 1.5, (2, V)).astype(np.float32)
    d0 = (t0[:1] * 0.7 + rng.normal(0, 1.0, (1, V))).astype(np.float32)
    q = softmax(d0[0].astype(np.float64) / np.float64(np.float32(T)))
    p = softmax(t0[0].astype(np.float64) / np.float64(np.float32(T)))
    tok = rng.choice(V, size=(n, 1), p=q).astype(np.int32)
    u = rng.random((n, 2, 2)).astype(np.float32)
    r = run(np.broadcast_to(t0, (n, 2, V)), np.broadcast_to(d0, (n, 1, V)), tok, u, T=T)
    counts = np.bincount(r.out_tokens[:, 0], minlength=V)
    _, pval = stats.chisquare(counts, p * n)
    assert pval > 1e-3, pval
    # the same test must be able to see a wrong rule: accepting every draft
    # yields q, not p
    _, pbad = stats.chisquare(np.bincount(tok[:, 0], minlength=V), p * n)
    assert pbad < 1e-6


def test_accept_length_law_and_printed_expected_tokens():
    # With the same (p, q) at every position, accept events are iid with
    # probability alpha = sum min(p, q): P(a = j) = (1 - alpha) alpha^j (j < k),
    # P(a = k) = alpha^k, and E[a + 1] = (1 - alpha^(k+1)) / (1 - alpha)
    # ("Physics of Stolen Time", section 3). The page evaluates it at
    # alpha = 0.4, k = 4 as about 1.6 (section 4).
    g = json.load(open(os.path.join(HERE, "golden", "pages_printed.json")))["expected_tokens_per_step"]
    alpha, k = g["alpha"], g["k"]
    closed = (1 - alpha ** (k + 1)) / (1 - alpha)
    assert abs(closed - g["printed"]) < g["tolerance"]
    # p = (0.4, 0.6), q = (1, 0): sum min(p, q) = 0.4
    rng = np.random.default_rng(9)
    n, V = 400_000, 2
    t = np.broadcast_to(logits_of([0.4, 0.6]), (n, k + 1, V))
    d = np.broadcast_to(logits_of([1.0, 0.0]), (n, k, V))
    tok = np.zeros((n, k), np.int32)
    u = rng.random((n, k + 1, 2)).astype(np.float32)
    r = run(t, d, tok, u)
    law = np.array([(1 - alpha) * alpha ** j for j in range(k)] + [alpha ** k])
    counts = np.bincount(r.accepted_len, minlength=k + 1)
    _, pval = stats.chisquare(counts, law * n)
    assert pval > 1e-3, (counts, law * n)
    mean = (r.accepted_len + 1).mean()
    sd = (r.accepted_len + 1).std() / math.sqrt(n)
    assert abs(mean - closed) < 5 * sd


def test_accept_length_law_random_pq():
    # Same law with a generic (p, q) pair and x ~ q at every position.
    rng = np.random.default_rng(10)
    n, k, V, T = 300_000, 3, 10, 1.0
    t1 = rng.normal(0, 1, V).astype(np.float32)
    d1 = (t1 + rng.normal(0, 1, V)).astype(np.float32)
    p = softmax(t1.astype(np.float64))
    q = softmax(d1.astype(np.float64))
    alpha = np.minimum(p, q).sum()
    tok = rng.choice(V, size=(n, k), p=q).astype(np.int32)
    u = rng.random((n, k + 1, 2)).astype(np.float32)
    r = run(np.broadcast_to(t1, (n, k + 1, V)), np.broadcast_to(d1, (n, k, V)), tok, u, T=T)
    law = np.array([(1 - alpha) * alpha ** j for j in range(k)] + [alpha ** k])
    counts = np.bincount(r.accepted_len, minlength=k + 1)
    _, pval = stats.chisquare(counts, law * n)
    assert pval > 1e-3, (counts, law * n)


# ---------------------------------------------------------------- invalid inputs


def test_invalid_rows():
    rng = np.random.default_rng(11)
    B, k, V = 6, 2, 8
    t = rng.normal(0, 1, (B, k + 1, V)).astype(np.float32)
    d = rng.normal(0, 1, (B, k, V)).astype(np.float32)
    tok = rng.integers(0, V, (B, k)).astype(np.int32)
    u = rng.random((B, k + 1, 2)).astype(np.float32)
    t[0, 1, 3] = np.nan              # NaN in a target row
    d[1, 0, 5] = np.inf              # +inf in a draft row
    t[2, 2, :] = NEG                 # bonus row with no finite entry
    tok[3, 1] = V                    # token out of range
    t[4, 0, :4] = NEG                # -inf masks are fine
    r = run(t, d, tok, u)
    assert list(r.accepted_len[:4]) == [-1, -1, -1, -1]
    assert (r.out_tokens[:4] == -1).all()
    assert r.accepted_len[4] >= 0 and r.accepted_len[5] >= 0
    # greedy mode ignores draft logits but still checks the target and tokens
    g = run(t, None, tok, None, mode=oracle.GREEDY)
    assert list(g.accepted_len[:4]) == [-1, 0 if tok[1, 0] != np.argmax(t[1, 0]) else g.accepted_len[1], -1, -1]


def test_argument_errors():
    t = np.zeros((1, 2, 4), np.float32)
    with pytest.raises(ValueError):
        run(t, np.zeros((1, 1, 4)), [[0]], np.zeros((1, 2, 2)), T=0.0)
    with pytest.raises(ValueError):
        run(t, np.zeros((1, 1, 4)), [[0]], np.zeros((1, 2, 2)), T=float("nan"))


def test_residual_below_fp64_resolution_is_flagged():
    # Two nearly one-hot distributions on the same token (T = 0.05): the exact
    # residual mass max(0, p - q) is ~1e-17 of p's total mass, below what fp64
    # can resolve in p - q, so the draw is flagged (bit 1). An ordinary pair
    # (residual mass ~0.4) is not.
    t = np.array([[[0.3046875, 0.36328125, -0.20019531, 0.0390625, -0.27734375, -3.140625, 2.546875],
                   [0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0]]], np.float32)
    d = np.array([[[1.0078125, -0.640625, -1.125, 0.6015625, -1.0859375, -2.546875, 2.953125]]], np.float32)
    tok = np.array([[0]], np.int32)
    u = np.array([[[0.21016294, 0.44941747], [0.5, 0.5]]], np.float32)
    r = oracle.spec_verify_ref(t, d, tok, u, 0.05, oracle.SAMPLE)
    assert r.accepted_len[0] == 0
    assert r.flags[0] & 2
    rng = np.random.default_rng(11)
    t2 = rng.normal(0, 2, (1, 2, 50)).astype(np.float32)
    d2 = (t2[:, :1] + rng.normal(0, 1, (1, 1, 50))).astype(np.float32)
    u2 = np.array([[[0.999, 0.3], [0.5, 0.5]]], np.float32)   # u = 0.999 rejects
    # the draft token's target logit is -inf, so p(x) = 0 and the test rejects
    # for every u: the ordinary residual draw always happens and is not flagged
    x2 = int(np.argmax(d2[0, 0]))
    t2[0, 0, x2] = NEG
    r2 = oracle.spec_verify_ref(t2, d2, np.array([[x2]], np.int32), u2, 1.0, oracle.SAMPLE)
    assert r2.accepted_len[0] == 0
    assert r2.flags[0] == 0
    p = softmax(t2[0, 0].astype(np.float64))
    q = softmax(d2[0, 0].astype(np.float64))
    w = np.maximum(0.0, p - q)
    assert r2.out_tokens[0, 0] == np.searchsorted(np.cumsum(w) / w.sum(), np.float64(np.float32(0.3)),
                                                  side="right")


def test_zero_residual_mass_falls_back_to_target():
    # R12: target and draft rows agree exactly and both give the draft token
    # probability 0 (-inf logit), so r = 0 rejects at position 0 and the
    # residual max(0, p - q) is identically zero: the draw falls back to p_0
    # itself (its inverse CDF at u[0,1]) and the row is flagged (bit 0). A
    # mistake that draws from the next target row, or forgets the flag, fails.
    rng = np.random.default_rng(13)
    V = 9
    row = rng.normal(0, 1.5, V).astype(np.float32)
    row[4] = NEG
    nxt = rng.normal(0, 1.5, V).astype(np.float32)
    t = np.stack([row, nxt])[None]
    d = row[None, None].copy()
    for u1 in (0.05, 0.37, 0.81, 0.999):
        u = np.array([[[0.5, u1], [0.5, 0.5]]], np.float32)
        r = run(t, d, [[4]], u)
        assert r.accepted_len[0] == 0
        assert r.flags[0] & 1
        assert r.flagged(1e-6, 1e-12)[0]
        p = softmax(row.astype(np.float64))
        assert r.out_tokens[0, 0] == np.searchsorted(np.cumsum(p), np.float64(np.float32(u1)), side="right")
        assert r.out_tokens[0, 1] == -1


# ---------------------------------------------------------------- alternatives of near-tie rows
# A flagged row may legitimately differ across implementations, but only by
# taking its nearest decision the other way. The oracle reports that outcome;
# these pins tie it to the oracle itself re-run with the uniform moved across
# the boundary.


def test_alternative_of_a_near_tie_acceptance():
    P, Q = [0.1, 0.2, 0.3, 0.4], [0.4, 0.3, 0.2, 0.1]
    t = np.array([[logits_of(P), np.zeros(4)]], np.float32)
    d = np.array([[logits_of(Q)]], np.float32)
    r_true = float(np.float64(softmax(t[0, 0].astype(np.float64))[1] / softmax(d[0, 0].astype(np.float64))[1]))
    f = np.float32(r_true)
    if float(f) < r_true:                                        # float32 neighbours of r
        below, above = f, np.nextafter(f, np.float32(1))
    else:
        below, above = np.nextafter(f, np.float32(0)), f
    assert float(below) < r_true <= float(above)                 # below accepts, above rejects
    for u0, other in ((below, above), (above, below)):
        u = np.array([[[u0, 0.6], [0.3, 0.7]]], np.float32)
        r = oracle.spec_verify_ref(t, d, np.array([[1]], np.int32), u, 1.0, oracle.SAMPLE,
                                   dtype=oracle.F32, flip_delta=1e-6)
        assert r.margin_acc[0] < 1e-6
        u2 = u.copy()
        u2[0, 0, 0] = other
        f = oracle.spec_verify_ref(t, d, np.array([[1]], np.int32), u2, 1.0, oracle.SAMPLE, dtype=oracle.F32)
        assert f.accepted_len[0] != r.accepted_len[0]
        assert r.alt_accepted_len[0] == f.accepted_len[0]
        assert (r.alt_out_tokens[0] == f.out_tokens[0]).all()
    # a row far from every boundary repeats its own outcome
    u = np.array([[[0.9, 0.6], [0.3, 0.7]]], np.float32)
    r = oracle.spec_verify_ref(t, d, np.array([[1]], np.int32), u, 1.0, oracle.SAMPLE, dtype=oracle.F32,
                               flip_delta=1e-6)
    assert r.alt_accepted_len[0] == r.accepted_len[0] and (r.alt_out_tokens[0] == r.out_tokens[0]).all()


def test_alternative_token_across_the_nearest_cdf_edge():
    # k = 0: the draw is textbook sampling from p (cumsum + searchsorted). With
    # u just below / above the edge C_2, the draw gives 2 / 3, and the
    # alternative is the token on the other side (a zero-mass token between is
    # skipped: token 3 has p = 0, so above the edge comes token 4).
    p = np.array([0.1, 0.2, 0.3, 0.0, 0.4])
    t = logits_of(p)[None, None]
    c = np.cumsum(softmax(t[0, 0].astype(np.float64)))
    edge = np.float32(c[2])
    lo = edge if float(edge) < c[2] else np.nextafter(edge, np.float32(0))
    hi = np.nextafter(lo, np.float32(1))
    for u1, tok, alt in ((lo, 2, 4), (hi, 4, 2)):
        assert np.searchsorted(c, np.float64(u1), side="right") == tok
        r = oracle.spec_verify_ref(t, None, np.zeros((1, 0), np.int32), np.array([[[0.5, u1]]], np.float32),
                                   1.0, oracle.SAMPLE, dtype=oracle.F32, flip_delta=1e-6)
        assert r.out_tokens[0, 0] == tok and r.alt_token[0] == alt
        assert r.margin_cdf[0] < 1e-7



# ---------------------------------------------------------------- ragged drafts
# A batch row with draft_len kb is, by definition, the verify rule with k = kb
# on its first kb positions (the design note and the stolen-time article let
# each sequence guess its own number of tokens). Pinned by identities with the
# fixed-length rule (itself pinned above): the equal-length case, truncation to
# kb, rows past kb that are never read, and out-of-range lengths.

def _ragged_case(rng, B, k, V):
    t = rng.normal(0, 2, (B, k + 1, V)).astype(np.float32)
    d = (t[:, :k] + rng.normal(0, 1, (B, k, V))).astype(np.float32)
    tok = rng.integers(0, V, (B, k)).astype(np.int32)
    u = rng.random((B, k + 1, 2)).astype(np.float32)
    return t, d, tok, u


@pytest.mark.parametrize("mode", [oracle.SAMPLE, oracle.GREEDY])
def test_ragged_full_length_equals_fixed(mode):
    rng = np.random.default_rng(21)
    t, d, tok, u = _ragged_case(rng, 40, 4, 30)
    dd, uu = (d, u) if mode == oracle.SAMPLE else (None, None)
    a = oracle.spec_verify_ref(t, dd, tok, uu, 0.8, mode, dtype=oracle.F32)
    r = oracle.spec_verify_ref(t, dd, tok, uu, 0.8, mode, dtype=oracle.F32,
                               draft_len=np.full(40, 4, np.int32))
    for f in ("accepted_len", "out_tokens", "flags"):
        assert (getattr(a, f) == getattr(r, f)).all(), f
    for f in ("gap", "p_tok", "q_tok", "margin_acc", "margin_cdf"):
        np.testing.assert_array_equal(getattr(a, f), getattr(r, f))


@pytest.mark.parametrize("mode", [oracle.SAMPLE, oracle.GREEDY])
def test_ragged_row_equals_truncated_fixed_call(mode):
    rng = np.random.default_rng(22)
    B, k, V = 30, 5, 24
    t, d, tok, u = _ragged_case(rng, B, k, V)
    if mode == oracle.GREEDY:
        am = np.argmax(t[:, :k], axis=2).astype(np.int32)
        tok = np.where(rng.random((B, k)) < 0.7, am, tok).astype(np.int32)
    dl = rng.integers(0, k + 1, B).astype(np.int32)
    dd, uu = (d, u) if mode == oracle.SAMPLE else (None, None)
    r = oracle.spec_verify_ref(t, dd, tok, uu, 1.3, mode, dtype=oracle.F32, draft_len=dl)
    for b in range(B):
        kb = int(dl[b])
        f = oracle.spec_verify_ref(t[b:b + 1, :kb + 1].copy(),
                                   None if dd is None else d[b:b + 1, :kb].copy(),
                                   tok[b:b + 1, :kb].copy(),
                                   None if uu is None else u[b:b + 1, :kb + 1].copy(),
                                   1.3, mode, dtype=oracle.F32)
        assert r.accepted_len[b] == f.accepted_len[0]
        assert (r.out_tokens[b, :kb + 1] == f.out_tokens[0]).all()
        assert (r.out_tokens[b, kb + 1:] == -1).all()
        np.testing.assert_array_equal(r.gap[b, :kb + 1], f.gap[0])
        assert np.isnan(r.gap[b, kb + 1:]).all()
        np.testing.assert_array_equal(r.p_tok[b, :kb], f.p_tok[0])
        assert np.isnan(r.p_tok[b, kb:]).all() and np.isnan(r.q_tok[b, kb:]).all()
        assert r.margin_acc[b] == f.margin_acc[0] and r.margin_cdf[b] == f.margin_cdf[0]
        assert r.flags[b] == f.flags[0]


def test_ragged_rows_past_the_length_are_not_read():
    rng = np.random.default_rng(23)
    B, k, V = 12, 4, 20
    t, d, tok, u = _ragged_case(rng, B, k, V)
    dl = rng.integers(0, k + 1, B).astype(np.int32)
    r = oracle.spec_verify_ref(t, d, tok, u, 1.0, oracle.SAMPLE, dtype=oracle.F32, draft_len=dl)
    t2, d2, tok2 = t.copy(), d.copy(), tok.copy()
    for b in range(B):                 # poison everything the row must not read
        t2[b, dl[b] + 1:] = np.nan
        d2[b, dl[b]:] = np.inf
        tok2[b, dl[b]:] = -5
    r2 = oracle.spec_verify_ref(t2, d2, tok2, u, 1.0, oracle.SAMPLE, dtype=oracle.F32, draft_len=dl)
    assert (r.accepted_len == r2.accepted_len).all() and (r.accepted_len >= 0).all()
    assert (r.out_tokens == r2.out_tokens).all()
    np.testing.assert_array_equal(r.gap, r2.gap)


def test_ragged_length_out_of_range_is_invalid():
    rng = np.random.default_rng(24)
    t, d, tok, u = _ragged_case(rng, 3, 2, 10)
    r = oracle.spec_verify_ref(t, d, tok, u, 1.0, oracle.SAMPLE, dtype=oracle.F32,
                               draft_len=np.array([-1, 3, 2], np.int32))
    assert list(r.accepted_len[:2]) == [-1, -1] and r.accepted_len[2] >= 0
    assert (r.out_tokens[:2] == -1).all() and np.isnan(r.gap[:2]).all()
