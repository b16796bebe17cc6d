"""Property tests of the oracle on random small shapes (hypothesis), CPU only.

Each property follows from the definitions in the pages without restating the
oracle's arithmetic:
* acceptance depends only on p(x)/q(x), so permuting the vocabulary (logits and
  token ids alike) leaves the accepted lengths and the gaps unchanged ("The
  Physics of Stolen Time", section 2);
* softmax(l/T) is what the rule sees: l/2 at T = 1 is the same call as l at
  T = 2, and adding a constant to a row changes nothing but nothing else
  (section 2; the gap of "Speculative Pre-Positioning", Eq. 11, is on the raw
  logits, so it halves and is shift-invariant);
* the output layout (accepted drafts, one emitted token, -1 padding);
* ragged rows never accept more than their length;
* the gate's coverage is monotone in tau row by row (Eq. 13).
Logits are multiples of 1/64 of modest size, so halving and shifting by an
integer are exact in float32.
"""
import numpy as np
from hypothesis import given, settings, strategies as st

import oracle

SET = settings(max_examples=60, deadline=None)


@st.composite
def calls(draw, greedy=False):
    B = draw(st.integers(1, 4))
    k = draw(st.integers(0, 4))
    V = draw(st.integers(1, 24))
    seed = draw(st.integers(0, 2 ** 31 - 1))
    rng = np.random.default_rng(seed)
    t = (rng.integers(-400, 400, (B, k + 1, V)) / 64.0).astype(np.float32)
    d = (t[:, :k] + rng.integers(-64, 64, (B, k, V)) / 64.0).astype(np.float32)
    tok = rng.integers(0, V, (B, k)).astype(np.int32)
    if greedy:
        am = np.argmax(t[:, :k], axis=2).astype(np.int32) if k else tok
        tok = np.where(rng.random((B, k)) < 0.6, am, tok).astype(np.int32)
    u = rng.random((B, k + 1, 2)).astype(np.float32)
    return t, d, tok, u, rng


def layout_ok(r, tok, k):
    for b in range(len(r.accepted_len)):
        a = r.accepted_len[b]
        if a < 0:
            assert (r.out_tokens[b] == -1).all()
            continue
        assert 0 <= a <= k
        assert (r.out_tokens[b, :a] == tok[b, :a]).all()
        assert r.out_tokens[b, a] >= 0
        assert (r.out_tokens[b, a + 1:] == -1).all()


@SET
@given(calls())
def test_layout_and_vocabulary_permutation(c):
    t, d, tok, u, rng = c
    r = oracle.spec_verify_ref(t, d, tok, u, 1.0, oracle.SAMPLE, dtype=oracle.F32)
    layout_ok(r, tok, tok.shape[1])
    perm = rng.permutation(t.shape[2])
    inv = np.argsort(perm)
    r2 = oracle.spec_verify_ref(np.ascontiguousarray(t[:, :, perm]), np.ascontiguousarray(d[:, :, perm]),
                                inv[tok].astype(np.int32), u, 1.0, oracle.SAMPLE, dtype=oracle.F32)
    assert (r2.accepted_len == r.accepted_len).all()
    np.testing.assert_array_equal(r2.gap, r.gap)
    np.testing.assert_allclose(r2.p_tok, r.p_tok, rtol=1e-12, atol=0)


@SET
@given(calls(), st.sampled_from([oracle.SAMPLE, oracle.GREEDY]))
def test_temperature_and_shift(c, mode):
    t, d, tok, u, rng = c
    if mode == oracle.GREEDY:
        d, u = None, None
    r = oracle.spec_verify_ref(t, d, tok, u, 2.0, mode, dtype=oracle.F32)
    half = oracle.spec_verify_ref(t / 2, None if d is None else d / 2, tok, u, 1.0, mode, dtype=oracle.F32)
    assert (half.accepted_len == r.accepted_len).all() and (half.out_tokens == r.out_tokens).all()
    np.testing.assert_array_equal(half.gap * 2, r.gap)
    shift = rng.integers(-8, 8, (t.shape[0], t.shape[1], 1)).astype(np.float32)
    s = oracle.spec_verify_ref(t + shift, d, tok, u, 2.0, mode, dtype=oracle.F32)
    assert (s.accepted_len == r.accepted_len).all()
    np.testing.assert_array_equal(s.gap, r.gap)
    if mode == oracle.SAMPLE:
        # the draw may move only where the shifted softmax rounds differently
        ok = (s.out_tokens == r.out_tokens).all(axis=1) | (r.margin_cdf < 1e-9)
        assert ok.all()


@SET
@given(calls(), st.sampled_from([oracle.SAMPLE, oracle.GREEDY]))
def test_ragged_lengths_bound_the_accepted_length(c, mode):
    t, d, tok, u, rng = c
    k = tok.shape[1]
    dl = rng.integers(0, k + 1, t.shape[0]).astype(np.int32)
    r = oracle.spec_verify_ref(t, None if mode else d, tok, None if mode else u, 1.0, mode,
                               dtype=oracle.F32, draft_len=dl)
    ok = r.accepted_len >= 0
    assert (r.accepted_len[ok] <= dl[ok]).all()
    for b in range(t.shape[0]):
        if ok[b]:
            assert (r.out_tokens[b, dl[b] + 1:] == -1).all()


@SET
@given(st.integers(1, 30), st.integers(1, 40), st.integers(0, 2 ** 31 - 1))
def test_gate_coverage_monotone_per_row(n, V, seed):
    rng = np.random.default_rng(seed)
    x = (rng.integers(-300, 300, (n, V)) / 32.0).astype(np.float32)
    A = oracle.admit_mask(rng.choice(V, max(1, V // 2), replace=False), V)
    taus = sorted(rng.uniform(-1, 12, 6))
    fires = [oracle.spec_gate_ref(x, oracle.MARGIN, t, A).fire for t in taus]
    for f0, f1 in zip(fires, fires[1:]):
        assert (f1 <= f0).all()
    cert = [oracle.spec_gate_ref(x, oracle.CERTIFIED, max(t, 0.0) / 2, A).fire for t in taus]
    for f0, f1 in zip(cert, cert[1:]):
        assert (f1 <= f0).all()
