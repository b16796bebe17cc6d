"""Pins of the int8 LM-head oracle (oracle.lmhead), CPU only: the integer
products against Python integers, the float32 scaling against a hand-worked
example, the greedy rule on the result against the pinned verify oracle, and
the sampling composition against hand-worked two-token examples and the
q = p invariant."""
import math

import numpy as np

import oracle
from oracle.lmhead import lmhead_greedy_ref, lmhead_logits_ref, lmhead_sample_ref


def test_integer_products_are_exact():
    rng = np.random.default_rng(0)
    for d in (1, 7, 64, 4096):
        h = rng.integers(-128, 128, (3, d)).astype(np.int8)
        w = rng.integers(-128, 128, (5, d)).astype(np.int8)
        got = lmhead_logits_ref(h, np.ones(3, np.float32), w, np.ones(5, np.float32))
        for m in range(3):
            for v in range(5):
                exact = sum(int(a) * int(b) for a, b in zip(h[m], w[v]))
                assert got[m, v] == np.float32(exact)


def test_extreme_products_and_rounding_to_float32():
    d = 4096
    h = np.full((1, d), -128, np.int8)
    w = np.full((1, d), -128, np.int8)
    got = lmhead_logits_ref(h, np.ones(1, np.float32), w, np.ones(1, np.float32))
    assert got[0, 0] == 2.0 ** 26                           # 128 * 128 * 4096, exact
    # Above 2^25 float32 steps by 4: 127*127*4095 + 127 = 66048382 is a tie
    # between 66048380 and 66048384 and goes to the even mantissa (...384);
    # 127*127*4095 + 254 = 66048509 rounds down to 66048508.
    h = np.full((1, d), 127, np.int8)
    w = np.full((2, d), 127, np.int8)
    w[0, 0], w[1, 0] = 1, 2
    got = lmhead_logits_ref(h, np.ones(1, np.float32), w, np.ones(2, np.float32))
    assert float(got[0, 0]) == 66048384.0 and float(got[0, 1]) == 66048508.0


def test_scaling_worked_example():
    # acc = 3*5 + (-2)*4 = 7; 7 * 0.5 = 3.5; 3.5 * 0.25 = 0.875
    h = np.array([[3, -2]], np.int8)
    w = np.array([[5, 4]], np.int8)
    got = lmhead_logits_ref(h, np.array([0.5], np.float32), w, np.array([0.25], np.float32))
    assert got[0, 0] == np.float32(0.875)
    # float32 products, in that order: (acc * hs) * ws
    hs, ws = np.float32(0.1), np.float32(0.3)
    got = lmhead_logits_ref(h, np.array([hs]), w, np.array([ws]))
    assert got[0, 0] == (np.float32(7.0) * hs) * ws


def test_two_float32_roundings_not_one():
    # acc = 680962: the oracle rounds after each product,
    # fl32(fl32(acc * hs) * ws) = 5408.3408203125, where one rounding of the
    # exact product gives 5408.34033203125, and so does the swapped order.
    hs = np.float32(0.006459721829742193)
    ws = np.float32(1.2294965982437134)
    pairs = [(127, 127)] * 42 + [(127, 27), (115, 1)]      # 42 * 16129 + 3429 + 115
    d = 128
    h = np.zeros((1, d), np.int8)
    w = np.zeros((1, d), np.int8)
    for j, (x, y) in enumerate(pairs):
        h[0, j], w[0, j] = x, y
    assert int((h.astype(np.int64) @ w.astype(np.int64).T)[0, 0]) == 680962
    got = lmhead_logits_ref(h, np.array([hs]), w, np.array([ws]))[0, 0]
    assert float(got) == 5408.3408203125


def test_greedy_on_the_logits():
    rng = np.random.default_rng(1)
    B, k, V, d = 4, 3, 50, 32
    h = rng.integers(-20, 20, (B * (k + 1), d)).astype(np.int8)
    w = rng.integers(-20, 20, (V, d)).astype(np.int8)
    hs = rng.uniform(0.01, 0.02, B * (k + 1)).astype(np.float32)
    ws = rng.uniform(0.5, 1.5, V).astype(np.float32)
    logits = lmhead_logits_ref(h, hs, w, ws).reshape(B, k + 1, V)
    am = np.argmax(logits, axis=2)
    tok = am[:, :k].astype(np.int32).copy()
    tok[1, 1] = (tok[1, 1] + 1) % V
    r = lmhead_greedy_ref(h, hs, w, ws, tok, B, k)
    assert list(r.accepted_len) == [3, 1, 3, 3]
    assert r.out_tokens[1, 1] == am[1, 1] and r.out_tokens[0, 3] == am[0, 3]
    np.testing.assert_array_equal(r.gap[0], np.sort(logits[0], axis=1)[:, -1].astype(np.float64)
                                  - np.sort(logits[0], axis=1)[:, -2])
    ref = oracle.spec_verify_ref(logits, None, tok, None, 1.0, oracle.GREEDY, dtype=oracle.F32)
    assert (ref.out_tokens == r.out_tokens).all()


def _one_by_one(th, tw, dh, dw):
    f = lambda a: np.array(a, np.int8)                      # noqa: E731
    return f(th), f(tw), f(dh), None if dw is None else f(dw)


def test_sampling_worked_example_shared_head():
    # V = 2, d = 1, scales 1. Target row 0: logits (2, 0), so p = (e^2, 1) / (e^2 + 1);
    # target row 1 and the draft row: logits (0, 0), q = (1/2, 1/2). Draft token 1:
    # p/q = 2 / (e^2 + 1) = 0.23840584... A uniform of 0.2 accepts it and the bonus
    # comes from target row 1 = (1/2, 1/2): u = 0.4 gives token 0, u = 0.6 token 1.
    # A uniform of 0.3 rejects it, and the residual max(0, p - q) = (p_0 - 1/2, 0)
    # gives token 0 whatever the second uniform.
    th, tw, dh, _ = _one_by_one([[1], [0]], [[2], [0]], [[0]], None)
    one2, one1 = np.ones(2, np.float32), np.ones(1, np.float32)
    tok = np.array([[1]], np.int32)
    for u0, u1, want_acc, want_tok in ((0.2, 0.4, 1, [1, 0]), (0.2, 0.6, 1, [1, 1]),
                                       (0.3, 0.99, 0, [0, -1]), (0.3, 0.0, 0, [0, -1])):
        u = np.array([[[u0, u1], [0.0, u1]]], np.float32)   # channel 1 of the row drawn from
        r = lmhead_sample_ref(th, one2, tw, one2, dh, one1, None, None, tok, u, 1.0, 1, 1)
        assert int(r.accepted_len[0]) == want_acc
        assert r.out_tokens[0].tolist() == want_tok
        assert abs(r.p_tok[0, 0] - 1.0 / (math.e ** 2 + 1.0)) < 1e-7
        assert abs(r.q_tok[0, 0] - 0.5) < 1e-7


def test_sampling_worked_example_draft_head():
    # The draft's own head: w_d = (0, 3) on draft hidden 1 gives draft logits (0, 3),
    # q(1) = e^3 / (1 + e^3), p(1)/q(1) = (1 + e^3) / ((e^2 + 1) e^3) = 0.12514...,
    # so a uniform of 0.2 rejects and the residual (p_0 - q_0, 0) gives token 0;
    # a uniform of 0.1 accepts.
    th, tw, dh, dw = _one_by_one([[1], [0]], [[2], [0]], [[1]], [[0], [3]])
    one2, one1 = np.ones(2, np.float32), np.ones(1, np.float32)
    tok = np.array([[1]], np.int32)
    q1 = math.e ** 3 / (1.0 + math.e ** 3)
    for u0, want_acc, want_tok in ((0.2, 0, [0, -1]), (0.1, 1, [1, 1])):
        u = np.array([[[u0, 0.7], [0.0, 0.7]]], np.float32)
        r = lmhead_sample_ref(th, one2, tw, one2, dh, one1, dw, one2, tok, u, 1.0, 1, 1)
        assert int(r.accepted_len[0]) == want_acc and r.out_tokens[0].tolist() == want_tok
        assert abs(r.q_tok[0, 0] - q1) < 1e-7


def test_sampling_identical_rows_accept_every_draft():
    # A draft that shares the head and the hidden states has q = p at every
    # position, so p/q = 1 > u for every uniform in [0, 1): all k drafts are
    # accepted and the reported p(x) and q(x) agree.
    rng = np.random.default_rng(2)
    B, k, V, d = 6, 4, 300, 64
    th = rng.integers(-60, 60, (B * (k + 1), d)).astype(np.int8)
    tw = rng.integers(-60, 60, (V, d)).astype(np.int8)
    ths = rng.uniform(0.002, 0.004, B * (k + 1)).astype(np.float32)
    tws = rng.uniform(0.5, 1.5, V).astype(np.float32)
    sel = (np.arange(B)[:, None] * (k + 1) + np.arange(k)[None, :]).ravel()
    dh, dhs = th[sel], ths[sel]
    tok = rng.integers(0, V, (B, k)).astype(np.int32)
    u = rng.random((B, k + 1, 2)).astype(np.float32)
    r = lmhead_sample_ref(th, ths, tw, tws, dh, dhs, None, None, tok, u, 0.8, B, k)
    assert (r.accepted_len == k).all()
    assert (r.out_tokens[:, :k] == tok).all() and (r.out_tokens[:, k] >= 0).all()
    assert np.array_equal(r.p_tok, r.q_tok)
