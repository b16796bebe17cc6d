"""Pins of the int8 LM-head oracle (oracle.lmhead), CPU only: the integer
products against Python integers, the float32 scaling against a hand-worked
example, and the greedy rule on the result against the pinned verify oracle."""
import numpy as np

import oracle
from oracle.lmhead import lmhead_greedy_ref, lmhead_logits_ref


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
