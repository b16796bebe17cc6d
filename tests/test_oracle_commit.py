"""Pins of the commit / rollback oracle (oracle.commit.commit_ref), CPU only.

A toy recurrent model whose state is a closed form of the tokens it consumed
(a polynomial hash per state element) supplies the checkpoint slots the way a
verify forward would; the committed state must equal that closed form over the
committed tokens alone, and a position-indexed KV cache truncated to the new
length must hold exactly the committed sequence. These fix the slot index (a,
not a+1 or a-1) and the length rule (1 + a) independently of the oracle.
"""
import numpy as np

from oracle.commit import commit_ref

P = 2_147_483_629           # a prime below 2^31


def closed_form(s0, tokens, mult):
    """State after consuming `tokens` from s0: s <- (s * mult + t) mod P per element."""
    s = s0.astype(np.int64).copy()
    for t in tokens:
        s = (s * mult + int(t)) % P
    return s


def test_commit_is_the_state_of_the_committed_prefix():
    rng = np.random.default_rng(0)
    B, k, D, maxlen = 12, 5, 7, 64
    mult = rng.integers(2, 1000, D)
    s0 = rng.integers(0, P, (B, D))
    L = rng.integers(0, 40, B)
    pending = rng.integers(0, 50000, B)
    drafts = rng.integers(0, 50000, (B, k))
    hist = rng.integers(0, 50000, (B, maxlen))           # committed history before the step
    kv = hist.copy()
    slots = np.zeros((B, k + 1, D), np.int64)
    for b in range(B):
        seq = [pending[b]] + list(drafts[b])
        kv[b, L[b]:L[b] + k + 1] = seq                      # the verify forward's KV writes
        for j in range(k + 1):
            slots[b, j] = closed_form(s0[b], seq[:j + 1], mult)
    acc = rng.integers(-1, k + 1, B)
    acc[:3] = [0, k, -1]
    new_kv, new_state = commit_ref(acc, L, slots, s0)
    for b in range(B):
        if acc[b] < 0:
            assert new_kv[b] == L[b] and (new_state[b] == s0[b]).all()
            continue
        committed = [pending[b]] + list(drafts[b, :acc[b]])
        assert (new_state[b] == closed_form(s0[b], committed, mult)).all()
        # the truncated cache holds the history, then exactly the committed tokens
        assert new_kv[b] == L[b] + len(committed)
        assert list(kv[b, :new_kv[b]]) == list(hist[b, :L[b]]) + committed


def test_inputs_are_not_modified_and_state_is_optional():
    acc = np.array([2, -1], np.int32)
    kv = np.array([5, 7], np.int32)
    new_kv, st = commit_ref(acc, kv, k=3)
    assert list(new_kv) == [8, 7] and st is None and list(kv) == [5, 7]


def test_lengths_outside_the_slots_commit_nothing():
    slots = np.arange(2 * 3 * 2).reshape(2, 3, 2)
    state = np.full((2, 2), -1)
    new_kv, st = commit_ref(np.array([3, 2]), np.array([0, 0]), slots, state)
    assert list(new_kv) == [0, 3]
    assert (st[0] == -1).all() and (st[1] == slots[1, 2]).all()
