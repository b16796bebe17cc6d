"""The parity rules themselves (host logic, no GPU): a flagged row is accepted
only with the oracle's outcome or its near-tie alternative, and the flag budget
is 0.01% of a workload's rows."""
from types import SimpleNamespace

import numpy as np
import pytest
import torch
from scipy.special import softmax

import oracle
from parity import DELTA_ACC, compare, within_budget


def fake_gpu(acc, tok, gap):
    return SimpleNamespace(accepted_len=torch.as_tensor(acc, dtype=torch.int32),
                           out_tokens=torch.as_tensor(tok, dtype=torch.int32),
                           gap=torch.as_tensor(gap, dtype=torch.float32),
                           target_prob=None, draft_prob=None)


def near_tie_case():
    # one draft position, u0 the float32 just below r = p(1)/q(1): accepted,
    # flagged, and the alternative rejects at position 0
    P, Q = np.array([0.1, 0.2, 0.3, 0.4]), np.array([0.4, 0.3, 0.2, 0.1])
    t = np.array([[np.log(P), np.zeros(4)]], np.float32)
    d = np.array([[np.log(Q)]], np.float32)
    p = softmax(t[0, 0].astype(np.float64))
    q = softmax(d[0, 0].astype(np.float64))
    r = p[1] / q[1]
    f = np.float32(r)
    u0 = f if float(f) < r else np.nextafter(f, np.float32(0))
    u = np.array([[[u0, 0.6], [0.3, 0.7]]], np.float32)
    return t, d, np.array([[1]], np.int32), u


def test_flagged_row_accepts_oracle_or_alternative_only():
    t, d, tok, u = near_tie_case()
    ref = oracle.spec_verify_ref(t, d, tok, u, 1.0, oracle.SAMPLE, dtype=oracle.F32, flip_delta=DELTA_ACC)
    assert ref.flagged(DELTA_ACC, 1e-12)[0] and ref.accepted_len[0] == 1
    assert ref.alt_accepted_len[0] == 0
    st = compare(fake_gpu(ref.accepted_len, ref.out_tokens, ref.gap), ref, "f32", False)
    assert st["flagged"] == 1 and st["mismatch_flagged"] == 0
    st = compare(fake_gpu(ref.alt_accepted_len, ref.alt_out_tokens, ref.gap), ref, "f32", False)
    assert st["mismatch_flagged"] == 1
    wrong = ref.alt_out_tokens.copy()
    wrong[0, 0] = (wrong[0, 0] + 1) % 4
    with pytest.raises(AssertionError):
        compare(fake_gpu(ref.alt_accepted_len, wrong, ref.gap), ref, "f32", False)


def test_flagged_row_needs_the_alternatives():
    t, d, tok, u = near_tie_case()
    ref = oracle.spec_verify_ref(t, d, tok, u, 1.0, oracle.SAMPLE, dtype=oracle.F32)
    with pytest.raises(ValueError):
        compare(fake_gpu(ref.accepted_len * 0, ref.out_tokens, ref.gap), ref, "f32", False)


def test_unflagged_mismatch_fails():
    t, d, tok, u = near_tie_case()
    u[0, 0, 0] = 0.9                               # far from the ratio: rejects
    ref = oracle.spec_verify_ref(t, d, tok, u, 1.0, oracle.SAMPLE, dtype=oracle.F32, flip_delta=DELTA_ACC)
    assert not ref.flagged(DELTA_ACC, 1e-12)[0]
    with pytest.raises(AssertionError):
        compare(fake_gpu(ref.alt_accepted_len + 1, ref.out_tokens, ref.gap), ref, "f32", False)


def test_budget_is_one_in_ten_thousand():
    assert within_budget(10_000, 1) and not within_budget(10_000, 2)
    assert within_budget(12_800, 1) and not within_budget(9_999, 1)
