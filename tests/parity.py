"""Parity rules between the HIP path and the fp64 oracle (shared by the tests).

Integer outputs (accepted_len, out_tokens) must be bit-exact on every row
except rows the oracle flags as near-ties:
  * acceptance: |u - p/q| < DELTA_ACC for a test actually taken (1e-6, the
    stated decision-margin threshold);
  * inverse-CDF draw: the uniform lies within DELTA_CDF of an edge of the
    chosen token's normalized CDF interval. The stated 1e-6 cannot be the
    intended unit here: at V ~ 1.5e5 most tokens carry less than 1e-6 of the
    mass, so about 11% of rows would be flagged. The GPU computes this draw in
    double precision (normalized CDF error ~1e-15), so 1e-12 is used; the
    literal-threshold fraction is reported next to it.
  * rows whose residual mass rounded to zero (oracle flag bit 0), and rows
    whose residual draw lies within 1e-13 of the target's total mass of a CDF
    boundary (flag bit 1): the residual max(0, p - q) is a difference of two
    probability vectors, so every fp64 evaluation of it carries absolute
    errors near 1e-15, and such a draw is decided by rounding (this happens
    when p and q nearly coincide, e.g. both one-hot at a low temperature).
Flagged rows must stay at or below MAX_FLAG_FRACTION (0.01% of rows) in
aggregate over the seeds of a workload. A flagged row is still checked: its
outcome must be the oracle's, or the oracle's with the near-tie decision taken
the other way (the acceptance test nearest its boundary flipped, or the draw's
token replaced by its neighbour across the nearest CDF edge); the oracle
reports both alternatives when called with flip_delta = DELTA_ACC. Rows whose
residual mass rounded to zero (flag bit 0) must match the oracle exactly.

Floating outputs: gap and p(x)/q(x) within 1e-5 absolute for float32 inputs
and 2e-3 for bfloat16 inputs (the gap of bf16 inputs is a difference of two
bf16 values and is compared exactly in practice). The kernel forms the gap as
one float32 subtraction of two exact float32 logits, so a gap may also differ
by half a float32 ulp of itself (2^-24 of its size), which is the larger bound
once gaps pass ~170.
"""
from __future__ import annotations

import numpy as np

DELTA_ACC = 1e-6
DELTA_CDF = 1e-12
DELTA_CDF_LITERAL = 1e-6
MAX_FLAG_FRACTION = 1e-4


def float_tol(dtype: str) -> float:
    return 1e-5 if dtype == "f32" else 2e-3


def flagged_ok(acc, tok, ref, flagged):
    """Per flagged row: is the GPU outcome one of the admissible ones?"""
    if ref.alt_accepted_len is None:
        raise ValueError("call the oracle with flip_delta=DELTA_ACC to check flagged rows")
    ok = np.ones(acc.shape[0], bool)
    for b in np.nonzero(flagged)[0]:
        same = acc[b] == ref.accepted_len[b] and (tok[b] == ref.out_tokens[b]).all()
        if same:
            continue
        good = False
        if ref.margin_acc[b] < DELTA_ACC:
            good |= acc[b] == ref.alt_accepted_len[b] and (tok[b] == ref.alt_out_tokens[b]).all()
        if (ref.margin_cdf[b] < DELTA_CDF or ref.flags[b] & 2) and acc[b] == ref.accepted_len[b] >= 0:
            a = int(ref.accepted_len[b])
            want = ref.out_tokens[b].copy()
            want[a] = ref.alt_token[b]
            good |= bool((tok[b] == want).all())
        ok[b] = good
    return ok


def compare(gpu, ref, dtype: str, greedy: bool):
    """Compare one call's GPU outputs (torch tensors) with a RefResult.

    Returns a dict of statistics; raises AssertionError on a parity failure.
    In sampling mode the oracle must have been called with flip_delta=DELTA_ACC
    when any row is flagged.
    """
    acc = gpu.accepted_len.cpu().numpy()
    tok = gpu.out_tokens.cpu().numpy()
    gap = gpu.gap.cpu().numpy().astype(np.float64)
    B = acc.shape[0]
    if greedy:
        flagged = np.zeros(B, bool)
    else:
        flagged = ref.flagged(DELTA_ACC, DELTA_CDF)
    row_ok = (acc == ref.accepted_len) & (tok == ref.out_tokens).all(axis=1)
    bad = ~row_ok & ~flagged
    stats = {
        "rows": B,
        "flagged": int(flagged.sum()),
        "flagged_literal": int(ref.flagged(DELTA_ACC, DELTA_CDF_LITERAL).sum()) if not greedy else 0,
        "flag_bits": int((ref.flags != 0).sum()) if not greedy else 0,
        "mismatch_flagged": int((~row_ok & flagged).sum()),
    }
    assert not bad.any(), (
        f"{int(bad.sum())} unflagged rows differ; first b={int(np.argmax(bad))}: "
        f"gpu acc={acc[bad][0]} tok={tok[bad][0]} ref acc={ref.accepted_len[bad][0]} "
        f"tok={ref.out_tokens[bad][0]} margins acc={ref.margin_acc[bad][0]:.3g} "
        f"cdf={ref.margin_cdf[bad][0]:.3g}")
    if (~row_ok & flagged).any():
        fok = flagged_ok(acc, tok, ref, flagged & ~row_ok)
        assert fok.all(), (
            f"flagged row b={int(np.argmin(fok))} has an outcome that is neither the oracle's nor "
            f"its near-tie alternative: gpu acc={acc[~fok][0]} tok={tok[~fok][0]} "
            f"ref acc={ref.accepted_len[~fok][0]} tok={ref.out_tokens[~fok][0]}")
    valid = ref.accepted_len >= 0
    tol = float_tol(dtype)
    g_ref = ref.gap[valid]
    g_gpu = gap[valid]
    fin = np.isfinite(g_ref)
    assert (np.isfinite(g_gpu) == fin).all(), "gap finiteness differs"
    assert (np.isnan(g_gpu) == np.isnan(g_ref)).all(), "gap NaN positions differ"
    if fin.any():
        dev = np.abs(g_gpu[fin] - g_ref[fin])
        bound = np.maximum(tol, 2.0 ** -24 * np.abs(g_ref[fin]))
        stats["gap_err"] = float(dev.max())
        assert (dev <= bound).all(), f"gap error {float(dev.max())} beyond max({tol}, 2^-24 |gap|)"
    if not greedy and gpu.target_prob is not None and ref.p_tok.size:
        for name, g, r in (("p", gpu.target_prob, ref.p_tok), ("q", gpu.draft_prob, ref.q_tok)):
            gg = g.cpu().numpy().astype(np.float64)[valid]
            rr = r[valid]
            # positions a row does not verify (ragged drafts) are NaN on both sides
            nan = np.isnan(rr)
            assert (np.isnan(gg) == nan).all(), f"{name}(x) NaN positions differ"
            err = np.abs(gg[~nan] - rr[~nan]).max() if (~nan).any() else 0.0
            stats[f"{name}_err"] = float(err)
            assert err <= tol, f"{name}(x) error {err} > {tol}"
    return stats


def within_budget(rows: int, flagged: int) -> bool:
    """Aggregate flag budget of one workload: at most 0.01% of its rows."""
    return flagged <= MAX_FLAG_FRACTION * rows
