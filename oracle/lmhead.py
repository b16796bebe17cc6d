"""Oracle of greedy verification fused with an int8 LM head (plain numpy).

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``.

The verify forward ends with the LM-head projection of the hidden states of
the k+1 verified positions ("Speculative Decoding: The Physics of Stolen Time",
section 1, the target's parallel verification pass; the speculative-decoding
design note, "Cost / correctness constraints", batched verify forward). The
pages run quantized targets (a 4-bit 70B-class model in "Speculative
Pre-Positioning", section 4; quantized GGUF weights in the design note); the
head here is int8 with one fp32 scale per vocabulary row and per hidden row:

    acc[m, v]    = sum_d h[m, d] * w[v, d]                 (exact integer)
    logit[m, v]  = fl32( fl32( float32(acc) * h_scale[m] ) * w_scale[v] )

where float32(acc) rounds the integer to nearest even and fl32 is one
float32 multiplication. The greedy rule ("The Inference Wall" part 7) and the
gap ("Speculative Pre-Positioning", Eq. 11) then apply to these logits exactly
as in oracle.spec_verify_ref.

Each product of two int8 values is at most 2^14 in magnitude, so for d up to
2^38 every partial sum is an integer below 2^53: a float64 matrix product is
exact, which is how acc is formed here. Pinned in tests/test_oracle_lmhead.py
against Python integers.
"""
from __future__ import annotations

import numpy as np

import oracle


def lmhead_logits_ref(h, h_scale, w, w_scale) -> np.ndarray:
    """float32 logits [M, V] of int8 h [M, d], w [V, d] and fp32 scales [M], [V]."""
    h = np.asarray(h, np.int8)
    w = np.asarray(w, np.int8)
    acc = h.astype(np.float64) @ w.astype(np.float64).T        # exact integers
    a32 = acc.astype(np.float32)                                 # round to nearest even
    hs = np.asarray(h_scale, np.float32)[:, None]
    ws = np.asarray(w_scale, np.float32)[None, :]
    return (a32 * hs) * ws                                       # two float32 products


def lmhead_greedy_ref(h, h_scale, w, w_scale, tokens, B: int, k: int):
    """Greedy verify of B batch rows whose k+1 target rows are h[b*(k+1)+i]."""
    logits = lmhead_logits_ref(h, h_scale, w, w_scale).reshape(B, k + 1, -1)
    return oracle.spec_verify_ref(np.ascontiguousarray(logits), None, np.asarray(tokens, np.int32), None,
                                  1.0, oracle.GREEDY, dtype=oracle.F32)
