"""Oracle of verification fused with int8 LM heads, greedy and sampling (plain numpy).

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
as in oracle.spec_verify_ref; so does modified rejection sampling, with the
draft's logits from its own hidden rows and head (or the target's head, when
the draft shares it).

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


def lmhead_sample_ref(th, ths, tw, tws, dh, dhs, dw, dws, tokens, uniforms, temperature: float, B: int, k: int,
                      flip_delta: float = 0.0):
    """Sampling-mode verify of B batch rows through two int8 heads.

    Target rows th[b*(k+1)+i] (i = 0..k) and draft rows dh[b*k+i] (i < k) are
    projected by their heads as in lmhead_logits_ref (dw / dws None: the draft
    shares the target's head); modified rejection sampling ("Speculative
    Decoding: The Physics of Stolen Time", section 2) then runs on those
    float32 logits as in oracle.spec_verify_ref.
    """
    t = lmhead_logits_ref(th, ths, tw, tws).reshape(B, k + 1, -1)
    V = t.shape[2]
    if dw is None:
        dw, dws = tw, tws
    if k > 0:
        q = lmhead_logits_ref(dh, dhs, dw, dws).reshape(B, k, V)
    else:
        q = np.zeros((B, 0, V), np.float32)
    return oracle.spec_verify_ref(np.ascontiguousarray(t), np.ascontiguousarray(q),
                                  np.asarray(tokens, np.int32).reshape(B, k), np.asarray(uniforms, np.float32),
                                  float(temperature), oracle.SAMPLE, dtype=oracle.F32, flip_delta=flip_delta)
