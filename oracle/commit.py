"""Oracle of the commit / rollback step after a verify (plain numpy).

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``.

Definition (the KV truncation on rejection in "Speculative Decoding: The
Physics of Stolen Time", section 6, "KV-cache management"; the speculative
KV rollback of the speculative-decoding design note, "Cost / correctness
constraints"; the per-position state checkpoints of hybrid models in "The
Inference Wall" part 7, "Why it inverts, mechanism 2"):

* The verify forward of batch row b consumed k+1 tokens, the pending token and
  the drafts x_0..x_{k-1}, appending their KV entries at positions
  kv_len[b] .. kv_len[b]+k, and wrote recurrent-state checkpoint slot j
  (j = 0..k) = the state after the pending token and drafts x_0..x_{j-1}.
* With a = accepted_len[b] >= 0 the committed tokens are the pending token and
  x_0..x_{a-1}: the KV entries of the rejected drafts are dropped, so
  kv_len[b] becomes kv_len[b] + 1 + a, and the live recurrent state becomes
  slot a. The emitted (resampled or bonus) token is the next pending token:
  its KV and state come with the next forward.
* An invalid row (a = -1) commits nothing: kv_len and the state are unchanged.
  Nor does a row whose accepted_len lies outside [0, k] (no such slot exists;
  a verify step never produces one).

Parity: pinned in tests/test_oracle_commit.py against a model whose state is a
closed form of the committed tokens.
"""
from __future__ import annotations

import numpy as np


def commit_ref(accepted_len, kv_len, slots=None, state=None, k=None):
    """Return (new kv_len, new state) for accepted_len [B], kv_len [B] and,
    optionally, slots [B, k+1, ...] and state [B, ...] (any dtype: a copy).
    k defaults to slots.shape[1] - 1 (required without slots)."""
    a = np.asarray(accepted_len, np.int64)
    if k is None:
        k = slots.shape[1] - 1
    kv = np.asarray(kv_len, np.int64).copy()
    B = a.shape[0]
    new_state = None if state is None else np.array(state, copy=True)
    for b in range(B):
        if a[b] < 0 or a[b] > k:
            continue
        kv[b] = kv[b] + 1 + a[b]
        if new_state is not None:
            new_state[b] = slots[b, a[b]]
    return kv.astype(np.int32), new_state
