"""Verification fused with int8 LM heads at the row count that makes the 0.01%
near-tie budget testable. Sampling: 10,000 batch rows (20 calls of B = 500,
k = 3, V = 32000, d = 256; half with a separate draft head, temperatures 1.0
and 0.7), every row against the oracle (oracle.lmhead.lmhead_sample_ref).
Greedy: 10,000 batch rows (10 calls of B = 1000, k = 3), every row exact.

Per call the rules of tests/parity.py apply: unflagged rows bit-exact, flagged
rows equal to the oracle's outcome or its near-tie alternative, p(x), q(x) and
gaps within 1e-5; over all calls the flagged rows stay within 0.01% ("The
Inference Wall", Part 7: near-ties may flip across kernels). V and d are
smaller than a model's so that the fp64 oracle over every row finishes in
seconds; the kernels, tiles and pipeline are the ones the full-size calls use.
"""
import json
import sys
import time

import pytest
import torch

import token_verification_amd as tv
import workloads
from oracle.lmhead import lmhead_sample_ref
from parity import DELTA_ACC, compare, within_budget

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
B, K, V, D = 500, 3, 32000, 256
CALLS = 20


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.timeout(900)
def test_lmhead_sample_parity_at_scale():
    tot = {"rows": 0, "flagged": 0, "flagged_literal": 0, "flag_bits": 0, "mismatch_flagged": 0}
    errs = {}
    t0 = time.time()
    for seed in range(CALLS):
        own = seed % 2 == 1
        T = 1.0 if seed % 4 < 2 else 0.7
        x = workloads.make_lmhead_sample(B, K, V, D, seed=100 + seed, device=DEV, draft_head=own)
        r = tv.spec_verify_lmhead_sample(x["hidden"], x["hidden_scale"], x["weight"], x["weight_scale"],
                                         x["draft_hidden"], x["draft_hidden_scale"], x["tokens"], x["uniforms"],
                                         T, draft_weight=x["draft_weight"],
                                         draft_weight_scale=x["draft_weight_scale"])
        torch.cuda.synchronize()
        h = {n: (None if x[n] is None else x[n].cpu().numpy())
             for n in ("hidden", "hidden_scale", "weight", "weight_scale", "draft_hidden", "draft_hidden_scale",
                       "draft_weight", "draft_weight_scale", "tokens", "uniforms")}
        ref = lmhead_sample_ref(h["hidden"], h["hidden_scale"], h["weight"], h["weight_scale"], h["draft_hidden"],
                                h["draft_hidden_scale"], h["draft_weight"], h["draft_weight_scale"], h["tokens"],
                                h["uniforms"], T, B, K, flip_delta=DELTA_ACC)
        st = compare(r, ref, "f32", False)
        for key in tot:
            tot[key] += st[key]
        for key in ("gap_err", "p_err", "q_err"):
            if key in st:
                errs[key] = max(errs.get(key, 0.0), st[key])
        acc = r.accepted_len.cpu()
        assert (acc >= 0).all()
        say(f"  call {seed} own={own} T={T}: {st}")
    summary = {"workload": f"lmhead_sample_b{B}_k{K}_v{V}_d{D}", **tot, **errs,
               "seconds": round(time.time() - t0, 1)}
    say("PARITY_SUMMARY " + json.dumps(summary))
    assert tot["rows"] == B * CALLS
    assert within_budget(tot["rows"], tot["flagged"]), summary


@pytest.mark.timeout(900)
def test_lmhead_greedy_parity_at_scale():
    # greedy verification fused with the int8 head over 10,000 batch rows:
    # tokens, lengths and gaps against the oracle, every row (greedy mode
    # has no near-tie flags: the logits are bit-identical on both sides)
    from oracle.lmhead import lmhead_greedy_ref
    rows = 0
    for seed in range(10):
        Bg, Kg = 1000, 3
        x = workloads.make_lmhead(Bg, Kg, V, D, seed=200 + seed, device=DEV)
        r = tv.spec_verify_lmhead(x["hidden"], x["hidden_scale"], x["weight"], x["weight_scale"], x["tokens"])
        torch.cuda.synchronize()
        ref = lmhead_greedy_ref(*(x[n].cpu().numpy() for n in ("hidden", "hidden_scale", "weight", "weight_scale",
                                                               "tokens")), Bg, Kg)
        st = compare(r, ref, "f32", True)
        assert st["flagged"] == 0
        rows += st["rows"]
    say(f"PARITY_SUMMARY greedy lmhead rows={rows}")
    assert rows == 10_000
