"""Parity at the seed counts that make the 0.01% near-tie budget testable.

Every workload is run over enough seeds to give at least 10^4 batch rows:
B=1 k=4 V=1000 fp32 over 10,000 seeds, B=8 k=5 V=32000 fp32 over 2,000,
B=64 k=5 V=151936 bf16 over 200, B=256 k=3 V=128256 bf16 greedy over 50 and
B=512 k=8 V=262144 bf16 over 20 (every row of every seed). The three large
workloads run one seed per call at their real shape, in the launch
configuration the benchmark times; the two small ones stack many seeds along
the batch dimension (batch rows are independent, so a stacked call is the
same computation per row).

Per workload: every unflagged row bit-exact against the fp64 oracle, every
flagged row equal to the oracle's outcome or its near-tie alternative
(tests/parity.py), probabilities and gaps within tolerance, and the flagged
rows at most 0.01% of all rows ("The Inference Wall", Part 7: near-ties may
flip across kernels; the budget bounds how often that may happen). A summary
line per workload (PARITY_SUMMARY) gives the row count, the flagged counts
under the 1e-12 CDF threshold and under the literal 1e-6 reading, the rows
with oracle flag bits, and the largest probability / gap errors.
"""
import json
import sys
import time

import pytest
import torch

import oracle
import token_verification_amd as tv
import workloads
from parity import DELTA_ACC, compare, within_budget

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def stacked(w, seeds, device):
    """Inputs of several seeds stacked along the batch dimension."""
    xs = [workloads.make(w, s, device=device) for s in seeds]
    out = {}
    for key in ("target", "draft", "tokens", "uniforms"):
        out[key] = None if xs[0][key] is None else torch.cat([x[key] for x in xs]).to(DEV)
    out["T"], out["mode"] = w.T, w.mode
    return out


def run_chunk(x, w):
    greedy = w.mode == workloads.GREEDY
    res = tv.spec_verify(x["target"], x["draft"], x["tokens"], x["uniforms"], x["T"], x["mode"],
                         return_probs=not greedy)
    torch.cuda.synchronize()
    host = {key: (None if x[key] is None else x[key].cpu()) for key in ("target", "draft", "tokens", "uniforms")}
    ref = oracle.spec_verify_ref(host["target"], host["draft"], host["tokens"], host["uniforms"], x["T"],
                                 x["mode"], flip_delta=DELTA_ACC)
    return compare(res, ref, w.dtype, greedy)


SCALE = [
    # workload, seeds, seeds per call, where the inputs are drawn
    ("b1_k4_v1000_f32", 10_000, 2_500, "cpu"),
    ("b8_k5_v32000_f32", 2_000, 100, DEV),
    ("b64_k5_v151936_bf16", 200, 1, DEV),
    ("b256_k3_v128256_bf16_greedy", 50, 1, DEV),
    ("b512_k8_v262144_bf16", 20, 1, DEV),
]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,nseeds,per_call,gen", SCALE, ids=[s[0] for s in SCALE])
def test_parity_at_scale(name, nseeds, per_call, gen):
    w = workloads.WORKLOADS[name]
    tot = {"rows": 0, "flagged": 0, "flagged_literal": 0, "flag_bits": 0, "mismatch_flagged": 0}
    errs = {}
    t0 = time.time()
    for s0 in range(0, nseeds, per_call):
        seeds = range(s0, min(nseeds, s0 + per_call))
        x = stacked(w, seeds, gen)
        st = run_chunk(x, w)
        del x
        for key in tot:
            tot[key] += st[key]
        for key in ("p_err", "q_err", "gap_err"):
            if key in st:
                errs[key] = max(errs.get(key, 0.0), st[key])
        if s0 % max(per_call, max(1, nseeds // 10)) == 0:
            say(f"{name} seeds {seeds.start}..{seeds.stop - 1}: {tot} ({time.time() - t0:.0f} s)")
    summary = {"workload": name, "seeds": nseeds, **tot, **errs}
    say("PARITY_SUMMARY " + json.dumps(summary))
    assert tot["rows"] == nseeds * w.B
    assert tot["rows"] >= 10_000
    assert within_budget(tot["rows"], tot["flagged"]), summary
