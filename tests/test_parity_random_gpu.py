"""Seeded random sweep of the verify step against the fp64 oracle.

Each case draws its shape and contents at random: B, k, V (odd sizes and
vector tails included), logit dtype, sampling or greedy mode, temperature,
logit spread, draft noise, independent draft rows, -inf masks, coarse values
that tie exactly, per-row draft lengths (some out of range) and uniforms at
0 and just below 1. The HIP path (through the C ABI) and the oracle see the
same bytes, and every row is compared under the rules of tests/parity.py
(bit-exact outside near-ties; a flagged row must take the oracle's outcome
or its near-tie alternative). Sizes stay at most 12M logits per case, so
inputs and oracle take at most a few seconds each on the host.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import token_verification_amd as tv
from parity import DELTA_ACC, compare

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
MAX_ELEMS = 12_000_000


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def draw_case(rng):
    while True:
        B = int(rng.integers(1, 41))
        k = int(rng.choice([0, 1, 2, 3, 5, 8, 13, 31, 64]))
        V = max(1, int(np.exp(rng.uniform(0.0, np.log(70_000)))) + int(rng.integers(-3, 4)))
        if B * (2 * k + 1) * V <= MAX_ELEMS:
            break
    c = {"B": B, "k": k, "V": V,
         "dtype": str(rng.choice(["f32", "bf16"])),
         "greedy": bool(rng.random() < 0.3),
         "T": float(rng.choice([0.25, 0.7, 1.0, 1.6])),
         "spread": float(rng.choice([0.5, 2.0, 6.0])),
         "noise": float(rng.choice([0.05, 1.0, 3.0])),
         "indep": float(rng.choice([0.0, 0.2, 1.0])),
         "mask": float(rng.choice([0.0, 0.0, 0.3, 0.9])),
         "coarse": bool(rng.random() < 0.2),
         "ragged": bool(rng.random() < 0.3)}
    return c


def build(rng, c):
    B, k, V = c["B"], c["k"], c["V"]
    t = rng.normal(0.0, c["spread"], (B, k + 1, V)).astype(np.float32)
    d = t[:, :k] + rng.normal(0.0, c["noise"], (B, k, V)).astype(np.float32)
    indep = rng.random((B, k)) < c["indep"]
    d[indep] = rng.normal(0.0, c["spread"], (int(indep.sum()), V)).astype(np.float32)
    if c["coarse"]:
        t = np.round(t * 2.0) / 2.0
        d = np.round(d * 2.0) / 2.0
    if c["mask"] > 0:
        t[rng.random(t.shape) < c["mask"]] = -np.inf
        d[rng.random(d.shape) < c["mask"]] = -np.inf
        t[:, :, 0] = np.where(np.isfinite(t[:, :, 0]), t[:, :, 0], 0.0)   # a finite entry per row
        d[:, :, 0] = np.where(np.isfinite(d[:, :, 0]), d[:, :, 0], 0.0)
        if B > 2:
            t[B - 1, 0, :] = -np.inf                                        # one all -inf row: invalid
    td = torch.float32 if c["dtype"] == "f32" else torch.bfloat16
    tt = torch.from_numpy(np.ascontiguousarray(t)).to(td)
    dt = torch.from_numpy(np.ascontiguousarray(d)).to(td)
    if c["greedy"]:
        am = torch.argmax(tt.float(), dim=2)[:, :k].to(torch.int32)
        tok = torch.from_numpy(rng.integers(0, V, (B, k)).astype(np.int32))
        keep = torch.from_numpy(rng.random((B, k)) < 0.7)
        tok = torch.where(keep, am, tok)
    else:
        # draft tokens drawn from the draft rows (a few out of range: invalid rows)
        tok = torch.zeros((B, k), dtype=torch.int32)
        if k > 0:
            q = torch.softmax(dt.float() / c["T"], dim=2).reshape(-1, V)
            q = torch.nan_to_num(q, nan=1.0 / V) + 1e-12
            g = torch.Generator().manual_seed(int(rng.integers(1 << 30)))
            tok = torch.multinomial(q, 1, generator=g).reshape(B, k).to(torch.int32)
            if B > 3:
                tok[1, 0] = V
    u = rng.random((B, k + 1, 2)).astype(np.float32)
    if B > 1:
        u[0, 0, :] = 0.0
        u[-1, -1, :] = np.nextafter(np.float32(1.0), np.float32(0.0))
    x = {"target": tt, "draft": None if c["greedy"] else dt, "tokens": tok,
         "uniforms": None if c["greedy"] else torch.from_numpy(u), "T": c["T"], "mode": 1 if c["greedy"] else 0}
    dl = None
    if c["ragged"]:
        dl = rng.integers(0, k + 1, B).astype(np.int32)
        if B > 4:
            dl[2] = -1
            dl[3] = k + 1
    return x, dl


@pytest.mark.parametrize("seed", range(200))
def test_random_case(seed):
    rng = np.random.default_rng(10_000 + seed)
    c = draw_case(rng)
    say("case", seed, c)
    x, dl = build(rng, c)
    dev = {key: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for key, v in x.items()}
    res = tv.spec_verify(dev["target"], dev["draft"], dev["tokens"], dev["uniforms"], x["T"], x["mode"],
                         return_probs=not c["greedy"],
                         draft_len=None if dl is None else torch.from_numpy(dl).to(DEV))
    torch.cuda.synchronize()
    ref = oracle.spec_verify_ref(x["target"], x["draft"], x["tokens"], x["uniforms"], x["T"], x["mode"],
                                 draft_len=dl, flip_delta=DELTA_ACC)
    st = compare(res, ref, c["dtype"], c["greedy"])
    say("  ", st)
