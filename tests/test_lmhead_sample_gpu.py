"""Sampling-mode verification fused with int8 LM heads (spec_verify_lmhead_sample)
against the oracle (oracle.lmhead.lmhead_sample_ref: exact integer products,
the two float32 scalings, then the sampling verify oracle).

Both sides see bit-identical float32 logits, so the rules of tests/parity.py
apply unchanged: accepted lengths and tokens bit-exact outside flagged
near-ties, gaps and p(x), q(x) within 1e-5. Small shapes cover partial
vocabulary and hidden-row tiles of all three tile widths, k = 0, the largest
k, a shared and a separate draft head; full sizes are checked on sampled
batch rows.
"""
import sys

import numpy as np
import pytest
import torch

import token_verification_amd as tv
import workloads
from oracle.lmhead import lmhead_sample_ref
from parity import DELTA_ACC, compare

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
NAMES = ("hidden", "hidden_scale", "weight", "weight_scale", "draft_hidden", "draft_hidden_scale",
         "draft_weight", "draft_weight_scale", "tokens", "uniforms")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(x):
    return {n: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for n, v in x.items()}


def run(y, T, **kw):
    return tv.spec_verify_lmhead_sample(y["hidden"], y["hidden_scale"], y["weight"], y["weight_scale"],
                                        y["draft_hidden"], y["draft_hidden_scale"], y["tokens"], y["uniforms"], T,
                                        draft_weight=y["draft_weight"], draft_weight_scale=y["draft_weight_scale"],
                                        **kw)


def oracle_of(x, T, rows=None):
    B, k = x["B"], x["k"]
    a = {n: (None if x[n] is None else x[n].cpu().numpy()) for n in NAMES}
    if rows is not None:
        rows = np.asarray(rows)
        ht = (rows[:, None] * (k + 1) + np.arange(k + 1)[None, :]).ravel()
        hd = (rows[:, None] * k + np.arange(k)[None, :]).ravel()
        a["hidden"], a["hidden_scale"] = a["hidden"][ht], a["hidden_scale"][ht]
        if k > 0:
            a["draft_hidden"], a["draft_hidden_scale"] = a["draft_hidden"][hd], a["draft_hidden_scale"][hd]
        a["tokens"], a["uniforms"], B = a["tokens"][rows], a["uniforms"][rows], len(rows)
    return lmhead_sample_ref(a["hidden"], a["hidden_scale"], a["weight"], a["weight_scale"], a["draft_hidden"],
                             a["draft_hidden_scale"], a["draft_weight"], a["draft_weight_scale"], a["tokens"],
                             a["uniforms"], T, B, k, flip_delta=DELTA_ACC)


def subset(r, rows):
    idx = torch.as_tensor(np.asarray(rows), device=r.accepted_len.device)
    return tv.binding.VerifyResult(*(None if t is None else t.index_select(0, idx) for t in r))


@pytest.mark.parametrize("B,k,V,d,T,own", [
    (1, 4, 1000, 128, 1.0, False),     # one partial tile each way
    (3, 2, 700, 256, 0.7, True),       # partial vocabulary tile, separate draft head
    (50, 3, 5000, 512, 1.0, False),    # 200 target rows: 256-row tiles; 150 draft rows
    (7, 0, 257, 128, 1.0, False),      # k = 0: only the bonus draw
    (2, 64, 300, 384, 1.0, False),     # the largest k (decisions over more than 64 rows)
    (40, 5, 32000, 1024, 0.4, True),   # sharp rows, separate head, 125 vocabulary tiles
    (96, 3, 3000, 640, 1.0, False),    # 384 / 288 rows: 192-row tiles
    (160, 3, 3000, 640, 1.6, True),    # 640 / 480 rows: 128-row tiles (the narrow kernel)
    (1, 4, 128256, 4096, 1.0, False),  # one batch row over a full-size shared head (one pass, 9 rows)
    (3, 7, 50000, 512, 0.8, False),    # 24 + 21 rows in one pass: the draft's rows start mid-tile
    (2, 3, 40000, 1536, 0.7, True),    # 8 / 6 rows, separate heads: 32-row tiles with 512-byte stages
    (1, 2, 5000, 512, 1.0, False),     # 3 + 2 rows in one pass, the 512-byte stages at their fewest
    (6, 3, 9000, 512, 0.9, False),     # 24 + 18 rows in one pass: one 128-row tile (the uncapped kernel)
    (10, 4, 3000, 1024, 1.0, True),    # 50 / 40 rows, separate heads: 128-row tiles
])
def test_lmhead_sample_matches_oracle(B, k, V, d, T, own):
    say("lmhead sample", B, k, V, d, T, own)
    x = workloads.make_lmhead_sample(B, k, V, d, seed=3, draft_head=own)
    r = run(to_dev(x), T)
    torch.cuda.synchronize()
    st = compare(r, oracle_of(x, T), "f32", False)
    acc = r.accepted_len.cpu().numpy()
    say("  ", st, "accepted", np.bincount(acc[acc >= 0], minlength=k + 1).tolist())


@pytest.mark.parametrize("B,k,V,d,own", [(1, 2, 1000, 65536, False), (2, 1, 700, 65408, True)])
def test_lmhead_sample_largest_d(B, k, V, d, own):
    # the largest d through both 32-row tiles (512- and 64-byte stages)
    say("lmhead sample largest d", B, k, V, d, own)
    x = workloads.make_lmhead_sample(B, k, V, d, seed=5, draft_head=own)
    r = run(to_dev(x), 1.0)
    torch.cuda.synchronize()
    st = compare(r, oracle_of(x, 1.0), "f32", False)
    say("  ", st)


def test_lmhead_sample_invalid_rows_and_extreme_uniforms():
    B, k, V, d, T = 50, 3, 3000, 256, 1.0
    x = workloads.make_lmhead_sample(B, k, V, d, seed=4)
    x["hidden_scale"][0] = float("nan")            # batch row 0: NaN target logits
    x["draft_hidden_scale"][3] = float("inf")      # batch row 1: +-inf / NaN draft logits
    x["tokens"][2, 1] = V                          # batch row 2: token out of range
    x["tokens"][4, 0] = -1                         # batch row 4: negative token
    x["hidden_scale"][24:28] = 3.0e38              # batch row 6: overflow to +-inf
    x["uniforms"][7, :, :] = 0.0                   # batch row 7: u = 0 everywhere
    x["uniforms"][8, :, :] = float(np.nextafter(np.float32(1.0), np.float32(0.0)))
    # batch row 9: the draft's rows equal the target's, so q = p and every draft is accepted
    x["draft_hidden"][27:30] = x["hidden"][36:39]
    x["draft_hidden_scale"][27:30] = x["hidden_scale"][36:39]
    r = run(to_dev(x), T)
    torch.cuda.synchronize()
    compare(r, oracle_of(x, T), "f32", False)
    acc = r.accepted_len.cpu().numpy()
    assert acc[0] == -1 and acc[1] == -1 and acc[2] == -1 and acc[4] == -1 and acc[6] == -1
    assert acc[9] == k
    assert (r.out_tokens[9, :k].cpu() == x["tokens"][9]).all()


@pytest.mark.parametrize("B,k,V,own", [(256, 3, 128256, False), (64, 5, 151936, True)])
def test_lmhead_sample_full_size_sampled_rows(B, k, V, own):
    d = workloads.LMHEAD_D
    T = 1.0
    say("lmhead sample full", B, k, V, d, own)
    x = workloads.make_lmhead_sample(B, k, V, d, seed=0, device=DEV, draft_head=own)
    r = run(x, T)
    torch.cuda.synchronize()
    rows = np.random.default_rng(0).choice(B, 6, replace=False)
    rows = np.unique(np.concatenate([rows, [0, B - 1]]))
    st = compare(subset(r, rows), oracle_of(x, T, rows), "f32", False)
    acc = r.accepted_len.cpu().numpy()
    say("  ", st, "accepted", np.bincount(acc[acc >= 0], minlength=k + 1).tolist())
    assert (acc >= 0).all()
    # a second call on the same workspace gives the same bits
    r2 = run(x, T)
    torch.cuda.synchronize()
    for a, b in zip(r, r2):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_lmhead_sample_graph_replays_and_timed_entry():
    B, k, V, d, T = 16, 3, 20000, 512, 0.8
    x = to_dev(workloads.make_lmhead_sample(B, k, V, d, seed=5))
    ws = torch.empty(tv.lib().spec_lmhead_sample_workspace_size(B, k, V, d), dtype=torch.uint8, device=DEV)
    eager = run(x, T, workspace=ws)
    torch.cuda.synchronize()
    eager = [t.clone() for t in eager]
    out = tv.binding.VerifyResult(torch.empty(B, dtype=torch.int32, device=DEV),
                                  torch.empty((B, k + 1), dtype=torch.int32, device=DEV),
                                  torch.empty((B, k + 1), dtype=torch.float32, device=DEV),
                                  torch.empty((B, k), dtype=torch.float32, device=DEV),
                                  torch.empty((B, k), dtype=torch.float32, device=DEV))
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            run(x, T, workspace=ws, out=out)
    torch.cuda.synchronize()
    for _ in range(3):
        for t in out:
            t.fill_(-7)
        junk = torch.randn(1 << 20, device=DEV).sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(eager, out):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32))
        del junk
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    r = run(x, T, phase_events=evs)
    torch.cuda.synchronize()
    for a, b in zip(eager, r):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    t = [evs[i].elapsed_time(evs[i + 1]) for i in range(3)]
    say("phases ms", [round(v, 4) for v in t])
    assert t[0] > 0 and t[1] >= 0 and t[2] >= 0


def test_lmhead_sample_equals_verify_on_stored_logits():
    # The fused call against spec_verify on the same float32 logits,
    # materialised by the oracle's projection on the host: the decisions,
    # tokens and gaps must agree exactly. p(x) and q(x) may differ in the last
    # bits, since the two paths sum a row's exponentials over different
    # partitions of the vocabulary.
    B, k, V, d, T = 24, 4, 9000, 256, 0.9
    x = workloads.make_lmhead_sample(B, k, V, d, seed=6, draft_head=True)
    from oracle.lmhead import lmhead_logits_ref
    tl = lmhead_logits_ref(x["hidden"].numpy(), x["hidden_scale"].numpy(), x["weight"].numpy(),
                           x["weight_scale"].numpy()).reshape(B, k + 1, V)
    dl = lmhead_logits_ref(x["draft_hidden"].numpy(), x["draft_hidden_scale"].numpy(), x["draft_weight"].numpy(),
                           x["draft_weight_scale"].numpy()).reshape(B, k, V)
    y = to_dev(x)
    fused = run(y, T)
    plain = tv.spec_verify(torch.from_numpy(tl).to(DEV), torch.from_numpy(dl).to(DEV), y["tokens"], y["uniforms"],
                           T, tv.SAMPLE, return_probs=True)
    torch.cuda.synchronize()
    for a, b in zip(fused[:3], plain[:3]):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    for a, b in zip(fused[3:], plain[3:]):
        assert torch.allclose(a, b, rtol=1e-6, atol=0.0, equal_nan=True)


def draw_shape(rng):
    while True:
        B = int(rng.integers(1, 41))
        k = int(rng.choice([0, 1, 2, 3, 5, 8, 13]))
        V = max(1, int(np.exp(rng.uniform(0.0, np.log(40_000)))) + int(rng.integers(-3, 4)))
        d = int(rng.choice([128, 256, 384, 640, 1024]))
        if B * (2 * k + 1) * V * d <= 2e10:
            return B, k, V, d


@pytest.mark.parametrize("seed", range(40))
def test_lmhead_sample_random_shapes(seed):
    # seeded random shapes (every tile width, vocabulary tails of any length,
    # k up to 13), temperatures, shared or separate draft heads, and injected
    # invalid rows and extreme uniforms, each against the oracle
    rng = np.random.default_rng(20_000 + seed)
    B, k, V, d = draw_shape(rng)
    T = float(rng.choice([0.3, 0.7, 1.0, 1.6]))
    own = bool(rng.random() < 0.5)
    say("lmhead sample random", seed, B, k, V, d, T, own)
    x = workloads.make_lmhead_sample(B, k, V, d, seed=seed, draft_head=own)
    if B > 3 and rng.random() < 0.3:
        x["hidden_scale"][int(rng.integers(0, B * (k + 1)))] = float("nan")
    if B > 3 and k > 0 and rng.random() < 0.3:
        x["tokens"][int(rng.integers(0, B)), int(rng.integers(0, k))] = V
    if B > 1:
        x["uniforms"][0, :, :] = 0.0
        x["uniforms"][-1, :, :] = float(np.nextafter(np.float32(1.0), np.float32(0.0)))
    r = run(to_dev(x), T)
    torch.cuda.synchronize()
    st = compare(r, oracle_of(x, T), "f32", False)
    say("  ", st)
