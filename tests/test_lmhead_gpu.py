"""Greedy verification fused with an int8 LM head (spec_verify_lmhead) against
the oracle (oracle.lmhead: exact integer products, the two float32 scalings,
then the greedy verify oracle).

Tokens and accepted lengths must be bit-exact (the logits are bit-identical on
both sides: exact int32 sums, one rounding to float32, two float32 products);
gaps agree within 1e-5, or half a float32 ulp of the gap where that is larger
(the kernel subtracts in float32, the oracle in fp64).
Small shapes cover partial vocabulary and hidden-row tiles, several LDS stages,
k = 0 and the largest k; full sizes are checked on sampled batch rows.
"""
import sys

import numpy as np
import pytest
import torch

import token_verification_amd as tv
import workloads
from oracle.lmhead import lmhead_greedy_ref

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(x):
    return {n: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for n, v in x.items()}


def check(gpu, ref, rows=None):
    acc = gpu.accepted_len.cpu().numpy()
    tok = gpu.out_tokens.cpu().numpy()
    gap = gpu.gap.cpu().numpy().astype(np.float64)
    if rows is not None:
        acc, tok, gap = acc[rows], tok[rows], gap[rows]
    assert (acc == ref.accepted_len).all(), (np.nonzero(acc != ref.accepted_len)[0][:8])
    assert (tok == ref.out_tokens).all()
    valid = ref.accepted_len >= 0
    g, r = gap[valid], ref.gap[valid]
    assert (np.isnan(g) == np.isnan(r)).all() and (np.isinf(g) == np.isinf(r)).all()
    fin = np.isfinite(r)
    # one float32 subtraction of exact float32 logits: within half an ulp of
    # the gap, or 1e-5 for small gaps
    dev = np.abs(g[fin] - r[fin])
    assert (dev <= np.maximum(1e-5, 2.0 ** -24 * np.abs(r[fin]))).all(), float(dev.max(initial=0.0))
    return acc


def run(x):
    y = to_dev(x)
    return tv.spec_verify_lmhead(y["hidden"], y["hidden_scale"], y["weight"], y["weight_scale"], y["tokens"])


def oracle_of(x, rows=None):
    B, k = x["B"], x["k"]
    h, hs, w, ws = (x[n].cpu().numpy() for n in ("hidden", "hidden_scale", "weight", "weight_scale"))
    tok = x["tokens"].cpu().numpy()
    if rows is not None:
        hr = (np.asarray(rows)[:, None] * (k + 1) + np.arange(k + 1)[None, :]).ravel()
        h, hs, tok, B = h[hr], hs[hr], tok[rows], len(rows)
    return lmhead_greedy_ref(h, hs, w, ws, tok, B, k)


@pytest.mark.parametrize("B,k,V,d", [
    (1, 4, 1000, 128),          # one partial tile each way
    (3, 2, 700, 256),           # partial vocabulary tile, two LDS stages
    (50, 3, 5000, 512),         # two hidden-row tiles, 20 vocabulary tiles
    (7, 0, 257, 128),           # k = 0: only the bonus argmax
    (2, 64, 300, 384),          # the largest k (decision over more than 64 rows)
    (40, 5, 32000, 1024),       # 8 XCD runs of tiles and a remainder
    (64, 3, 1000, 128),         # 256-row tiles with the fewest stages (two)
    (64, 3, 2000, 256),         # 256-row tiles, four stages (the prologue fills three)
    (96, 3, 3000, 640),         # 384 rows: two 192-row tiles, ten stages
    (160, 3, 3000, 640),        # 640 rows: five 128-row tiles (the narrow kernel), ten stages
    (2, 4, 70001, 1536),        # 10 rows: a 32-row tile with 512-byte stages (12), vocabulary tail
    (4, 7, 3000, 512),          # 32 rows: the 512-byte stages at their fewest (four)
    (10, 4, 5000, 768),         # 50 rows: one 128-row tile, d not a multiple of 512, vocabulary tail
    (2, 3, 1, 512),             # V = 1: one vocabulary row in a 256-row tile, 512-byte stages
    (3, 1, 255, 1024),          # V = 255: one partial vocabulary tile, 512-byte stages
])
def test_lmhead_matches_oracle(B, k, V, d):
    say("lmhead", B, k, V, d)
    x = workloads.make_lmhead(B, k, V, d, seed=3)
    r = run(x)
    torch.cuda.synchronize()
    acc = check(r, oracle_of(x))
    say("accepted", np.bincount(acc[acc >= 0], minlength=k + 1).tolist())


@pytest.mark.parametrize("B,k,V,d", [
    (1, 2, 1000, 65536),        # the largest d: 512 stages of 512 bytes (32-row tile)
    (2, 1, 700, 65408),         # the largest d that is not a multiple of 512 (32-row tile, 64-byte stages)
    (16, 3, 300, 65536),        # 64 rows at the largest d (128-row tile), |acc| up to 2^30
])
def test_lmhead_largest_d(B, k, V, d):
    say("lmhead largest d", B, k, V, d)
    x = workloads.make_lmhead(B, k, V, d, seed=5)
    x["hidden"][0] = 127                           # extreme rows: the int32 sums at their largest
    x["weight"][:8] = -128
    r = run(x)
    torch.cuda.synchronize()
    check(r, oracle_of(x))


def test_lmhead_invalid_rows_and_ties():
    B, k, V, d = 50, 3, 3000, 256
    x = workloads.make_lmhead(B, k, V, d, seed=4)
    x["hidden_scale"][0] = float("nan")            # batch row 0: NaN logits
    x["hidden_scale"][5] = float("inf")            # batch row 1: +-inf / NaN logits
    x["tokens"][2, 1] = V                          # batch row 2: token out of range
    x["tokens"][4, 0] = -1                         # batch row 4: negative token
    x["hidden"][12:16] = 0                         # batch row 3: all logits 0, argmax 0 by the tie rule
    x["tokens"][3, :] = 0
    x["weight"][1] = x["weight"][2]                # equal rows 1 and 2 with equal scales: tied logits
    x["weight_scale"][1] = x["weight_scale"][2]
    x["hidden_scale"][24:28] = 3.0e38              # batch row 6: overflow to +-inf
    r = run(x)
    torch.cuda.synchronize()
    acc = check(r, oracle_of(x))
    assert acc[0] == -1 and acc[1] == -1 and acc[2] == -1 and acc[4] == -1
    assert acc[3] == 3 and r.out_tokens[3].tolist() == [0, 0, 0, 0]


@pytest.mark.parametrize("B,k,V", [(256, 3, 128256), (64, 5, 151936)])
def test_lmhead_full_size_sampled_rows(B, k, V):
    d = workloads.LMHEAD_D
    say("lmhead full", B, k, V, d)
    x = workloads.make_lmhead(B, k, V, d, seed=0, device=DEV)
    r = tv.spec_verify_lmhead(x["hidden"], x["hidden_scale"], x["weight"], x["weight_scale"], x["tokens"])
    torch.cuda.synchronize()
    rows = np.random.default_rng(0).choice(B, 6, replace=False)
    rows = np.unique(np.concatenate([rows, [0, B - 1]]))
    check(r, oracle_of(x, rows), rows)
    acc = r.accepted_len.cpu().numpy()
    say("accepted", np.bincount(acc[acc >= 0], minlength=k + 1).tolist())
    # a second call on the same workspace gives the same bits
    r2 = tv.spec_verify_lmhead(x["hidden"], x["hidden_scale"], x["weight"], x["weight_scale"], x["tokens"])
    torch.cuda.synchronize()
    for a, b in zip(r[:3], r2[:3]):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_lmhead_graph_replays_and_timed_entry():
    x = to_dev(workloads.make_lmhead(16, 3, 20000, 512, seed=5))
    args = (x["hidden"], x["hidden_scale"], x["weight"], x["weight_scale"], x["tokens"])
    ws = torch.empty(tv.lib().spec_lmhead_workspace_size(16, 3, 20000, 512), dtype=torch.uint8, device=DEV)
    eager = tv.spec_verify_lmhead(*args, workspace=ws)
    torch.cuda.synchronize()
    eager = [t.clone() for t in eager[:3]]
    out = tv.binding.VerifyResult(torch.empty(16, dtype=torch.int32, device=DEV),
                                  torch.empty((16, 4), dtype=torch.int32, device=DEV),
                                  torch.empty((16, 4), dtype=torch.float32, device=DEV), None, None)
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            tv.spec_verify_lmhead(*args, workspace=ws, out=out)
    torch.cuda.synchronize()
    for _ in range(3):
        for t in out[:3]:
            t.fill_(-7)
        junk = torch.randn(1 << 20, device=DEV).sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(eager, out[:3]):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32))
        del junk
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    r = tv.spec_verify_lmhead(*args, phase_events=evs)
    torch.cuda.synchronize()
    for a, b in zip(eager, r[:3]):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    t = [evs[0].elapsed_time(evs[1]), evs[1].elapsed_time(evs[2])]
    say("phases ms", [round(v, 4) for v in t])
    assert t[0] > 0 and t[1] >= 0


@pytest.mark.parametrize("B,k", [(1, 0), (64, 3)])     # 128-row and 256-row tiles
def test_lmhead_float32_order_decides_the_argmax(B, k):
    # Vocabulary rows 0 and 1 share their int8 weights; every hidden row gives
    # acc = 680962 against them. With hs = 0.006459721829742193 the two float32
    # products give 5408.34033203125 for row 0 (ws 1.2294964790344238) and
    # 5408.3408203125 for row 1 (ws 1.2294965982437134), one ulp apart; one
    # rounding of the exact product, or the swapped order, would give row 1
    # 5408.34033203125 too, and the tie would go to row 0.
    V, d = 300, 128
    pairs = [(127, 127)] * 42 + [(127, 27), (115, 1)]
    M = B * (k + 1)
    h = torch.zeros((M, d), dtype=torch.int8)
    w = torch.zeros((V, d), dtype=torch.int8)
    for j, (x, y) in enumerate(pairs):
        h[:, j] = x
        w[0, j] = w[1, j] = y
    hs = torch.full((M,), 0.006459721829742193, dtype=torch.float32)
    ws = torch.full((V,), 1.0, dtype=torch.float32)
    ws[0], ws[1] = 1.2294964790344238, 1.2294965982437134
    tok = torch.ones((B, k), dtype=torch.int32)
    x = {"hidden": h, "hidden_scale": hs, "weight": w, "weight_scale": ws, "tokens": tok, "B": B, "k": k,
         "V": V, "d": d}
    r = run(x)
    torch.cuda.synchronize()
    check(r, oracle_of(x))
    assert r.accepted_len.tolist() == [k] * B
    assert (r.out_tokens.cpu() == 1).all()
    assert (r.gap.cpu() == 0.00048828125).all()
