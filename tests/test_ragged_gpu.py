"""Parity of the ragged-draft entry point with the fp64 oracle.

Every test calls token_verification_amd.spec_verify with ``draft_len``, which
enqueues spec_verify_ragged of libspecverify.so, and compares with
oracle.spec_verify_ref(..., draft_len=...) on the same seeded inputs (rules in
tests/parity.py). Draft lengths come from workloads.draft_lengths, plus
out-of-range values where a test says so.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import token_verification_amd as tv
import workloads
from parity import DELTA_ACC, compare

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(x):
    y = dict(x)
    for key in ("target", "draft", "tokens", "uniforms"):
        if y[key] is not None:
            y[key] = y[key].to(DEV)
    return y


def run_ragged(x, dl, dtype, greedy, rows=None):
    """GPU call with per-row draft lengths dl (int32 [B]); oracle on host copies."""
    dl = torch.as_tensor(dl, dtype=torch.int32)
    res = tv.spec_verify(x["target"], x["draft"], x["tokens"], x["uniforms"], x["T"], x["mode"],
                         return_probs=not greedy, draft_len=dl.to(DEV))
    torch.cuda.synchronize()
    sel = slice(None) if rows is None else rows
    host = {key: (None if x[key] is None else x[key][sel].cpu())
            for key in ("target", "draft", "tokens", "uniforms")}
    dlh = dl[sel.cpu() if isinstance(sel, torch.Tensor) else sel].numpy()
    ref = oracle.spec_verify_ref(host["target"], host["draft"], host["tokens"], host["uniforms"],
                                 x["T"], x["mode"], draft_len=dlh, flip_delta=DELTA_ACC)
    if rows is not None:
        res = tv.binding.VerifyResult(res.accepted_len[sel], res.out_tokens[sel], res.gap[sel],
                                      None if res.target_prob is None else res.target_prob[sel],
                                      None if res.draft_prob is None else res.draft_prob[sel])
    st = compare(res, ref, dtype, greedy)
    # what the layout fixes for every row, valid or not
    k = x["tokens"].shape[1]
    gap = res.gap.cpu().numpy()
    tok = res.out_tokens.cpu().numpy()
    acc = res.accepted_len.cpu().numpy()
    bad_len = (dlh < 0) | (dlh > k)
    assert (acc[bad_len] == -1).all() and (tok[bad_len] == -1).all() and np.isnan(gap[bad_len]).all()
    past = np.arange(k + 1)[None, :] > dlh[:, None]
    assert np.isnan(gap[past & ~bad_len[:, None]]).all()
    assert (tok[past] == -1).all()
    ok = acc >= 0
    assert (acc[ok] <= dlh[ok]).all()
    return st


@pytest.mark.parametrize("name,seeds", [
    ("b1_k4_v1000_f32", range(200)),
    ("b8_k5_v32000_f32", range(40)),
])
def test_small_workloads_ragged(name, seeds):
    w = workloads.WORKLOADS[name]
    tot = {"rows": 0, "flagged": 0, "mismatch_flagged": 0}
    for s in seeds:
        dl = workloads.draft_lengths(w, s)
        if s % 7 == 3:
            dl[0] = -1 if s % 2 else w.k + 1            # out of range: invalid row
        st = run_ragged(to_dev(workloads.make(w, s)), dl, w.dtype, w.mode == workloads.GREEDY)
        for key in tot:
            tot[key] += st[key]
    say(name, tot)
    assert tot["flagged"] <= max(1, 1e-4 * tot["rows"])


@pytest.mark.parametrize("name,seeds", [
    ("b64_k5_v151936_bf16", range(3)),
    ("b256_k3_v128256_bf16_greedy", range(2)),
])
def test_full_size_workloads_ragged(name, seeds):
    w = workloads.WORKLOADS[name]
    for s in seeds:
        say(f"{name} ragged seed {s}")
        x = workloads.make(w, s, device=DEV)
        st = run_ragged(x, workloads.draft_lengths(w, s), w.dtype, w.mode == workloads.GREEDY)
        say(name, s, st)


def test_largest_workload_ragged_sampled_rows():
    w = workloads.WORKLOADS["b512_k8_v262144_bf16"]
    say("b512 ragged generate")
    x = workloads.make(w, 0, device=DEV)
    rows = torch.tensor(sorted(set(list(range(0, 512, 29)) + [1, 510, 511])), device=DEV)
    st = run_ragged(x, workloads.draft_lengths(w, 0), w.dtype, False, rows=rows)
    say("b512 ragged", st)


def test_full_length_is_the_fixed_call():
    # draft_len = k everywhere: bit-identical to spec_verify
    w = workloads.WORKLOADS["b64_k5_v151936_bf16"]
    x = workloads.make(w, 1, device=DEV)
    a = tv.spec_verify(x["target"], x["draft"], x["tokens"], x["uniforms"], x["T"], 0, return_probs=True)
    torch.cuda.synchronize()
    a = [t.clone() for t in a]
    dl = torch.full((w.B,), w.k, dtype=torch.int32, device=DEV)
    b = tv.spec_verify(x["target"], x["draft"], x["tokens"], x["uniforms"], x["T"], 0, return_probs=True,
                       draft_len=dl)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u.view(torch.int32), v.view(torch.int32))


def rand_case(rng, B, k, V, dtype, T, mode=0):
    t = torch.from_numpy(rng.normal(0, 2.0, (B, k + 1, V)).astype(np.float32))
    d = t[:, :k] + torch.from_numpy(rng.normal(0, 1.0, (B, k, V)).astype(np.float32))
    td = torch.float32 if dtype == "f32" else torch.bfloat16
    tok = torch.from_numpy(rng.integers(0, V, (B, k)).astype(np.int32))
    if mode == 1:
        t = torch.round(t * 2) / 2
        am = torch.argmax(t.to(td).float(), dim=2)[:, :k].to(torch.int32)
        tok = torch.where(torch.from_numpy(rng.random((B, k)) < 0.7), am, tok)
    uni = torch.from_numpy(rng.random((B, k + 1, 2)).astype(np.float32))
    return {"target": t.to(td), "draft": None if mode else d.to(td), "tokens": tok,
            "uniforms": None if mode else uni, "T": T, "mode": mode}


@pytest.mark.parametrize("mode", [0, 1])
def test_ragged_edges(mode):
    rng = np.random.default_rng(40 + mode)
    greedy = mode == 1
    for dtype in ("f32", "bf16"):
        for V in (1, 7, 4097):
            x = rand_case(rng, 6, 3, V, dtype, 0.9, mode)
            for dl in ([0] * 6, [3] * 6, [-1] * 6, [4, -2, 0, 3, 1, 2]):
                say(f"edges mode={mode} {dtype} V={V} draft_len={dl}")
                run_ragged(to_dev(x), np.array(dl, np.int32), dtype, greedy)
        # rows decided by one workgroup (more than 64 rows per batch row)
        x = rand_case(rng, 7, 40, 500, dtype, 1.1, mode)
        run_ragged(to_dev(x), rng.integers(-1, 42, 7).astype(np.int32), dtype, greedy)
    # more batch rows than one chunk of the row-packing scan
    x = rand_case(rng, 1500, 2, 33, "f32", 1.0, mode)
    run_ragged(to_dev(x), rng.integers(-1, 4, 1500).astype(np.int32), "f32", greedy)


def test_rows_past_the_length_are_not_read():
    # NaN in every row past a row's draft length changes nothing
    rng = np.random.default_rng(44)
    x = rand_case(rng, 10, 4, 3000, "bf16", 1.0)
    dl = np.array([0, 1, 2, 3, 4, 0, 1, 2, 3, 4], np.int32)
    for b in range(10):
        x["target"][b, dl[b] + 1:] = float("nan")
        x["draft"][b, dl[b]:] = float("nan")
        x["tokens"][b, dl[b]:] = -3
    st = run_ragged(to_dev(x), dl, "bf16", False)
    assert st["rows"] == 10
    res = tv.spec_verify(*(to_dev(x)[key] for key in ("target", "draft", "tokens", "uniforms")), 1.0, 0,
                         draft_len=torch.from_numpy(dl).to(DEV))
    assert (res.accepted_len.cpu() >= 0).all()
