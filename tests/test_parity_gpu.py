"""Parity of the HIP verify step (through the C ABI) with the fp64 oracle.

Every test here calls token_verification_amd.spec_verify, which enqueues the
HIP kernel through libspecverify.so, and compares against oracle.spec_verify_ref
on the same seeded inputs (see tests/parity.py for the rules).
"""
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import token_verification_amd as tv
import workloads
from parity import DELTA_ACC, DELTA_CDF, compare

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_pair(x, dtype, greedy, rows=None):
    """GPU call on device tensors x; oracle on host copies (optionally a row subset)."""
    res = tv.spec_verify(x["target"], x["draft"], x["tokens"], x["uniforms"], x["T"], x["mode"],
                         return_probs=not greedy)
    torch.cuda.synchronize()
    sel = slice(None) if rows is None else rows
    tgt = x["target"][sel].cpu()
    dft = None if x["draft"] is None else x["draft"][sel].cpu()
    tok = x["tokens"][sel].cpu()
    uni = None if x["uniforms"] is None else x["uniforms"][sel].cpu()
    ref = oracle.spec_verify_ref(tgt, dft, tok, uni, x["T"], x["mode"], flip_delta=DELTA_ACC)
    if rows is not None:
        res = tv.binding.VerifyResult(res.accepted_len[sel], res.out_tokens[sel], res.gap[sel],
                                      None if res.target_prob is None else res.target_prob[sel],
                                      None if res.draft_prob is None else res.draft_prob[sel])
    return compare(res, ref, dtype, greedy)


def to_dev(x):
    y = dict(x)
    for key in ("target", "draft", "tokens", "uniforms"):
        if y[key] is not None:
            y[key] = y[key].to(DEV)
    return y


# The five workloads at full size, over enough seeds for the near-tie budget,
# are in test_parity_scale_gpu.py.


# ---------------------------------------------------------------- edge cases


def rand_case(rng, B, k, V, dtype, T, mask_frac=0.0, spread=2.0):
    t = torch.from_numpy(rng.normal(0, spread, (B, k + 1, V)).astype(np.float32))
    d = t[:, :k] + torch.from_numpy(rng.normal(0, 1.0, (B, k, V)).astype(np.float32))
    if mask_frac > 0:
        m = torch.from_numpy(rng.random((B, k + 1, V)) < mask_frac)
        t[m] = -float("inf")
        md = torch.from_numpy(rng.random((B, k, V)) < mask_frac)
        d[md] = -float("inf")
        t[:, :, 0] = 0.0                       # keep a finite entry per row
        d[:, :, 0] = 0.0
    td = torch.float32 if dtype == "f32" else torch.bfloat16
    tok = torch.from_numpy(rng.integers(0, V, (B, k)).astype(np.int32))
    uni = torch.from_numpy(rng.random((B, k + 1, 2)).astype(np.float32))
    return {"target": t.to(td), "draft": d.to(td), "tokens": tok, "uniforms": uni, "T": T, "mode": 0}


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V", [1, 2, 3, 7, 8, 63, 65, 1001, 4097, 40961])
def test_odd_vocab_sampling(dtype, V):
    rng = np.random.default_rng(V)
    for k, T in ((0, 1.0), (1, 0.05), (3, 10.0), (5, 0.7)):
        x = rand_case(rng, 7, k, V, dtype, T)
        run_pair(to_dev(x), dtype, False)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V", [1, 2, 5, 64, 129, 3001, 70001])
def test_odd_vocab_greedy(dtype, V):
    rng = np.random.default_rng(1000 + V)
    for k in (0, 1, 4):
        x = rand_case(rng, 9, k, V, dtype, 1.0)
        # coarse values force exact ties at the top
        x["target"] = (torch.round(x["target"].float() * 2) / 2).to(x["target"].dtype)
        am = torch.argmax(x["target"].float(), dim=2)[:, :k].to(torch.int32)
        keep = torch.from_numpy(rng.random((9, k)) < 0.7)
        x["tokens"] = torch.where(keep, am, x["tokens"])
        x["mode"] = 1
        x["draft"] = None
        x["uniforms"] = None
        run_pair(to_dev(x), dtype, True)


def test_masks_and_large_k():
    rng = np.random.default_rng(5)
    for dtype in ("f32", "bf16"):
        x = rand_case(rng, 5, 64, 300, dtype, 0.9, mask_frac=0.5)
        run_pair(to_dev(x), dtype, False)


def test_q_equals_p_and_disjoint_supports():
    rng = np.random.default_rng(6)
    x = rand_case(rng, 16, 5, 5000, "bf16", 1.0)
    x["draft"] = x["target"][:, :5].clone()
    x["uniforms"][:, :, 0] = 1.0 - 2.0 ** -24
    st = run_pair(to_dev(x), "bf16", False)
    res = tv.spec_verify(*(to_dev(x)[key] for key in ("target", "draft", "tokens", "uniforms")), 1.0, 0)
    assert (res.accepted_len.cpu() == 5).all()
    y = rand_case(rng, 16, 3, 5000, "f32", 1.0)
    y["target"][:, :, 2500:] = -float("inf")
    y["draft"][:, :, :2500] = -float("inf")
    y["tokens"] = torch.from_numpy(rng.integers(2500, 5000, (16, 3)).astype(np.int32))
    y["uniforms"][:, 0, 0] = 0.0
    run_pair(to_dev(y), "f32", False)
    res = tv.spec_verify(*(to_dev(y)[key] for key in ("target", "draft", "tokens", "uniforms")), 1.0, 0)
    assert (res.accepted_len.cpu() == 0).all()
    say(st)


def test_invalid_rows():
    rng = np.random.default_rng(7)
    for dtype in ("f32", "bf16"):
        x = rand_case(rng, 8, 3, 777, dtype, 1.0)
        t = x["target"].float()
        d = x["draft"].float()
        t[0, 1, 3] = float("nan")
        d[1, 0, 5] = float("inf")
        t[2, 3, :] = -float("inf")
        x["tokens"][3, 2] = 777
        x["tokens"][4, 0] = -1
        t[5, 0, :100] = -float("inf")
        td = x["target"].dtype
        x["target"], x["draft"] = t.to(td), d.to(td)
        run_pair(to_dev(x), dtype, False)
        g = dict(x)
        g["mode"], g["draft"], g["uniforms"] = 1, None, None
        run_pair(to_dev(g), dtype, True)


def test_deterministic_and_exact_path():
    w = workloads.WORKLOADS["b8_k5_v32000_f32"]
    x = to_dev(workloads.make(w, 3))
    a = tv.spec_verify(x["target"], x["draft"], x["tokens"], x["uniforms"], x["T"], 0, return_probs=True)
    torch.cuda.synchronize()
    a = [t.clone() for t in a]
    b = tv.spec_verify(x["target"], x["draft"], x["tokens"], x["uniforms"], x["T"], 0, return_probs=True)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)
    os.environ["SPEC_VERIFY_FORCE_EXACT_PATH"] = "1"
    try:
        c = tv.spec_verify(x["target"], x["draft"], x["tokens"], x["uniforms"], x["T"], 0, return_probs=True)
        torch.cuda.synchronize()
    finally:
        del os.environ["SPEC_VERIFY_FORCE_EXACT_PATH"]
    assert torch.equal(a[0], c.accepted_len)
    assert torch.equal(a[1], c.out_tokens)


def test_chi_square_on_gpu():
    # 10^6 trials: x ~ q, u ~ U(0,1); the first emitted token is distributed as p.
    from scipy import stats
    from scipy.special import softmax
    rng = np.random.default_rng(77)
    V, n, T = 16, 1_000_000, 0.8
    t0 = rng.normal(0, 1.5, (2, V)).astype(np.float32)
    d0 = (t0[:1] * 0.7 + rng.normal(0, 1.0, (1, V))).astype(np.float32)
    q = softmax(d0[0].astype(np.float64) / np.float64(np.float32(T)))
    p = softmax(t0[0].astype(np.float64) / np.float64(np.float32(T)))
    tok = torch.from_numpy(rng.choice(V, size=(n, 1), p=q).astype(np.int32)).to(DEV)
    u = torch.from_numpy(rng.random((n, 2, 2)).astype(np.float32)).to(DEV)
    tgt = torch.from_numpy(t0).to(DEV).expand(n, 2, V).contiguous()
    dft = torch.from_numpy(d0).to(DEV).expand(n, 1, V).contiguous()
    res = tv.spec_verify(tgt, dft, tok, u, T, 0)
    counts = np.bincount(res.out_tokens[:, 0].cpu().numpy(), minlength=V)
    _, pval = stats.chisquare(counts, p * n)
    say("chi2 p-value", pval)
    assert pval > 1e-3


def test_noncontiguous_rejected_and_errors():
    x = to_dev(rand_case(np.random.default_rng(8), 2, 2, 64, "f32", 1.0))
    with pytest.raises(tv.SpecVerifyError) as e:
        tv.spec_verify(x["target"], x["draft"], x["tokens"], x["uniforms"], 0.0, 0)
    assert e.value.code == -5
    with pytest.raises(tv.SpecVerifyError) as e:
        tv.spec_verify(x["target"], None, x["tokens"], x["uniforms"], 1.0, 0)
    assert e.value.code == -1


def _band_case(rng, B, k, V, clusters):
    """Draft rows equal to the target except a few low-mass entries: the exact
    lambda is within 1e-5 of 1, so elements with x_t == x_d (and, with
    clusters, tiny-magnitude elements one or two bf16 ulps apart) fall inside
    pass 2's band around it."""
    t = torch.from_numpy(rng.normal(0, 2.0, (B, k + 1, V)).astype(np.float32)).to(torch.bfloat16)
    d = t[:, :k].clone()
    for b in range(B):
        for i in range(k):
            low = torch.argsort(t[b, i].float())[:5]
            d[b, i, low] = (t[b, i, low].float() - 4.0).to(torch.bfloat16)
            if clusters:
                # tiny magnitudes: x_t - x_d of +-1 and +-2 ulps at 2^-10
                idx = torch.from_numpy(rng.choice(V, 64, replace=False))
                base = torch.full((64,), 2.0 ** -10)
                t[b, i, idx] = base.to(torch.bfloat16)
                steps = torch.tensor([0, 1, -1, 2, -2] * 13)[:64].float() * 2.0 ** -17
                d[b, i, idx] = (base + steps).to(torch.bfloat16)
    tok = torch.from_numpy(rng.integers(0, V, (B, k)).astype(np.int32))
    uni = torch.from_numpy(rng.random((B, k + 1, 2)).astype(np.float32))
    uni[:, :, 0] = 0.999                     # reject at the first position: a residual draw
    return {"target": t, "draft": d, "tokens": tok, "uniforms": uni, "T": 1.0, "mode": 0}


@pytest.mark.parametrize("clusters", [False, True])
def test_band_groups(clusters):
    # one band group per segment (x_t == x_d), or more distinct keys than the
    # groups a segment records (the draw then recomputes those segments)
    rng = np.random.default_rng(71 + clusters)
    for V in (20000, 151936):
        x = _band_case(rng, 6, 2, V, clusters)
        st = run_pair(to_dev(x), "bf16", False)
        say("band groups", clusters, V, st)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("seed", range(6))
def test_exact_enumeration_on_gpu(dtype, seed):
    # For V <= 8 the output distribution, enumerated over the draft token and
    # the uniforms' cells (each probed at a float32 midpoint, far from every
    # boundary), equals p_0 within 1e-12, the bonus given acceptance is p_1,
    # and acceptance has probability sum min(p, q) ("Speculative Decoding:
    # The Physics of Stolen Time", section 2, the losslessness proof). Every
    # enumerated row must also be bit-exact with the oracle.
    from oracle import exact_enum
    rng = np.random.default_rng(300 + seed)
    V = int(rng.integers(2, 9))
    T = float(rng.choice([0.5, 1.0, 1.7]))
    t = rng.normal(0, 1.5, (2, V)).astype(np.float32)
    d = (t[:1] + rng.normal(0, 1.0, (1, V))).astype(np.float32)
    if seed % 3 == 2:
        d[0, : V // 2] = -np.inf                      # draft misses part of the support
    if dtype == "bf16":                               # bf16 values, exactly representable in f32
        t = torch.from_numpy(t).to(torch.bfloat16).float().numpy()
        d = torch.from_numpy(d).to(torch.bfloat16).float().numpy()
    tgt, dft, tok, uni, wts = exact_enum.cells_k1(t, d, T)
    td = torch.float32 if dtype == "f32" else torch.bfloat16
    x = {"target": torch.from_numpy(tgt).to(td), "draft": torch.from_numpy(dft).to(td),
         "tokens": torch.from_numpy(tok), "uniforms": torch.from_numpy(uni), "T": T, "mode": 0}
    st = run_pair(to_dev(x), dtype, False)
    assert st["flagged"] == 0                          # midpoints are far from every edge
    res = tv.spec_verify(*(to_dev(x)[key] for key in ("target", "draft", "tokens", "uniforms")), T, 0)
    dist0, dist1, acc = exact_enum.distribution(res.out_tokens.cpu().numpy(), res.accepted_len.cpu().numpy(),
                                                wts, V)
    out0, acc_exact, p0, p1 = exact_enum.closed_form(t, d, T)
    say(f"enumeration V={V} T={T} rows={len(wts)}: max |dist0 - p0| = {np.abs(dist0 - p0).max():.2e}")
    assert np.abs(dist0 - p0).max() < 1e-12
    assert abs(acc - float(acc_exact)) < 1e-12
    assert np.abs(dist1 - acc * p1).max() < 1e-12


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_zero_residual_mass_on_gpu(dtype):
    # Target and draft rows agree exactly and both put the draft token at -inf:
    # r = 0 rejects at position 0, max(0, p - q) is identically zero and the
    # draw falls back to p_0 (the oracle flags the row with bit 0; the kernel
    # must give the same token).
    rng = np.random.default_rng(91)
    B, V = 8, 1000
    x = rand_case(rng, B, 2, V, dtype, 0.9)
    x["draft"][:, 0] = x["target"][:, 0]
    for b in range(B):
        x["target"][b, 0, int(x["tokens"][b, 0])] = -float("inf")
        x["draft"][b, 0, int(x["tokens"][b, 0])] = -float("inf")
    st = run_pair(to_dev(x), dtype, False)
    assert st["flag_bits"] == B and st["mismatch_flagged"] == 0
