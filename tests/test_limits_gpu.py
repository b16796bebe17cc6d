"""Parity at the documented size limits (through the C ABI): the largest sampling
vocabulary (2^23), a greedy vocabulary past it, the largest batch (2^21 rows) and
the largest draft count (64), each against the oracle on every row."""
import sys

import numpy as np
import pytest
import torch

import oracle
import token_verification_amd as tv
from parity import DELTA_ACC, compare

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def case(B, k, V, dtype, seed, spread=2.0):
    g = torch.Generator(device=DEV).manual_seed(seed)
    t = torch.randn((B, k + 1, V), generator=g, device=DEV) * spread
    d = t[:, :k] + torch.randn((B, k, V), generator=g, device=DEV)
    td = torch.float32 if dtype == "f32" else torch.bfloat16
    tok = torch.randint(0, V, (B, k), generator=g, device=DEV, dtype=torch.int32)
    uni = torch.rand((B, k + 1, 2), generator=g, device=DEV)
    return t.to(td), d.to(td), tok, uni


def check(t, d, tok, uni, T, mode, dtype, threads=0, draft_len=None):
    greedy = mode == tv.GREEDY
    res = tv.spec_verify(t, None if greedy else d, tok, None if greedy else uni, T, mode,
                         return_probs=not greedy, draft_len=draft_len)
    torch.cuda.synchronize()
    ref = oracle.spec_verify_ref(t.cpu(), None if greedy else d.cpu(), tok.cpu(),
                                 None if greedy else uni.cpu(), T, mode, threads=threads,
                                 draft_len=None if draft_len is None else draft_len.cpu().numpy(),
                                 flip_delta=DELTA_ACC)
    return compare(res, ref, dtype, greedy)


@pytest.mark.parametrize("dtype,B", [("bf16", 2), ("f32", 1)])
def test_largest_sampling_vocabulary(dtype, B):
    V = 1 << 23
    say(f"V=2^23 {dtype} B={B}")
    t, d, tok, uni = case(B, 1, V, dtype, 11)
    say(check(t, d, tok, uni, 1.0, tv.SAMPLE, dtype, threads=2))


def test_greedy_vocabulary_past_the_sampling_cap():
    V = (1 << 25) + 3
    say("greedy V=2^25+3")
    t, d, tok, uni = case(1, 1, V, "bf16", 12)
    tok[0, 0] = int(torch.argmax(t[0, 0].float()))
    say(check(t, d, tok, uni, 1.0, tv.GREEDY, "bf16", threads=1))


@pytest.mark.parametrize("mode", [tv.SAMPLE, tv.GREEDY])
def test_largest_batch(mode):
    B = 1 << 21
    say(f"B=2^21 mode={mode}")
    t, d, tok, uni = case(B, 1, 4, "f32", 13)
    st = check(t, d, tok, uni, 0.7, mode, "f32")
    say(st)
    assert st["flagged"] <= max(1, 1e-4 * B)


def test_largest_draft_count():
    say("k=64 V=20000")
    t, d, tok, uni = case(3, 64, 20000, "bf16", 14)
    say(check(t, d, tok, uni, 1.0, tv.SAMPLE, "bf16"))
    dl = torch.tensor([64, 0, 37], dtype=torch.int32, device=DEV)
    say(check(t, d, tok, uni, 1.0, tv.SAMPLE, "bf16", draft_len=dl))
    say(check(t, d, tok, uni, 1.0, tv.GREEDY, "bf16", draft_len=dl))
