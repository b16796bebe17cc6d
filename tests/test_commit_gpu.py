"""Parity of the commit / rollback step (spec_commit through the C ABI) with
oracle.commit.commit_ref: KV lengths and the committed state bit for bit."""
import numpy as np
import pytest
import torch

import token_verification_amd as tv
import workloads
from oracle.commit import commit_ref

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def run(acc, k, kv, slots, state):
    kv_d = None if kv is None else torch.from_numpy(kv).to(DEV)
    sl_d = None if slots is None else slots.to(DEV)
    st_d = None if state is None else state.to(DEV)
    tv.spec_commit(torch.from_numpy(acc).to(DEV), k, kv_d, sl_d, st_d)
    torch.cuda.synchronize()
    ref_kv, ref_st = commit_ref(acc, kv if kv is not None else np.zeros(len(acc), np.int32),
                                None if slots is None else slots.view(torch.int16).numpy(),
                                None if state is None else state.view(torch.int16).numpy(), k=k)
    if kv is not None:
        assert (kv_d.cpu().numpy() == ref_kv).all()
    if state is not None:
        assert torch.equal(st_d.cpu().view(torch.int16), torch.from_numpy(ref_st))


def test_commit_after_the_headline_verify():
    # accepted lengths from a real verify call; 1 MiB of fp32 state per row
    w = workloads.WORKLOADS["b64_k5_v151936_bf16"]
    x = workloads.make(w, 0, device=DEV)
    res = tv.spec_verify(x["target"], x["draft"], x["tokens"], x["uniforms"], x["T"], 0)
    acc = res.accepted_len.cpu().numpy()
    acc[3] = -1
    g = torch.Generator().manual_seed(1)
    slots = torch.randn((w.B, w.k + 1, 262144), generator=g)
    state = torch.randn((w.B, 262144), generator=g)
    kv = np.random.default_rng(2).integers(0, 4000, w.B).astype(np.int32)
    run(acc, w.k, kv, slots, state)


@pytest.mark.parametrize("B,k,shape,dtype", [
    (9, 3, (1002,), torch.bfloat16),          # 2004 bytes per row: 4-byte copies
    (17, 0, (7, 64), torch.float32),          # 1792 bytes: 16-byte copies
    (3, 64, (5000,), torch.float32),          # largest k
    (130, 2, (3, 34), torch.bfloat16),        # 204 bytes
    (2, 1, (70000,), torch.float32),          # several chunks per row
])
def test_commit_shapes(B, k, shape, dtype):
    rng = np.random.default_rng(B)
    acc = rng.integers(-1, k + 2, B).astype(np.int32)
    acc[0] = k
    kv = rng.integers(0, 100, B).astype(np.int32)
    slots = torch.from_numpy(rng.normal(size=(B, k + 1) + shape).astype(np.float32)).to(dtype)
    state = torch.from_numpy(rng.normal(size=(B,) + shape).astype(np.float32)).to(dtype)
    run(acc, k, kv, slots, state)
    run(acc, k, kv, None, None)                # KV lengths only
    run(acc, k, None, slots, state)            # state only


def test_verify_then_commit_ragged():
    w = workloads.WORKLOADS["b8_k5_v32000_f32"]
    x = workloads.make(w, 0, device=DEV)
    dl = workloads.draft_lengths(w, 0).to(DEV)
    res = tv.spec_verify(x["target"], x["draft"], x["tokens"], x["uniforms"], x["T"], 0, draft_len=dl)
    kv = torch.full((w.B,), 100, dtype=torch.int32, device=DEV)
    tv.spec_commit(res.accepted_len, w.k, kv)
    torch.cuda.synchronize()
    a = res.accepted_len.cpu()
    assert (a <= dl.cpu()).all()
    assert torch.equal(kv.cpu(), torch.where(a >= 0, 101 + a, torch.full_like(a, 100)))
