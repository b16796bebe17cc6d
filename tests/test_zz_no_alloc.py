"""spec_verify_noalloc (the library's own device scratch in place of a
workspace) against spec_verify on the same inputs, through the C ABI: two calls
in a row, the second smaller, both bit-exact with the workspace entry point."""
import sys

import pytest
import torch

import token_verification_amd as tv
import workloads
from token_verification_amd import binding

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def outs(B, k, probs):
    return binding.VerifyResult(torch.empty(B, dtype=torch.int32, device=DEV),
                                torch.empty((B, k + 1), dtype=torch.int32, device=DEV),
                                torch.empty((B, k + 1), dtype=torch.float32, device=DEV),
                                torch.empty((B, k), dtype=torch.float32, device=DEV) if probs else None,
                                torch.empty((B, k), dtype=torch.float32, device=DEV) if probs else None)


def same(a, b):
    for u, v in zip(a, b):
        if u is None:
            assert v is None
        else:
            assert torch.equal(u, v)


@pytest.mark.parametrize("first,second", [
    ("b64_k5_v151936_bf16", "b8_k5_v32000_f32"),
    ("b256_k3_v128256_bf16_greedy", "b1_k4_v1000_f32"),
])
def test_noalloc_matches_workspace_entry(first, second):
    for name in (first, second):
        w = workloads.WORKLOADS[name]
        say(f"noalloc {name}")
        x = workloads.make(w, 1, device=DEV)
        probs = w.mode == workloads.SAMPLE
        ref = tv.spec_verify(x["target"], x["draft"], x["tokens"], x["uniforms"], x["T"], x["mode"],
                             return_probs=probs)
        o = outs(w.B, w.k, probs)
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated()
        got = binding.spec_verify_noalloc(x["target"], x["draft"], x["tokens"], x["uniforms"], x["T"],
                                          x["mode"], return_probs=probs, out=o)
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated() == before   # nothing allocated through torch
        same(got, ref)
        del x, ref, o, got                                 # free before the next, smaller call


def test_noalloc_rejects_sizes_beyond_its_scratch():
    # B=8192 k=4 V=151936 needs more workspace than the scratch holds; the check
    # is host-side and nothing is enqueued (no tensor is even read).
    lib = tv.lib()
    need = tv.workspace_size(8192, 4, 151936, 1, 0)
    assert need > (16 << 20)
    fake = 0x10000
    rc = lib.spec_verify_noalloc(fake, fake, fake, fake, 1.0, 0, 8192, 4, 151936, 1, fake, fake, fake,
                                 None, None, None)
    assert rc == -6
    assert "scratch" in tv.binding.last_error()
