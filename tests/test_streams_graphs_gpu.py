"""The entry points under HIP graph capture and on concurrent streams.

A serving loop captures the verify step once and replays it. Every entry point
here only enqueues kernels (no allocation, no host synchronisation, no memset
nodes), so a captured call must reproduce the eager results on every replay,
with unrelated eager work and synchronisations between replays. Two streams
with their own workspaces must not disturb each other.
"""
import sys

import pytest
import torch

import token_verification_amd as tv
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def outputs(B, k):
    return tv.binding.VerifyResult(torch.empty(B, dtype=torch.int32, device=DEV),
                                   torch.empty((B, k + 1), dtype=torch.int32, device=DEV),
                                   torch.empty((B, k + 1), dtype=torch.float32, device=DEV),
                                   torch.empty((B, k), dtype=torch.float32, device=DEV),
                                   torch.empty((B, k), dtype=torch.float32, device=DEV))


def same(a, b):
    for u, v in zip(a, b):
        if u is not None:
            assert torch.equal(u.view(torch.int32), v.view(torch.int32))


@pytest.mark.parametrize("ragged", [False, True])
def test_verify_graph_replays_match_eager(ragged):
    w = workloads.WORKLOADS["b8_k5_v32000_f32"]
    x = workloads.make(w, 0, device=DEV)
    dl = workloads.draft_lengths(w, 0).to(DEV) if ragged else None
    B, k = w.B, w.k
    ws = torch.empty(tv.workspace_size(B, k, w.V, 0, 0), dtype=torch.uint8, device=DEV)
    eager = outputs(B, k)
    tv.spec_verify(x["target"], x["draft"], x["tokens"], x["uniforms"], x["T"], 0, workspace=ws,
                   return_probs=True, out=eager, draft_len=dl)
    torch.cuda.synchronize()
    eager = [t.clone() for t in eager]

    s = torch.cuda.Stream()
    out = outputs(B, k)
    g = torch.cuda.CUDAGraph()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            tv.spec_verify(x["target"], x["draft"], x["tokens"], x["uniforms"], x["T"], 0, workspace=ws,
                           return_probs=True, out=out, draft_len=dl)
    torch.cuda.synchronize()
    for r in range(4):
        for t in out:
            t.fill_(-7)
        junk = torch.randn(1 << 20, device=DEV).sum()        # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        same(eager, out)
        del junk
    say("replays ok", ragged)


def test_gate_and_commit_graph_replays():
    x, A = workloads.make_gate(8, 5000, 3, "bf16", device=DEV)
    m = workloads.admit_bits(A, 5000).to(DEV)
    ws = torch.empty(tv.lib().spec_gate_workspace_size(8, 5000, 1), dtype=torch.uint8, device=DEV)
    eager = tv.spec_gate(x, 2.0, m, workspace=ws)
    torch.cuda.synchronize()
    eager = [t.clone() for t in eager]
    out = tv.binding.GateResult(torch.empty(8, dtype=torch.int32, device=DEV),
                                torch.empty(8, device=DEV), torch.empty(8, dtype=torch.int32, device=DEV))
    acc = torch.tensor([0, 2, -1, 1], dtype=torch.int32, device=DEV)
    kv = torch.zeros(4, dtype=torch.int32, device=DEV)
    slots = torch.randn((4, 3, 1000), device=DEV)
    state = torch.zeros((4, 1000), device=DEV)
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            tv.spec_gate(x, 2.0, m, workspace=ws, out=out)
            tv.spec_commit(acc, 2, kv, slots, state)
    torch.cuda.synchronize()
    for r in range(3):
        out.fire.fill_(-7)
        state.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        same(eager, out)
        for b, a in enumerate([0, 2, -1, 1]):
            want = slots[b, a] if a >= 0 else torch.zeros(1000, device=DEV)
            assert torch.equal(state[b], want)
    assert kv.tolist() == [3, 9, 0, 6]                        # three replays of += 1 + a


def test_two_streams_with_own_workspaces():
    w = workloads.WORKLOADS["b64_k5_v151936_bf16"]
    xs = [workloads.make(w, s, device=DEV) for s in (0, 1)]
    ref = []
    for x in xs:
        r = tv.spec_verify(x["target"], x["draft"], x["tokens"], x["uniforms"], x["T"], 0)
        torch.cuda.synchronize()
        ref.append([t.clone() for t in r[:3]])
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    wss = [torch.empty(tv.workspace_size(w.B, w.k, w.V, 1, 0), dtype=torch.uint8, device=DEV)
           for _ in range(2)]
    outs = [outputs(w.B, w.k) for _ in range(2)]
    torch.cuda.synchronize()
    for it in range(5):
        for i in (0, 1):
            with torch.cuda.stream(streams[i]):
                x = xs[i]
                tv.spec_verify(x["target"], x["draft"], x["tokens"], x["uniforms"], x["T"], 0,
                               workspace=wss[i], out=outs[i])
        torch.cuda.synchronize()
        for i in (0, 1):
            same(ref[i], outs[i][:3])


@pytest.mark.parametrize("ragged,mode", [(False, 0), (True, 0), (False, 1)])
def test_timed_entry_matches_and_orders_its_events(ragged, mode):
    w = workloads.WORKLOADS["b64_k5_v151936_bf16"]
    x = workloads.make(w, 2, device=DEV)
    dl = workloads.draft_lengths(w, 2).to(DEV) if ragged else None
    d, u = (x["draft"], x["uniforms"]) if mode == 0 else (None, None)
    a = tv.spec_verify(x["target"], d, x["tokens"], u, x["T"], mode, draft_len=dl)
    torch.cuda.synchronize()
    a = [t.clone() for t in a[:3]]
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    b = tv.spec_verify(x["target"], d, x["tokens"], u, x["T"], mode, draft_len=dl, phase_events=evs)
    torch.cuda.synchronize()
    same(a, b[:3])
    t = [evs[i].elapsed_time(evs[i + 1]) for i in range(3)]
    say("phases ms", [round(v, 4) for v in t])
    assert t[0] > 0 and t[1] >= 0 and t[2] >= 0
    assert t[0] < 1.0                          # pass 1 of this shape takes tens of microseconds
