"""Parity of the confidence gate (spec_gate through the C ABI) with the oracle.

argmax and fire are compared bit for bit, the float32 gap exactly (it is the
rounded difference of two stored logits on both sides). Inputs come from
workloads.make_gate (seeded ready distributions and an admissible set) plus
hand-placed ties, single finite entries and invalid rows.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import token_verification_amd as tv
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def check(x, rule, tau, admit=None):
    res = tv.spec_gate(x, tau, admit, rule)
    torch.cuda.synchronize()
    am = None if admit is None else admit.cpu().numpy().view(np.uint32)
    ref = oracle.spec_gate_ref(x.cpu(), rule, tau, am)
    arg = res.argmax.cpu().numpy()
    gap = res.gap.cpu().numpy()
    fire = res.fire.cpu().numpy()
    assert (arg == ref.argmax).all(), np.nonzero(arg != ref.argmax)[0][:5]
    assert (fire.astype(bool) == ref.fire).all() and set(np.unique(fire)) <= {0, 1}
    assert (np.isnan(gap) == np.isnan(ref.gap)).all()
    ok = ~np.isnan(ref.gap)
    assert (gap[ok] == ref.gap[ok].astype(np.float32)).all()
    return fire.astype(bool)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_single_ready_distribution(dtype):
    # the fast-path case: one cached distribution of a 70B-class vocabulary
    for seed in range(40):
        x, A = workloads.make_gate(1, workloads.GATE_V, seed, dtype, device=DEV)
        m = workloads.admit_bits(A, workloads.GATE_V).to(DEV)
        check(x, tv.MARGIN, 2.0, m)
        check(x, tv.CERTIFIED, 1.0, m)


def test_many_rows_and_coverage_sweep():
    x, A = workloads.make_gate(1024, workloads.GATE_V, 7, "bf16", device=DEV)
    m = workloads.admit_bits(A, workloads.GATE_V).to(DEV)
    cov = []
    for tau in (0.0, 0.5, 1.0, 2.0, 4.0, 8.0, 16.0, 24.0):
        cov.append(check(x, tv.MARGIN, tau, m).mean())
    say("coverage", [round(c, 4) for c in cov])
    assert all(a >= b for a, b in zip(cov, cov[1:]))
    assert cov[-1] == 0.0 and cov[0] > 0.8


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("V", [1, 2, 31, 33, 4097, 70001])
def test_odd_vocab_and_special_rows(dtype, V):
    x, A = workloads.make_gate(37, V, V, dtype, device=DEV)
    x = x.clone()
    x[0, :] = -float("inf")                    # no finite entry: invalid
    x[1, V // 2] = float("nan")                # invalid
    x[2, :] = 0.5                              # all tied: gap 0 (or +inf when V = 1)
    x[3, :] = -float("inf")
    x[3, V - 1] = 1.0                          # one finite entry: gap +inf
    x[4, 0] = float("inf")                     # invalid
    m = workloads.admit_bits(A, V).to(DEV)
    for rule, tau in ((tv.MARGIN, 2.0), (tv.MARGIN, -1.0), (tv.CERTIFIED, 0.0), (tv.CERTIFIED, 3.0)):
        check(x, rule, tau, m)
        check(x, rule, tau, None)


def test_gate_on_verify_target_rows():
    # the gate over the target rows of a verify batch agrees with the oracle,
    # and its gap with spec_verify's gap output
    w = workloads.WORKLOADS["b64_k5_v151936_bf16"]
    x = workloads.make(w, 0, device=DEV)
    rows = x["target"].view(w.B * (w.k + 1), w.V)
    check(rows, tv.MARGIN, 2.0)
    g = tv.spec_gate(rows, 2.0)
    v = tv.spec_verify(x["target"], x["draft"], x["tokens"], x["uniforms"], x["T"], 0)
    torch.cuda.synchronize()
    assert torch.equal(g.gap.view(w.B, w.k + 1), v.gap)


def test_gate_errors():
    x = torch.zeros((2, 8), device=DEV)
    with pytest.raises(tv.SpecVerifyError) as e:
        tv.spec_gate(x, float("nan"))
    assert e.value.code == -9
    with pytest.raises(tv.SpecVerifyError) as e:
        tv.spec_gate(x, -1.0, None, tv.CERTIFIED)
    assert e.value.code == -9
