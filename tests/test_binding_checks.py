"""The binding's checks of caller-supplied outputs and workspaces (host logic;
the checks run before any library call, so CPU tensors exercise them)."""
import pytest
import torch

from token_verification_amd import binding

CPU = torch.device("cpu")


def outs(B, k, probs=True, **over):
    t = {"accepted_len": torch.empty(B, dtype=torch.int32),
         "out_tokens": torch.empty((B, k + 1), dtype=torch.int32),
         "gap": torch.empty((B, k + 1), dtype=torch.float32),
         "target_prob": torch.empty((B, k), dtype=torch.float32) if probs else None,
         "draft_prob": torch.empty((B, k), dtype=torch.float32) if probs else None}
    t.update(over)
    return binding.VerifyResult(**t)


def test_good_outputs_pass():
    binding._check_out(outs(4, 3), 4, 3, CPU, True)
    binding._check_out(outs(4, 3, probs=False), 4, 3, CPU, False)


@pytest.mark.parametrize("field,bad", [
    ("accepted_len", torch.empty(5, dtype=torch.int32)),                 # shape
    ("accepted_len", torch.empty(4, dtype=torch.int64)),                 # dtype
    ("out_tokens", torch.empty((4, 3), dtype=torch.int32)),              # k instead of k+1
    ("out_tokens", torch.empty((4, 8), dtype=torch.int32)[:, ::2]),      # not contiguous
    ("gap", torch.empty((4, 4), dtype=torch.float64)),
    ("target_prob", torch.empty((4, 4), dtype=torch.float32)),
    ("draft_prob", torch.empty((4, 3), dtype=torch.bfloat16)),
])
def test_bad_outputs_raise(field, bad):
    with pytest.raises(ValueError, match=field):
        binding._check_out(outs(4, 3, **{field: bad}), 4, 3, CPU, True)


def test_probs_requested_without_prob_tensors():
    with pytest.raises(ValueError, match="return_probs"):
        binding._check_out(outs(4, 3, probs=False), 4, 3, CPU, True)


def test_wrong_device_output():
    with pytest.raises(ValueError, match="accepted_len"):
        binding._check_out(outs(4, 3), 4, 3, torch.device("cuda:0"), True)


def test_workspace_checks():
    ws = torch.empty(1024, dtype=torch.uint8)
    assert binding._user_workspace(ws, CPU, 1024) is ws
    assert binding._user_workspace(torch.empty(256, dtype=torch.float32), CPU, 1024) is not None
    with pytest.raises(ValueError, match="needs"):
        binding._user_workspace(ws, CPU, 1025)
    with pytest.raises(ValueError, match="device"):
        binding._user_workspace(ws, torch.device("cuda:0"), 16)
    with pytest.raises(ValueError, match="contiguous"):
        binding._user_workspace(torch.empty(4096, dtype=torch.uint8)[::2], CPU, 16)
