"""C-ABI checks that need no GPU: the library loads, exports exactly what the
header declares, sizes its workspace consistently, and rejects bad arguments
with the documented codes (spec_verify_check_args makes no HIP call)."""
import ctypes
import os
import re
import subprocess

import pytest

import token_verification_amd as tv
from token_verification_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spec_verify.h")


def declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return set(re.findall(r"\b(spec_(?:verify|gate|commit|lmhead)\w*)\s*\(", src))


def test_exports_match_header():
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    exported = {s for s in exported if s.startswith("spec_")}
    assert declared() == exported
    assert len(exported) == 21


def test_version():
    assert b"gfx950" in tv.lib().spec_verify_version()


def test_workspace_size():
    assert tv.workspace_size(64, 5, 151936, 1, 0) > 0
    assert tv.workspace_size(0, 5, 100, 1, 0) == 0
    assert tv.workspace_size(1, 65, 100, 1, 0) == 0
    assert tv.workspace_size(1, 2, 0, 1, 0) == 0
    assert tv.workspace_size(1, 2, 100, 7, 0) == 0
    assert tv.workspace_size(1, 2, 100, 1, 3) == 0
    # greedy needs no pass-2 records
    assert tv.workspace_size(64, 5, 151936, 1, 1) < tv.workspace_size(64, 5, 151936, 1, 0)
    for B, k, V in ((1, 0, 1), (3, 64, 7), (512, 8, 262144), (1, 4, 1 << 23)):
        n = tv.workspace_size(B, k, V, 0, 0)
        assert n % 256 == 0 and n >= 256
    # the sampling draw supports V up to 2^23; greedy mode has no such cap
    assert tv.workspace_size(1, 4, (1 << 23) + 1, 1, 0) == 0
    assert tv.workspace_size(1, 4, 1 << 24, 1, 1) > 0


FAKE = 0x10000          # aligned fake device address (never dereferenced)


def args(**kw):
    a = dict(target=FAKE, draft=FAKE, tokens=FAKE, uniforms=FAKE, T=1.0, mode=0, B=4, k=3, V=100,
             dtype=0, acc=FAKE, out=FAKE, gap=FAKE, ws=0x100000, ws_bytes=tv.workspace_size(4, 3, 100, 0, 0))
    a.update(kw)
    return a


def check(**kw):
    a = args(**kw)
    return tv.check_args(a["target"], a["draft"], a["tokens"], a["uniforms"], a["T"], a["mode"],
                         a["B"], a["k"], a["V"], a["dtype"], a["acc"], a["out"], a["gap"], a["ws"],
                         a["ws_bytes"])


@pytest.mark.parametrize("kw,code", [
    ({}, 0),
    ({"target": None}, -1),
    ({"draft": None}, -1),
    ({"draft": None, "mode": 1, "uniforms": None}, 0),
    ({"tokens": None}, -1),
    ({"tokens": None, "k": 0}, 0),
    ({"uniforms": None}, -1),
    ({"acc": None}, -1),
    ({"gap": None}, -1),
    ({"B": 0}, -2),
    ({"k": -1}, -2),
    ({"k": 65}, -2),
    ({"V": 0}, -2),
    ({"dtype": 2}, -3),
    ({"mode": 2}, -4),
    ({"T": 0.0}, -5),
    ({"T": -1.0}, -5),
    ({"T": float("nan")}, -5),
    ({"T": float("inf")}, -5),
    ({"T": 0.0, "mode": 1, "draft": None, "uniforms": None}, 0),
    ({"ws": None}, -6),
    ({"ws_bytes": 16}, -6),
    ({"target": FAKE + 2}, -7),
    ({"target": FAKE + 2, "dtype": 1}, 0),
    ({"target": FAKE + 1, "dtype": 1}, -7),
    ({"tokens": FAKE + 2}, -7),
    ({"ws": 0x100000 + 64}, -7),
])
def test_check_args_codes(kw, code):
    assert check(**kw) == code
    if code != 0:
        assert binding.last_error()


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(tv.SpecVerifyError):
        binding.lib()


def test_cpu_tensors_rejected():
    import torch
    t = torch.zeros(1, 2, 4)
    with pytest.raises(ValueError):
        tv.spec_verify(t, torch.zeros(1, 1, 4), torch.zeros(1, 1, dtype=torch.int32),
                       torch.zeros(1, 2, 2), 1.0, 0)


@pytest.mark.parametrize("kw,dlen,code", [
    ({}, None, -1),                 # draft_len is required by the ragged entry
    ({}, FAKE + 2, -7),             # and 4-byte aligned
    ({"B": 0}, FAKE, -2),
    ({"tokens": None}, FAKE, -1),
])
def test_ragged_entry_rejects_synchronously(kw, dlen, code):
    # every case fails the host-side checks, so no HIP call is made
    a = args(**kw)
    L = tv.lib()
    rc = L.spec_verify_ragged(a["target"], a["draft"], a["tokens"], dlen, a["uniforms"],
                              ctypes.c_float(a["T"]), a["mode"], a["B"], a["k"], a["V"], a["dtype"],
                              a["acc"], a["out"], a["gap"], None, None, a["ws"], a["ws_bytes"], None)
    assert rc == code
    assert binding.last_error()


@pytest.mark.parametrize("kw,code", [
    ({"rule": 2}, -4),
    ({"n": 0}, -2),
    ({"V": 0}, -2),
    ({"tau": float("nan")}, -9),
    ({"tau": -1.0, "rule": 1}, -9),
    ({"logits": None}, -1),
    ({"fire": None}, -1),
    ({"admit": FAKE + 2}, -7),
    ({"dtype": 5}, -3),
    ({"ws": None}, -6),
])
def test_gate_rejects_synchronously(kw, code):
    a = dict(logits=FAKE, n=3, V=100, dtype=1, rule=0, tau=2.0, admit=None, argmax=FAKE, gap=FAKE,
             fire=FAKE, ws=0x100000, ws_bytes=1 << 20)
    a.update(kw)
    rc = tv.lib().spec_gate(a["logits"], a["n"], a["V"], a["dtype"], a["rule"], ctypes.c_float(a["tau"]),
                            a["admit"], a["argmax"], a["gap"], a["fire"], a["ws"], a["ws_bytes"], None)
    assert rc == code
    assert binding.last_error()


def test_gate_workspace_size():
    assert tv.lib().spec_gate_workspace_size(1, 128256, 1) > 0
    assert tv.lib().spec_gate_workspace_size(0, 128256, 1) == 0


@pytest.mark.parametrize("kw,code", [
    ({"B": 0}, -2),
    ({"k": 65}, -2),
    ({"acc": None}, -1),
    ({"slots": None}, -1),
    ({"row": 6}, -7),
    ({"state": FAKE + 2}, -7),
])
def test_commit_rejects_synchronously(kw, code):
    a = dict(acc=FAKE, B=4, k=3, kv=FAKE, slots=FAKE, state=0x200000, row=64)
    a.update(kw)
    rc = tv.lib().spec_commit(a["acc"], a["B"], a["k"], a["kv"], a["slots"], a["state"], a["row"], None)
    assert rc == code
    assert binding.last_error()


def test_lmhead_workspace_size():
    L = tv.lib()
    assert L.spec_lmhead_workspace_size(256, 3, 128256, 4096) > 0
    assert L.spec_lmhead_workspace_size(256, 3, 128256, 4096) % 256 == 0
    assert L.spec_lmhead_workspace_size(0, 3, 100, 128) == 0
    assert L.spec_lmhead_workspace_size(1, 65, 100, 128) == 0
    assert L.spec_lmhead_workspace_size(1, 3, 100, 100) == 0       # d not a multiple of 128
    assert L.spec_lmhead_workspace_size(1, 3, 100, 65536 + 128) == 0


@pytest.mark.parametrize("kw,code", [
    ({"B": 0}, -2),
    ({"k": 65}, -2),
    ({"d": 192}, -2),
    ({"d": 0}, -2),
    ({"hidden": None}, -1),
    ({"w_scale": None}, -1),
    ({"tokens": None}, -1),
    ({"gap": None}, -1),
    ({"hidden": FAKE + 4}, -7),
    ({"weight": FAKE + 8}, -7),
    ({"h_scale": FAKE + 2}, -7),
    ({"ws": None}, -6),
    ({"ws_bytes": 256}, -6),
    ({"ws": 0x100010}, -7),
])
def test_lmhead_rejects_synchronously(kw, code):
    a = dict(hidden=FAKE, h_scale=FAKE, weight=FAKE, w_scale=FAKE, tokens=FAKE, B=4, k=3, V=1000, d=256,
             acc=FAKE, out=FAKE, gap=FAKE, ws=0x100000, ws_bytes=1 << 24)
    a.update(kw)
    rc = tv.lib().spec_verify_lmhead(a["hidden"], a["h_scale"], a["weight"], a["w_scale"], a["tokens"], a["B"],
                                     a["k"], a["V"], a["d"], a["acc"], a["out"], a["gap"], a["ws"],
                                     a["ws_bytes"], None)
    assert rc == code
    assert binding.last_error()
    ev = (ctypes.c_void_p * 3)(None, None, None)
    rc = tv.lib().spec_verify_lmhead_timed(a["hidden"], a["h_scale"], a["weight"], a["w_scale"], a["tokens"],
                                           a["B"], a["k"], a["V"], a["d"], a["acc"], a["out"], a["gap"],
                                           a["ws"], a["ws_bytes"], None, ctypes.cast(ev, ctypes.c_void_p))
    assert rc in (code, -1)
    # the tile-major entry point validates the same arguments the same way
    rc = tv.lib().spec_verify_lmhead_packed(a["hidden"], a["h_scale"], a["weight"], a["w_scale"], a["tokens"],
                                            a["B"], a["k"], a["V"], a["d"], a["acc"], a["out"], a["gap"],
                                            a["ws"], a["ws_bytes"], None, None)
    assert rc == code


def test_lmhead_packed_size_and_pack_rejects():
    L = tv.lib()
    assert L.spec_lmhead_packed_size(1000, 4096) == 4 * 256 * 4096     # whole 256-row tiles
    assert L.spec_lmhead_packed_size(256, 128) == 256 * 128
    assert L.spec_lmhead_packed_size(257, 128) == 512 * 128
    assert L.spec_lmhead_packed_size(0, 128) == 0
    assert L.spec_lmhead_packed_size(100, 100) == 0                    # d not a multiple of 128
    assert L.spec_lmhead_packed_size(100, 65536 + 128) == 0
    need = L.spec_lmhead_packed_size(1000, 256)
    for args, code in (((FAKE, 0, 256, FAKE, need, None), -2), ((None, 1000, 256, FAKE, need, None), -1),
                       ((FAKE, 1000, 256, None, need, None), -1), ((FAKE + 8, 1000, 256, FAKE, need, None), -7),
                       ((FAKE, 1000, 256, FAKE, need - 16, None), -6)):
        assert L.spec_lmhead_pack(*args) == code
        assert binding.last_error()


def test_lmhead_sample_workspace_size():
    L = tv.lib()
    n = L.spec_lmhead_sample_workspace_size(256, 3, 128256, 4096)
    assert n > 0 and n % 256 == 0
    # per-tile records of both heads and the two recomputed logit rows per batch row
    assert n > 2 * 256 * 128256 * 4
    assert L.spec_lmhead_sample_workspace_size(0, 3, 100, 128) == 0
    assert L.spec_lmhead_sample_workspace_size(1, 65, 100, 128) == 0
    assert L.spec_lmhead_sample_workspace_size(1, 3, 100, 100) == 0
    assert L.spec_lmhead_sample_workspace_size(1, 3, (1 << 23) + 1, 128) == 0
    assert L.spec_lmhead_sample_workspace_size(1, 0, 100, 128) > 0


@pytest.mark.parametrize("kw,code", [
    ({"B": 0}, -2),
    ({"k": 65}, -2),
    ({"d": 192}, -2),
    ({"V": (1 << 23) + 1}, -2),
    ({"T": 0.0}, -5),
    ({"T": float("inf")}, -5),
    ({"hidden": None}, -1),
    ({"uniforms": None}, -1),
    ({"dhidden": None}, -1),
    ({"tokens": None}, -1),
    ({"dweight": FAKE}, -1),                  # a draft head without its scales
    ({"gap": None}, -1),
    ({"hidden": FAKE + 4}, -7),
    ({"dhidden": FAKE + 8}, -7),
    ({"tprob": FAKE + 2}, -7),
    ({"ws": None}, -6),
    ({"ws_bytes": 256}, -6),
    ({"ws": 0x100010}, -7),
])
def test_lmhead_sample_rejects_synchronously(kw, code):
    a = dict(hidden=FAKE, h_scale=FAKE, weight=FAKE, w_scale=FAKE, dhidden=FAKE, dh_scale=FAKE, dweight=None,
             dw_scale=None, tokens=FAKE, uniforms=FAKE, T=1.0, B=4, k=3, V=1000, d=256, acc=FAKE, out=FAKE,
             gap=FAKE, tprob=None, dprob=None, ws=0x100000, ws_bytes=1 << 26)
    a.update(kw)
    args = (a["hidden"], a["h_scale"], a["weight"], a["w_scale"], a["dhidden"], a["dh_scale"], a["dweight"],
            a["dw_scale"], a["tokens"], a["uniforms"], a["T"], a["B"], a["k"], a["V"], a["d"], a["acc"],
            a["out"], a["gap"], a["tprob"], a["dprob"], a["ws"], a["ws_bytes"], None)
    rc = tv.lib().spec_verify_lmhead_sample(*args)
    assert rc == code, binding.last_error()
    assert binding.last_error()
    ev = (ctypes.c_void_p * 4)(None, None, None, None)
    rc = tv.lib().spec_verify_lmhead_sample_timed(*args, ctypes.cast(ev, ctypes.c_void_p))
    assert rc in (code, -1)
    assert tv.lib().spec_verify_lmhead_sample_packed(*args, None) == code


def test_noalloc_rejects_sizes_beyond_its_scratch_on_the_host():
    # the size check comes before any HIP call, so it runs without a GPU
    need = tv.workspace_size(8192, 4, 151936, 1, 0)
    assert need > (16 << 20)
    rc = tv.lib().spec_verify_noalloc(FAKE, FAKE, FAKE, FAKE, 1.0, 0, 8192, 4, 151936, 1, FAKE, FAKE, FAKE,
                                      None, None, None)
    assert rc == -6 and "scratch" in binding.last_error()
