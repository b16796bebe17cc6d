"""The LM heads in the tile-major layout (pack_lmhead, spec_lmhead_pack and the
*_packed entry points of include/spec_verify.h) against the row-major calls.

The layout only moves the head's bytes; the kernels form the same exact int32
sums and the same epilogues, so every output must be bit-identical to the
row-major call on the same inputs (which the other LM-head tests check against
the oracle). The packed bytes themselves are checked against the layout's
definition, written out here in numpy.
"""
import sys

import numpy as np
import pytest
import torch

import token_verification_amd as tv
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def layout_ref(w: np.ndarray) -> np.ndarray:
    # vocabulary tile vt (256 rows, zeros past V), 64 bytes of d per block:
    # row r at 64 r, physical 16-byte chunk p holding chunk p ^ ((r >> 2) & 3)
    V, d = w.shape
    nvt = (V + 255) // 256
    wp = np.zeros((nvt * 256, d), np.int8)
    wp[:V] = w
    t = wp.reshape(nvt, 256, d // 64, 4, 16)               # [vt, r, ks, logical chunk, byte]
    r = np.arange(256)[:, None]
    logical = np.arange(4)[None, :] ^ ((r >> 2) & 3)       # [r, p]
    out = t[:, r, :, logical, :]                           # [r, p, vt, ks, byte]
    return out.transpose(2, 3, 0, 1, 4).reshape(-1)        # [vt, ks, r, p, byte]


@pytest.mark.parametrize("V,d", [(600, 256), (257, 128), (1, 512)])
def test_pack_layout(V, d):
    g = torch.Generator().manual_seed(V + d)
    w = torch.randint(-128, 128, (V, d), generator=g, dtype=torch.int8)
    p = tv.pack_lmhead(w.to(DEV))
    torch.cuda.synchronize()
    assert p.V == V and p.d == d
    assert np.array_equal(p.data.cpu().numpy(), layout_ref(w.numpy()))


def same(a, b):
    for x, y in zip(a, b):
        if x is None or y is None:
            assert x is None and y is None
        else:
            assert torch.equal(x.view(torch.int32), y.view(torch.int32))


@pytest.mark.parametrize("B,k,V,d", [
    (1, 4, 1000, 512),          # 32-row tiles (the tile-major call keeps 64-byte stages)
    (10, 4, 3000, 256),         # one 128-row tile
    (96, 3, 3000, 640),         # 192-row tiles
    (64, 3, 2000, 256),         # 256-row tiles
    (1, 4, 128256, 4096),       # a full-size head, one batch row
])
def test_packed_greedy_equals_row_major(B, k, V, d):
    say("packed greedy", B, k, V, d)
    x = workloads.make_lmhead(B, k, V, d, seed=7, device=DEV)
    a = (x["hidden"], x["hidden_scale"], x["weight"], x["weight_scale"], x["tokens"])
    r0 = tv.spec_verify_lmhead(*a)
    p = tv.pack_lmhead(x["weight"])
    r1 = tv.spec_verify_lmhead(a[0], a[1], p, a[3], a[4])
    torch.cuda.synchronize()
    same(r0, r1)


@pytest.mark.parametrize("B,k,V,d,own", [
    (1, 4, 1000, 512, False),   # 9 rows in one pass: a 32-row tile
    (3, 2, 700, 256, True),     # separate heads, partial vocabulary tile
    (50, 3, 5000, 512, False),  # 350 rows in one pass: 256-row tiles
    (160, 3, 3000, 640, True),  # 640 / 480 rows: 128- and 256-row tiles
    (1, 4, 128256, 4096, False),
])
def test_packed_sample_equals_row_major(B, k, V, d, own):
    say("packed sample", B, k, V, d, own)
    x = workloads.make_lmhead_sample(B, k, V, d, seed=7, device=DEV, draft_head=own)

    def call(w, dw):
        return tv.spec_verify_lmhead_sample(x["hidden"], x["hidden_scale"], w, x["weight_scale"],
                                            x["draft_hidden"], x["draft_hidden_scale"], x["tokens"],
                                            x["uniforms"], 0.8, draft_weight=dw,
                                            draft_weight_scale=x["draft_weight_scale"])
    r0 = call(x["weight"], x["draft_weight"])
    pw = tv.pack_lmhead(x["weight"])
    pd = None if x["draft_weight"] is None else tv.pack_lmhead(x["draft_weight"])
    r1 = call(pw, pd)
    torch.cuda.synchronize()
    same(r0, r1)


def test_packed_rejects_mixed_heads():
    x = workloads.make_lmhead_sample(2, 2, 300, 256, seed=1, device=DEV, draft_head=True)
    with pytest.raises(ValueError):
        tv.spec_verify_lmhead_sample(x["hidden"], x["hidden_scale"], tv.pack_lmhead(x["weight"]),
                                     x["weight_scale"], x["draft_hidden"], x["draft_hidden_scale"], x["tokens"],
                                     x["uniforms"], 1.0, draft_weight=x["draft_weight"],
                                     draft_weight_scale=x["draft_weight_scale"])
