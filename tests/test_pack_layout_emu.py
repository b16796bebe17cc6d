"""The tile-major head layout (spec_lmhead_pack) on the CPU: the library's
pack kernel, run through the emulation harness (tests/emu), against the
layout's definition written out in numpy (the same reference the GPU test
uses, tests/test_lmhead_packed_gpu.py)."""
import ctypes
import os
import subprocess

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
EMU = os.path.join(HERE, "emu")
ROOT = os.path.dirname(HERE)
CLANG = "/opt/rocm/llvm/bin/clang++"


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


def test_layout_ref_by_loops():
    # the vectorised reference against the definition taken element by element
    rng = np.random.default_rng(0)
    V, d = 300, 128
    w = rng.integers(-128, 128, (V, d)).astype(np.int8)
    ref = np.zeros(512 * d, np.int8)
    for vt in range(2):
        for ks in range(d // 64):
            for r in range(256):
                for p in range(4):
                    c, v = p ^ ((r >> 2) & 3), vt * 256 + r
                    o = ((vt * (d // 64) + ks) * 256 + r) * 64 + 16 * p
                    if v < V:
                        ref[o:o + 16] = w[v, ks * 64 + 16 * c:ks * 64 + 16 * c + 16]
    assert np.array_equal(layout_ref(w), ref)


@pytest.fixture(scope="module")
def emu():
    out = os.path.join(EMU, "libspecverify_emu_pack.so")
    subprocess.run([CLANG, "-std=c++17", "-O1", "-fPIC", "-shared", "-I", EMU, "-I", os.path.join(ROOT, "include"),
                    "-Wno-unknown-pragmas", "-Wno-pass-failed", "-Wno-psabi", "-o", out,
                    os.path.join(EMU, "spec_verify_emu.cpp"), "-lpthread"], check=True)
    L = ctypes.CDLL(out)
    L.spec_lmhead_packed_size.argtypes = [ctypes.c_int32, ctypes.c_int32]
    L.spec_lmhead_packed_size.restype = ctypes.c_size_t
    L.spec_lmhead_pack.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                   ctypes.c_size_t, ctypes.c_void_p]
    L.spec_lmhead_pack.restype = ctypes.c_int
    return L


@pytest.mark.parametrize("V,d", [(600, 256), (257, 128), (1, 512), (256, 384)])
def test_pack_kernel_matches_layout(emu, V, d):
    rng = np.random.default_rng(V + d)
    w = rng.integers(-128, 128, (V, d)).astype(np.int8)
    n = emu.spec_lmhead_packed_size(V, d)
    assert n == (V + 255) // 256 * 256 * d
    buf = np.frombuffer(os.urandom(n + 16), np.uint8).copy()      # garbage where nothing is written
    o = (-buf.ctypes.data) % 16
    out = buf[o:o + n]
    assert emu.spec_lmhead_pack(w.ctypes.data, V, d, out.ctypes.data, n, None) == 0
    assert np.array_equal(out.view(np.int8), layout_ref(w))
