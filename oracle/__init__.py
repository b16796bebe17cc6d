"""fp64 CPU oracle of the speculative-decoding verify step.

TEST INFRASTRUCTURE ONLY: only the tests, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import this package. The product path (the
HIP library and its binding) never imports, links or calls it, and it shares
no code with them.

The arithmetic lives in ``spec_verify_ref.c`` (plain C, double precision,
Neumaier sums); this module builds it with gcc and wraps it with ctypes on
host numpy arrays. ``exact_enum`` holds the small exact-enumeration checker.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
(closed forms, hand-worked examples, exact enumeration, a chi-square test and
the accept-length law). The specific token chosen at a given uniform is fixed
by the inverse-CDF convention, which the pages do not print an example of; it
is pinned against ``numpy.searchsorted`` on the cumulative sum.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "spec_verify_ref.c")
_LIB = os.path.join(_HERE, "libspecverify_ref.so")

F32, BF16 = 0, 1
SAMPLE, GREEDY = 0, 1

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (OpenMP, strict IEEE double arithmetic)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
               "-fno-fast-math", "-ffp-contract=off", "-Wall", "-Wextra", "-Werror",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        lib.spec_verify_ref.argtypes = [P, P, P, P, ctypes.c_float, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        P, P, P, P, P, P, P, P, ctypes.c_int]
        lib.spec_verify_ref.restype = ctypes.c_int
        lib.spec_verify_ref_ragged.argtypes = [P, P, P, P, P, ctypes.c_float, ctypes.c_int,
                                               ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                               P, P, P, P, P, P, P, P, ctypes.c_int]
        lib.spec_verify_ref_ragged.restype = ctypes.c_int
        lib.spec_verify_ref_full.argtypes = [P, P, P, P, P, ctypes.c_float, ctypes.c_int,
                                             ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                             P, P, P, P, P, P, P, P, ctypes.c_double, P, P, P, ctypes.c_int]
        lib.spec_verify_ref_full.restype = ctypes.c_int
        lib.spec_verify_ref_max_threads.restype = ctypes.c_int
        lib.spec_gate_ref.argtypes = [P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_float, P, P, P, P]
        lib.spec_gate_ref.restype = ctypes.c_int
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().spec_verify_ref_max_threads())


@dataclass
class RefResult:
    accepted_len: np.ndarray   # [B] int32
    out_tokens: np.ndarray     # [B,k+1] int32
    gap: np.ndarray            # [B,k+1] float64
    p_tok: np.ndarray          # [B,k] float64 (NaN in greedy mode / invalid rows)
    q_tok: np.ndarray          # [B,k] float64
    margin_acc: np.ndarray     # [B] float64, +inf where no test was taken
    margin_cdf: np.ndarray     # [B] float64, +inf where no draw was taken
    flags: np.ndarray          # [B] int32, bit 0: residual mass was zero; bit 1: the
                               # residual draw is within 1e-13 (of p's total mass) of a
                               # CDF boundary, below what fp64 resolves
    # Alternatives (only with flip_delta > 0; else None): the outcome with the
    # acceptance test nearest its boundary decided the other way (rows whose
    # smallest margin is below flip_delta; other rows repeat the outcome), and
    # the token the final draw gives with its uniform across the nearest CDF
    # edge.
    alt_accepted_len: Optional[np.ndarray] = None   # [B] int32
    alt_out_tokens: Optional[np.ndarray] = None     # [B,k+1] int32
    alt_token: Optional[np.ndarray] = None          # [B] int32

    def flagged(self, delta_acc: float, delta_cdf: float) -> np.ndarray:
        return (self.margin_acc < delta_acc) | (self.margin_cdf < delta_cdf) | (self.flags != 0)


def _as_logits(x, dtype: int) -> np.ndarray:
    """Accept float32 arrays, uint16 bf16 bit patterns, or torch tensors."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().contiguous()
            if x.dtype == torch.bfloat16:
                x = x.view(torch.int16).numpy().view(np.uint16)
            else:
                x = x.numpy()
    except ImportError:  # pragma: no cover
        pass
    x = np.ascontiguousarray(x)
    if dtype == F32:
        assert x.dtype == np.float32, x.dtype
    else:
        assert x.dtype == np.uint16, x.dtype
    return x


def _np(x, dt):
    if x is None:
        return None
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().contiguous().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(x, dtype=dt)


def spec_verify_ref(target, draft, tokens, uniforms, temperature: float, mode: int,
                    dtype: Optional[int] = None, threads: int = 0, draft_len=None,
                    flip_delta: float = 0.0) -> RefResult:
    """Run the oracle on host arrays shaped [B,k+1,V], [B,k,V], [B,k], [B,k+1,2].

    draft_len: optional [B] int32, the number of draft positions each batch row
    verifies (ragged drafts; None means k for every row). flip_delta > 0 also
    returns the alternative outcomes of near-tie rows (see RefResult).
    """
    if dtype is None:
        dtype = BF16 if str(getattr(target, "dtype", "")) in ("torch.bfloat16", "uint16") else F32
    tgt = _as_logits(target, dtype)
    B, k1, V = tgt.shape
    k = k1 - 1
    dft = _as_logits(draft, dtype) if draft is not None else None
    if dft is not None:
        assert dft.shape == (B, k, V), dft.shape
    tok = _np(tokens, np.int32)
    if tok is None:
        tok = np.zeros((B, k), np.int32)
    assert tok.shape == (B, k), tok.shape
    uni = _np(uniforms, np.float32)
    if uni is not None:
        assert uni.shape == (B, k + 1, 2), uni.shape

    acc = np.zeros(B, np.int32)
    out = np.zeros((B, k + 1), np.int32)
    gap = np.zeros((B, k + 1), np.float64)
    pt = np.zeros((B, k), np.float64)
    qt = np.zeros((B, k), np.float64)
    ma = np.zeros(B, np.float64)
    mc = np.zeros(B, np.float64)
    fl = np.zeros(B, np.int32)

    def ptr(a):
        return None if a is None else a.ctypes.data_as(ctypes.c_void_p)

    dl = _np(draft_len, np.int32)
    if dl is not None:
        assert dl.shape == (B,), dl.shape
    alts = flip_delta > 0
    aa = np.zeros(B, np.int32) if alts else None
    ao = np.zeros((B, k + 1), np.int32) if alts else None
    at = np.zeros(B, np.int32) if alts else None
    rc = _load().spec_verify_ref_full(ptr(tgt), ptr(dft), ptr(tok), ptr(dl), ptr(uni),
                                      ctypes.c_float(temperature), int(mode), int(B), int(k),
                                      int(V), int(dtype), ptr(acc), ptr(out), ptr(gap), ptr(pt),
                                      ptr(qt), ptr(ma), ptr(mc), ptr(fl), float(flip_delta),
                                      ptr(aa), ptr(ao), ptr(at), int(threads))
    if rc != 0:
        raise ValueError(f"spec_verify_ref rejected its arguments (rc={rc})")
    return RefResult(acc, out, gap, pt, qt, ma, mc, fl, aa, ao, at)


MARGIN, CERTIFIED = 0, 1


@dataclass
class GateResult:
    argmax: np.ndarray    # [n] int32, -1 for an invalid row
    gap: np.ndarray       # [n] float64 (NaN for an invalid row)
    fire: np.ndarray      # [n] bool


def spec_gate_ref(logits, rule: int, tau: float, admit=None, dtype: Optional[int] = None) -> GateResult:
    """Confidence gate over ready distributions logits [n, V] (float32 or bf16).

    admit: optional uint32 [(V + 31) // 32] bit mask of admissible tokens.
    """
    if dtype is None:
        dtype = BF16 if str(getattr(logits, "dtype", "")) in ("torch.bfloat16", "uint16") else F32
    x = _as_logits(logits, dtype)
    n, V = x.shape
    am = _np(admit, np.uint32)
    if am is not None:
        assert am.shape == ((V + 31) // 32,), am.shape
    arg = np.zeros(n, np.int32)
    gap = np.zeros(n, np.float64)
    fire = np.zeros(n, np.int32)

    def ptr(a):
        return None if a is None else a.ctypes.data_as(ctypes.c_void_p)

    rc = _load().spec_gate_ref(ptr(x), int(n), int(V), int(dtype), int(rule), ctypes.c_float(tau),
                               ptr(am), ptr(arg), ptr(gap), ptr(fire))
    if rc != 0:
        raise ValueError(f"spec_gate_ref rejected its arguments (rc={rc})")
    return GateResult(arg, gap, fire.astype(bool))


def admit_mask(tokens, V: int) -> np.ndarray:
    """The V-bit admissible-set mask of a list of token ids."""
    m = np.zeros((V + 31) // 32, np.uint32)
    for t in tokens:
        m[int(t) >> 5] |= np.uint32(1) << np.uint32(int(t) & 31)
    return m
