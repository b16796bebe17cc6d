"""Run the CPU-emulated HIP library on host inputs and compare with the oracle.

TEST INFRASTRUCTURE ONLY. Invoked in a subprocess with the sanitizer runtime
preloaded (see tests/test_emulation.py). Usage: run_emu.py <case> [<case> ...]
"""
import ctypes
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.dirname(HERE))

import torch  # noqa: E402

import oracle  # noqa: E402
import workloads  # noqa: E402
from parity import DELTA_ACC, DELTA_CDF  # noqa: E402

L = ctypes.CDLL(os.path.join(HERE, os.environ.get("SPEC_EMU_LIB", "libspecverify_emu.so")))
P, I, F, S = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
L.spec_verify.argtypes = [P, P, P, P, F, ctypes.c_int, I, I, I, ctypes.c_int, P, P, P, P, P, P, S, P]
L.spec_verify.restype = ctypes.c_int
L.spec_verify_ragged.argtypes = [P, P, P, P, P, F, ctypes.c_int, I, I, I, ctypes.c_int, P, P, P, P, P, P, S, P]
L.spec_verify_ragged.restype = ctypes.c_int
L.spec_verify_workspace_size.argtypes = [I, I, I, ctypes.c_int, ctypes.c_int]
L.spec_verify_workspace_size.restype = S
L.spec_verify_last_error.restype = ctypes.c_char_p
L.spec_gate.argtypes = [P, I, I, ctypes.c_int, ctypes.c_int, F, P, P, P, P, P, S, P]
L.spec_gate.restype = ctypes.c_int
L.spec_gate_workspace_size.argtypes = [I, I, ctypes.c_int]
L.spec_gate_workspace_size.restype = S
L.spec_commit.argtypes = [P, I, I, P, P, P, S, P]
L.spec_commit.restype = ctypes.c_int
L.spec_verify_lmhead.argtypes = [P, P, P, P, P, I, I, I, I, P, P, P, P, S, P]
L.spec_verify_lmhead.restype = ctypes.c_int
L.spec_lmhead_workspace_size.argtypes = [I, I, I, I]
L.spec_lmhead_workspace_size.restype = S
L.spec_verify_emu_set_cu_count.argtypes = [ctypes.c_int]
L.spec_verify_emu_set_pool.argtypes = [ctypes.c_int]



def host(x, dtype):
    if x is None:
        return None
    if isinstance(x, torch.Tensor):
        if x.dtype == torch.bfloat16:
            return np.ascontiguousarray(x.view(torch.int16).numpy().view(np.uint16))
        return np.ascontiguousarray(x.numpy())
    return np.ascontiguousarray(x)


def ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def run_case(x, cus=1, ws_reuse=None, pool=1):
    tgt = x["target"]
    dtype = 1 if tgt.dtype == torch.bfloat16 else 0
    B, k1, V = tgt.shape
    k = k1 - 1
    mode = x["mode"]
    t = host(tgt, dtype)
    d = host(x["draft"], dtype)
    tok = host(x["tokens"], None).astype(np.int32)
    u = host(x["uniforms"], None)
    acc = np.full(B, -7, np.int32)
    out = np.full((B, k + 1), -7, np.int32)
    gap = np.zeros((B, k + 1), np.float32)
    tp = np.zeros((B, k), np.float32)
    dp = np.zeros((B, k), np.float32)
    n = L.spec_verify_workspace_size(B, k, V, dtype, mode)
    # uninitialised workspace: every record must be written before it is read
    ws = ws_reuse if ws_reuse is not None else np.frombuffer(os.urandom(n + 256), np.uint8).copy()
    base = ws.ctypes.data
    off = (-base) % 256
    L.spec_verify_emu_set_cu_count(cus)
    L.spec_verify_emu_set_pool(pool)
    dl = x.get("draft_len")
    dlh = None if dl is None else np.ascontiguousarray(np.asarray(dl, np.int32))

    def call(acc, out, gap, tp, dp):
        if dlh is None:
            return L.spec_verify(ptr(t), ptr(d), ptr(tok), ptr(u), ctypes.c_float(x["T"]), mode, B, k, V, dtype,
                                 ptr(acc), ptr(out), ptr(gap), ptr(tp), ptr(dp), ctypes.c_void_p(base + off), n,
                                 None)
        return L.spec_verify_ragged(ptr(t), ptr(d), ptr(tok), ptr(dlh), ptr(u), ctypes.c_float(x["T"]), mode, B,
                                    k, V, dtype, ptr(acc), ptr(out), ptr(gap), ptr(tp), ptr(dp),
                                    ctypes.c_void_p(base + off), n, None)

    rc = call(acc, out, gap, tp if mode == 0 else None, dp if mode == 0 else None)
    assert rc == 0, (rc, L.spec_verify_last_error())
    # a second call on the same workspace must reproduce the first bit for bit
    acc2, out2, gap2 = acc.copy(), out.copy(), gap.copy()
    rc = call(acc2, out2, gap2, None, None)
    assert rc == 0
    assert (acc2 == acc).all() and (out2 == out).all() and (gap2.view(np.uint32) == gap.view(np.uint32)).all()
    ref = oracle.spec_verify_ref(x["target"], x["draft"], x["tokens"], x["uniforms"], x["T"], mode,
                                 draft_len=dlh)
    flagged = ref.flagged(DELTA_ACC, DELTA_CDF) if mode == 0 else np.zeros(B, bool)
    same = (acc == ref.accepted_len) & (out == ref.out_tokens).all(axis=1)
    bad = ~same & ~flagged
    assert not bad.any(), (np.nonzero(bad)[0][:5], acc[bad][:3], ref.accepted_len[bad][:3],
                           out[bad][:3], ref.out_tokens[bad][:3])
    valid = ref.accepted_len >= 0
    g = gap.astype(np.float64)[valid]
    r = ref.gap[valid]
    fin = np.isfinite(r)
    assert (np.isfinite(g) == fin).all()
    assert np.abs(g[fin] - r[fin]).max(initial=0) <= (1e-5 if dtype == 0 else 2e-3)
    if mode == 0 and k > 0:
        for gg, rr in ((tp, ref.p_tok), (dp, ref.q_tok)):
            gg = gg.astype(np.float64)[valid]
            rr = rr[valid]
            assert (np.isnan(gg) == np.isnan(rr)).all()
            assert np.abs(gg - rr)[~np.isnan(rr)].max(initial=0) <= 1e-5
    if dlh is not None:
        # draft lengths outside [0, k]: invalid, every gap NaN
        bad_len = (dlh < 0) | (dlh > k)
        assert (acc[bad_len] == -1).all() and np.isnan(gap[bad_len]).all()
        # rows past kb: NaN gaps
        past = np.arange(k + 1)[None, :] > dlh[:, None]
        assert np.isnan(gap[past & valid[:, None]]).all()
    return int(flagged.sum())


def rand_case(rng, B, k, V, dtype, T, mode=0, coarse=False):
    t = torch.from_numpy(rng.normal(0, 2.0, (B, k + 1, V)).astype(np.float32))
    if coarse:
        t = torch.round(t * 2) / 2
    d = t[:, :k] + torch.from_numpy(rng.normal(0, 1.0, (B, k, V)).astype(np.float32))
    td = torch.float32 if dtype == 0 else torch.bfloat16
    tok = torch.from_numpy(rng.integers(0, V, (B, k)).astype(np.int32))
    if mode == 1:
        am = torch.argmax(t.to(td).float(), dim=2)[:, :k].to(torch.int32)
        keep = torch.from_numpy(rng.random((B, k)) < 0.7)
        tok = torch.where(keep, am, tok)
    uni = torch.from_numpy(rng.random((B, k + 1, 2)).astype(np.float32))
    return {"target": t.to(td), "draft": None if mode == 1 else d.to(td), "tokens": tok,
            "uniforms": None if mode == 1 else uni, "T": T, "mode": mode}


CASES = {}


def case(fn):
    CASES[fn.__name__] = fn
    return fn


@case
def smoke_b8():
    w = workloads.WORKLOADS["b8_k5_v32000_f32"]
    run_case(workloads.make(w, 0), cus=1)
    run_case(workloads.make(w, 1), cus=3)


@case
def concurrent_b8():
    # the real launch shape of this workload on 256 CUs: 680 workers, 8 at a time
    w = workloads.WORKLOADS["b8_k5_v32000_f32"]
    run_case(workloads.make(w, 0), cus=256, pool=8)


@case
def smoke_b1():
    w = workloads.WORKLOADS["b1_k4_v1000_f32"]
    for s in range(5):
        run_case(workloads.make(w, s))


@case
def odd_shapes():
    rng = np.random.default_rng(1)
    for dtype in (0, 1):
        for V in (1, 2, 3, 7, 9, 63, 65, 1001, 4097, 9001):
            for k, T in ((0, 1.0), (1, 0.05), (3, 7.0)):
                run_case(rand_case(rng, 3, k, V, dtype, T))
            for k in (0, 2):
                run_case(rand_case(rng, 3, k, V, dtype, 1.0, mode=1, coarse=True))


@case
def masks_large_k():
    # -inf entries (probability 0) in half of every row, k at its maximum
    rng = np.random.default_rng(4)
    for dtype, T in ((0, 0.9), (1, 1.3), (1, 1.0)):
        x = rand_case(rng, 3, 64, 300, dtype, T)
        for key in ("target", "draft"):
            t = x[key].float()
            m = torch.from_numpy(rng.random(tuple(t.shape)) < 0.5)
            t[m] = -float("inf")
            t[:, :, 0] = 0.0
            x[key] = t.to(x[key].dtype)
        run_case(x, cus=2)


@case
def bf16_long_rows():
    # bf16 rows long enough that each pass-2 wave loads several groups of
    # vectors (one CU: one workgroup per batch row), aligned and unaligned rows
    rng = np.random.default_rng(5)
    for V in (60000, 60001):
        run_case(rand_case(rng, 8, 2, V, 1, 1.0), cus=1)


@case
def ragged():
    # per-row draft lengths 0..k, with two out-of-range lengths; sampling and
    # greedy, one wave deciding (rpb <= 64) and one workgroup (k = 40)
    rng = np.random.default_rng(6)
    for dtype, k, V, mode, cus in ((0, 5, 3001, 0, 2), (1, 5, 4100, 0, 1), (1, 4, 2000, 1, 2),
                                   (0, 40, 97, 0, 1), (1, 40, 130, 1, 1)):
        B = 9
        x = rand_case(rng, B, k, V, dtype, 1.1, mode=mode, coarse=mode == 1)
        dl = rng.integers(0, k + 1, B).astype(np.int32)
        dl[2], dl[5] = -1, k + 1
        dl[0], dl[1] = 0, k
        x["draft_len"] = dl
        run_case(x, cus=cus)
    # more batch rows than one chunk of the row-packing scan (greedy: no pass 2)
    x = rand_case(rng, 1100, 2, 5, 0, 1.0, mode=1, coarse=True)
    x["draft_len"] = rng.integers(-1, 4, 1100).astype(np.int32)
    run_case(x, cus=4)


def run_gate(x, rule, tau, admit=None, cus=1):
    dtype = 1 if x.dtype == torch.bfloat16 else 0
    n, V = x.shape
    h = host(x, dtype)
    am = None if admit is None else np.ascontiguousarray(np.asarray(admit).view(np.uint32))
    arg = np.full(n, -7, np.int32)
    gap = np.zeros(n, np.float32)
    fire = np.full(n, -7, np.int32)
    nb = L.spec_gate_workspace_size(n, V, dtype)
    ws = np.frombuffer(os.urandom(nb + 256), np.uint8).copy()
    base = ws.ctypes.data
    off = (-base) % 256
    L.spec_verify_emu_set_cu_count(cus)
    L.spec_verify_emu_set_pool(1)
    rc = L.spec_gate(ptr(h), n, V, dtype, rule, ctypes.c_float(tau), ptr(am), ptr(arg), ptr(gap), ptr(fire),
                     ctypes.c_void_p(base + off), nb, None)
    assert rc == 0, (rc, L.spec_verify_last_error())
    ref = oracle.spec_gate_ref(x, rule, tau, am)
    assert (arg == ref.argmax).all(), (np.nonzero(arg != ref.argmax)[0][:5])
    assert (fire.astype(bool) == ref.fire).all()
    assert (np.isnan(gap) == np.isnan(ref.gap)).all()
    ok = ~np.isnan(ref.gap)
    assert (gap[ok] == ref.gap[ok].astype(np.float32)).all()


@case
def gate():
    # the confidence gate: seeded ready distributions, both rules, with and
    # without an admissible set, plus ties, single finite entries and invalid rows
    rng = np.random.default_rng(8)
    for dtype, n, V, cus in (("bf16", 1, 50000, 2), ("f32", 40, 3001, 2), ("bf16", 300, 97, 1)):
        x, A = workloads.make_gate(n, V, 1, dtype)
        x = x.clone()
        if n >= 40:
            x[0, :] = -float("inf")
            x[1, 5] = float("nan")
            x[2, :] = 1.0                      # all tied
            x[3, :] = -float("inf")
            x[3, 7] = 2.0                      # one finite entry
            x[4, 3] = float("inf")
        am = workloads.admit_bits(A, V).numpy()
        for rule, tau in ((0, 2.0), (0, -1.0), (1, 0.75), (1, 0.0)):
            run_gate(x, rule, tau, am, cus=cus)
            run_gate(x, rule, tau, None, cus=cus)
    del rng


@case
def commit():
    # commit / rollback: 16-byte and 4-byte copies, several chunks per row,
    # invalid and out-of-range accepted lengths, no KV lengths, no state
    from oracle.commit import commit_ref
    rng = np.random.default_rng(9)
    L.spec_verify_emu_set_cu_count(2)
    L.spec_verify_emu_set_pool(1)
    for B, k, words in ((5, 3, 3 * 8192 + 100), (7, 0, 333), (4, 5, 0), (3, 2, 4096)):
        acc = rng.integers(-1, k + 2, B).astype(np.int32)
        acc[0] = k
        kv = rng.integers(0, 1000, B).astype(np.int32)
        slots = rng.integers(0, 2 ** 31, (B, k + 1, words)).astype(np.int32)
        state = rng.integers(0, 2 ** 31, (B, words)).astype(np.int32)
        ref_kv, ref_state = commit_ref(acc, kv, slots, state, k=k)
        kv2, st2 = kv.copy(), state.copy()
        rc = L.spec_commit(ptr(acc), B, k, ptr(kv2), ptr(slots) if words else None,
                           ptr(st2) if words else None, 4 * words, None)
        assert rc == 0, L.spec_verify_last_error()
        assert (kv2 == ref_kv).all() and (st2 == ref_state).all()
        kv3 = kv.copy()
        assert L.spec_commit(ptr(acc), B, k, ptr(kv3), None, None, 0, None) == 0
        assert (kv3 == ref_kv).all()


@case
def greedy_bf16():
    rng = np.random.default_rng(2)
    run_case(rand_case(rng, 6, 3, 20000, 1, 1.0, mode=1, coarse=True), cus=2)


@case
def exact_path():
    os.environ["SPEC_VERIFY_FORCE_EXACT_PATH"] = "1"
    rng = np.random.default_rng(3)
    run_case(rand_case(rng, 4, 3, 9000, 0, 0.9))
    del os.environ["SPEC_VERIFY_FORCE_EXACT_PATH"]


def pack_head(w, V, d):
    """The tile-major copy of a head, written by the library's pack kernel
    (kept referenced by the caller while the library reads it)."""
    L.spec_lmhead_packed_size.argtypes = [I, I]
    L.spec_lmhead_packed_size.restype = S
    L.spec_lmhead_pack.argtypes = [P, I, I, P, S, P]
    L.spec_lmhead_pack.restype = ctypes.c_int
    n = L.spec_lmhead_packed_size(V, d)
    buf = np.frombuffer(os.urandom(n + 16), np.uint8).copy()
    o = (-buf.ctypes.data) % 16
    view = buf[o:o + n]
    assert L.spec_lmhead_pack(ptr(w), V, d, ptr(view), n, None) == 0, L.spec_verify_last_error()
    return view


def run_lmhead(x, pool=1, packed=False):
    from oracle.lmhead import lmhead_greedy_ref
    B, k, V, d = x["B"], x["k"], x["V"], x["d"]
    h, hs, w, ws = (np.ascontiguousarray(x[n].numpy()) for n in ("hidden", "hidden_scale", "weight", "weight_scale"))
    tok = np.ascontiguousarray(x["tokens"].numpy().astype(np.int32))
    acc = np.full(B, -7, np.int32)
    out = np.full((B, k + 1), -7, np.int32)
    gap = np.zeros((B, k + 1), np.float32)
    nb = L.spec_lmhead_workspace_size(B, k, V, d)
    assert nb > 0
    wsp = np.frombuffer(os.urandom(nb + 256), np.uint8).copy()
    base = wsp.ctypes.data
    off = (-base) % 256
    L.spec_verify_emu_set_pool(pool)
    if packed:
        L.spec_verify_lmhead_packed.argtypes = [P, P, P, P, P, I, I, I, I, P, P, P, P, S, P, P]
        L.spec_verify_lmhead_packed.restype = ctypes.c_int
        pw = pack_head(w, V, d)
        rc = L.spec_verify_lmhead_packed(ptr(h), ptr(hs), ptr(pw), ptr(ws), ptr(tok), B, k, V, d, ptr(acc),
                                         ptr(out), ptr(gap), ctypes.c_void_p(base + off), nb, None, None)
    else:
        rc = L.spec_verify_lmhead(ptr(h), ptr(hs), ptr(w), ptr(ws), ptr(tok), B, k, V, d, ptr(acc), ptr(out),
                                  ptr(gap), ctypes.c_void_p(base + off), nb, None)
    assert rc == 0, (rc, L.spec_verify_last_error())
    ref = lmhead_greedy_ref(h, hs, w, ws, tok, B, k)
    assert (acc == ref.accepted_len).all(), (acc, ref.accepted_len)
    assert (out == ref.out_tokens).all()
    valid = ref.accepted_len >= 0                           # gaps are compared on valid rows
    g, r = gap.astype(np.float64)[valid], ref.gap[valid]
    assert (np.isnan(g) == np.isnan(r)).all() and (np.isinf(g) == np.isinf(r)).all()
    fin = np.isfinite(r)
    assert np.abs(g[fin] - r[fin]).max(initial=0.0) <= 1e-5
    return acc


@case
def lmhead():
    # int8 LM head fused with greedy verification: partial vocabulary and
    # hidden-row tiles, several LDS stages, k = 0, NaN / inf scales, a token
    # outside [0, V), ties at the top
    # then 16 and 18 tiles of 256 rows (one hidden tile ragged), 32-row tiles
    # with 512-byte stages (d = 512, 1536), and 50 and 48 rows in a 128-row
    # tile (d = 512, 768)
    for B, k, V, d, pool in ((3, 2, 700, 256, 1), (50, 3, 300, 128, 2), (4, 0, 257, 128, 1), (64, 3, 600, 256, 2),
                             (48, 3, 500, 128, 2), (64, 3, 4000, 128, 2), (125, 3, 2100, 256, 2),
                             (3, 2, 700, 512, 1), (2, 5, 1300, 1536, 2), (10, 4, 1300, 512, 2),
                             (12, 3, 900, 768, 1), (2, 3, 1, 512, 1), (3, 1, 255, 1024, 2)):
        x = workloads.make_lmhead(B, k, V, d, seed=1)
        if B >= 50:
            x["hidden_scale"][0] = float("nan")            # batch row 0: NaN logits
            x["hidden_scale"][5] = float("inf")            # batch row 1: +-inf / NaN logits
            x["tokens"][2, 1] = V                          # batch row 2: token out of range
            x["hidden"][12:16] = 0                         # batch row 3: all logits 0, a tie at 0
            x["tokens"][3, :] = 0
        acc = run_lmhead(x, pool=pool)
        if d in (256, 512) and V > 1:                       # the same through the tile-major layout
            assert (run_lmhead(x, pool=pool, packed=True) == acc).all()
        if B >= 50:
            assert acc[0] == -1 and acc[1] == -1 and acc[2] == -1 and acc[3] == 3


def run_lmhead_sample(x, T, pool=1, packed=False):
    # set here, not at import: libraries built from older sources lack the symbol
    from oracle.lmhead import lmhead_sample_ref
    L.spec_verify_lmhead_sample.argtypes = [P, P, P, P, P, P, P, P, P, P, F, I, I, I, I, P, P, P, P, P, P, S, P]
    L.spec_verify_lmhead_sample.restype = ctypes.c_int
    L.spec_lmhead_sample_workspace_size.argtypes = [I, I, I, I]
    L.spec_lmhead_sample_workspace_size.restype = S
    B, k, V, d = x["B"], x["k"], x["V"], x["d"]
    arr = {n: (None if x[n] is None else np.ascontiguousarray(x[n].numpy()))
           for n in ("hidden", "hidden_scale", "weight", "weight_scale", "draft_hidden", "draft_hidden_scale",
                     "draft_weight", "draft_weight_scale", "uniforms")}
    tok = np.ascontiguousarray(x["tokens"].numpy().astype(np.int32))
    acc = np.full(B, -7, np.int32)
    out = np.full((B, k + 1), -7, np.int32)
    gap = np.zeros((B, k + 1), np.float32)
    tp = np.zeros((B, k), np.float32)
    dp = np.zeros((B, k), np.float32)
    nb = L.spec_lmhead_sample_workspace_size(B, k, V, d)
    assert nb > 0
    wsp = np.frombuffer(os.urandom(nb + 256), np.uint8).copy()
    base = wsp.ctypes.data
    off = (-base) % 256
    L.spec_verify_emu_set_pool(pool)
    wt, wd = arr["weight"], arr["draft_weight"]
    fn = L.spec_verify_lmhead_sample
    tail = ()
    if packed:
        L.spec_verify_lmhead_sample_packed.argtypes = [P, P, P, P, P, P, P, P, P, P, F, I, I, I, I, P, P, P, P, P,
                                                       P, S, P, P]
        L.spec_verify_lmhead_sample_packed.restype = ctypes.c_int
        wt = pack_head(wt, V, d)
        wd = None if wd is None else pack_head(wd, V, d)
        fn, tail = L.spec_verify_lmhead_sample_packed, (None,)
    rc = fn(
        ptr(arr["hidden"]), ptr(arr["hidden_scale"]), ptr(wt), ptr(arr["weight_scale"]),
        ptr(arr["draft_hidden"]), ptr(arr["draft_hidden_scale"]), ptr(wd),
        ptr(arr["draft_weight_scale"]), ptr(tok), ptr(arr["uniforms"]), ctypes.c_float(T), B, k, V, d,
        ptr(acc), ptr(out), ptr(gap), ptr(tp), ptr(dp), ctypes.c_void_p(base + off), nb, None, *tail)
    assert rc == 0, (rc, L.spec_verify_last_error())
    ref = lmhead_sample_ref(arr["hidden"], arr["hidden_scale"], arr["weight"], arr["weight_scale"],
                            arr["draft_hidden"], arr["draft_hidden_scale"], arr["draft_weight"],
                            arr["draft_weight_scale"], tok, arr["uniforms"], T, B, k)
    flagged = ref.flagged(DELTA_ACC, DELTA_CDF)
    same = (acc == ref.accepted_len) & (out == ref.out_tokens).all(axis=1)
    bad = ~same & ~flagged
    assert not bad.any(), (np.nonzero(bad)[0][:5], acc[bad][:3], ref.accepted_len[bad][:3],
                           out[bad][:3], ref.out_tokens[bad][:3])
    valid = ref.accepted_len >= 0
    g, r = gap.astype(np.float64)[valid], ref.gap[valid]
    assert (np.isnan(g) == np.isnan(r)).all() and (np.isinf(g) == np.isinf(r)).all()
    fin = np.isfinite(r)
    assert np.abs(g[fin] - r[fin]).max(initial=0.0) <= 1e-5
    for gg, rr in ((tp, ref.p_tok), (dp, ref.q_tok)):
        gg, rr = gg.astype(np.float64)[valid], rr[valid]
        assert (np.isnan(gg) == np.isnan(rr)).all()
        assert np.abs(gg - rr)[~np.isnan(rr)].max(initial=0) <= 1e-5
    return acc


@case
def lmhead_sample():
    # sampling-mode verify fused with int8 heads: shared and separate draft
    # heads, partial tiles, k = 0, NaN / inf scales, a token outside [0, V);
    # two take 32-row tiles with 512-byte stages, the last two (36 and 42
    # rows in one pass) a 128-row tile
    for B, k, V, d, T, own, pool in ((3, 2, 700, 256, 1.0, False, 1), (50, 3, 300, 128, 0.7, True, 2),
                                     (4, 0, 257, 128, 1.3, False, 1), (48, 3, 500, 128, 1.0, False, 2),
                                     (16, 5, 1500, 384, 0.3, True, 2), (5, 2, 1, 128, 0.7, True, 1),
                                     (3, 13, 6, 128, 1.0, False, 2), (64, 3, 600, 256, 0.9, False, 2),
                                     (3, 2, 700, 512, 1.0, False, 1), (2, 4, 1300, 1536, 0.8, True, 2),
                                     (4, 4, 900, 1024, 1.0, False, 2), (6, 3, 700, 256, 0.7, False, 1)):
        x = workloads.make_lmhead_sample(B, k, V, d, seed=1, draft_head=own)
        if B >= 48:
            x["hidden_scale"][0] = float("nan")            # batch row 0: NaN target logits
            x["draft_hidden_scale"][3] = float("inf")      # batch row 1: +-inf / NaN draft logits
            x["tokens"][2, 1] = V                          # batch row 2: token out of range
        acc = run_lmhead_sample(x, T, pool=pool)
        if d in (256, 512, 1024) and B <= 16:               # the same through the tile-major layout
            assert (run_lmhead_sample(x, T, pool=pool, packed=True) == acc).all()
        if B >= 48:
            assert acc[0] == -1 and acc[1] == -1 and acc[2] == -1
        print("  accepted", np.bincount(acc[acc >= 0], minlength=k + 1).tolist(), flush=True)


if __name__ == "__main__":
    names = sys.argv[1:] or list(CASES)
    for nm in names:
        print("case", nm, flush=True)
        CASES[nm]()
        print("ok", nm, flush=True)
