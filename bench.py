"""Throughput of the batched speculative-decoding verify step on one MI355X.

One step = one spec_verify call (the whole path: pass-1 row scans, decisions,
pass-2 residual / bonus draws) over one batch of synthetic logits already
resident in HBM. The default workload is B=64 rows, k=5 drafts, V=151936,
bfloat16 logits, sampling mode, T=1.0. Inputs rotate over several device copies
(>= 1 GiB in total) so the 256 MB Infinity Cache cannot serve them.

Prints one JSON line: verified draft positions per second (B*k per step), the
HBM roofline fraction of the kernel (algorithmic bytes / measured kernel time /
8 TB/s), and the fp64 CPU oracle timed on a bounded sample of the same work.

--ragged times spec_verify_ragged instead, with per-row draft lengths from
workloads.draft_lengths: positions are sum(draft_len) per step, and the
algorithmic bytes count only the rows those lengths use.

--gate N times the confidence gate (spec_gate) over N ready distributions of
workloads.make_gate (V=128256 bf16, margin rule, tau=2, 64 admissible tokens):
rows per second, the per-call latency (N=1 is the single-distribution fast
path), the roofline of its logit read, and the coverage c(tau) of the rows.

--commit times the commit / rollback step (spec_commit) after the headline
verify call: B=64 rows, k=5, 4 MiB of recurrent state per row and k+1
checkpoint slots, accepted lengths from the verify call itself.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
METRIC = "verified draft positions/sec + % of HBM roofline, B=64 k=5 V=151936 bf16"


def algorithmic_bytes(w, draft_len=None) -> int:
    """Every logit the step must read, read once, plus the small inputs and
    outputs. With per-row draft lengths kb: target rows 0..kb, draft rows and
    tokens 0..kb-1 and uniforms 0..kb of each row, and the lengths."""
    B, k, V, s = w.B, w.k, w.V, w.elem_bytes
    outs = 4 * B + 4 * B * (k + 1) + 4 * B * (k + 1)
    if draft_len is None:
        rows = B * (k + 1) + (B * k if w.mode == 0 else 0)
        small = 4 * B * k + (8 * B * (k + 1) if w.mode == 0 else 0)
        return rows * V * s + small + outs
    kb = [int(v) for v in draft_len]
    n_t = sum(v + 1 for v in kb)
    n_d = sum(kb)
    rows = n_t + (n_d if w.mode == 0 else 0)
    small = 4 * n_d + (8 * n_t if w.mode == 0 else 0) + 4 * B
    return rows * V * s + small + outs


def counter_traffic(name: str, key: str = "traffic_bytes_per_call"):
    """HBM bytes per call (or, with key="traffic_bytes_pass1", of pass 1 alone)
    from the committed rocprofv3 counter summary profiles/<name>.md
    (FETCH_SIZE + WRITE_SIZE, calibrated against a plain copy), or None when
    there is none or the kernel source changed since."""
    import hashlib
    summary = os.path.join(ROOT, "profiles", f"{name}.md")
    src = os.path.join(ROOT, "token_verification_amd", "csrc", "spec_verify.hip")
    if not os.path.exists(summary):
        return None
    fields = {}
    for line in open(summary):
        if ":" in line and line.split(":")[0] in ("source_sha256", key):
            name_, val = line.split(":", 1)
            fields[name_] = val.strip()
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if fields.get("source_sha256") != sha or key not in fields:
        return None
    return int(fields[key])


def metric_name(w, ragged: bool) -> str:
    """The headline metric's wording, with the sizes of the workload actually run."""
    kind = "" if w.mode == 0 else "greedy, "
    if ragged:
        return (f"verified draft positions/sec + % of HBM roofline, {kind}ragged drafts, "
                f"B={w.B} k<={w.k} V={w.V} {w.dtype}")
    return f"verified draft positions/sec + % of HBM roofline, {kind}B={w.B} k={w.k} V={w.V} {w.dtype}"


def inputs_sha256(x) -> str:
    """SHA-256 over the bytes of the input tensors, in argument order."""
    import hashlib
    import torch
    h = hashlib.sha256()
    for key in ("target", "draft", "tokens", "uniforms", "draft_len"):
        v = x.get(key)
        if isinstance(v, torch.Tensor):
            t = v.detach().cpu().contiguous()
            if t.dtype == torch.bfloat16:
                t = t.view(torch.int16)
            h.update(t.numpy().tobytes())
    return h.hexdigest()


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--ragged", action="store_true",
                    help="per-row draft lengths (spec_verify_ragged)")
    ap.add_argument("--gate", type=int, default=0, metavar="N",
                    help="time the confidence gate over N ready distributions instead")
    ap.add_argument("--commit", action="store_true",
                    help="time the commit / rollback step after the headline verify instead")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle baseline sample (0 disables it)")
    ap.add_argument("--rotate-bytes", type=float, default=1.1e9)
    ap.add_argument("--lmhead", action="store_true",
                    help="time greedy verification fused with an int8 LM head instead "
                         "(B=256 k=3 V=128256 d=4096 unless --lmhead-shape)")
    ap.add_argument("--lmhead-shape", default="256,3,128256,4096", metavar="B,k,V,d")
    ap.add_argument("--lmhead-sample", action="store_true",
                    help="time sampling-mode verification fused with int8 LM heads (target and draft "
                         "hidden rows; the draft shares the head unless --draft-head)")
    ap.add_argument("--draft-head", action="store_true",
                    help="with --lmhead-sample: the draft has an int8 head of its own")
    ap.add_argument("--packed", action="store_true",
                    help="with --lmhead / --lmhead-sample: the heads in the tile-major layout (pack_lmhead, "
                         "written once before the timed region)")
    ap.add_argument("--no-context", action="store_true",
                    help="with --lmhead / --lmhead-sample: skip the library and unfused comparisons "
                         "(run after the timed region), so a profile holds only the fused call")
    ap.add_argument("--probe", choices=["copy", "sum"], default=None,
                    help="instead of the verify step, time a plain 1 GiB device copy (or a "
                         "read-only sum): achievable-bandwidth context and the known-size "
                         "kernel used to calibrate HBM traffic counters")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(batch rows shard with no communication, see the design notes)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    if args.probe:
        return probe(args, torch, np)
    if args.gate:
        return gate_bench(args, torch, np)
    if args.commit:
        return commit_bench(args, torch, np)
    if args.lmhead_sample:
        return lmhead_sample_bench(args, torch, np)
    if args.lmhead:
        return lmhead_bench(args, torch, np)

    import token_verification_amd as tv
    import workloads

    name = args.workload or workloads.HEADLINE
    w = workloads.WORKLOADS[name]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    print(f"bench: generating {name}", file=sys.stderr, flush=True)
    x = workloads.make(w, 0, device=dev)
    dlen = workloads.draft_lengths(w, 0) if args.ragged else None
    if dlen is not None:
        x["draft_len"] = dlen.to(dev)
    per_copy = x["target"].numel() * w.elem_bytes + (
        x["draft"].numel() * w.elem_bytes if x["draft"] is not None else 0)
    # enough copies that the 256 MB Infinity Cache cannot hold them, at most 64
    # (tiny workloads stay cache-resident whatever the count)
    R = min(64, max(1, math.ceil(args.rotate_bytes / per_copy)))
    copies = [x] + [{key: (v.clone() if isinstance(v, torch.Tensor) else v) for key, v in x.items()}
                    for _ in range(R - 1)]
    B, k = w.B, w.k
    outs = [tv.binding.VerifyResult(torch.empty(B, dtype=torch.int32, device=dev),
                                    torch.empty((B, k + 1), dtype=torch.int32, device=dev),
                                    torch.empty((B, k + 1), dtype=torch.float32, device=dev),
                                    None, None) for _ in range(R)]

    def step(i):
        c = copies[i % R]
        tv.spec_verify(c["target"], c["draft"], c["tokens"], c["uniforms"], c["T"], c["mode"],
                       out=outs[i % R], draft_len=c.get("draft_len"))

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # The timed region: K calls back to back, bracketed by one event pair on
    # the stream the kernels run on (events between the calls would add their
    # own gaps to the stream), so the GPU time per step includes every kernel
    # and every gap between them.
    stream = torch.cuda.current_stream(dev)
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g0.record(stream)
    for i in range(args.steps):
        step(i)
    g1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    k_avg = g0.elapsed_time(g1) / args.steps
    ms_per_step = wall * 1e3 / args.steps

    # spread of single calls: event pairs around each call, in a loop of its own
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    for i in range(args.steps):
        ev[i][0].record(stream)
        step(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    kms = np.array([a.elapsed_time(b) for a, b in ev])

    positions = B * k if dlen is None else int(dlen.sum())
    alg = algorithmic_bytes(w, dlen)
    label = name + ("_ragged" if dlen is not None else "")

    # the dominant kernel, pass 1 (every logit streamed once), timed live with
    # events the library records between its kernels (spec_verify_timed)
    pev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        c = copies[i % R]
        tv.spec_verify(c["target"], c["draft"], c["tokens"], c["uniforms"], c["T"], c["mode"],
                       out=outs[i % R], draft_len=c.get("draft_len"), phase_events=pev[i])
    torch.cuda.synchronize()
    ph = np.array([[a[j].elapsed_time(a[j + 1]) for j in range(3)] for a in pev])
    p1_ms = float(ph[:, 0].mean())
    if dlen is None:
        logit_rows = B * (k + 1) + (B * k if w.mode == 0 else 0)
    else:
        logit_rows = int((dlen + 1).sum()) + (int(dlen.sum()) if w.mode == 0 else 0)
    p1_bytes = logit_rows * w.V * w.elem_bytes
    p1_gbs = p1_bytes / (p1_ms * 1e-3) / 1e9
    achieved = alg / (k_avg * 1e-3) / 1e9
    value = positions / (ms_per_step * 1e-3)

    acc = outs[0].accepted_len.cpu().numpy()
    valid = (acc >= 0) & (acc <= k)
    kb = np.full(B, k) if dlen is None else dlen.cpu().numpy()
    line = {
        "metric": metric_name(w, dlen is not None),
        "value": round(value, 1),
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32+f64",
        "data": "synthetic",
        "config": {"workload": label, "B": B, "k": k, "V": w.V, "logits": w.dtype,
                   "mode": "sample" if w.mode == 0 else "greedy", "T": w.T,
                   "rotated_copies": R},
        # mean: GPU time per step over the timed region; the percentiles: single calls
        "kernel_us": {"mean": round(k_avg * 1e3, 2), "p10": round(float(np.percentile(kms, 10)) * 1e3, 2),
                      "p50": round(float(np.percentile(kms, 50)) * 1e3, 2),
                      "p90": round(float(np.percentile(kms, 90)) * 1e3, 2)},
        "acceptance": {"mean_accepted_len": round(float(acc[valid].mean()), 4),
                       "acceptance_rate": round(float(acc[valid].sum() / max(1, kb[valid].sum())), 4),
                       "invalid_rows": int((~valid).sum())},
        "inputs_sha256": inputs_sha256(x),
        "positions_per_s_kernel": round(positions / (k_avg * 1e-3), 1),
        "phase_us": {"pass1": round(p1_ms * 1e3, 2), "pass2": round(float(ph[:, 1].mean()) * 1e3, 2),
                     "draw": round(float(ph[:, 2].mean()) * 1e3, 2)},
        # the dominant kernel: pass 1 reads every logit once
        "roofline": {"bound": "hbm", "kernel": "scan_kernel (pass 1)", "achieved": round(p1_gbs, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(p1_gbs / PEAK_HBM_GBS, 4),
                     "traffic": counter_traffic("spec_verify_" + label, "traffic_bytes_pass1"),
                     "algorithmic_bytes_per_launch": p1_bytes},
        # the whole call (all kernels) against the same bytes plus the small tensors
        "roofline_call": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                          "frac": round(achieved / PEAK_HBM_GBS, 4),
                          "traffic": counter_traffic("spec_verify_" + label),
                          "algorithmic_bytes_per_launch": alg,
                          "bytes_per_position": round(alg / positions, 1)},
    }

    if dlen is not None:
        line["config"]["draft_len"] = {"recipe": "successes before the first failure, p=0.8, capped at k",
                                       "mean": round(positions / B, 3)}
    if args.cpu_seconds > 0:
        import oracle
        host = {key: (v.cpu() if isinstance(v, torch.Tensor) else v) for key, v in x.items()}
        hl = None if dlen is None else dlen.numpy()
        ref = oracle.spec_verify_ref(host["target"], host["draft"], host["tokens"], host["uniforms"],
                                     host["T"], host["mode"], draft_len=hl)    # also warms (page-in)
        # this call's outputs against the oracle's, row by row (flagged: near-ties)
        out0 = outs[0].out_tokens.cpu().numpy()
        same = (acc == ref.accepted_len) & (out0 == ref.out_tokens).all(axis=1)
        if w.mode == 0:
            fl12 = ref.flagged(1e-6, 1e-12)
            fl6 = ref.flagged(1e-6, 1e-6)
        else:
            fl12 = fl6 = np.zeros(B, bool)
        line["parity"] = {"rows": B, "mismatch_unflagged": int((~same & ~fl12).sum()),
                          "mismatch_flagged": int((~same & fl12).sum()),
                          "flagged_1e-12": int(fl12.sum()), "flagged_literal_1e-6": int(fl6.sum()),
                          "flag_bits": int((ref.flags != 0).sum())}
        n, t_cpu = 0, 0.0
        while t_cpu < args.cpu_seconds:
            c0 = time.perf_counter()
            oracle.spec_verify_ref(host["target"], host["draft"], host["tokens"], host["uniforms"],
                                   host["T"], host["mode"], draft_len=hl)
            t_cpu += time.perf_counter() - c0
            n += 1
        cores = len(os.sched_getaffinity(0))
        line["cpu_baseline"] = {"value": round(positions * n / t_cpu, 1), "unit": "positions/s",
                                "cores": min(cores, oracle.max_threads()), "kind": "oracle",
                                "sample": f"{n} full calls of {label} (B={B}) on host copies, "
                                          f"{t_cpu:.1f} s of oracle time",
                                "cpu_model": cpu_model(), "affinity_cores": cores}
        # one thread, on the first batch rows (rows are independent)
        bs = max(1, B // 16)
        sub = {key: (v[:bs] if isinstance(v, torch.Tensor) else v) for key, v in host.items()}
        hs = None if hl is None else hl[:bs]
        n1, t1 = 0, 0.0
        while t1 < args.cpu_seconds / 4:
            c0 = time.perf_counter()
            oracle.spec_verify_ref(sub["target"], sub["draft"], sub["tokens"], sub["uniforms"],
                                   sub["T"], sub["mode"], draft_len=hs, threads=1)
            t1 += time.perf_counter() - c0
            n1 += 1
        pos1 = bs * k if hs is None else int(hs.sum())
        line["cpu_baseline_1thread"] = {"value": round(pos1 * n1 / t1, 1), "unit": "positions/s", "cores": 1,
                                        "sample": f"{n1} calls on the first {bs} batch rows, {t1:.1f} s"}
    print(json.dumps(line), flush=True)
    return 0


def gate_bench(args, torch, np) -> int:
    import token_verification_amd as tv
    import workloads

    n, V = args.gate, workloads.GATE_V
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    x, A = workloads.make_gate(n, V, 0, "bf16", device=dev)
    mask = workloads.admit_bits(A, V).to(dev)
    per_copy = x.numel() * 2
    # rotate over copies (>= 1 GiB) so every call reads its rows from HBM
    R = max(1, min(8192, math.ceil(args.rotate_bytes / per_copy)))
    pool = x.repeat(R, 1)
    copies = [pool[i * n:(i + 1) * n] for i in range(R)]
    out = tv.binding.GateResult(torch.empty(n, dtype=torch.int32, device=dev),
                                torch.empty(n, dtype=torch.float32, device=dev),
                                torch.empty(n, dtype=torch.int32, device=dev))
    for i in range(args.warmup):
        tv.spec_gate(copies[i % R], 2.0, mask, out=out)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        tv.spec_gate(copies[i % R], 2.0, mask, out=out)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kms = np.array([a.elapsed_time(b) for a, b in ev])
    k_avg = float(kms.mean())
    alg = n * V * 2 + mask.numel() * 4 + 12 * n
    achieved = alg / (k_avg * 1e-3) / 1e9
    cov = {}
    for tau in (0.5, 1.0, 2.0, 4.0, 8.0):
        r = tv.spec_gate(x, tau, mask)
        cov[str(tau)] = round(float(r.fire.float().mean()), 4)
    line = {
        "metric": f"confidence-gate rows/sec, n={n} V={V} bf16",
        "value": round(n / (wall / args.steps), 1),
        "unit": "rows/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"gate_n{n}_v{V}_bf16", "n": n, "V": V, "rule": "margin", "tau": 2.0,
                   "admissible": int(A.numel()), "rotated_copies": R},
        "latency_us": {"mean": round(k_avg * 1e3, 2), "p50": round(float(np.percentile(kms, 50)) * 1e3, 2),
                       "p90": round(float(np.percentile(kms, 90)) * 1e3, 2)},
        "coverage": cov,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": counter_traffic(f"spec_gate_n{n}_v{V}_bf16"),
                     "algorithmic_bytes_per_launch": alg},
    }
    if args.cpu_seconds > 0:
        import oracle
        xh = x.cpu()
        mh = mask.cpu().numpy().view(np.uint32)
        oracle.spec_gate_ref(xh, 0, 2.0, mh)
        m, t_cpu = 0, 0.0
        while t_cpu < args.cpu_seconds:
            c0 = time.perf_counter()
            oracle.spec_gate_ref(xh, 0, 2.0, mh)
            t_cpu += time.perf_counter() - c0
            m += 1
        line["cpu_baseline"] = {"value": round(n * m / t_cpu, 1), "unit": "rows/s", "cores": 1,
                                "kind": "oracle",
                                "sample": f"{m} calls over the same {n} rows, {t_cpu:.1f} s of oracle time"}
    print(json.dumps(line), flush=True)
    return 0


def commit_bench(args, torch, np) -> int:
    import token_verification_amd as tv
    import workloads

    w = workloads.WORKLOADS[workloads.HEADLINE]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    x = workloads.make(w, 0, device=dev)
    acc = tv.spec_verify(x["target"], x["draft"], x["tokens"], x["uniforms"], x["T"], 0).accepted_len
    del x
    row = 4 << 20
    B, k = w.B, w.k
    g = torch.Generator(device=dev).manual_seed(5)
    slots = torch.randint(-2 ** 31, 2 ** 31 - 1, (B, k + 1, row // 4), generator=g, dtype=torch.int32, device=dev)
    state = torch.zeros((B, row // 4), dtype=torch.int32, device=dev)
    kv = torch.zeros(B, dtype=torch.int32, device=dev)
    for _ in range(args.warmup):
        tv.spec_commit(acc, k, kv, slots, state)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        tv.spec_commit(acc, k, kv, slots, state)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kms = np.array([a.elapsed_time(b) for a, b in ev])
    k_avg = float(kms.mean())
    nvalid = int((acc >= 0).sum())
    alg = 2 * nvalid * row + 4 * B + 8 * nvalid
    achieved = alg / (k_avg * 1e-3) / 1e9
    line = {
        "metric": f"committed rows/sec (KV truncation + {row >> 20} MiB state-slot copy), B={B} k={k}",
        "value": round(B / (wall / args.steps), 1), "unit": "rows/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bytes", "data": "synthetic",
        "config": {"workload": f"commit_b{B}_k{k}_state{row >> 20}mib", "B": B, "k": k,
                   "state_bytes": row, "accepted_from": workloads.HEADLINE},
        "kernel_us": {"mean": round(k_avg * 1e3, 2), "p50": round(float(np.percentile(kms, 50)) * 1e3, 2)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": counter_traffic(f"spec_commit_b{B}_k{k}_state{row >> 20}mib"),
                     "algorithmic_bytes_per_launch": alg},
    }
    if args.cpu_seconds > 0:
        from oracle.commit import commit_ref
        a_h, kv_h = acc.cpu().numpy(), kv.cpu().numpy()
        sl_h, st_h = slots.cpu().numpy(), state.cpu().numpy()
        m, t_cpu = 0, 0.0
        while t_cpu < min(args.cpu_seconds, 5.0):
            c0 = time.perf_counter()
            commit_ref(a_h, kv_h, sl_h, st_h, k=k)
            t_cpu += time.perf_counter() - c0
            m += 1
        line["cpu_baseline"] = {"value": round(B * m / t_cpu, 1), "unit": "rows/s", "cores": 1,
                                "kind": "oracle", "sample": f"{m} commits of the same {B} rows"}
    print(json.dumps(line), flush=True)
    return 0


PEAK_INT8_TOPS = 5000.0    # MI355X dense int8 matrix peak, TOP/s


def head_roofline(ops: float, nbytes: int, seconds: float, traffic):
    """Roofline of LM-head kernels taking `seconds`: against the int8 MFMA peak
    when the 2-op multiply-adds take longer there than the algorithmic bytes
    (weights and hidden rows, read once) take at the HBM peak, else against
    the HBM peak (a handful of hidden rows: the call streams the head)."""
    if ops / (PEAK_INT8_TOPS * 1e12) >= nbytes / (PEAK_HBM_GBS * 1e9):
        a = ops / seconds / 1e12
        return {"bound": "mfma", "achieved": round(a, 1), "peak": PEAK_INT8_TOPS, "unit": "TOP/s",
                "frac": round(a / PEAK_INT8_TOPS, 4), "traffic": traffic, "algorithmic_ops_per_launch": ops,
                "algorithmic_bytes_per_launch": nbytes}
    a = nbytes / seconds / 1e9
    return {"bound": "hbm", "achieved": round(a, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(a / PEAK_HBM_GBS, 4), "traffic": traffic, "algorithmic_bytes_per_launch": nbytes,
            "algorithmic_ops_per_launch": ops}


def timed_calls(torch, fn, steps):
    """Wall seconds for `steps` calls of fn back to back, and the GPU ms per
    call between one event pair on the current stream around all of them."""
    stream = torch.cuda.current_stream()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g0.record(stream)
    for _ in range(steps):
        fn()
    g1.record(stream)
    torch.cuda.synchronize()
    return time.perf_counter() - t0, g0.elapsed_time(g1) / steps


def materialized_events(torch, steps, n):
    """steps x n timing events, each recorded once beforehand: torch creates an
    event's handle at its first record, which would otherwise add a record of
    its own inside the timed loop."""
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n)] for _ in range(steps)]
    for e in evs:
        for ev in e:
            ev.record()
    torch.cuda.synchronize()
    return evs


def lmhead_bench(args, torch, np) -> int:
    import token_verification_amd as tv
    import workloads

    B, k, V, d = (int(v) for v in args.lmhead_shape.split(","))
    M = B * (k + 1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"bench: generating the int8 LM head B={B} k={k} V={V} d={d}", file=sys.stderr, flush=True)
    x = workloads.make_lmhead(B, k, V, d, seed=0, device=dev)
    hw = tv.pack_lmhead(x["weight"]) if args.packed else x["weight"]
    a = (x["hidden"], x["hidden_scale"], hw, x["weight_scale"], x["tokens"])
    out = tv.binding.VerifyResult(torch.empty(B, dtype=torch.int32, device=dev),
                                  torch.empty((B, k + 1), dtype=torch.int32, device=dev),
                                  torch.empty((B, k + 1), dtype=torch.float32, device=dev), None, None)
    for _ in range(args.warmup):
        tv.spec_verify_lmhead(*a, out=out)
    torch.cuda.synchronize()
    # the timed region: plain calls back to back (events between the calls
    # would add their own gaps to the stream); then, in a loop of its own, the
    # phases from events the library records between its kernels
    wall, k_ms = timed_calls(torch, lambda: tv.spec_verify_lmhead(*a, out=out), args.steps)
    evs = materialized_events(torch, args.steps, 3)
    for i in range(args.steps):
        tv.spec_verify_lmhead(*a, out=out, phase_events=evs[i])
    torch.cuda.synchronize()
    head = np.array([e[0].elapsed_time(e[1]) for e in evs])
    tail = np.array([e[1].elapsed_time(e[2]) for e in evs])
    call = np.array([e[0].elapsed_time(e[2]) for e in evs])
    ops = 2.0 * M * V * d                                  # int8 multiply-adds, counted as two ops
    wbytes = V * d + M * d + 4 * (V + M)
    positions = B * k
    acc = out.accepted_len.cpu().numpy()
    line = {
        "metric": f"verified draft positions/sec, greedy verify fused with an int8 LM head, "
                  f"B={B} k={k} V={V} d={d}" + (", tile-major head" if args.packed else ""),
        "value": round(positions / (wall / args.steps), 1),
        "unit": "positions/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "int8", "data": "synthetic",
        "config": {"workload": f"lmhead_b{B}_k{k}_v{V}_d{d}_int8" + ("_packed" if args.packed else ""),
                   "B": B, "k": k, "V": V, "d": d, "hidden_rows": M,
                   "weight_layout": "tile-major" if args.packed else "row-major"},
        "gpu_us_per_step": round(k_ms * 1e3, 2),
        "phase_us": {"lmhead_kernel": round(float(head.mean()) * 1e3, 2),
                     "merge_and_decide": round(float(tail.mean()) * 1e3, 2),
                     "call": round(float(call.mean()) * 1e3, 2)},
        "roofline": head_roofline(ops, wbytes, float(head.mean()) * 1e-3,
                                  counter_traffic(f"spec_verify_lmhead_b{B}_k{k}_v{V}_d{d}_int8"
                                                  + ("_packed" if args.packed else ""),
                                                  "traffic_bytes_lmhead_kernel")),
        "hbm_context": {"weight_and_hidden_bytes": wbytes,
                        "GB_per_s": round(wbytes / (float(head.mean()) * 1e-3) / 1e9, 1)},
        "accepted_mean": round(float(acc[acc >= 0].mean()), 3) if (acc >= 0).any() else None,
    }
    # context: the library int8 GEMM alone (hipBLASLt through torch._int_mm, int32
    # logits written out), which an unfused path would follow with scaling and a verify
    try:
        if args.no_context:
            raise RuntimeError("skipped (--no-context)")
        wt = x["weight"].t()
        for _ in range(3):
            torch._int_mm(x["hidden"], wt)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            torch._int_mm(x["hidden"], wt)
        e1.record()
        torch.cuda.synchronize()
        lib_us = e0.elapsed_time(e1) / 10 * 1e3
        line["library_gemm_context"] = {"op": "torch._int_mm(hidden, weight.t()) -> int32 [M, V]",
                                        "us": round(lib_us, 1), "TOP/s": round(ops / lib_us / 1e6, 1)}
    except Exception as ex:                                # context only; never fails the bench
        line["library_gemm_context"] = {"error": f"{type(ex).__name__}: {str(ex)[:120]}"}
    if args.cpu_seconds > 0:
        from oracle.lmhead import lmhead_greedy_ref
        hh, hs, ww, wsc = (t.cpu().numpy() for t in (x["hidden"], x["hidden_scale"], x["weight"], x["weight_scale"]))
        tok = a[4].cpu().numpy()
        n, t_cpu, b = 0, 0.0, 0
        while t_cpu < args.cpu_seconds:
            rows = np.arange(b * (k + 1), (b + 1) * (k + 1))
            c0 = time.perf_counter()
            lmhead_greedy_ref(hh[rows], hs[rows], ww, wsc, tok[b:b + 1], 1, k)
            t_cpu += time.perf_counter() - c0
            n += 1
            b = (b + 1) % B
        line["cpu_baseline"] = {"value": round(n * k / t_cpu, 1), "unit": "positions/s",
                                "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
                                "sample": f"{n} batch rows one at a time (k+1 hidden rows against the "
                                          f"whole head), {t_cpu:.1f} s of oracle time"}
    print(json.dumps(line), flush=True)
    return 0


def lmhead_sample_bench(args, torch, np) -> int:
    import token_verification_amd as tv
    import workloads

    B, k, V, d = (int(v) for v in args.lmhead_shape.split(","))
    MT, MD = B * (k + 1), B * k
    own = args.draft_head
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"bench: generating int8 heads and hidden rows B={B} k={k} V={V} d={d} draft_head={own}",
          file=sys.stderr, flush=True)
    x = workloads.make_lmhead_sample(B, k, V, d, seed=0, device=dev, draft_head=own)
    T = 1.0
    hw = tv.pack_lmhead(x["weight"]) if args.packed else x["weight"]
    hdw = x["draft_weight"]
    if args.packed and hdw is not None:
        hdw = tv.pack_lmhead(hdw)
    out = tv.binding.VerifyResult(torch.empty(B, dtype=torch.int32, device=dev),
                                  torch.empty((B, k + 1), dtype=torch.int32, device=dev),
                                  torch.empty((B, k + 1), dtype=torch.float32, device=dev),
                                  torch.empty((B, k), dtype=torch.float32, device=dev),
                                  torch.empty((B, k), dtype=torch.float32, device=dev))

    def call(**kw):
        tv.spec_verify_lmhead_sample(x["hidden"], x["hidden_scale"], hw, x["weight_scale"],
                                     x["draft_hidden"], x["draft_hidden_scale"], x["tokens"], x["uniforms"], T,
                                     draft_weight=hdw, draft_weight_scale=x["draft_weight_scale"],
                                     out=out, **kw)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    wall, k_ms = timed_calls(torch, call, args.steps)     # as in lmhead_bench
    evs = materialized_events(torch, args.steps, 4)
    for i in range(args.steps):
        call(phase_events=evs[i])
    torch.cuda.synchronize()
    ph = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(3)] for e in evs])
    callt = np.array([e[0].elapsed_time(e[3]) for e in evs])
    heads = ph[:, 0]
    ops = 2.0 * (MT + MD) * V * d                          # int8 multiply-adds of both heads, two ops each
    wbytes = (2 if own else 1) * (V * d + 4 * V) + (MT + MD) * (d + 4)
    positions = B * k
    acc = out.accepted_len.cpu().numpy()
    tag = f"lmhead_sample_b{B}_k{k}_v{V}_d{d}_int8" + ("_drafthead" if own else "") + ("_packed" if args.packed else "")
    line = {
        "metric": f"verified draft positions/sec, sampling verify fused with int8 LM heads, "
                  f"B={B} k={k} V={V} d={d}" + (", separate draft head" if own else ", shared head")
                  + (", tile-major heads" if args.packed else ""),
        "value": round(positions / (wall / args.steps), 1),
        "unit": "positions/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "int8", "data": "synthetic",
        "config": {"workload": tag, "B": B, "k": k, "V": V, "d": d, "T": T,
                   "target_rows": MT, "draft_rows": MD, "draft_head": "own" if own else "shared",
                   "weight_layout": "tile-major" if args.packed else "row-major"},
        "gpu_us_per_step": round(k_ms * 1e3, 2),
        "phase_us": {"head_passes": round(float(heads.mean()) * 1e3, 2),
                     "merges": round(float(ph[:, 1].mean()) * 1e3, 2),
                     "decide_and_draw": round(float(ph[:, 2].mean()) * 1e3, 2),
                     "call": round(float(callt.mean()) * 1e3, 2)},
        "roofline": head_roofline(ops, wbytes, float(heads.mean()) * 1e-3,
                                  counter_traffic(f"spec_verify_{tag}", "traffic_bytes_head_passes")),
        "hbm_context": {"weight_and_hidden_bytes": wbytes,
                        "GB_per_s": round(wbytes / (float(heads.mean()) * 1e-3) / 1e9, 1)},
        "accepted_mean": round(float(acc[acc >= 0].mean()), 3) if (acc >= 0).any() else None,
    }
    # context: the unfused path on this GPU -- the library int8 GEMMs (hipBLASLt
    # through torch._int_mm) writing int32 logits, float32 scaling by torch, and
    # spec_verify over the stored [B, k+1, V] and [B, k, V] logits
    try:
        if args.no_context:
            raise RuntimeError("skipped (--no-context)")
        wt = x["weight"].t()
        wd = wt if not own else x["draft_weight"].t()
        wsd = x["weight_scale"] if not own else x["draft_weight_scale"]

        def unfused():
            tl = (torch._int_mm(x["hidden"], wt).float() * x["hidden_scale"][:, None]) * x["weight_scale"][None, :]
            dl = (torch._int_mm(x["draft_hidden"], wd).float() * x["draft_hidden_scale"][:, None]) * wsd[None, :]
            return tv.spec_verify(tl.view(B, k + 1, V), dl.view(B, k, V), x["tokens"], x["uniforms"], T, tv.SAMPLE,
                                  return_probs=True)

        for _ in range(3):
            ref = unfused()
        torch.cuda.synchronize()
        same = all(torch.equal(a.view(torch.int32), b.view(torch.int32)) for a, b in zip(ref[:3], out[:3]))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            unfused()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / 10 * 1e3
        line["unfused_context"] = {"op": "torch._int_mm x2 -> int32 logits, float32 scaling, spec_verify (SAMPLE)",
                                   "us": round(us, 1), "fused_speedup": round(us / (float(callt.mean()) * 1e3), 3),
                                   "same_outputs": bool(same)}
    except Exception as ex:                                # context only; never fails the bench
        line["unfused_context"] = {"error": f"{type(ex).__name__}: {str(ex)[:120]}"}
    if args.cpu_seconds > 0:
        from oracle.lmhead import lmhead_sample_ref
        a = {n: (None if x[n] is None else x[n].cpu().numpy())
             for n in ("hidden", "hidden_scale", "weight", "weight_scale", "draft_hidden", "draft_hidden_scale",
                       "draft_weight", "draft_weight_scale", "tokens", "uniforms")}
        n, t_cpu, b = 0, 0.0, 0
        while t_cpu < args.cpu_seconds:
            rt = np.arange(b * (k + 1), (b + 1) * (k + 1))
            rd = np.arange(b * k, (b + 1) * k)
            c0 = time.perf_counter()
            lmhead_sample_ref(a["hidden"][rt], a["hidden_scale"][rt], a["weight"], a["weight_scale"],
                              a["draft_hidden"][rd], a["draft_hidden_scale"][rd], a["draft_weight"],
                              a["draft_weight_scale"], a["tokens"][b:b + 1], a["uniforms"][b:b + 1], T, 1, k)
            t_cpu += time.perf_counter() - c0
            n += 1
            b = (b + 1) % B
        line["cpu_baseline"] = {"value": round(n * k / t_cpu, 1), "unit": "positions/s",
                                "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
                                "sample": f"{n} batch rows one at a time (2k+1 hidden rows against the "
                                          f"whole heads), {t_cpu:.1f} s of oracle time"}
    print(json.dumps(line), flush=True)
    return 0


def probe(args, torch, np) -> int:
    n = 1 << 30
    dev = torch.device("cuda:0")
    src = torch.empty(n, dtype=torch.uint8, device=dev).random_(0, 255)
    dst = torch.empty_like(src)
    src16 = src.view(torch.bfloat16)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    for i in range(args.warmup + args.steps):
        if i >= args.warmup:
            ev[i - args.warmup][0].record()
        if args.probe == "copy":
            dst.copy_(src)
        else:
            src16.sum(dtype=torch.float32)
        if i >= args.warmup:
            ev[i - args.warmup][1].record()
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    moved = 2 * n if args.probe == "copy" else n
    print(json.dumps({"probe": args.probe, "bytes_read": n, "bytes_written": n if args.probe == "copy" else 0,
                      "ms": round(ms, 4), "GBps": round(moved / ms / 1e6, 1)}), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
