"""Throughput of the batched speculative-decoding verify step on one MI355X.

One step = one spec_verify call (the whole path: pass-1 row scans, decisions,
pass-2 residual / bonus draws) over one batch of synthetic logits already
resident in HBM. The default workload is B=64 rows, k=5 drafts, V=151936,
bfloat16 logits, sampling mode, T=1.0. Inputs rotate over several device copies
(>= 1 GiB in total) so the 256 MB Infinity Cache cannot serve them.

Prints one JSON line: verified draft positions per second (B*k per step), the
HBM roofline fraction of the kernel (algorithmic bytes / measured kernel time /
8 TB/s), and the fp64 CPU oracle timed on a bounded sample of the same work.
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


def algorithmic_bytes(w) -> int:
    """Every logit read once plus the small inputs and outputs."""
    B, k, V, s = w.B, w.k, w.V, w.elem_bytes
    rows = B * (k + 1) + (B * k if w.mode == 0 else 0)
    small = 4 * B * k + (8 * B * (k + 1) if w.mode == 0 else 0)
    outs = 4 * B + 4 * B * (k + 1) + 4 * B * (k + 1)
    return rows * V * s + small + outs


def counter_traffic(name: str):
    """HBM bytes per call from the committed rocprofv3 counter summary of this
    workload (FETCH_SIZE + WRITE_SIZE, calibrated against a plain copy), or None
    when there is none or the kernel source changed since it was taken."""
    import hashlib
    summary = os.path.join(ROOT, "profiles", f"spec_verify_{name}.md")
    src = os.path.join(ROOT, "token_verification_amd", "csrc", "spec_verify.hip")
    if not os.path.exists(summary):
        return None
    fields = {}
    for line in open(summary):
        if ":" in line and line.split(":")[0] in ("source_sha256", "traffic_bytes_per_call"):
            key, val = line.split(":", 1)
            fields[key] = val.strip()
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if fields.get("source_sha256") != sha or "traffic_bytes_per_call" not in fields:
        return None
    return int(fields["traffic_bytes_per_call"])


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle baseline sample (0 disables it)")
    ap.add_argument("--rotate-bytes", type=float, default=1.1e9)
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

    import token_verification_amd as tv
    import workloads

    name = args.workload or workloads.HEADLINE
    w = workloads.WORKLOADS[name]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    print(f"bench: generating {name}", file=sys.stderr, flush=True)
    x = workloads.make(w, 0, device=dev)
    per_copy = x["target"].numel() * w.elem_bytes + (
        x["draft"].numel() * w.elem_bytes if x["draft"] is not None else 0)
    R = max(1, math.ceil(args.rotate_bytes / per_copy))
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
                       out=outs[i % R])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # per-launch kernel time: event pairs on the stream the kernel runs on
    stream = torch.cuda.current_stream(dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        step(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kms = np.array([a.elapsed_time(b) for a, b in ev])
    k_avg = float(kms.mean())
    ms_per_step = wall * 1e3 / args.steps

    positions = B * k if w.mode == 0 else B * k
    alg = algorithmic_bytes(w)
    achieved = alg / (k_avg * 1e-3) / 1e9
    value = positions / (ms_per_step * 1e-3)

    line = {
        "metric": METRIC,
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
        "config": {"workload": name, "B": B, "k": k, "V": w.V, "logits": w.dtype,
                   "mode": "sample" if w.mode == 0 else "greedy", "T": w.T,
                   "rotated_copies": R},
        "kernel_us": {"mean": round(k_avg * 1e3, 2), "p10": round(float(np.percentile(kms, 10)) * 1e3, 2),
                      "p50": round(float(np.percentile(kms, 50)) * 1e3, 2),
                      "p90": round(float(np.percentile(kms, 90)) * 1e3, 2)},
        "positions_per_s_kernel": round(positions / (k_avg * 1e-3), 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": counter_traffic(name),
                     "algorithmic_bytes_per_launch": alg,
                     "bytes_per_position": round(alg / positions, 1)},
    }

    if args.cpu_seconds > 0:
        import oracle
        host = {key: (v.cpu() if isinstance(v, torch.Tensor) else v) for key, v in x.items()}
        oracle.spec_verify_ref(host["target"], host["draft"], host["tokens"], host["uniforms"],
                               host["T"], host["mode"])          # warm (page-in)
        n, t_cpu = 0, 0.0
        while t_cpu < args.cpu_seconds:
            c0 = time.perf_counter()
            oracle.spec_verify_ref(host["target"], host["draft"], host["tokens"], host["uniforms"],
                                   host["T"], host["mode"])
            t_cpu += time.perf_counter() - c0
            n += 1
        line["cpu_baseline"] = {"value": round(positions * n / t_cpu, 1), "unit": "positions/s",
                                "cores": oracle.max_threads(), "kind": "oracle",
                                "sample": f"{n} full calls of {name} (B={B}) on host copies, "
                                          f"{t_cpu:.1f} s of oracle time"}
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
