"""bench.py on the CPU: the one-GPU contract, the algorithmic byte counts its
roofline divides by, and the shape of the committed profile summaries it reads
`traffic` from (no GPU needed)."""
import os
import re
import subprocess
import sys

import bench
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_algorithmic_bytes_of_the_headline():
    w = workloads.WORKLOADS["b64_k5_v151936_bf16"]
    logits = 64 * (2 * 5 + 1) * 151936 * 2                     # every target and draft logit once
    assert logits == 213925888
    small = 4 * 64 * 5 + 8 * 64 * 6 + 4 * 64 + 2 * 4 * 64 * 6   # tokens, uniforms, outputs
    assert bench.algorithmic_bytes(w) == logits + small


def test_algorithmic_bytes_ragged_and_greedy():
    w = workloads.WORKLOADS["b64_k5_v151936_bf16"]
    kb = [5] * w.B                                               # full lengths equal the fixed call
    assert bench.algorithmic_bytes(w, kb) == bench.algorithmic_bytes(w) + 4 * w.B
    kb0 = [0] * w.B                                              # only the bonus rows
    assert bench.algorithmic_bytes(w, kb0) == (w.B * 151936 * 2 + 8 * w.B + 4 * w.B
                                               + 4 * w.B + 8 * w.B * 6)
    g = workloads.WORKLOADS["b256_k3_v128256_bf16_greedy"]      # greedy reads no draft logits
    assert bench.algorithmic_bytes(g) == 256 * 4 * 128256 * 2 + 4 * 256 * 3 + 4 * 256 + 8 * 256 * 4


def test_profile_summaries_carry_hash_command_and_traffic():
    d = os.path.join(ROOT, "profiles")
    names = sorted(f for f in os.listdir(d) if f.endswith(".md"))
    assert names
    for nm in names:
        text = open(os.path.join(d, nm)).read()
        assert re.search(r"^source_sha256: [0-9a-f]{64}$", text, re.M), nm
        assert "rocprofv3" in text and "--kernel-trace --stats" in text, nm
        keys = re.findall(r"^(traffic_bytes_\w+): (\d+)$", text, re.M)
        assert keys, nm
        for _, v in keys:
            assert int(v) > 0


def test_metric_names_the_workload_run():
    assert bench.metric_name(workloads.WORKLOADS[workloads.HEADLINE], False) == bench.METRIC
    assert "B=512 k=8 V=262144 bf16" in bench.metric_name(workloads.WORKLOADS["b512_k8_v262144_bf16"], False)
    g = bench.metric_name(workloads.WORKLOADS["b256_k3_v128256_bf16_greedy"], False)
    assert "greedy" in g and "B=256 k=3 V=128256 bf16" in g
    assert "ragged" in bench.metric_name(workloads.WORKLOADS[workloads.HEADLINE], True)


def test_inputs_hash_follows_the_bytes():
    w = workloads.WORKLOADS["b1_k4_v1000_f32"]
    a, b = workloads.make(w, 0), workloads.make(w, 0)
    assert bench.inputs_sha256(a) == bench.inputs_sha256(b)
    b["uniforms"] = b["uniforms"].clone()
    b["uniforms"][0, 0, 0] += 0.25
    assert bench.inputs_sha256(a) != bench.inputs_sha256(b)
