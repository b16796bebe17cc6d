"""CPU runs of the unchanged HIP source through the emulation harness.

tests/emu/hip/hip_runtime.h maps the HIP subset the kernels use onto host C++
(fibers per workgroup), so these tests execute the product kernels on the CPU
and compare them with the oracle, with a random (uninitialised) workspace.
SPEC_EMU_ASAN=1 rebuilds the harness with AddressSanitizer (slow, ~10 min).
"""
import ctypes
import os
import subprocess
import sys

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
EMU = os.path.join(HERE, "emu")
ROOT = os.path.dirname(HERE)
ASAN = os.environ.get("SPEC_EMU_ASAN") == "1"
CLANG = "/opt/rocm/llvm/bin/clang++"   # host clang: native vector types as in the device code


@pytest.fixture(scope="module")
def emu_lib():
    out = os.path.join(EMU, "libspecverify_emu.so")
    cmd = [CLANG, "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fno-omit-frame-pointer",
           "-I", EMU, "-I", os.path.join(ROOT, "include"), "-Wno-unknown-pragmas",
           "-Wno-pass-failed",
           "-o", out, os.path.join(EMU, "spec_verify_emu.cpp"), "-lpthread"]
    if ASAN:
        cmd[5:5] = ["-fsanitize=address,undefined"]
    subprocess.run(cmd, check=True)
    return out


def run_cases(*names, timeout=1200):
    env = dict(os.environ)
    if ASAN:
        asan = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"],
                              capture_output=True, text=True).stdout.strip()
        env["LD_PRELOAD"] = asan
        env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:detect_stack_use_after_return=0"
    r = subprocess.run([sys.executable, os.path.join(EMU, "run_emu.py"), *names], env=env,
                       capture_output=True, text=True, timeout=timeout)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]


def test_emulated_small_workloads(emu_lib):
    run_cases("smoke_b1", "smoke_b8")


def test_emulated_odd_shapes_greedy_and_exact_path(emu_lib):
    run_cases("odd_shapes", "greedy_bf16", "exact_path")


def test_emulated_concurrent_workgroups(emu_lib):
    run_cases("concurrent_b8")


def test_pass2_exp_accuracy(emu_lib):
    # the table-driven exp used by the fp64 draw stays within 2 ulp of libm's
    # exp over the whole argument range the draw uses, (-745, 0]
    if ASAN:
        pytest.skip("plain build only")
    L = ctypes.CDLL(emu_lib)
    L.spec_verify_emu_exp.argtypes = [ctypes.c_double]
    L.spec_verify_emu_exp.restype = ctypes.c_double
    rng = np.random.default_rng(0)
    xs = np.concatenate([-rng.random(200_000) * 745.0, -rng.random(100_000) * 30.0,
                         -rng.random(20_000) * 1e-3, [0.0, -1e-300, -0.5, -700.0, -744.9]])
    worst = 0.0
    for x in xs:
        got = L.spec_verify_emu_exp(float(x))
        ref = float(np.exp(x))
        if ref == 0.0:
            assert got == 0.0
            continue
        ulp = np.spacing(ref)
        worst = max(worst, abs(got - ref) / ulp)
    assert worst <= 2.0, worst
    assert L.spec_verify_emu_exp(-float("inf")) == 0.0
    assert L.spec_verify_emu_exp(-746.0) == 0.0
