"""CPU runs of the unchanged HIP source through the emulation harness.

tests/emu/hip/hip_runtime.h maps the HIP subset the kernels use onto host C++
(fibers per workgroup), so these tests execute the product kernels on the CPU
and compare them with the oracle, with a random (uninitialised) workspace.
SPEC_EMU_ASAN=1 builds the harness with AddressSanitizer and UndefinedBehavior-
Sanitizer into a library of its own and runs every case under it (slow: the
whole set took about 2 h 06 min on 8 cores; the per-case time limits grow to
match).
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
LIBNAME = "libspecverify_emu_asan.so" if ASAN else "libspecverify_emu.so"
CLANG = "/opt/rocm/llvm/bin/clang++"   # host clang: native vector types as in the device code


@pytest.fixture(scope="module")
def emu_lib():
    out = os.path.join(EMU, LIBNAME)
    cmd = [CLANG, "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fno-omit-frame-pointer",
           "-I", EMU, "-I", os.path.join(ROOT, "include"), "-Wno-unknown-pragmas",
           "-Wno-pass-failed", "-Wno-psabi",
           "-o", out, os.path.join(EMU, "spec_verify_emu.cpp"), "-lpthread"]
    if ASAN:
        cmd[5:5] = ["-fsanitize=address,undefined"]
    subprocess.run(cmd, check=True)
    return out


def run_cases(*names, timeout=1200):
    env = dict(os.environ)
    env["SPEC_EMU_LIB"] = LIBNAME
    if ASAN:
        timeout *= 8
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


def test_emulated_masks_and_largest_k(emu_lib):
    run_cases("masks_large_k")


def test_emulated_bf16_long_rows(emu_lib):
    run_cases("bf16_long_rows")


def test_emulated_ragged_drafts(emu_lib):
    run_cases("ragged")


def test_emulated_gate(emu_lib):
    run_cases("gate")


def test_emulated_commit(emu_lib):
    run_cases("commit")


def test_emulated_lmhead(emu_lib):
    run_cases("lmhead")


def test_emulated_lmhead_sample(emu_lib):
    run_cases("lmhead_sample")


def test_emulated_concurrent_workgroups(emu_lib):
    run_cases("concurrent_b8")


def test_pass2_exp_accuracy(emu_lib):
    # the table-driven exp used by the fp64 draw stays within 8 ulp of libm's
    # exp over the argument range it serves, (-708, 0]; at or below -708 it is
    # 0. Its truncation error r^4/24 < 5.6e-16 relative is up to ~5 ulp at the
    # bottom of a binade; the draw needs ~1e-13.
    if ASAN:
        pytest.skip("plain build only")
    L = ctypes.CDLL(emu_lib)
    L.spec_verify_emu_exp.argtypes = [ctypes.c_double]
    L.spec_verify_emu_exp.restype = ctypes.c_double
    rng = np.random.default_rng(0)
    xs = np.concatenate([-rng.random(200_000) * 707.99, -rng.random(100_000) * 30.0,
                         -rng.random(20_000) * 1e-3, [0.0, -1e-300, -0.5, -700.0, -707.9, 1e-17]])
    worst = 0.0
    for x in xs:
        got = L.spec_verify_emu_exp(float(x))
        ref = float(np.exp(x))
        worst = max(worst, abs(got - ref) / np.spacing(ref))
    assert worst <= 8.0, worst
    for x in (-float("inf"), -708.0, -746.0, -1e300):
        assert L.spec_verify_emu_exp(x) == 0.0


def test_decision_log2_exp2_accuracy(emu_lib):
    # the lean double log2 / exp2 of the acceptance decisions against libm
    if ASAN:
        pytest.skip("plain build only")
    L = ctypes.CDLL(emu_lib)
    for f in (L.spec_verify_emu_log2, L.spec_verify_emu_exp2):
        f.argtypes = [ctypes.c_double]
        f.restype = ctypes.c_double
    rng = np.random.default_rng(1)
    xs = np.concatenate([0.5 + rng.random(50_000) * 3.0, np.exp(rng.random(50_000) * 40.0),
                         [1.0, 0.5, 2.0, 0.7071067811865476, 1.4142135623730951, 1e300]])
    worst = max(abs(L.spec_verify_emu_log2(float(x)) - np.log2(x)) for x in xs)
    assert worst <= 8e-15, worst
    ds = np.concatenate([rng.uniform(-60, 60, 100_000), [0.0, 0.5, -0.5, 1023.0, -1022.0, -1070.0]])
    worst = 0.0
    for d in ds:
        got, ref = L.spec_verify_emu_exp2(float(d)), float(np.exp2(d))
        worst = max(worst, abs(got - ref) / np.spacing(ref))
    assert worst <= 4.0, worst
    assert L.spec_verify_emu_exp2(-float("inf")) == 0.0
    assert L.spec_verify_emu_exp2(float("inf")) == float("inf")
