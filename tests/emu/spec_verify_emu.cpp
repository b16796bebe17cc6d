// Host build of the HIP library source for the CPU emulation tests.
// TEST INFRASTRUCTURE ONLY: compiled with host clang++ against tests/emu/hip/hip_runtime.h.
#include "../../token_verification_amd/csrc/spec_verify.hip"

extern "C" void spec_verify_emu_set_cu_count(int n) { emu_cu_count() = n; }
extern "C" void spec_verify_emu_set_pool(int n) { emu_pool() = n; }

// The table-driven double exp of pass 2, evaluated on the host with the same
// 2^(j/N) table construction, for accuracy tests against libm.
extern "C" double spec_verify_emu_exp(double x) {
    static double T[EXP_N];
    static bool init = false;
    if (!init) {
        for (int j = 0; j < EXP_N; ++j) T[j] = exp2(static_cast<double>(j) / EXP_N);
        init = true;
    }
    return exp_fast(x, T);
}

// The lean double log2 / exp2 of the decisions, for accuracy tests against libm.
extern "C" double spec_verify_emu_log2(double x) { return log2_lean(x); }
extern "C" double spec_verify_emu_exp2(double x) { return exp2_lean(x); }
