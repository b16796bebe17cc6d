// Host build of the HIP library source for the CPU emulation tests.
// TEST INFRASTRUCTURE ONLY: compiled with host clang++ against tests/emu/hip/hip_runtime.h.
#include "../../token_verification_amd/csrc/spec_verify.hip"

extern "C" void spec_verify_emu_set_cu_count(int n) { emu_cu_count() = n; }
extern "C" void spec_verify_emu_set_pool(int n) { emu_pool() = n; }

// The table-driven double exp of pass 2, evaluated on the host with the same
// 2^(j/64) table construction, for accuracy tests against libm.
extern "C" double spec_verify_emu_exp(double x) {
    static double T[64];
    static bool init = false;
    if (!init) {
        for (int j = 0; j < 64; ++j) T[j] = exp2(static_cast<double>(j) / 64.0);
        init = true;
    }
    return exp_tab(x, T);
}
