// Host build of the HIP library source for the CPU emulation tests.
// TEST INFRASTRUCTURE ONLY: compiled with g++ against tests/emu/hip/hip_runtime.h.
#include "../../token_verification_amd/csrc/spec_verify.hip"

extern "C" void spec_verify_emu_set_cu_count(int n) { emu_cu_count() = n; }
extern "C" void spec_verify_emu_set_pool(int n) { emu_pool() = n; }
