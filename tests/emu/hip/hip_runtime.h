// CPU emulation of the small HIP subset that spec_verify.hip uses.
//
// TEST INFRASTRUCTURE ONLY. It lets the unchanged kernel source be compiled as
// host C++ (see ../spec_verify_emu.cpp) and run on the CPU, optionally under
// AddressSanitizer.
//
// Model: a launch runs its workgroups on a pool of OS threads (emu_set_pool,
// default 1 = workgroups strictly one after another). Inside a workgroup the
// lanes are cooperative fibers (ucontext) on that OS thread, so __shared__
// (mapped to static thread_local) is private to the workgroup. The scheduler
// resumes the lanes round-robin; a workgroup barrier waits for every live lane
// of the workgroup and each half of a shuffle or vote waits for the 64 lanes
// of its wave, so waves may diverge between workgroup barriers as they may on
// the hardware (each wave's lanes must meet the same wave exchanges, and
// every live lane the same workgroup barriers: the kernel's contract).
// Global atomics are the GCC __atomic builtins, so workgroups on different OS
// threads really race, spin-waits included.
#pragma once

#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <ucontext.h>

#include <atomic>
#include <chrono>
#include <tuple>
#include <thread>
#include <vector>

#define __global__
#define __device__
#define __host__
#define __forceinline__ inline
#define __launch_bounds__(...)
#define __shared__ static thread_local

struct dim3 {
    unsigned x, y, z;
    dim3(unsigned a = 1, unsigned b = 1, unsigned c = 1) : x(a), y(b), z(c) {}
};
struct EmuIdx { unsigned x, y, z; };
inline thread_local EmuIdx threadIdx{0, 0, 0};
inline thread_local EmuIdx blockIdx{0, 0, 0};
inline EmuIdx gridDim{1, 1, 1};
inline EmuIdx blockDim{1, 1, 1};




inline float __uint_as_float(unsigned u) { float f; memcpy(&f, &u, 4); return f; }
inline int min(int a, int b) { return a < b ? a : b; }
inline int max(int a, int b) { return a > b ? a : b; }

inline float emu_fmed3f(float a, float b, float c) {
    return fmaxf(fminf(a, b), fminf(fmaxf(a, b), c));
}
inline float emu_exp2f(float x) { return exp2f(x); }
#define __builtin_amdgcn_fmed3f emu_fmed3f
#define __builtin_amdgcn_exp2f emu_exp2f
#define __builtin_amdgcn_s_sleep(n) std::this_thread::yield()

// raw buffer loads: base + byte range; a load past the range reads zeros
typedef unsigned emu_u32x4 __attribute__((ext_vector_type(4)));
struct EmuRsrc { const char* base; unsigned bytes; };
#define __amdgpu_buffer_rsrc_t EmuRsrc
inline EmuRsrc emu_make_rsrc(void* p, int, int bytes, int) {
    return EmuRsrc{static_cast<const char*>(p), static_cast<unsigned>(bytes)};
}
inline emu_u32x4 emu_raw_load_b128(EmuRsrc r, int voff, int soff, int) {
    const unsigned off = static_cast<unsigned>(voff) + static_cast<unsigned>(soff);
    emu_u32x4 v = {0u, 0u, 0u, 0u};
    if (static_cast<unsigned long long>(off) + 16ull <= r.bytes) memcpy(&v, r.base + off, 16);
    return v;
}
#define __builtin_amdgcn_make_buffer_rsrc emu_make_rsrc
#define __builtin_amdgcn_raw_buffer_load_b128 emu_raw_load_b128
// 16-byte buffer load with the LDS as destination: lane l's bytes land at
// the (wave-uniform) LDS address + 16*l; past the range they are zeros
template <class LdsPtr>
inline void emu_raw_load_lds(EmuRsrc r, LdsPtr lds, unsigned size, int voff, int soff, unsigned off, unsigned) {
    const unsigned lane = threadIdx.x & 63u;
    unsigned char* dst = (unsigned char*)(lds) + static_cast<size_t>(lane) * size;
    const unsigned o = static_cast<unsigned>(voff) + static_cast<unsigned>(soff) + off;
    if (static_cast<unsigned long long>(o) + size <= r.bytes) memcpy(dst, r.base + o, size);
    else memset(dst, 0, size);
}
#define __builtin_amdgcn_raw_ptr_buffer_load_lds emu_raw_load_lds

inline int __double2loint(double d) { uint64_t u; memcpy(&u, &d, 8); return static_cast<int>(static_cast<uint32_t>(u)); }
inline int __double2hiint(double d) { uint64_t u; memcpy(&u, &d, 8); return static_cast<int>(static_cast<uint32_t>(u >> 32)); }
inline double __hiloint2double(int hi, int lo) {
    const uint64_t u = (static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) | static_cast<uint32_t>(lo);
    double d; memcpy(&d, &u, 8); return d;
}
#define __builtin_amdgcn_sched_barrier(n) ((void)0)
#define __builtin_amdgcn_sched_group_barrier(mask, size, id) ((void)0)
#define __builtin_amdgcn_s_waitcnt(n) __atomic_thread_fence(__ATOMIC_SEQ_CST)
#define __builtin_amdgcn_fence(...) __atomic_thread_fence(__ATOMIC_SEQ_CST)
#define __builtin_amdgcn_s_barrier() __syncthreads()
#define __builtin_amdgcn_readfirstlane(x) (x)
// the occupancy hint of a kernel means nothing here
#define amdgpu_waves_per_eu(...) unused

// Optional random delays at every device-scope atomic (EMU_JITTER=1), so that
// concurrent workgroups interleave in many different orders.
inline int emu_jitter_on() {
    static const int on = [] { const char* e = getenv("EMU_JITTER"); return e && e[0] == '1'; }();
    return on;
}
inline void emu_jitter() {
    if (!emu_jitter_on()) return;
    thread_local unsigned long long x = 0x9E3779B97F4A7C15ull ^ reinterpret_cast<uintptr_t>(&x);
    x ^= x << 13; x ^= x >> 7; x ^= x << 17;
    const unsigned r = static_cast<unsigned>(x % 1000);
    if (r < 30) std::this_thread::sleep_for(std::chrono::microseconds(r));
    else if (r < 200) std::this_thread::yield();
}
template <class T, class V> inline T emu_atomic_add(T* p, V v, int o) {
    emu_jitter(); T r = __atomic_fetch_add(p, static_cast<T>(v), o); emu_jitter(); return r;
}
template <class T, class V> inline void emu_atomic_store(T* p, V v, int o) {
    emu_jitter(); __atomic_store_n(p, static_cast<T>(v), o); emu_jitter();
}
template <class T> inline T emu_atomic_load(const T* p, int o) {
    emu_jitter(); T r = __atomic_load_n(p, o); emu_jitter(); return r;
}
#define __HIP_MEMORY_SCOPE_AGENT 0
#define __hip_atomic_fetch_add(p, v, o, s) emu_atomic_add((p), (v), (o))
#define __hip_atomic_store(p, v, o, s) emu_atomic_store((p), (v), (o))
#define __hip_atomic_load(p, o, s) emu_atomic_load((p), (o))
template <class T> inline T atomicAdd(T* p, T v) { return __atomic_fetch_add(p, v, __ATOMIC_SEQ_CST); }
template <class T> inline T atomicAnd(T* p, T v) { return __atomic_fetch_and(p, v, __ATOMIC_SEQ_CST); }
template <class T> inline T atomicOr(T* p, T v) { return __atomic_fetch_or(p, v, __ATOMIC_SEQ_CST); }
template <class T> inline T atomicMin(T* p, T v) {
    T old = __atomic_load_n(p, __ATOMIC_SEQ_CST);
    while (v < old && !__atomic_compare_exchange_n(p, &old, v, false, __ATOMIC_SEQ_CST, __ATOMIC_SEQ_CST)) {}
    return old;
}
template <class T> inline T atomicMax(T* p, T v) {
    T old = __atomic_load_n(p, __ATOMIC_SEQ_CST);
    while (v > old && !__atomic_compare_exchange_n(p, &old, v, false, __ATOMIC_SEQ_CST, __ATOMIC_SEQ_CST)) {}
    return old;
}
inline void __threadfence() { __atomic_thread_fence(__ATOMIC_SEQ_CST); }

// static device arrays are host arrays; a symbol's address is its own
#define __align__(n) __attribute__((aligned(n)))
#define HIP_SYMBOL(x) (&(x))

// ---------------------------------------------------------------- fibers
// Lanes are fibers run round-robin. A workgroup barrier releases once every
// live lane of the workgroup has arrived; a wave-level exchange (shuffle,
// vote, wave barrier) releases once the 64 lanes of that wave have arrived,
// so waves may take different paths between workgroup barriers, as on the
// hardware. Arrival counts use generation numbers.
struct EmuWG {
    static constexpr size_t STACK = 512 * 1024;
    static constexpr unsigned MAXW = 1024 / 64;
    ucontext_t sched;
    std::vector<ucontext_t> ctx;
    char* stacks = nullptr;     // fiber stacks, pages committed only as they are touched
    size_t stacks_bytes = 0;
    EmuWG() = default;
    EmuWG(const EmuWG&) = delete;
    EmuWG& operator=(const EmuWG&) = delete;
    ~EmuWG() { delete[] stacks; }
    std::vector<char> done;
    unsigned n = 0;
    unsigned ndone = 0;
    unsigned blk_arrive = 0, blk_gen = 0;
    unsigned wave_arrive[MAXW] = {}, wave_gen[MAXW] = {};
    void (*body)(void*) = nullptr;
    void* arg = nullptr;
    alignas(8) unsigned char shfl[1024][8];
    alignas(16) unsigned char mfa[1024][16], mfb[1024][16];
};
inline thread_local EmuWG* emu_wg = nullptr;

inline void emu_yield() {
    EmuWG* w = emu_wg;
    const unsigned me = threadIdx.x;
    swapcontext(&w->ctx[me], &w->sched);
    threadIdx.x = me;
}

// every live lane of the workgroup
inline void __syncthreads() {
    EmuWG* w = emu_wg;
    const unsigned gen = w->blk_gen;
    if (++w->blk_arrive == w->n - w->ndone) {
        w->blk_arrive = 0;
        ++w->blk_gen;
        return;
    }
    while (w->blk_gen == gen) emu_yield();
}

// the 64 lanes of this thread's wave
inline void emu_wave_sync() {
    EmuWG* w = emu_wg;
    const unsigned wv = threadIdx.x >> 6;
    const unsigned width = (w->n - wv * 64) < 64 ? (w->n - wv * 64) : 64;
    const unsigned gen = w->wave_gen[wv];
    if (++w->wave_arrive[wv] == width) {
        w->wave_arrive[wv] = 0;
        ++w->wave_gen[wv];
        return;
    }
    while (w->wave_gen[wv] == gen) emu_yield();
}

inline void __builtin_amdgcn_wave_barrier() { emu_wave_sync(); }

template <class T>
inline T __shfl_xor(T v, int mask, int width = 64) {
    (void)width;
    EmuWG* w = emu_wg;
    const unsigned me = threadIdx.x;
    const unsigned base = me & ~63u, lane = me & 63u;
    memcpy(w->shfl[me], &v, sizeof(T));
    emu_wave_sync();
    T r;
    memcpy(&r, w->shfl[base + (lane ^ static_cast<unsigned>(mask))], sizeof(T));
    emu_wave_sync();
    return r;
}

template <class T>
inline T __shfl(T v, int src, int width = 64) {
    (void)width;
    EmuWG* w = emu_wg;
    const unsigned me = threadIdx.x;
    const unsigned base = me & ~63u;
    memcpy(w->shfl[me], &v, sizeof(T));
    emu_wave_sync();
    T r;
    memcpy(&r, w->shfl[base + (static_cast<unsigned>(src) & 63u)], sizeof(T));
    emu_wave_sync();
    return r;
}

// wave votes over this thread's wave
inline unsigned long long __ballot(int pred) {
    EmuWG* w = emu_wg;
    const unsigned me = threadIdx.x;
    const unsigned base = me & ~63u;
    const int p = pred != 0;
    memcpy(w->shfl[me], &p, sizeof(int));
    emu_wave_sync();
    unsigned long long r = 0;
    for (unsigned l = base; l < base + 64 && l < w->n; ++l) {
        int q;
        memcpy(&q, w->shfl[l], sizeof(int));
        if (q) r |= 1ull << (l - base);
    }
    emu_wave_sync();
    return r;
}
inline int __any(int pred) { return __ballot(pred) != 0; }
inline int __ffsll(long long x) { return __builtin_ffsll(x); }
inline int __clzll(long long x) { return __builtin_clzll(static_cast<unsigned long long>(x)); }

template <class T>
inline T __shfl_up(T v, unsigned delta, int width = 64) {
    (void)width;
    EmuWG* w = emu_wg;
    const unsigned me = threadIdx.x;
    const unsigned base = me & ~63u, lane = me & 63u;
    memcpy(w->shfl[me], &v, sizeof(T));
    emu_wave_sync();
    T r;
    memcpy(&r, w->shfl[lane >= delta ? base + lane - delta : me], sizeof(T));
    emu_wave_sync();
    return r;
}

// v_mfma_i32_32x32x32_i8 over the 64 lanes of this thread's wave (the lane
// layout of the gfx950 instruction): A(i, k) is byte k % 16 of lane
// i + 32 (k / 16)'s a, B(k, j) byte k % 16 of lane j + 32 (k / 16)'s b, and
// D(i, j) = C(i, j) + sum_k A(i, k) B(k, j) is register 4 (i / 8) + i % 4 of
// lane j + 32 ((i / 4) % 2).
typedef int emu_i32x4 __attribute__((ext_vector_type(4)));
typedef int emu_i32x16 __attribute__((ext_vector_type(16)));
inline emu_i32x16 emu_mfma_i32_32x32x32_i8(emu_i32x4 a, emu_i32x4 b, emu_i32x16 c, int, int, int) {
    EmuWG* w = emu_wg;
    const unsigned me = threadIdx.x, base = me & ~63u, lane = me & 63u;
    memcpy(w->mfa[me], &a, 16);
    memcpy(w->mfb[me], &b, 16);
    emu_wave_sync();
    const unsigned j = lane & 31, h = lane >> 5;
    emu_i32x16 d = c;
    for (int q = 0; q < 16; ++q) {
        const unsigned i = 8 * (q / 4) + 4 * h + q % 4;
        long long s = 0;
        for (int kk = 0; kk < 32; ++kk)
            s += static_cast<long long>(static_cast<signed char>(w->mfa[base + i + 32 * (kk / 16)][kk % 16])) *
                 static_cast<signed char>(w->mfb[base + j + 32 * (kk / 16)][kk % 16]);
        d[q] = static_cast<int>(static_cast<long long>(d[q]) + s);
    }
    emu_wave_sync();
    return d;
}
#define __builtin_amdgcn_mfma_i32_32x32x32_i8 emu_mfma_i32_32x32x32_i8

inline void emu_fiber_entry(unsigned lo, unsigned hi) {
    (void)lo; (void)hi;
    EmuWG* w = emu_wg;
    const unsigned me = threadIdx.x;
    w->body(w->arg);
    w->done[me] = 1;
    // a lane that leaves no longer counts for the workgroup barrier
    ++w->ndone;
    if (w->blk_arrive > 0 && w->blk_arrive == w->n - w->ndone) {
        w->blk_arrive = 0;
        ++w->blk_gen;
    }
}

inline void emu_run_wg(EmuWG& w, unsigned wg, unsigned nthreads) {
    emu_wg = &w;
    blockIdx = EmuIdx{wg, 0, 0};
    w.n = nthreads;
    w.ndone = 0;
    w.blk_arrive = w.blk_gen = 0;
    for (unsigned q = 0; q < EmuWG::MAXW; ++q) w.wave_arrive[q] = w.wave_gen[q] = 0;
    w.ctx.assign(nthreads, ucontext_t{});
    w.done.assign(nthreads, 0);
    if (w.stacks_bytes < nthreads * EmuWG::STACK) {
        delete[] w.stacks;
        w.stacks_bytes = nthreads * EmuWG::STACK;
        w.stacks = new char[w.stacks_bytes];
    }
    for (unsigned t = 0; t < nthreads; ++t) {
        getcontext(&w.ctx[t]);
        w.ctx[t].uc_stack.ss_sp = w.stacks + t * EmuWG::STACK;
        w.ctx[t].uc_stack.ss_size = EmuWG::STACK;
        w.ctx[t].uc_link = &w.sched;
        makecontext(&w.ctx[t], reinterpret_cast<void (*)()>(emu_fiber_entry), 2, 0u, 0u);
    }
    for (;;) {
        bool any = false;
        for (unsigned t = 0; t < nthreads; ++t) {
            if (w.done[t]) continue;
            any = true;
            threadIdx = EmuIdx{t, 0, 0};
            swapcontext(&w.sched, &w.ctx[t]);
        }
        if (!any) break;
    }
}

inline int& emu_pool() { static int n = 1; return n; }

template <class... P>
struct EmuLaunch {
    void (*kernel)(P...);
    std::tuple<P...> params;
    static void call(void* self) {
        auto* s = static_cast<EmuLaunch*>(self);
        std::apply(s->kernel, s->params);
    }
};

template <class... P, class... A>
inline void emu_launch(void (*kernel)(P...), dim3 grid, dim3 block, A... args) {
    gridDim = EmuIdx{grid.x, 1, 1};
    blockDim = EmuIdx{block.x, 1, 1};
    EmuLaunch<P...> L{kernel, std::tuple<P...>(args...)};
    std::atomic<unsigned> next{0};
    auto worker = [&] {
        EmuWG w;
        w.body = &EmuLaunch<P...>::call;
        w.arg = &L;
        for (;;) {
            const unsigned wg = next.fetch_add(1);
            if (wg >= grid.x) break;
            emu_run_wg(w, wg, block.x);
        }
    };
    const int pool = emu_pool() < 1 ? 1 : emu_pool();
    std::vector<std::thread> th;
    for (int i = 0; i < pool; ++i) th.emplace_back(worker);
    for (auto& t : th) t.join();
}

// ---------------------------------------------------------------- host API
typedef int hipError_t;
typedef void* hipStream_t;
typedef void* hipEvent_t;
inline hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return 0; }
enum { hipSuccess = 0, hipErrorInvalidValue = 1 };
enum hipMemcpyKind { hipMemcpyDeviceToHost = 2 };
enum hipDeviceAttribute_t { hipDeviceAttributeMultiprocessorCount = 0 };

inline int& emu_cu_count() { static int n = 1; return n; }
inline hipError_t hipGetDevice(int* d) { *d = 0; return hipSuccess; }
inline hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t, int) { *v = emu_cu_count(); return hipSuccess; }
inline hipError_t hipGetSymbolAddress(void** p, const void* sym) { *p = const_cast<void*>(sym); return hipSuccess; }
inline hipError_t hipGetLastError() { return hipSuccess; }
inline int& emu_blocks_per_cu() { static int n = 8; return n; }
template <class K>
inline hipError_t hipOccupancyMaxActiveBlocksPerMultiprocessor(int* n, K, int, size_t) {
    *n = emu_blocks_per_cu();
    return hipSuccess;
}
inline const char* hipGetErrorString(hipError_t) { return "emulated"; }
inline hipError_t hipMemsetAsync(void* p, int v, size_t n, hipStream_t) { memset(p, v, n); return hipSuccess; }
inline hipError_t hipMemcpy(void* d, const void* s, size_t n, hipMemcpyKind) { memcpy(d, s, n); return hipSuccess; }

#define hipLaunchKernelGGL(kernel, grid, block, shmem, stream, ...) \
    emu_launch(kernel, dim3(grid), dim3(block), __VA_ARGS__)
