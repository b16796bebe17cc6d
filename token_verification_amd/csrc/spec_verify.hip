// spec_verify.hip -- batched speculative-decoding verify step for MI355X (gfx950).
//
// What is computed is stated in include/spec_verify.h (the modified rejection
// sampling rule of "Speculative Decoding: The Physics of Stolen Time", section 2;
// greedy argmax matching of "The Inference Wall" part 7; the top-1 minus top-2
// logit gap of "Speculative Pre-Positioning", Eq. 11).
//
// Pipeline (stream-ordered kernels; no workgroup ever waits on another):
//
//  1. row_scan_kernel -- one resident round of workgroups, each streaming an
//     equal slice of the flattened (row, element) space (a slice may span row
//     boundaries and emits one record per row segment). 16-byte vector loads,
//     ping-pong pipelined; per lane the top-2 raw logits (v_max/v_med3 on pairs) and,
//     in sampling mode, an online sum s = sum 2^(x*c - ref) with c = log2(e)/T in
//     fp32 and an integer reference ref = ceil(max*c), so rescaling when the
//     running max grows is an exact power-of-two ldexp. Lanes, waves and segments
//     merge the same way. Greedy mode also finds the first index of the max.
//  2. decide_kernel -- one workgroup per batch row: merges the segments of its
//     rows, writes the gaps, evaluates every acceptance test
//     r_i = p_i(x_i)/q_i(x_i) in the log2 domain in fp64 from the pass-1 sums,
//     finds the first rejection a and writes every output except the one token
//     the sampling draw will produce.
//  3. residual_chunk_kernel (sampling) -- the residual max(0, p_a - q_a), or the
//     bonus p_k, is drawn by an inverse CDF that must resolve ~1e-13 of the mass
//     at V ~ 10^5, so this pass is fp64 (table-driven double exp). One
//     workgroup covers CHUNK elements of the selected row pair. The residual is
//     linearised, w_x = (e_x - lambda f_x)/S_p with lambda = S_p/S_q, so a single
//     read gives S_p, S_q and, over the elements whose sign is certain under
//     pass 1's estimate of lambda (relative band ETA), the sums E, F; elements
//     inside the band are recorded by index and settled once lambda is exact.
//  4. draw_kernel (sampling) -- one workgroup per batch row: exact lambda, chunk
//     masses, ordered block scan to the chunk holding u*Z, fp64 rescan of that
//     chunk in vocabulary order.
//
// Every reduction uses a fixed order, so results are bitwise reproducible.

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "spec_verify.h"

namespace {

constexpr int NT = 256;                 // threads per workgroup (4 wave64)
constexpr int NWAVE = NT / 64;
constexpr int MAX_AMB = 4;              // band elements recorded per chunk
constexpr int MAXC = 2048;              // max pass-2 chunks per row (LDS capacity)
constexpr int CHUNK = 4096;             // pass-2 chunk length (elements)
constexpr int EPT = CHUNK / NT;         // pass-2 elements per thread (contiguous)
constexpr int MAX_V = MAXC * CHUNK;     // largest supported vocabulary
constexpr double ETA = 1e-5;            // relative band around pass 1's lambda estimate
constexpr int G_MAX = 16384;            // most pass-1 workgroups one launch uses
constexpr int MIN_SLICE = 8192;         // smallest pass-1 slice (elements) worth a workgroup

enum : int { K_TARGET = 0, K_DRAFT = 1, K_GREEDY = 2 };

// ------------------------------------------------------------------ element types

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Each element type streams 16-byte vectors. stream() is a non-temporal load
// (the logits are read once per call): on MI355X it sustains ~7 TB/s where
// ordinary loads level off near 6.
struct Bf16 {
    static constexpr int VE = 8;        // elements per 16-byte vector
    static constexpr int ES = 2;
    using vec = u32x4;
    __device__ static inline vec stream(const vec* p) { return __builtin_nontemporal_load(p); }
    __device__ static inline float load1(const void* base, size_t i) {
        const unsigned short h = reinterpret_cast<const unsigned short*>(base)[i];
        return __uint_as_float(static_cast<unsigned>(h) << 16);
    }
    __device__ static inline void unpack(const vec& w, float (&x)[8]) {
        x[0] = __uint_as_float(w.x << 16); x[1] = __uint_as_float(w.x & 0xffff0000u);
        x[2] = __uint_as_float(w.y << 16); x[3] = __uint_as_float(w.y & 0xffff0000u);
        x[4] = __uint_as_float(w.z << 16); x[5] = __uint_as_float(w.z & 0xffff0000u);
        x[6] = __uint_as_float(w.w << 16); x[7] = __uint_as_float(w.w & 0xffff0000u);
    }
};

struct F32 {
    static constexpr int VE = 4;
    static constexpr int ES = 4;
    using vec = f32x4;
    __device__ static inline vec stream(const vec* p) { return __builtin_nontemporal_load(p); }
    __device__ static inline float load1(const void* base, size_t i) {
        return reinterpret_cast<const float*>(base)[i];
    }
    __device__ static inline void unpack(const vec& w, float (&x)[4]) {
        x[0] = w.x; x[1] = w.y; x[2] = w.z; x[3] = w.w;
    }
};

// ------------------------------------------------------------------ workspace records

struct alignas(32) TileRec {   // one split of one row
    float t1, t2, ref;
    int idx;                   // greedy: row index of the first maximum (INT_MAX if none)
    double s;                  // sampling: sum 2^(x*c - ref)
    int nan;                   // greedy: a NaN was seen
    int pad;
};

struct alignas(32) RowRec {
    float m, t2, ref;
    int idx;
    double s;
    int valid;
    int pad;
};

struct alignas(64) ChunkRec {
    double sp, sq, e, f;       // sum e, sum f, sums over the certain-positive set
    int namb;                  // band elements seen (> MAX_AMB: overflow)
    int amb[MAX_AMB];
    int pad[3];
};

struct Params {
    const void* tgt;
    const void* dft;
    const int* tok;
    const float* uni;
    int* acc_len;
    int* out_tok;
    float* gap;
    float* tprob;
    float* dprob;
    int B, k, V, rpb, nchunk, chunk;
    int G;                     // pass-1 workgroups: one resident round
    long long L;               // elements per pass-1 workgroup (last one may get fewer)
    long long N;               // B * rpb * V: the flattened (row, element) space
    int mode, force_exact;
    int vec_ok;                // rows start 16-byte aligned: pass 2 may use vector loads
    float c;                   // log2(e)/T (fp32), pass-1 exponent scale
    double invT;               // 1/T in double, pass 2
    TileRec* tiles;            // [B*rpb + G] segment records, slot = row + workgroup
    RowRec* rows;              // [B*rpb]
    int* desc;                 // [B] row of the sampling draw, -1 = none
    double* lam_hat;           // [B] pass-1 estimate of S_p/S_q at that row
    ChunkRec* chunks;          // [B*nchunk]
};

// ------------------------------------------------------------------ small helpers

// s * 2^d for d <= 0 given as an integer-valued float; exact unless underflow.
__device__ inline double scale2(double s, float d) {
    if (s == 0.0) return 0.0;
    if (d < -1100.0f) return 0.0;
    return ldexp(s, static_cast<int>(d));
}

// second largest of the multiset {a1 >= a2} U {b1 >= b2}
__device__ inline void top2_merge(float& a1, float& a2, float b1, float b2) {
    const float n2 = __builtin_amdgcn_fmed3f(a1, b1, fmaxf(a2, b2));
    a1 = fmaxf(a1, b1);
    a2 = n2;
}

// merge two (ref, s) sums: result relative to the larger reference. An empty
// partner (s == 0) carries no reference, so it cannot push the other's scale
// into underflow.
__device__ inline void sref_merge(float& ra, double& sa, float rb, double sb) {
    if (sb == 0.0) return;
    if (sa == 0.0) { ra = rb; sa = sb; return; }
    const float r = fmaxf(ra, rb);
    sa = scale2(sa, ra - r) + scale2(sb, rb - r);
    ra = r;
}

__device__ inline double wave_sum(double v) {
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

__device__ inline int wave_min(int v) {
    for (int m = 32; m >= 1; m >>= 1) v = min(v, __shfl_xor(v, m, 64));
    return v;
}

__device__ inline int wave_max(int v) {
    for (int m = 32; m >= 1; m >>= 1) v = max(v, __shfl_xor(v, m, 64));
    return v;
}

// ------------------------------------------------------------------ block reductions

struct Red {
    float t1[NWAVE], t2[NWAVE], ref[NWAVE];
    double s[NWAVE];
    int i[NWAVE];
    int j[NWAVE];
    double d[4][NWAVE];
    float bt1, bt2;
};

// Block top-2 of (t1, t2): every thread returns the block's top-2.
__device__ void block_top2(Red& R, float& t1, float& t2) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    for (int m = 32; m >= 1; m >>= 1) {
        const float o1 = __shfl_xor(t1, m, 64), o2 = __shfl_xor(t2, m, 64);
        top2_merge(t1, t2, o1, o2);
    }
    if (lane == 0) { R.t1[w] = t1; R.t2[w] = t2; }
    __syncthreads();
    if (threadIdx.x == 0) {
        float a1 = R.t1[0], a2 = R.t2[0];
        for (int q = 1; q < NWAVE; ++q) top2_merge(a1, a2, R.t1[q], R.t2[q]);
        R.bt1 = a1; R.bt2 = a2;
    }
    __syncthreads();
    t1 = R.bt1; t2 = R.bt2;
    __syncthreads();
}

// Block merge of (ref, s); result valid in thread 0.
__device__ void block_sref(Red& R, float& ref, double& s) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    for (int m = 32; m >= 1; m >>= 1) {
        const float orf = __shfl_xor(ref, m, 64);
        const double os = __shfl_xor(s, m, 64);
        sref_merge(ref, s, orf, os);
    }
    if (lane == 0) { R.ref[w] = ref; R.s[w] = s; }
    __syncthreads();
    if (threadIdx.x == 0) {
        float r = R.ref[0];
        double a = R.s[0];
        for (int q = 1; q < NWAVE; ++q) sref_merge(r, a, R.ref[q], R.s[q]);
        ref = r; s = a;
    }
    __syncthreads();
}

__device__ int block_min(Red& R, int v) {
    v = wave_min(v);
    if ((threadIdx.x & 63) == 0) R.i[threadIdx.x >> 6] = v;
    __syncthreads();
    int r = R.i[0];
    for (int q = 1; q < NWAVE; ++q) r = min(r, R.i[q]);
    __syncthreads();
    return r;
}

__device__ int block_max(Red& R, int v) {
    v = wave_max(v);
    if ((threadIdx.x & 63) == 0) R.j[threadIdx.x >> 6] = v;
    __syncthreads();
    int r = R.j[0];
    for (int q = 1; q < NWAVE; ++q) r = max(r, R.j[q]);
    __syncthreads();
    return r;
}

// Ordered block sum of up to 4 doubles; every thread returns the sums.
template <int N>
__device__ void block_sum(Red& R, double (&v)[N]) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int q = 0; q < N; ++q) {
        v[q] = wave_sum(v[q]);
        if (lane == 0) R.d[q][w] = v[q];
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < N; ++q) {
        double a = R.d[q][0];
        for (int z = 1; z < NWAVE; ++z) a += R.d[q][z];
        v[q] = a;
    }
    __syncthreads();
}

// Exclusive scan of one double per thread in thread order (fixed Hillis-Steele
// order: deterministic). `a` is NT doubles of shared memory. Returns the
// exclusive prefix and sets `total`.
__device__ double block_exscan(double* a, double v, double& total) {
    a[threadIdx.x] = v;
    __syncthreads();
    for (int off = 1; off < NT; off <<= 1) {
        const double add = threadIdx.x >= static_cast<unsigned>(off) ? a[threadIdx.x - off] : 0.0;
        __syncthreads();
        a[threadIdx.x] += add;
        __syncthreads();
    }
    const double incl = a[threadIdx.x];
    total = a[NT - 1];
    __syncthreads();
    return incl - v;
}

// ------------------------------------------------------------------ pass 1

struct Lane {
    float t1, t2, mref, ref;
    double s;
    int bvec;
    int nan;
};

__device__ inline void lane_rescale(Lane& st, float c) {
    if (st.t1 > st.mref) {
        const float nr = ceilf(st.t1 * c);
        if (!(nr <= 3.0e38f)) {           // +inf logit or overflow: poison the sum
            st.s = __builtin_nan("");
            st.ref = 0.0f;
            st.mref = INFINITY;
        } else {
            st.s = scale2(st.s, st.ref - nr);
            st.ref = nr;
            st.mref = st.t1;
        }
    }
}

template <int KIND, int VE>
__device__ inline void consume_vec(Lane& st, const float (&x)[VE], int vidx, float c) {
    if constexpr (KIND == K_DRAFT) {
#pragma unroll
        for (int j = 0; j < VE; j += 2) st.t1 = fmaxf(st.t1, fmaxf(x[j], x[j + 1]));
    } else {
        const float before = st.t1;
#pragma unroll
        for (int j = 0; j < VE; j += 2) {
            st.t2 = fmaxf(st.t2, __builtin_amdgcn_fmed3f(st.t1, x[j], x[j + 1]));
            st.t1 = fmaxf(st.t1, fmaxf(x[j], x[j + 1]));
        }
        if constexpr (KIND == K_GREEDY) {
            if (st.t1 > before) st.bvec = vidx;
            int n = 0;
#pragma unroll
            for (int j = 0; j < VE; ++j) n |= (x[j] != x[j]);
            st.nan |= n;
        }
    }
    if constexpr (KIND != K_GREEDY) {
        lane_rescale(st, c);
        float e[VE];
#pragma unroll
        for (int j = 0; j < VE; ++j) e[j] = __builtin_amdgcn_exp2f(fmaf(x[j], c, -st.ref));
#pragma unroll
        for (int w = 1; w < VE; w <<= 1) {
#pragma unroll
            for (int j = 0; j + w < VE; j += 2 * w) e[j] += e[j + w];
        }
        st.s += static_cast<double>(e[0]);
    }
}

template <int KIND>
__device__ inline void consume_one(Lane& st, float x, float c) {
    if constexpr (KIND == K_DRAFT) {
        st.t1 = fmaxf(st.t1, x);
    } else {
        st.t2 = fmaxf(st.t2, fminf(st.t1, x));
        st.t1 = fmaxf(st.t1, x);
        if constexpr (KIND == K_GREEDY) st.nan |= (x != x);
    }
    if constexpr (KIND != K_GREEDY) {
        lane_rescale(st, c);
        st.s += static_cast<double>(__builtin_amdgcn_exp2f(fmaf(x, c, -st.ref)));
    }
}

// Scan split [e0, e1) of the row at rowp; the split's record is complete in thread 0.
template <class E, int KIND>
__device__ TileRec tile_scan(const char* row, int e0, int e1, float c, Red& R) {
    using vec = typename E::vec;
    constexpr int VE = E::VE;
    const int tid = threadIdx.x;
    const char* start = row + static_cast<size_t>(e0) * E::ES;
    const int len = e1 - e0;
    int head = static_cast<int>(((16u - (reinterpret_cast<uintptr_t>(start) & 15u)) & 15u) / E::ES);
    if (head > len) head = len;
    const int nvec = (len - head) / VE;
    const int tail = len - head - nvec * VE;
    const vec* vp = reinterpret_cast<const vec*>(start + static_cast<size_t>(head) * E::ES);

    Lane st;
    st.t1 = -INFINITY; st.t2 = -INFINITY; st.mref = -INFINITY; st.ref = 0.0f;
    st.s = 0.0; st.bvec = -1; st.nan = 0;

    // Ping-pong pipelined body: while one batch of U vectors is consumed the
    // next batch is in flight. Loads are never skipped by a branch (a batch past
    // the end re-reads a valid address and is not consumed), so the compiler's
    // wait counts stay exact instead of draining every load each iteration.
    constexpr int U = 4;
    int v = tid;
    const int step = U * NT;
    auto batch_ok = [&](int at) { return at + (U - 1) * NT < nvec; };
    vec A[U], Bv[U];
    if (batch_ok(v)) {
#pragma unroll
        for (int u = 0; u < U; ++u) A[u] = E::stream(vp + v + u * NT);
    }
    while (batch_ok(v)) {
        const int v1 = v + step;
        const int l1 = batch_ok(v1) ? v1 : v;
#pragma unroll
        for (int u = 0; u < U; ++u) Bv[u] = E::stream(vp + l1 + u * NT);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float x[VE];
            E::unpack(A[u], x);
            consume_vec<KIND, VE>(st, x, v + u * NT, c);
        }
        v = v1;
        if (!batch_ok(v)) break;
        const int v2 = v + step;
        const int l2 = batch_ok(v2) ? v2 : v;
#pragma unroll
        for (int u = 0; u < U; ++u) A[u] = E::stream(vp + l2 + u * NT);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float x[VE];
            E::unpack(Bv[u], x);
            consume_vec<KIND, VE>(st, x, v + u * NT, c);
        }
        v = v2;
    }
    for (; v < nvec; v += NT) {
        float x[VE];
        E::unpack(E::stream(vp + v), x);
        consume_vec<KIND, VE>(st, x, v, c);
    }

    // head / tail elements: at most 2*VE-2 of them, one per thread
    const float vb = st.t1;
    const int bvec = st.bvec;
    float sx = -INFINITY;
    int sidx = 0x7fffffff;
    if (tid < head + tail) {
        const int rel = tid < head ? tid : head + nvec * VE + (tid - head);
        sx = E::load1(row, static_cast<size_t>(e0) + rel);
        sidx = e0 + rel;
        consume_one<KIND>(st, sx, c);
    }

    float t1 = st.t1, t2 = st.t2;
    block_top2(R, t1, t2);
    TileRec out;
    out.t1 = t1; out.t2 = t2; out.idx = 0x7fffffff; out.nan = 0; out.ref = 0.0f; out.s = 0.0; out.pad = 0;

    if constexpr (KIND == K_GREEDY) {
        int cand = 0x7fffffff;
        if (bvec >= 0 && vb == t1) {
            float x[VE];
            E::unpack(vp[bvec], x);
            int j = VE;
#pragma unroll
            for (int q = VE - 1; q >= 0; --q) if (x[q] == t1) j = q;
            if (j < VE) cand = e0 + head + bvec * VE + j;
        }
        if (sx == t1 && sidx < cand) cand = sidx;
        out.idx = block_min(R, cand);
        out.nan = block_max(R, st.nan);
    } else {
        float ref = st.ref;
        double s = st.s;
        block_sref(R, ref, s);
        out.ref = ref; out.s = s;
    }
    return out;
}

template <class E, int MODE>
__global__ __launch_bounds__(NT) void row_scan_kernel(Params P) {
    __shared__ Red R;
    // Workgroup w owns the flattened elements [w*L, (w+1)*L) of all B*rpb rows,
    // so every workgroup streams the same number of bytes and the grid is one
    // resident round. It emits one record per row segment, in slot row + w.
    const long long w = blockIdx.x;
    const long long g0 = w * P.L;
    const long long g1 = g0 + P.L < P.N ? g0 + P.L : P.N;
    const int k = P.k, V = P.V;
    for (long long g = g0; g < g1;) {
        const long long row = g / V;
        const int e0 = static_cast<int>(g - row * V);
        const long long rend = (row + 1) * V < g1 ? (row + 1) * V : g1;
        const int e1 = static_cast<int>(rend - row * V);
        const int b = static_cast<int>(row / P.rpb), j = static_cast<int>(row % P.rpb);
        const bool is_target = j <= k;
        const char* rowp;
        if (is_target)
            rowp = static_cast<const char*>(P.tgt) + (static_cast<size_t>(b) * (k + 1) + j) * V * E::ES;
        else
            rowp = static_cast<const char*>(P.dft) + (static_cast<size_t>(b) * k + (j - k - 1)) * V * E::ES;
        TileRec tr;
        if constexpr (MODE == SPEC_MODE_GREEDY) {
            tr = tile_scan<E, K_GREEDY>(rowp, e0, e1, P.c, R);
        } else {
            if (is_target) tr = tile_scan<E, K_TARGET>(rowp, e0, e1, P.c, R);
            else tr = tile_scan<E, K_DRAFT>(rowp, e0, e1, P.c, R);
        }
        if (threadIdx.x == 0) P.tiles[row + w] = tr;
        g = rend;
    }
}

// ------------------------------------------------------------------ decisions

struct Dec {
    RowRec rec[2 * SPEC_MAX_K + 1];
    int acc[SPEC_MAX_K + 1];
    int a;
    int valid;
};

template <class E, int MODE>
__global__ __launch_bounds__(NT) void decide_kernel(Params P) {
    __shared__ Dec D;
    const int tid = threadIdx.x;
    const int b = blockIdx.x;
    const int k = P.k, V = P.V, rpb = P.rpb;
    constexpr bool sample = MODE == SPEC_MODE_SAMPLE;

    // Independent loads first: the draft token of position tid, its uniform,
    // and (as soon as the token is known to be in range) the two logits it
    // picks; they overlap the merge of the split records below.
    int x = -1;
    bool inr = false;
    double u0 = 0.0, lt = 0.0, ld = 0.0;
    if (tid < k) {
        x = P.tok[static_cast<size_t>(b) * k + tid];
        inr = x >= 0 && x < V;
        const size_t rowT = static_cast<size_t>(b) * (k + 1) + tid;
        if constexpr (sample) {
            u0 = P.uni[rowT * 2 + 0];
            if (inr) {
                lt = E::load1(P.tgt, rowT * V + x);
                ld = E::load1(P.dft, (static_cast<size_t>(b) * k + tid) * V + x);
            }
        }
    }

    // merge the segments of every row of batch row b, in element order
    if (tid < rpb) {
        const size_t row = static_cast<size_t>(b) * rpb + tid;
        // segments of this row, in element order: workgroups w0..w1, slot row + w
        const long long r0 = static_cast<long long>(row) * V;
        const long long w0 = r0 / P.L, w1 = (r0 + V - 1) / P.L;
        const TileRec* t = P.tiles + row;
        TileRec m = t[w0];
        for (long long q0 = w0 + 1; q0 <= w1; q0 += 4) {
            TileRec o[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) if (q0 + u <= w1) o[u] = t[q0 + u];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (q0 + u > w1) break;
                const float prev = m.t1;
                top2_merge(m.t1, m.t2, o[u].t1, o[u].t2);
                if constexpr (MODE == SPEC_MODE_GREEDY) {
                    if (o[u].t1 > prev) m.idx = o[u].idx;    // earlier segment wins ties
                    m.nan |= o[u].nan;
                } else {
                    sref_merge(m.ref, m.s, o[u].ref, o[u].s);
                }
            }
        }
        RowRec rr;
        rr.m = m.t1; rr.t2 = m.t2; rr.ref = m.ref; rr.idx = m.idx; rr.s = m.s; rr.pad = 0;
        if constexpr (MODE == SPEC_MODE_GREEDY)
            rr.valid = !m.nan && m.t1 > -INFINITY && m.t1 < INFINITY;
        else
            rr.valid = (m.s == m.s) && m.s > 0.0 && m.s < INFINITY && m.t1 > -INFINITY && m.t1 < INFINITY;
        D.rec[tid] = rr;
        if constexpr (sample) P.rows[row] = rr;
        if (tid <= k) {
            const float g = (m.t2 == -INFINITY) ? INFINITY : m.t1 - m.t2;
            P.gap[static_cast<size_t>(b) * (k + 1) + tid] = g;
        }
    }
    if (tid == 0) { D.valid = 1; D.a = k; }
    __syncthreads();

    int ok = 1;
    if (tid <= k) ok = D.rec[tid].valid;                  // target rows 0..k
    if (tid < k) {
        if (!inr) ok = 0;
        if (sample && !D.rec[k + 1 + tid].valid) ok = 0;
        int acc = 0;
        float pf = __builtin_nanf(""), qf = __builtin_nanf("");
        if (ok) {
            const RowRec& rt = D.rec[tid];
            if constexpr (sample) {
                const RowRec& rd = D.rec[k + 1 + tid];
                const double c = P.c;
                const double lp = lt == -INFINITY ? -INFINITY : lt * c - rt.ref - log2(rt.s);
                const double lq = ld == -INFINITY ? -INFINITY : ld * c - rd.ref - log2(rd.s);
                double r;
                if (lq == -INFINITY) r = (lp == -INFINITY) ? 0.0 : INFINITY;
                else r = exp2(lp - lq);
                acc = u0 < r;
                pf = static_cast<float>(exp2(lp));
                qf = static_cast<float>(exp2(lq));
            } else {
                acc = (x == rt.idx);
            }
        }
        D.acc[tid] = acc;
        if (P.tprob) P.tprob[static_cast<size_t>(b) * k + tid] = ok ? pf : __builtin_nanf("");
        if (P.dprob) P.dprob[static_cast<size_t>(b) * k + tid] = ok ? qf : __builtin_nanf("");
    }
    if (!ok) atomicAnd(&D.valid, 0);
    __syncthreads();
    const int valid = D.valid;
    if (tid == 0) {
        int a = k;
        for (int i = 0; i < k; ++i) if (!D.acc[i]) { a = i; break; }
        D.a = a;
    }
    __syncthreads();
    const int a = D.a;
    if (tid <= k) {
        int o;
        if (!valid) o = -1;
        else if (tid < a) o = x;
        else if (tid == a) o = sample ? -1 : D.rec[a].idx;    // sampling: the draw kernel writes it
        else o = -1;
        P.out_tok[static_cast<size_t>(b) * (k + 1) + tid] = o;
    }
    if (tid == 0) {
        P.acc_len[b] = valid ? a : -1;
        if constexpr (sample) {
            P.desc[b] = valid ? a : -1;
            double lh = 0.0;
            if (valid && a < k) {
                const RowRec& rt = D.rec[a];
                const RowRec& rd = D.rec[k + 1 + a];
                const double c = P.c;
                // pass-1 sums rescaled to the exp((x - m)/T) normalisation of pass 2
                const double lp = static_cast<double>(rt.ref) - static_cast<double>(rt.m) * c;
                const double lq = static_cast<double>(rd.ref) - static_cast<double>(rd.m) * c;
                lh = (rt.s / rd.s) * exp2(lp - lq);
            }
            P.lam_hat[b] = lh;
        }
    }
}

// ------------------------------------------------------------------ pass 2

// exp(x) for x <= 0 in double precision, by the table-driven method of
// P. T. P. Tang ("Table-driven implementation of the exponential function in
// IEEE floating-point arithmetic", ACM TOMS 15(2), 1989): write
// x = (64 m + j) ln2/64 + r with |r| <= ln2/128, so exp(x) = 2^m 2^(j/64) e^r;
// ln2/64 is split into a 36-bit head (so (64 m + j) * head is exact) and a
// tail, and e^r - 1 is its Taylor polynomial of degree 6 (truncation below
// r^7/7! < 3e-20). T[j] = 2^(j/64) is built per workgroup with the device
// exp2. Total error is a few ulp. Inputs below -745 give 0 (also -inf).
constexpr double EXP_INV_L = 0x1.71547652b82fep+6;    // 64 / ln 2
constexpr double EXP_L1 = 0x1.62e42fefa0000p-7;       // ln 2 / 64, leading 36 bits
constexpr double EXP_L2 = 0x1.cf79abc9e3b3ap-46;      // ln 2 / 64 - EXP_L1
constexpr double EXP_C3 = 0x1.5555555555555p-3;       // 1/3!
constexpr double EXP_C4 = 0x1.5555555555555p-5;       // 1/4!
constexpr double EXP_C5 = 0x1.1111111111111p-7;       // 1/5!
constexpr double EXP_C6 = 0x1.6c16c16c16c17p-10;      // 1/6!

__device__ inline double exp_tab(double x, const double* T) {
    if (!(x > -745.0)) return 0.0;
    const double kf = rint(x * EXP_INV_L);
    double r = fma(-kf, EXP_L1, x);
    r = fma(-kf, EXP_L2, r);
    const int k = static_cast<int>(kf);
    double p = fma(r, EXP_C6, EXP_C5);
    p = fma(r, p, EXP_C4);
    p = fma(r, p, EXP_C3);
    p = fma(r, p, 0.5);
    p = fma(r, p, 1.0);
    p *= r;
    const double t = T[k & 63];
    return ldexp(fma(t, p, t), k >> 6);
}

__device__ inline void exp_table_init(double* T) {
    if (threadIdx.x < 64) T[threadIdx.x] = exp2(static_cast<double>(threadIdx.x) / 64.0);
}

// EPT contiguous elements [j0, j0 + EPT) of a row clipped to [.., hi): 16-byte
// vector loads when the row is aligned and the run is whole, else element loads.
// Elements at or past hi read as -inf (weight 0).
template <class E>
__device__ inline void load_run(const void* row, int j0, int hi, bool vec_ok, float (&x)[EPT]) {
    constexpr int VE = E::VE;
    if (vec_ok && j0 + EPT <= hi) {
        const typename E::vec* vp =
            reinterpret_cast<const typename E::vec*>(static_cast<const char*>(row) + static_cast<size_t>(j0) * E::ES);
        typename E::vec w[EPT / VE];
#pragma unroll
        for (int u = 0; u < EPT / VE; ++u) w[u] = vp[u];
#pragma unroll
        for (int u = 0; u < EPT / VE; ++u) {
            float y[VE];
            E::unpack(w[u], y);
#pragma unroll
            for (int q = 0; q < VE; ++q) x[u * VE + q] = y[q];
        }
    } else {
#pragma unroll
        for (int q = 0; q < EPT; ++q)
            x[q] = (j0 + q < hi) ? E::load1(row, static_cast<size_t>(j0) + q) : -INFINITY;
    }
}

struct Pass2 {
    const void* rowT;
    const void* rowD;
    double mp, mq, invT, lam;
    bool resid;
};

template <class E>
__device__ inline Pass2 pass2_setup(const Params& P, int b, int a) {
    const int k = P.k, V = P.V;
    const size_t rpbase = static_cast<size_t>(b) * P.rpb;
    Pass2 Q;
    Q.resid = a < k;
    Q.rowT = static_cast<const char*>(P.tgt) + (static_cast<size_t>(b) * (k + 1) + a) * V * E::ES;
    Q.rowD = Q.resid ? static_cast<const char*>(P.dft) + (static_cast<size_t>(b) * k + a) * V * E::ES
                     : nullptr;
    Q.mp = P.rows[rpbase + a].m;
    Q.mq = Q.resid ? P.rows[rpbase + k + 1 + a].m : 0.0;
    Q.invT = P.invT;
    Q.lam = 0.0;
    return Q;
}

// Residual weight e - lambda f (clamped at 0), or e for the bonus draw, of one
// element given its target and draft logits.
__device__ inline double weight_of(const Pass2& Q, float xt, float xd, const double* T) {
    const double e = exp_tab((static_cast<double>(xt) - Q.mp) * Q.invT, T);
    if (!Q.resid) return e;
    const double f = exp_tab((static_cast<double>(xd) - Q.mq) * Q.invT, T);
    const double w = e - Q.lam * f;
    return w > 0.0 ? w : 0.0;
}

template <class E>
__device__ inline double weight_at(const Pass2& Q, int j, const double* T) {
    const float xt = E::load1(Q.rowT, j);
    const float xd = Q.resid ? E::load1(Q.rowD, j) : 0.0f;
    return weight_of(Q, xt, xd, T);
}

struct ChunkLds {
    Red R;
    double T[64];
    int namb;
    int amb[MAX_AMB];
};

template <class E>
__global__ __launch_bounds__(NT) void residual_chunk_kernel(Params P) {
    __shared__ ChunkLds S;
    const int tid = threadIdx.x;
    const int b = blockIdx.x / P.nchunk, c = blockIdx.x % P.nchunk;
    const int a = P.desc[b];
    if (a < 0) return;                                     // uniform: whole block leaves
    exp_table_init(S.T);
    if (tid == 0) S.namb = 0;
    const Pass2 Q = pass2_setup<E>(P, b, a);
    const double lh = P.lam_hat[b];
    const double hi_b = lh * (1.0 + ETA), lo_b = lh * (1.0 - ETA);
    const int lo = c * CHUNK, hi = min(P.V, lo + CHUNK);
    const int j0 = lo + tid * EPT;
    float xt[EPT], xd[EPT];
    load_run<E>(Q.rowT, j0, hi, P.vec_ok, xt);
    if (Q.resid) load_run<E>(Q.rowD, j0, hi, P.vec_ok, xd);
    __syncthreads();                                       // table ready
    double v[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int q = 0; q < EPT; ++q) {
        const double e = exp_tab((static_cast<double>(xt[q]) - Q.mp) * Q.invT, S.T);
        v[0] += e;
        if (Q.resid) {
            const double f = exp_tab((static_cast<double>(xd[q]) - Q.mq) * Q.invT, S.T);
            v[1] += f;
            if (e > 0.0) {
                if (e > hi_b * f) { v[2] += e; v[3] += f; }
                else if (e >= lo_b * f) {
                    const int slot = atomicAdd(&S.namb, 1);
                    if (slot < MAX_AMB) S.amb[slot] = j0 + q;
                }
            }
        }
    }
    block_sum<4>(S.R, v);
    if (tid == 0) {
        ChunkRec r;
        r.sp = v[0]; r.sq = v[1]; r.e = v[2]; r.f = v[3];
        const int n = S.namb;
        r.namb = n < MAX_AMB + 1 ? n : MAX_AMB + 1;
        for (int q = 0; q < MAX_AMB; ++q) r.amb[q] = q < n ? S.amb[q] : 0;
        r.pad[0] = r.pad[1] = r.pad[2] = 0;
        P.chunks[static_cast<size_t>(b) * P.nchunk + c] = r;
    }
}

struct DrawLds {
    Red R;
    double T[64];
    double mass[MAXC];
    double scan[NT];
    double base;
};

// Mass of chunk c recomputed element by element (whole block, ordered).
template <class E>
__device__ double chunk_exact(const Params& P, const Pass2& Q, int c, DrawLds& S) {
    const int lo = c * CHUNK, hi = min(P.V, lo + CHUNK);
    double acc[1] = {0.0};
    for (int j = lo + static_cast<int>(threadIdx.x); j < hi; j += NT) acc[0] += weight_at<E>(Q, j, S.T);
    block_sum<1>(S.R, acc);
    return acc[0];
}

template <class E>
__global__ __launch_bounds__(NT) void draw_kernel(Params P) {
    __shared__ DrawLds S;
    const int tid = threadIdx.x;
    const int b = blockIdx.x;
    const int a = P.desc[b];
    if (a < 0) return;                                     // uniform: whole block leaves
    const int k = P.k, V = P.V, NC = P.nchunk;
    const ChunkRec* recs = P.chunks + static_cast<size_t>(b) * NC;
    exp_table_init(S.T);
    Pass2 Q = pass2_setup<E>(P, b, a);
    const double u1 = P.uni[(static_cast<size_t>(b) * (k + 1) + a) * 2 + 1];
    const double lh = P.lam_hat[b];

    // exact normalisers
    double sums[2] = {0.0, 0.0};
    for (int c = tid; c < NC; c += NT) { sums[0] += recs[c].sp; sums[1] += recs[c].sq; }
    block_sum<2>(S.R, sums);                               // also publishes the table
    Q.lam = Q.resid ? sums[0] / sums[1] : 0.0;
    const bool band_ok = !Q.resid ||
        (!P.force_exact && Q.lam >= lh * (1.0 - ETA) && Q.lam <= lh * (1.0 + ETA));

    double* M = S.mass;
    for (int attempt = 0; attempt < 2; ++attempt) {
        // chunk masses; NaN marks a chunk that must be recomputed exactly
        for (int c = tid; c < NC; c += NT) {
            const ChunkRec& r = recs[c];
            double m;
            if (!Q.resid) {
                m = r.sp;
            } else if (!band_ok || r.namb > MAX_AMB) {
                m = __builtin_nan("");
            } else {
                m = r.e - Q.lam * r.f;
                if (!(m > 0.0)) m = 0.0;
                int id[MAX_AMB];
                const int n = r.namb;
                for (int q = 0; q < n; ++q) id[q] = r.amb[q];
                for (int x = 1; x < n; ++x)                // sort: fixed summation order
                    for (int y = x; y > 0 && id[y - 1] > id[y]; --y) { const int t = id[y]; id[y] = id[y - 1]; id[y - 1] = t; }
                for (int q = 0; q < n; ++q) m += weight_at<E>(Q, id[q], S.T);
            }
            M[c] = m;
        }
        __syncthreads();
        for (int c = 0; c < NC; ++c) {                    // rare: exact recompute
            if (M[c] != M[c]) {
                __syncthreads();
                const double m = chunk_exact<E>(P, Q, c, S);
                if (tid == 0) M[c] = m;
                __syncthreads();
            }
        }
        __syncthreads();
        // contiguous chunk ranges per thread -> ordered scan
        const int cpt = (NC + NT - 1) / NT;
        const int c0 = min(NC, tid * cpt), c1 = min(NC, c0 + cpt);
        double mine = 0.0;
        for (int c = c0; c < c1; ++c) mine += M[c];
        double Z;
        const double pre = block_exscan(S.scan, mine, Z);
        if (Q.resid && !(Z > 0.0)) {                      // residual mass rounded to zero: use p_a
            Q.resid = false;
            __syncthreads();
            continue;
        }
        const double tgt = u1 * Z;
        // chunk holding the target
        int cstar = 0x7fffffff;
        {
            double run = pre;
            for (int c = c0; c < c1; ++c) {
                const double nx = run + M[c];
                if (nx > tgt) { cstar = c; break; }
                run = nx;
            }
        }
        cstar = block_min(S.R, cstar);
        if (cstar == 0x7fffffff) {                         // rounding: last chunk with mass
            int last = -1;
            for (int c = tid; c < NC; c += NT) if (M[c] > 0.0) last = max(last, c);
            cstar = block_max(S.R, last);
            if (cstar < 0) cstar = 0;
        }
        if (c0 <= cstar && cstar < c1) {
            double run = pre;
            for (int c = c0; c < cstar; ++c) run += M[c];
            S.base = run;                                   // mass before c*
        }
        // rescan c* in element order: EPT contiguous elements per thread, kept in registers
        const int lo = cstar * CHUNK, hi = min(V, lo + CHUNK);
        const int j0 = lo + tid * EPT;
        float xt[EPT], xd[EPT];
        load_run<E>(Q.rowT, j0, hi, P.vec_ok, xt);
        if (Q.resid) load_run<E>(Q.rowD, j0, hi, P.vec_ok, xd);
        double w[EPT];
        double wsum = 0.0;
#pragma unroll
        for (int q = 0; q < EPT; ++q) {
            w[q] = weight_of(Q, xt[q], Q.resid ? xd[q] : 0.0f, S.T);
            wsum += w[q];
        }
        __syncthreads();                                    // S.base visible
        const double base = S.base;
        double tot;
        const double wpre = block_exscan(S.scan, wsum, tot);
        int tok = 0x7fffffff, lastpos = -1;
        {
            double run = base + wpre;
#pragma unroll
            for (int q = 0; q < EPT; ++q) {
                if (w[q] > 0.0) lastpos = j0 + q;
                run += w[q];
                if (run > tgt && tok == 0x7fffffff) tok = j0 + q;
            }
        }
        tok = block_min(S.R, tok);
        if (tok == 0x7fffffff) {
            tok = block_max(S.R, lastpos);
            if (tok < 0) tok = lo;
        }
        if (tid == 0) P.out_tok[static_cast<size_t>(b) * (k + 1) + a] = tok;
        break;
    }
}

// ------------------------------------------------------------------ host side

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

struct Plan {
    int rpb, nchunk, chunk;
    size_t rows_total;
    // workspace offsets (bytes)
    size_t o_tiles, o_rows, o_desc, o_lam, o_chunks, total;
};

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

bool make_plan(int32_t B, int32_t k, int32_t V, int mode, Plan& p) {
    if (B < 1 || k < 0 || k > SPEC_MAX_K || V < 1) return false;
    if (mode != SPEC_MODE_SAMPLE && mode != SPEC_MODE_GREEDY) return false;
    p.rpb = mode == SPEC_MODE_SAMPLE ? 2 * k + 1 : k + 1;
    p.rows_total = static_cast<size_t>(B) * p.rpb;
    if (p.rows_total > (1u << 26)) return false;
    if (mode == SPEC_MODE_SAMPLE) {
        if (V > MAX_V) return false;
        p.chunk = CHUNK;
        p.nchunk = (V + CHUNK - 1) / CHUNK;
    } else {
        p.chunk = 0;
        p.nchunk = 0;
    }
    if (static_cast<size_t>(B) * static_cast<size_t>(p.nchunk) > 0x7fffffffUL) return false;
    size_t o = 0;
    p.o_tiles = o; o = align256(o + (p.rows_total + G_MAX) * sizeof(TileRec));
    p.o_rows = o; o = align256(o + p.rows_total * sizeof(RowRec));
    p.o_desc = o; o = align256(o + static_cast<size_t>(B) * sizeof(int));
    p.o_lam = o; o = align256(o + static_cast<size_t>(B) * sizeof(double));
    p.o_chunks = o; o = align256(o + static_cast<size_t>(B) * p.nchunk * sizeof(ChunkRec));
    p.total = o;
    return true;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check(const void* tgt, const void* dft, const int32_t* tok, const float* uni, float T, int mode,
          int32_t B, int32_t k, int32_t V, int dtype, const int32_t* acc, const int32_t* out,
          const float* gap, const void* ws, size_t ws_bytes, Plan& plan) {
    if (dtype != SPEC_DTYPE_F32 && dtype != SPEC_DTYPE_BF16)
        return fail(SPEC_ERR_DTYPE, "dtype %d is not SPEC_DTYPE_F32 or SPEC_DTYPE_BF16", dtype);
    if (mode != SPEC_MODE_SAMPLE && mode != SPEC_MODE_GREEDY)
        return fail(SPEC_ERR_MODE, "mode %d is not SPEC_MODE_SAMPLE or SPEC_MODE_GREEDY", mode);
    if (B < 1 || k < 0 || k > SPEC_MAX_K || V < 1)
        return fail(SPEC_ERR_SHAPE, "need B >= 1, 0 <= k <= %d, V >= 1 (got B=%d k=%d V=%d)", SPEC_MAX_K, B, k, V);
    if (!make_plan(B, k, V, mode, plan))
        return fail(SPEC_ERR_SHAPE, "sizes B=%d k=%d V=%d exceed the supported range", B, k, V);
    const unsigned long long elems = static_cast<unsigned long long>(B) * (k + 1) * static_cast<unsigned long long>(V);
    if (elems > (1ull << 46)) return fail(SPEC_ERR_SHAPE, "B*(k+1)*V = %llu is too large", elems);
    const bool sample = mode == SPEC_MODE_SAMPLE;
    if (!tgt) return fail(SPEC_ERR_NULL, "target_logits is NULL");
    if (k > 0 && !tok) return fail(SPEC_ERR_NULL, "draft_tokens is NULL");
    if (sample && k > 0 && !dft) return fail(SPEC_ERR_NULL, "draft_logits is NULL in sampling mode");
    if (sample && !uni) return fail(SPEC_ERR_NULL, "uniforms is NULL in sampling mode");
    if (!acc || !out || !gap) return fail(SPEC_ERR_NULL, "an output pointer is NULL");
    if (sample && !(T > 0.0f && T <= 3.0e38f))
        return fail(SPEC_ERR_TEMP, "temperature must be finite and > 0 in sampling mode (got %g)", (double)T);
    const size_t es = dtype == SPEC_DTYPE_F32 ? 4 : 2;
    if (!aligned(tgt, es) || (dft && !aligned(dft, es)) || (tok && !aligned(tok, 4)) ||
        (uni && !aligned(uni, 4)) || !aligned(acc, 4) || !aligned(out, 4) || !aligned(gap, 4))
        return fail(SPEC_ERR_ALIGN, "a tensor pointer is not aligned to its element size");
    if (!ws || ws_bytes < plan.total)
        return fail(SPEC_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu%s)", plan.total, ws_bytes,
                    ws ? "" : ", NULL");
    if (!aligned(ws, 256)) return fail(SPEC_ERR_ALIGN, "workspace must be 256-byte aligned");
    return SPEC_OK;
}

// Resident workgroups per CU of the pass-1 kernel, cached per device.
template <class E, int MODE>
int scan_blocks_per_cu(int dev) {
    static int cache[64] = {0};
    if (dev >= 0 && dev < 64 && cache[dev] > 0) return cache[dev];
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, row_scan_kernel<E, MODE>, NT, 0) != hipSuccess || n < 1)
        n = 1;
    if (dev >= 0 && dev < 64) cache[dev] = n;
    return n;
}

template <class E, int MODE>
hipError_t launch_all(Params& P, int dev, int ncu, hipStream_t s) {
    long long G = static_cast<long long>(ncu) * scan_blocks_per_cu<E, MODE>(dev);
    const long long by_size = (P.N + MIN_SLICE - 1) / MIN_SLICE;
    if (G > by_size) G = by_size;
    if (G > G_MAX) G = G_MAX;
    if (G < 1) G = 1;
    P.L = (P.N + G - 1) / G;
    P.G = static_cast<int>((P.N + P.L - 1) / P.L);
    hipLaunchKernelGGL((row_scan_kernel<E, MODE>), dim3(P.G), dim3(NT), 0, s, P);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decide_kernel<E, MODE>), dim3(P.B), dim3(NT), 0, s, P);
    e = hipGetLastError();
    if (e != hipSuccess || MODE == SPEC_MODE_GREEDY) return e;
    const unsigned nch = static_cast<unsigned>(P.B) * static_cast<unsigned>(P.nchunk);
    hipLaunchKernelGGL((residual_chunk_kernel<E>), dim3(nch), dim3(NT), 0, s, P);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((draw_kernel<E>), dim3(P.B), dim3(NT), 0, s, P);
    return hipGetLastError();
}

}  // namespace

extern "C" {

size_t spec_verify_workspace_size(int32_t B, int32_t k, int32_t V, int dtype, int mode) {
    if (dtype != SPEC_DTYPE_F32 && dtype != SPEC_DTYPE_BF16) return 0;
    Plan p;
    if (!make_plan(B, k, V, mode, p)) return 0;
    return p.total;
}

int spec_verify_check_args(const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                           const float* uniforms, float temperature, int mode, int32_t B, int32_t k, int32_t V,
                           int dtype, const int32_t* accepted_len, const int32_t* out_tokens, const float* gap,
                           const void* workspace, size_t workspace_bytes) {
    Plan p;
    return check(target_logits, draft_logits, draft_tokens, uniforms, temperature, mode, B, k, V, dtype,
                 accepted_len, out_tokens, gap, workspace, workspace_bytes, p);
}

int spec_verify(const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                const float* uniforms, float temperature, int mode, int32_t B, int32_t k, int32_t V, int dtype,
                int32_t* accepted_len, int32_t* out_tokens, float* gap, float* target_prob, float* draft_prob,
                void* workspace, size_t workspace_bytes, void* stream) {
    Plan plan;
    const int rc = check(target_logits, draft_logits, draft_tokens, uniforms, temperature, mode, B, k, V,
                         dtype, accepted_len, out_tokens, gap, workspace, workspace_bytes, plan);
    if (rc != SPEC_OK) return rc;

    char* ws = static_cast<char*>(workspace);
    Params P;
    P.tgt = target_logits;
    P.dft = draft_logits;
    P.tok = draft_tokens;
    P.uni = uniforms;
    P.acc_len = accepted_len;
    P.out_tok = out_tokens;
    P.gap = gap;
    P.tprob = k > 0 ? target_prob : nullptr;
    P.dprob = k > 0 ? draft_prob : nullptr;
    P.B = B; P.k = k; P.V = V;
    P.rpb = plan.rpb;
    P.nchunk = plan.nchunk; P.chunk = plan.chunk;
    P.N = static_cast<long long>(plan.rows_total) * V;
    P.G = 0; P.L = 0;
    P.mode = mode;
    const char* fe = getenv("SPEC_VERIFY_FORCE_EXACT_PATH");
    P.force_exact = (fe && fe[0] == '1') ? 1 : 0;
    const double Td = mode == SPEC_MODE_SAMPLE ? static_cast<double>(temperature) : 1.0;
    P.c = static_cast<float>(1.4426950408889634 / Td);
    P.invT = 1.0 / Td;
    P.vec_ok = aligned(target_logits, 16) && (draft_logits == nullptr || aligned(draft_logits, 16)) &&
               (static_cast<size_t>(V) * (dtype == SPEC_DTYPE_F32 ? 4 : 2)) % 16 == 0;
    P.tiles = reinterpret_cast<TileRec*>(ws + plan.o_tiles);
    P.rows = reinterpret_cast<RowRec*>(ws + plan.o_rows);
    P.desc = reinterpret_cast<int*>(ws + plan.o_desc);
    P.lam_hat = reinterpret_cast<double*>(ws + plan.o_lam);
    P.chunks = reinterpret_cast<ChunkRec*>(ws + plan.o_chunks);

    int dev = 0, ncu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu < 1)
        return fail(SPEC_ERR_HIP, "cannot query the current HIP device");
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (dtype == SPEC_DTYPE_BF16)
        e = mode == SPEC_MODE_SAMPLE ? launch_all<Bf16, SPEC_MODE_SAMPLE>(P, dev, ncu, s)
                                     : launch_all<Bf16, SPEC_MODE_GREEDY>(P, dev, ncu, s);
    else
        e = mode == SPEC_MODE_SAMPLE ? launch_all<F32, SPEC_MODE_SAMPLE>(P, dev, ncu, s)
                                     : launch_all<F32, SPEC_MODE_GREEDY>(P, dev, ncu, s);
    if (e != hipSuccess) return fail(SPEC_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return SPEC_OK;
}

const char* spec_verify_last_error(void) { return g_err; }

const char* spec_verify_version(void) { return "specverify 0.2.0 (gfx950)"; }

}  // extern "C"
