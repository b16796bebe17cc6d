// spec_verify.hip -- batched speculative-decoding verify step for MI355X (gfx950).
//
// What is computed is stated in include/spec_verify.h (the modified rejection
// sampling rule of "Speculative Decoding: The Physics of Stolen Time", section 2;
// greedy argmax matching of "The Inference Wall" part 7; the top-1 minus top-2
// logit gap of "Speculative Pre-Positioning", Eq. 11).
//
// Three stream-ordered kernels per call in sampling mode (two in greedy mode;
// ragged drafts over more than 1024 batch rows add rows_kernel first); no
// workgroup ever waits on another (every hand-over between them is a kernel
// boundary). The same file holds the confidence gate (gate_kernel,
// gate_row_kernel), the commit step (commit_kernel) and greedy verification
// fused with an int8 LM head on the matrix cores (head_kernel_wide /
// head_kernel_narrow, head_merge_kernel, then decide_kernel; described at
// those kernels).
//
//  1. scan_kernel -- one resident round of workgroups, each streaming an equal
//     slice of the flattened (row, element) space (a slice may span row
//     boundaries and emits one record per row segment). 16-byte non-temporal
//     buffer loads, ping-pong pipelined; per lane the top-2 raw logits
//     (v_max/v_med3 on pairs) and, in sampling mode, an online sum
//     s = sum 2^(x*c - ref) with c = log2(e)/T split into fp32 head and tail
//     (so the rounding of c to fp32 cannot shift p/q) and an integer reference
//     ref = ceil(max*c), so rescaling when the running max grows is an exact
//     power-of-two ldexp. The lane whose vector holds the row's draft token
//     keeps that logit. Greedy mode also finds the first index of the max.
//  2. The decision of a batch row (decide_wave / decide_batch): merges the segments of its
//     rows, writes the gaps, evaluates every acceptance test
//     r_i = p_i(x_i)/q_i(x_i) in the log2 domain in fp64, finds the first
//     rejection a and writes every output except the token the sampling draw
//     will produce. Greedy mode runs it as decide_kernel; sampling mode runs
//     it at the start of every pass-2 workgroup.
//  3. seg_kernel (sampling) -- the residual max(0, p_a - q_a), or the bonus
//     p_k, is drawn by an inverse CDF that must resolve ~1e-13 of the mass at
//     V ~ 10^5, so this pass is fp64 (a value table for bf16 logits, else a
//     table-driven double exp). The selected row pair is split into one
//     segment per wave. The residual is linearised, w_x = (e_x - lambda f_x)/S_p
//     with lambda = S_p/S_q, so a single read gives S_p, S_q and, over the
//     elements whose sign is certain under pass 1's estimate of lambda
//     (relative band ETA), the sums E, F; elements inside the band are
//     grouped by their exact logit difference (one ratio e/f per group) and
//     settled once lambda is exact.
//  4. draw_kernel (sampling) -- one workgroup per batch row: exact lambda,
//     segment masses, ordered scan to the segment holding u*Z, fp64 rescan of
//     that segment in vocabulary order.
//
// Every reduction uses a fixed order, so results are bitwise reproducible.

#include <hip/hip_runtime.h>

#include <math.h>
#include <mutex>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "spec_verify.h"

namespace {

constexpr int NT = 256;                 // threads per workgroup (4 wave64)
constexpr int NWAVE = NT / 64;
constexpr int MAX_AMB = 4;              // groups of band elements recorded per pass-2 segment
constexpr int NT2 = 512;                // threads per draw workgroup (8 wave64)
constexpr int NTS = 1024;               // threads per pass-2 segment workgroup (16 wave64)
constexpr int W_CAP = 256;              // most pass-2 workgroups per batch row
constexpr int MAXS = W_CAP * (NTS / 64); // most pass-2 segments per row (one per wave)
constexpr int SEG_U = 2;                // vectors per lane and row loaded together in pass 2
constexpr int SLOTS_CAP = 4096;         // most resident pass-2 workgroups assumed by the workspace
constexpr int MAX_V = SPEC_MAX_V_SAMPLE; // largest vocabulary of sampling mode
constexpr double ETA = 1e-5;            // relative band around pass 1's lambda estimate
constexpr int G_MAX = 16384;            // most pass-1 workgroups one launch uses
constexpr int MIN_SLICE = 8192;         // smallest pass-1 slice (elements) worth a workgroup
constexpr int EXP_N = 1024;             // entries of the 2^(j/N) table of the fp64 exp
constexpr unsigned TAB_BASE = 111u << 7;  // bf16 magnitude bits of 2^-16 (start of the value table)
constexpr unsigned TAB_RANGE = 24u << 7;  // magnitudes per sign: 24 binades, 2^-16 <= |v| < 2^8
constexpr unsigned TAB_NEG = 4096;      // entry of the first negative value
constexpr int TAB_MAX = TAB_NEG + TAB_RANGE;  // value-table entries (entries RANGE..NEG-1 unused)

// Row kinds of pass 1: K_TARGET (top-2 and exp-sum: target rows with a draft
// token), K_DRAFT (max and exp-sum), K_GREEDY (top-2, first argmax, NaN flag),
// K_TOP2 (top-2 and NaN flag: the bonus target row of sampling mode, whose
// normaliser only the bonus draw needs, and pass 2 computes it there).
enum : int { K_TARGET = 0, K_DRAFT = 1, K_GREEDY = 2, K_TOP2 = 3 };

// ------------------------------------------------------------------ element types

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Each element type streams 16-byte vectors (pass 1 loads them non-temporal:
// the logits are read once per call, and on MI355X non-temporal 16-byte loads
// sustain ~7 TB/s where ordinary loads level off near 6).
struct Bf16 {
    static constexpr int VE = 8;        // elements per 16-byte vector
    static constexpr int ES = 2;
    using vec = u32x4;
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
    __device__ static inline float load1(const void* base, size_t i) {
        return reinterpret_cast<const float*>(base)[i];
    }
    __device__ static inline void unpack(const vec& w, float (&x)[4]) {
        x[0] = w.x; x[1] = w.y; x[2] = w.z; x[3] = w.w;
    }
};

// ------------------------------------------------------------------ workspace records

struct alignas(32) TileRec {   // one segment of one row
    float t1, t2, ref;
    int idx;                   // greedy: row index of the first maximum (INT_MAX if none)
    double s;                  // sampling: sum 2^(x*c - ref)
    float lx;                  // sampling: the row's draft-token logit, if in this segment
    int flags;                 // bit 0: a NaN was seen (greedy); bit 1: lx is set
};

struct RowRec {
    float m, t2;
    int idx;
    int valid;
    double lg;                 // sampling: log2 of the row's normaliser sum 2^(x*c)
    float lx;                  // sampling: the draft-token logit (draft-token rows)
    int has_lx;
};

struct alignas(32) BatchRec {  // what pass 2 and the draw need of one batch row
    int a;                     // row of the draw (k = bonus), -1 = no draw (invalid row)
    float u1;                  // uniform of the draw, u[b, a, 1]
    float mp, mq;              // max raw logit of target row a and (a < k) draft row a
    double lam;                // pass-1 estimate of S_p/S_q at row a (a < k), max-normalised
    double lam_hat;            // the same in pass 2's units (written by pass 2)
    int kb;                    // this batch row's draft length (a < kb: residual draw)
};

struct alignas(64) SegRec {    // one pass-2 segment (one wave's share of a row pair)
    double sp, sq, e, f;       // sum e, sum f, sums over the certain-positive set
    double ae[MAX_AMB], af[MAX_AMB];  // sums of e and f over each group of band elements
    int namb;                  // groups (> MAX_AMB: overflow, the draw recomputes the segment)
    int pad[7];
};

struct Params {
    const void* tgt;
    const void* dft;
    const int* tok;
    const int* dlen;           // [B] per-row draft lengths (ragged drafts), or null: all k
    const float* uni;
    int* acc_len;
    int* out_tok;
    float* gap;
    float* tprob;
    float* dprob;
    int B, k, V, rpb;
    int nvec;                  // 16-byte vectors per row: ceil(V / VE)
    int wpb;                   // pass-2 workgroups per batch row (sampling)
    int nseg, vps;             // pass-2 segments per row (one per wave) and vectors per segment
    int G;                     // pass-1 workgroups: one resident round
    long long L;               // elements per pass-1 workgroup (last one may get fewer)
    long long N;               // B * rpb * V: the flattened (row, element) space
    int mode, force_exact;
    int vec_ok;                // rows start 16-byte aligned: pass 2 may use vector loads
    float ch, cl;              // log2(e)/T = ch + cl (fp32 head, fp32 tail), pass-1 exponent scale
    double c;                  // ch + cl in double: the scale the decisions use
    double invT;               // 1/T in double, pass 2
    TileRec* tiles;            // [B*rpb + G] segment records, slot = row + workgroup
    BatchRec* bat;             // [B]
    SegRec* segs;              // [B*nseg]
    double* exptab;            // [EXP_N] 2^(j/EXP_N), written by pass 1 for pass 2
    double* tautab;            // [TAB_MAX] exp(v/T - tab_c) of bf16 values v, written by pass 1
    // ragged drafts: only the rows a batch row uses enter pass 1's flattened
    // space, in batch-row order; written by rows_kernel before pass 1 (many
    // batch rows) or by pass 1's first workgroup (rowoff, rhdr)
    int* rowoff;               // [B] first packed row of each batch row
    int* rowmap;               // [rows] packed row -> (b << 9) | bonus << 8 | draft << 7 | position
    long long* rhdr;           // [2] pass 1's slice length L and element count N
    // confidence gate (greedy records of n rows): admissible-token mask (or
    // null: all), fire output (null: not a gate call), rule and threshold
    const unsigned* admit;
    int* fire;
    int gate_rule;
    float gate_tau;
    int tab_on;                // the bf16 value table is built and usable
    double tab_lim;            // the table covers 2^-16 <= |v| < tab_lim
    double tab_c;
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

// Workgroup barrier that orders LDS accesses only (every hand-over between the
// threads of a workgroup goes through LDS): global loads stay in flight across
// it instead of being drained, so a prefetch survives the reductions.
__device__ inline void lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// LDS of the block reductions of a workgroup of NW waves.
template <int NW>
struct RedT {
    float t1[NW], t2[NW], ref[NW];
    double s[NW];
    int i[NW];
    int j[NW];
    double d[4][NW];
    float bt1, bt2;
};
using Red = RedT<NWAVE>;

// Block top-2 of (t1, t2): every thread returns the block's top-2.
template <int NW>
__device__ void block_top2(RedT<NW>& R, float& t1, float& t2) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    for (int m = 32; m >= 1; m >>= 1) {
        const float o1 = __shfl_xor(t1, m, 64), o2 = __shfl_xor(t2, m, 64);
        top2_merge(t1, t2, o1, o2);
    }
    if (lane == 0) { R.t1[w] = t1; R.t2[w] = t2; }
    lds_sync();
    if (threadIdx.x == 0) {
        float a1 = R.t1[0], a2 = R.t2[0];
        for (int q = 1; q < NW; ++q) top2_merge(a1, a2, R.t1[q], R.t2[q]);
        R.bt1 = a1; R.bt2 = a2;
    }
    lds_sync();
    t1 = R.bt1; t2 = R.bt2;
    lds_sync();
}

template <int NW>
__device__ int block_min(RedT<NW>& R, int v) {
    v = wave_min(v);
    if ((threadIdx.x & 63) == 0) R.i[threadIdx.x >> 6] = v;
    lds_sync();
    int r = R.i[0];
    for (int q = 1; q < NW; ++q) r = min(r, R.i[q]);
    lds_sync();
    return r;
}

template <int NW>
__device__ int block_max(RedT<NW>& R, int v) {
    v = wave_max(v);
    if ((threadIdx.x & 63) == 0) R.j[threadIdx.x >> 6] = v;
    lds_sync();
    int r = R.j[0];
    for (int q = 1; q < NW; ++q) r = max(r, R.j[q]);
    lds_sync();
    return r;
}

// Ordered block sum of up to 4 doubles; every thread returns the sums.
template <int N, int NW>
__device__ void block_sum(RedT<NW>& R, double (&v)[N]) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int q = 0; q < N; ++q) {
        v[q] = wave_sum(v[q]);
        if (lane == 0) R.d[q][w] = v[q];
    }
    lds_sync();
#pragma unroll
    for (int q = 0; q < N; ++q) {
        double a = R.d[q][0];
        for (int z = 1; z < NW; ++z) a += R.d[q][z];
        v[q] = a;
    }
    lds_sync();
}

// Exclusive scan of one double per thread in thread order, in a fixed order
// (so it is deterministic): an inclusive Hillis-Steele scan inside each
// wave64 with lane shuffles, then the NW wave totals added in wave order
// through `wt` (NW doubles of shared memory). Returns the exclusive prefix
// and sets `total`.
template <int NW>
__device__ double block_exscan(double* wt, double v, double& total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    double x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const double y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    double ex = __shfl_up(x, 1, 64);                       // exclusive within the wave
    if (lane == 0) ex = 0.0;
    if (lane == 63) wt[w] = x;
    lds_sync();
    double before = 0.0, all = 0.0;
#pragma unroll
    for (int q = 0; q < NW; ++q) {
        const double t = wt[q];
        if (q < w) before += t;
        all += t;
    }
    lds_sync();
    total = all;
    return before + ex;
}

// ------------------------------------------------------------------ pass 1

struct Lane {
    float t1, t2, mref, ref;
    double s;
    int bvec;
    int nan;
};

__device__ inline void lane_rescale(Lane& st, float ch) {
    if (st.t1 > st.mref) {
        const float nr = ceilf(st.t1 * ch);
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

// 2^(x*c - ref) with c = ch + cl: the head product is exact for bf16 inputs
// (ch carries 16 significant bits), so only the final roundings remain.
__device__ inline float exp_term(float x, float ch, float cl, float ref) {
    return __builtin_amdgcn_exp2f(fmaf(x, cl, fmaf(x, ch, -ref)));
}

template <int KIND, int VE>
__device__ inline void consume_vec(Lane& st, const float (&x)[VE], int vidx, float ch, float cl) {
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
        }
        if constexpr (KIND == K_GREEDY || KIND == K_TOP2) {
            int n = 0;
#pragma unroll
            for (int j = 0; j < VE; ++j) n |= (x[j] != x[j]);
            st.nan |= n;
        }
    }
    if constexpr (KIND == K_TARGET || KIND == K_DRAFT) {
        lane_rescale(st, ch);
        float e[VE];
#pragma unroll
        for (int j = 0; j < VE; ++j) e[j] = exp_term(x[j], ch, cl, st.ref);
#pragma unroll
        for (int w = 1; w < VE; w <<= 1) {
#pragma unroll
            for (int j = 0; j + w < VE; j += 2 * w) e[j] += e[j + w];
        }
        st.s += static_cast<double>(e[0]);
    }
}

template <int KIND>
__device__ inline void consume_one(Lane& st, float x, float ch, float cl) {
    if constexpr (KIND == K_DRAFT) {
        st.t1 = fmaxf(st.t1, x);
    } else {
        st.t2 = fmaxf(st.t2, fminf(st.t1, x));
        st.t1 = fmaxf(st.t1, x);
        if constexpr (KIND == K_GREEDY || KIND == K_TOP2) st.nan |= (x != x);
    }
    if constexpr (KIND == K_TARGET || KIND == K_DRAFT) {
        lane_rescale(st, ch);
        st.s += static_cast<double>(exp_term(x, ch, cl, st.ref));
    }
}

// 16-byte loads through a buffer resource: one VGPR holds the lane's byte
// offset, the per-vector stride sits in an SGPR, and a load past num_records
// returns zeros instead of faulting (such lanes are never consumed).
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, unsigned bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), 0x00020000);
}

template <class E>
__device__ inline typename E::vec load_nt(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff) {
    const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(voff), static_cast<int>(soff), 2);
    return __builtin_bit_cast(typename E::vec, w);
}

// Wave-level part of a sampling segment's reduction: top-2 (or max), the
// (ref, s) sum rescaled to the wave's largest reference, the NaN flag; lane 0
// leaves them in R slot `w`.
template <int KIND, int NW>
__device__ inline void wave_rec(RedT<NW>& R, const Lane& st) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    float t1 = st.t1, t2 = st.t2;
    for (int m = 32; m >= 1; m >>= 1) {
        const float o1 = __shfl_xor(t1, m, 64);
        if constexpr (KIND == K_DRAFT) {
            t1 = fmaxf(t1, o1);
        } else {
            const float o2 = __shfl_xor(t2, m, 64);
            top2_merge(t1, t2, o1, o2);
        }
    }
    float ref = st.ref;
    double s = st.s;
    int nan = st.nan;
    if constexpr (KIND == K_TARGET || KIND == K_DRAFT) {
        // a lane with no sum carries no reference
        float r = s == 0.0 ? -INFINITY : ref;
        for (int m = 32; m >= 1; m >>= 1) r = fmaxf(r, __shfl_xor(r, m, 64));
        s = (s == 0.0 || s != s) ? s : scale2(s, ref - r);
        s = wave_sum(s);
        ref = r == -INFINITY ? 0.0f : r;
    } else {
        nan = __any(nan) ? 1 : 0;
    }
    if (lane == 0) { R.t1[w] = t1; R.t2[w] = t2; R.ref[w] = ref; R.s[w] = s; R.j[w] = nan; }
}

// Scan segment [e0, e1) of the row at `row`; the segment's record is complete
// in thread 0. tokp points at the row's draft token (or is null): thread 0
// reads it at once, and once the first batch has arrived (the token with it)
// loads that logit if it lies in the segment. The unaligned head and tail
// elements are loaded before the stream too, so no load waits at the end.
// R is used by this segment only: consecutive segments alternate between two.
template <class E, int KIND, int NTH = NT, int U = 4>
__device__ TileRec tile_scan(const char* row, int e0, int e1, const int* tokp, float ch, float cl,
                             RedT<NTH / 64>& R) {
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
    int xs = -1;
    if (tid == 0 && tokp) xs = *tokp;
    // head / tail elements: at most 2*VE-2 of them, one per thread
    float sx = -INFINITY;
    int sidx = 0x7fffffff;
    const bool has_ht = tid < head + tail;
    if (has_ht) {
        const int rel = tid < head ? tid : head + nvec * VE + (tid - head);
        sx = E::load1(row, static_cast<size_t>(e0) + rel);
        sidx = e0 + rel;
    }
    float lx = 0.0f;
    bool got = false;
    auto fetch_lx = [&]() {
        got = tid == 0 && xs >= e0 && xs < e1;
        if (got) lx = E::load1(row, static_cast<size_t>(xs));
    };

    Lane st;
    st.t1 = -INFINITY; st.t2 = -INFINITY; st.mref = -INFINITY; st.ref = 0.0f;
    st.s = 0.0; st.bvec = -1; st.nan = 0;

    // Batch i holds vectors (i*U + u)*NTH + tid, u < U. Batches are ping-pong
    // pipelined (one in flight while the other is consumed); every branch on i
    // is uniform, and only the last batch can hold vectors past nvec, which
    // load as zeros and are skipped.
    constexpr unsigned BSTRIDE = NTH * 16u;                // bytes between u and u+1
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(vp, static_cast<unsigned>(nvec) * 16u);
    const unsigned voff = static_cast<unsigned>(tid) * 16u;
    const int nb = (nvec + U * NTH - 1) / (U * NTH);
    auto consume = [&](const vec (&X)[U], int i) {
        const bool full = (i + 1) * U * NTH <= nvec;
        const int rem = nvec - i * U * NTH - tid;          // vectors of this batch left at u = 0
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int vi = (i * U + u) * NTH + tid;
            if (full || u * NTH < rem) {
                float x[VE];
                E::unpack(X[u], x);
                consume_vec<KIND, VE>(st, x, vi, ch, cl);
            }
        }
    };
    vec A[U], Bv[U];
    if (nb > 0) {
#pragma unroll
        for (int u = 0; u < U; ++u) A[u] = load_nt<E>(rs, voff, u * BSTRIDE);
    }
    if constexpr (KIND == K_TARGET || KIND == K_DRAFT) {
        if (nb == 0) fetch_lx();
    }
    for (int i = 0; i < nb; i += 2) {
        if (i + 1 < nb) {
#pragma unroll
            for (int u = 0; u < U; ++u) Bv[u] = load_nt<E>(rs, voff, ((i + 1) * U + u) * BSTRIDE);
        }
        consume(A, i);
        if constexpr (KIND == K_TARGET || KIND == K_DRAFT) {
            if (i == 0) fetch_lx();                        // the token arrived before batch 0
        }
        if (i + 1 >= nb) break;
        if (i + 2 < nb) {
#pragma unroll
            for (int u = 0; u < U; ++u) A[u] = load_nt<E>(rs, voff, ((i + 2) * U + u) * BSTRIDE);
        }
        consume(Bv, i + 1);
    }

    const float vb = st.t1;
    const int bvec = st.bvec;
    if (has_ht) consume_one<KIND>(st, sx, ch, cl);

    TileRec out;
    out.t1 = -INFINITY; out.t2 = -INFINITY;
    out.idx = 0x7fffffff; out.ref = 0.0f; out.s = 0.0; out.lx = 0.0f; out.flags = 0;
    if constexpr (KIND == K_GREEDY) {
        float t1 = st.t1, t2 = st.t2;
        block_top2(R, t1, t2);
        out.t1 = t1; out.t2 = t2;
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
        out.flags = block_max(R, st.nan) ? 1 : 0;
    } else {
        wave_rec<KIND>(R, st);
        lds_sync();
        if (tid == 0) {
            float a1 = R.t1[0], a2 = R.t2[0], r = R.ref[0];
            double sum = R.s[0];
            int nan = R.j[0];
            for (int q = 1; q < NTH / 64; ++q) {
                top2_merge(a1, a2, R.t1[q], R.t2[q]);
                sref_merge(r, sum, R.ref[q], R.s[q]);
                nan |= R.j[q];
            }
            out.t1 = a1;
            out.t2 = KIND == K_DRAFT ? -INFINITY : a2;
            if constexpr (KIND == K_TOP2) {
                out.flags = nan ? 1 : 0;
            } else {
                out.ref = r; out.s = sum;
                if (got) { out.lx = lx; out.flags = 2; }
            }
        }
    }
    return out;
}

// ------------------------------------------------------------------ decisions

// log2(s) for finite s > 0 in double precision with few registers (the
// library routine would raise the occupancy-limiting register count of the
// whole scan kernel): s = m 2^e with m in [sqrt(1/2), sqrt(2)), and
// ln m = 2 atanh(z), z = (m - 1)/(m + 1), |z| <= 0.172, by its odd series
// (terms through z^21, truncation below 3e-17).
__device__ inline double log2_lean(double s) {
    int e;
    double m = frexp(s, &e);                         // m in [0.5, 1)
    if (m < 0.70710678118654752) { m *= 2.0; --e; }
    const double z = (m - 1.0) / (m + 1.0);
    const double z2 = z * z;
    double t = 1.0 / 21.0;
    t = fma(t, z2, 1.0 / 19.0);
    t = fma(t, z2, 1.0 / 17.0);
    t = fma(t, z2, 1.0 / 15.0);
    t = fma(t, z2, 1.0 / 13.0);
    t = fma(t, z2, 1.0 / 11.0);
    t = fma(t, z2, 1.0 / 9.0);
    t = fma(t, z2, 1.0 / 7.0);
    t = fma(t, z2, 1.0 / 5.0);
    t = fma(t, z2, 1.0 / 3.0);
    t = fma(t, z2, 1.0);
    return static_cast<double>(e) + (2.0 * z * t) * 1.4426950408889634;
}

// 2^d in double precision with few registers: d = n + f, |f| <= 1/2, and
// 2^f = e^(f ln 2) by its Taylor series through degree 13 (truncation below
// 4e-18); 2^n by ldexp. -inf gives 0, +inf gives +inf.
__device__ inline double exp2_lean(double d) {
    if (!(d > -1100.0)) return 0.0;
    if (!(d < 1100.0)) return INFINITY;
    const double n = rint(d);
    const double g = (d - n) * 0.69314718055994531;
    double t = 1.0 / 6227020800.0;                   // 1/13!
    t = fma(t, g, 1.0 / 479001600.0);
    t = fma(t, g, 1.0 / 39916800.0);
    t = fma(t, g, 1.0 / 3628800.0);
    t = fma(t, g, 1.0 / 362880.0);
    t = fma(t, g, 1.0 / 40320.0);
    t = fma(t, g, 1.0 / 5040.0);
    t = fma(t, g, 1.0 / 720.0);
    t = fma(t, g, 1.0 / 120.0);
    t = fma(t, g, 1.0 / 24.0);
    t = fma(t, g, 1.0 / 6.0);
    t = fma(t, g, 0.5);
    t = fma(t, g, 1.0);
    t = fma(t, g, 1.0);
    return ldexp(t, static_cast<int>(n));
}


// Ragged drafts with at most RAG_INLINE batch rows: pass 1 packs the rows
// itself (four batch rows per thread, a workgroup scan into LDS) instead of
// waiting for rows_kernel.
constexpr int RAG_INLINE = 4 * NT;

template <class E, int MODE>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(7))) void scan_kernel(Params P) {
    __shared__ Red R2[2];
    __shared__ int RO[RAG_INLINE + 1];                     // ragged: first packed row of each batch row
    const int tid = threadIdx.x;
    const int k = P.k, V = P.V;
    // Workgroup w owns the flattened elements [w*L, (w+1)*L) of all B*rpb rows,
    // so every workgroup streams the same number of bytes and the grid is one
    // resident round. It emits one record per row segment, in slot row + w.
    const long long w = blockIdx.x;
    // pass 2's tables, a few entries per workgroup (entry j in workgroup
    // j mod G, thread j div G), so no workgroup starts its stream much later
    // than the others: 2^(j/N) of the fp64 exp, and (bf16) exp(v/T - C) of
    // every bf16 value v the table covers
    {
        if constexpr (MODE == SPEC_MODE_SAMPLE) {
            const long long ntab = EXP_N + (E::ES == 2 ? TAB_MAX : 0);
            const long long G = gridDim.x;
            for (long long j = w + G * tid; j < ntab; j += G * NT) {
                if (j < EXP_N) {
                    P.exptab[j] = exp2(static_cast<double>(j) / EXP_N);
                } else {
                    const long long t = j - EXP_N;
                    const unsigned sgn = t >= TAB_NEG ? 1u : 0u;
                    const unsigned mi = static_cast<unsigned>(t) - sgn * TAB_NEG;
                    const unsigned bits = (sgn << 15) | (mi + TAB_BASE);
                    const double v = __uint_as_float(bits << 16);
                    P.tautab[t] = mi < TAB_RANGE ? exp(fma(v, P.invT, -P.tab_c)) : 0.0;
                }
            }
        }
    }
    // ragged drafts: the packed rows, their slice length and element count
    long long L = P.L, N = P.N;
    const bool inl = P.dlen && P.B <= RAG_INLINE;          // uniform
    if (inl) {
        int n[4], loc = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int b = tid * 4 + q;
            int c = 0;
            if (b < P.B) {
                const int kb = P.dlen[b];
                if (kb >= 0 && kb <= k) c = MODE == SPEC_MODE_SAMPLE ? 2 * kb + 1 : kb + 1;
            }
            n[q] = c;
            loc += c;
        }
        const int lane = tid & 63, wv = tid >> 6;
        int x = loc;                                       // inclusive scan over the wave
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(x, off, 64);
            if (lane >= off) x += y;
        }
        if (lane == 63) R2[0].i[wv] = x;
        lds_sync();
        int pre = x - loc, tot = 0;
#pragma unroll
        for (int q = 0; q < NWAVE; ++q) {
            const int t = R2[0].i[q];
            pre += q < wv ? t : 0;
            tot += t;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int b = tid * 4 + q;
            if (b < P.B) {
                RO[b] = pre;
                if (w == 0) P.rowoff[b] = pre;
            }
            pre += n[q];
        }
        if (tid == 0) RO[P.B] = tot;
        N = static_cast<long long>(tot) * V;
        L = (N + gridDim.x - 1) / gridDim.x;
        if (L < 1) L = 1;
        if (w == 0 && tid == 0) { P.rhdr[0] = L; P.rhdr[1] = N; }
        lds_sync();                                        // RO complete; R2[0] free again
    } else if (P.dlen) {
        L = P.rhdr[0];
        N = P.rhdr[1];
    }
    const long long g0 = w * L;
    const long long g1 = g0 + L < N ? g0 + L : N;
    int seg = 0;
    for (long long g = g0; g < g1; ++seg) {
        Red& R = R2[seg & 1];
        const long long row = g / V;
        const int e0 = static_cast<int>(g - row * V);
        const long long rend = (row + 1) * V < g1 ? (row + 1) * V : g1;
        const int e1 = static_cast<int>(rend - row * V);
        // batch row, target or draft row, its position, and whether it is the
        // bonus row (the target row after the last draft position)
        int b, pos;
        bool draft, bonus;
        if (inl) {
            // the batch row holding packed row `row`: the largest b with RO[b] <= row
            int lo = 0, hi = P.B - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (RO[mid] <= row) lo = mid;
                else hi = mid - 1;
            }
            b = lo;
            const int j = static_cast<int>(row) - RO[b], nb = RO[b + 1] - RO[b];
            const int kb = MODE == SPEC_MODE_SAMPLE ? (nb - 1) >> 1 : nb - 1;
            draft = j > kb; pos = draft ? j - kb - 1 : j; bonus = j == kb;
        } else if (P.dlen) {
            const int code = P.rowmap[row];
            b = code >> 9; bonus = (code >> 8) & 1; draft = (code >> 7) & 1; pos = code & 127;
        } else {
            b = static_cast<int>(row / P.rpb);
            const int j = static_cast<int>(row % P.rpb);
            draft = j > k; pos = draft ? j - k - 1 : j; bonus = j == k;
        }
        const char* rowp;
        if (!draft)
            rowp = static_cast<const char*>(P.tgt) + (static_cast<size_t>(b) * (k + 1) + pos) * V * E::ES;
        else
            rowp = static_cast<const char*>(P.dft) + (static_cast<size_t>(b) * k + pos) * V * E::ES;
        TileRec tr;
        if constexpr (MODE == SPEC_MODE_GREEDY) {
            tr = tile_scan<E, K_GREEDY>(rowp, e0, e1, nullptr, P.ch, P.cl, R);
        } else {
            // the draft token of this row's position (every row but the bonus row)
            const int* tokp = P.tok + static_cast<size_t>(b) * k + pos;
            if (bonus) tr = tile_scan<E, K_TOP2>(rowp, e0, e1, nullptr, P.ch, P.cl, R);
            else if (!draft) tr = tile_scan<E, K_TARGET>(rowp, e0, e1, tokp, P.ch, P.cl, R);
            else tr = tile_scan<E, K_DRAFT>(rowp, e0, e1, tokp, P.ch, P.cl, R);
        }
        if (tid == 0) P.tiles[row + w] = tr;
        g = rend;
    }
}

// Ragged drafts: pack the rows each batch row uses (target rows 0..kb, then,
// in sampling mode, draft rows 0..kb-1) into pass 1's flattened space, so
// pass 1 reads only those. One workgroup scans the row counts in chunks of
// NTR batch rows; a draft length outside [0, k] contributes no rows. Also
// sets pass 1's slice length for its G workgroups.
constexpr int NTR = 1024;

__global__ __launch_bounds__(NTR) void rows_kernel(Params P) {
    __shared__ int wsum[NTR / 64];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const bool sample = P.mode == SPEC_MODE_SAMPLE;
    int carry = 0;
    for (int c0 = 0; c0 < P.B; c0 += NTR) {
        const int b = c0 + tid;
        int kb = -1, n = 0;
        if (b < P.B) {
            kb = P.dlen[b];
            if (kb >= 0 && kb <= P.k) n = sample ? 2 * kb + 1 : kb + 1;
        }
        int x = n;                                         // inclusive scan over the wave
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(x, off, 64);
            if (lane >= off) x += y;
        }
        if (lane == 63) wsum[wv] = x;
        __syncthreads();
        int pre = 0, tot = 0;
#pragma unroll
        for (int i = 0; i < NTR / 64; ++i) {
            const int t = wsum[i];
            pre += i < wv ? t : 0;
            tot += t;
        }
        const int r0 = carry + pre + x - n;
        if (b < P.B) {
            P.rowoff[b] = r0;
            for (int j = 0; j < n; ++j) {
                const int dr = j > kb;
                const int pos = dr ? j - kb - 1 : j;
                const int bonus = !dr && j == kb;
                P.rowmap[r0 + j] = (b << 9) | (bonus << 8) | (dr << 7) | pos;
            }
        }
        carry += tot;
        __syncthreads();                                   // wsum is reused
    }
    if (tid == 0) {
        const long long N = static_cast<long long>(carry) * P.V;
        const long long L = (N + P.G - 1) / P.G;
        P.rhdr[0] = L > 0 ? L : 1;
        P.rhdr[1] = N;
    }
}

// ------------------------------------------------------------------ decisions

struct Dec {
    RowRec rec[2 * SPEC_MAX_K + 1];
    int acc[SPEC_MAX_K + 1];
    float u1[SPEC_MAX_K + 1];
    int a;
    int valid;
    BatchRec br;
};

// Merge the segment records t[w0..w1] of one row in element order (earlier
// segments win ties of the greedy argmax); the first four are loaded together.
template <int MODE>
__device__ inline RowRec merge_row(const TileRec* t, long long w0, long long w1, bool with_sum) {
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
            m.flags |= o[u].flags & 1;
            if constexpr (MODE == SPEC_MODE_GREEDY) {
                if (o[u].t1 > prev) m.idx = o[u].idx;
            } else {
                sref_merge(m.ref, m.s, o[u].ref, o[u].s);
                if (o[u].flags & 2) { m.lx = o[u].lx; m.flags |= 2; }
            }
        }
    }
    RowRec rr;
    rr.m = m.t1; rr.t2 = m.t2; rr.idx = m.idx; rr.lg = 0.0; rr.lx = m.lx; rr.has_lx = (m.flags & 2) != 0;
    if (MODE == SPEC_MODE_GREEDY || !with_sum) {
        rr.valid = !(m.flags & 1) && m.t1 > -INFINITY && m.t1 < INFINITY;
    } else {
        rr.valid = (m.s == m.s) && m.s > 0.0 && m.s < INFINITY && m.t1 > -INFINITY && m.t1 < INFINITY;
        if (rr.valid) rr.lg = static_cast<double>(m.ref) + log2_lean(m.s);
    }
    return rr;
}

// Draft length, first row record and pass-1 slice length of batch row b. A
// draft length outside [0, k] gives kb = -1: the row has no records and is
// invalid.
struct RowSpan {
    int kb;
    long long row0, L;
};

__device__ inline RowSpan row_span(const Params& P, int b) {
    RowSpan r;
    if (P.dlen) {
        const int kb = P.dlen[b];
        r.kb = kb >= 0 && kb <= P.k ? kb : -1;
        r.row0 = P.rowoff[b];
        r.L = P.rhdr[0];
    } else {
        r.kb = P.k;
        r.row0 = static_cast<long long>(b) * P.rpb;
        r.L = P.L;
    }
    return r;
}

// Decide batch row b in one workgroup (any size of at least k + 1 and rpb
// threads): merge the segment records of its rows, evaluate the acceptance
// tests, and return (in every thread) what pass 2 needs. With `write`, also
// write the outputs and the batch record. A row with draft length kb < k
// decides positions 0..kb-1 with the bonus at row kb; its outputs past those
// are NaN (gap, p, q) and -1 (tokens).
template <class E, int MODE>
__device__ BatchRec decide_batch(const Params& P, Dec& D, int b, bool write) {
    const int tid = threadIdx.x;
    const int k = P.k, V = P.V;
    constexpr bool sample = MODE == SPEC_MODE_SAMPLE;
    const RowSpan sp = row_span(P, b);
    const bool kb_ok = sp.kb >= 0;
    const int kb = kb_ok ? sp.kb : 0;
    const int nrows = !kb_ok ? 0 : sample ? 2 * kb + 1 : kb + 1;

    // One round of independent loads: the draft token and uniform of position
    // tid, and the segment records of row tid (the draft-token logits came with
    // the records).
    int x = -1;
    double u0 = 0.0;
    if (tid < kb) {
        x = P.tok[static_cast<size_t>(b) * k + tid];
        if constexpr (sample) u0 = P.uni[(static_cast<size_t>(b) * (k + 1) + tid) * 2];
    }
    if (sample && tid <= kb) D.u1[tid] = P.uni[(static_cast<size_t>(b) * (k + 1) + tid) * 2 + 1];
    if (tid < nrows) {
        const long long row = sp.row0 + tid;
        const long long r0 = row * V;
        // the bonus target row kb of sampling mode carries no sum
        D.rec[tid] = merge_row<MODE>(P.tiles + row, r0 / sp.L, (r0 + V - 1) / sp.L, tid != kb);
    } else if (tid == 0) {
        D.rec[0].valid = 0;                                // no records: invalid draft length
    }
    if (write && tid <= k) {
        float g = __builtin_nanf("");
        if (tid < nrows && tid <= kb) {
            const RowRec& rr = D.rec[tid];
            g = (rr.t2 == -INFINITY) ? INFINITY : rr.m - rr.t2;
        }
        P.gap[static_cast<size_t>(b) * (k + 1) + tid] = g;
    }
    if (tid == 0) { D.valid = 1; D.a = kb; }
    lds_sync();

    int ok = 1;
    if (tid <= kb) ok = D.rec[tid].valid;                 // target rows 0..kb
    if (tid < k) {
        int acc = 0;
        float pf = __builtin_nanf(""), qf = __builtin_nanf("");
        if (tid < kb) {
            const bool inr = x >= 0 && x < V;
            if (!inr) ok = 0;
            if (sample && !D.rec[kb + 1 + tid].valid) ok = 0;
            if (sample && ok && !(D.rec[tid].has_lx && D.rec[kb + 1 + tid].has_lx)) ok = 0;
            if (ok) {
                const RowRec& rt = D.rec[tid];
                if constexpr (sample) {
                    // log2 p(x) = x*c - lg_p and log2 q(x) = x*c - lg_q, in double
                    const RowRec& rd = D.rec[kb + 1 + tid];
                    const double lt = rt.lx, ld = rd.lx;
                    const double c = P.c;
                    const double lp = lt == -INFINITY ? -INFINITY : lt * c - rt.lg;
                    const double lq = ld == -INFINITY ? -INFINITY : ld * c - rd.lg;
                    double r;
                    if (lq == -INFINITY) r = (lp == -INFINITY) ? 0.0 : INFINITY;
                    else r = exp2_lean(lp - lq);
                    acc = u0 < r;
                    pf = exp2f(static_cast<float>(lp));
                    qf = exp2f(static_cast<float>(lq));
                } else {
                    acc = (x == rt.idx);
                }
            }
            D.acc[tid] = acc;
        }
        const bool pq = tid < kb && ok;
        if (write && P.tprob) P.tprob[static_cast<size_t>(b) * k + tid] = pq ? pf : __builtin_nanf("");
        if (write && P.dprob) P.dprob[static_cast<size_t>(b) * k + tid] = pq ? qf : __builtin_nanf("");
    }
    if (!ok) atomicAnd(&D.valid, 0);
    lds_sync();
    const int valid = D.valid;
    if (tid == 0) {
        int a = kb;
        for (int i = 0; i < kb; ++i) if (!D.acc[i]) { a = i; break; }
        D.a = a;
    }
    lds_sync();
    const int a = D.a;
    if (write && tid <= k) {
        int o;
        if (!valid) o = -1;
        else if (tid < a) o = x;
        else if (tid == a) o = sample ? -1 : D.rec[a].idx;    // sampling: the draw writes it
        else o = -1;
        P.out_tok[static_cast<size_t>(b) * (k + 1) + tid] = o;
    }
    if (tid == 0) {
        if (write) P.acc_len[b] = valid ? a : -1;
        BatchRec br;
        br.a = valid ? a : -1;
        br.kb = kb;
        br.u1 = sample ? D.u1[a] : 0.0f;
        br.mp = D.rec[a].m;
        br.mq = sample && a < kb ? D.rec[kb + 1 + a].m : 0.0f;
        br.lam = 0.0;
        br.lam_hat = 0.0;
        if (sample && valid && a < kb) {
            // S_p/S_q in the exp((x - m)/T) normalisation of pass 2: only
            // used to place a relative band of ETA, so 2^d is taken as
            // 2^round(d) * exp2f(d - round(d)) (relative error ~1e-7)
            const RowRec& rt = D.rec[a];
            const RowRec& rd = D.rec[kb + 1 + a];
            const double c = P.c;
            const double d = (rt.lg - static_cast<double>(rt.m) * c) - (rd.lg - static_cast<double>(rd.m) * c);
            const double n = rint(d);
            br.lam = ldexp(static_cast<double>(exp2f(static_cast<float>(d - n))), static_cast<int>(n));
        }
        D.br = br;
    }
    lds_sync();
    return D.br;
}


// The same decision made by one wave when the batch row has at most 64 rows
// (rpb <= 64): lane r merges row r, and the acceptance tests, validity, the
// first rejection and the outputs use shuffles and ballots only, with no
// workgroup barrier. Called by the 64 lanes of one wave; the returned record
// is complete in every lane.
template <class E, int MODE>
__device__ BatchRec decide_wave(const Params& P, int b, bool write) {
    const int lane = threadIdx.x & 63;
    const int k = P.k, V = P.V;
    constexpr bool sample = MODE == SPEC_MODE_SAMPLE;
    const RowSpan sp = row_span(P, b);
    const bool kb_ok = sp.kb >= 0;
    const int kb = kb_ok ? sp.kb : 0;
    const int nrows = !kb_ok ? 0 : sample ? 2 * kb + 1 : kb + 1;
    int x = -1;
    double u0 = 0.0;
    float u1 = 0.0f;
    if (lane < kb) {
        x = P.tok[static_cast<size_t>(b) * k + lane];
        if constexpr (sample) u0 = P.uni[(static_cast<size_t>(b) * (k + 1) + lane) * 2];
    }
    if (sample && lane <= kb) u1 = P.uni[(static_cast<size_t>(b) * (k + 1) + lane) * 2 + 1];
    RowRec rr;
    rr.m = -INFINITY; rr.t2 = -INFINITY; rr.idx = 0x7fffffff; rr.valid = 0; rr.lg = 0.0; rr.lx = 0.0f; rr.has_lx = 0;
    if (lane < nrows) {
        const long long row = sp.row0 + lane;
        const long long r0 = row * V;
        // the bonus target row kb of sampling mode carries no sum
        rr = merge_row<MODE>(P.tiles + row, r0 / sp.L, (r0 + V - 1) / sp.L, lane != kb);
    }
    if (write && lane <= k) {
        const float g = lane >= nrows || lane > kb ? __builtin_nanf("")
                      : (rr.t2 == -INFINITY) ? INFINITY : rr.m - rr.t2;
        P.gap[static_cast<size_t>(b) * (k + 1) + lane] = g;
    }
    // draft row of position lane (lane < kb): lane kb + 1 + lane
    const int dl = lane < kb ? kb + 1 + lane : lane;
    const int d_valid = __shfl(rr.valid, dl, 64);
    const int d_has = __shfl(rr.has_lx, dl, 64);
    const float d_lx = __shfl(rr.lx, dl, 64);
    const double d_lg = __shfl(rr.lg, dl, 64);
    int ok = lane <= kb ? rr.valid : 1;                    // target rows 0..kb (none: invalid)
    int acc = 0;
    float pf = __builtin_nanf(""), qf = __builtin_nanf("");
    if (lane < kb) {
        if (!(x >= 0 && x < V)) ok = 0;
        if (sample && !d_valid) ok = 0;
        if (sample && ok && !(rr.has_lx && d_has)) ok = 0;
        if (ok) {
            if constexpr (sample) {
                // log2 p(x) = x*c - lg_p and log2 q(x) = x*c - lg_q, in double
                const double c = P.c;
                const double lt = rr.lx, ld = d_lx;
                const double lp = lt == -INFINITY ? -INFINITY : lt * c - rr.lg;
                const double lq = ld == -INFINITY ? -INFINITY : ld * c - d_lg;
                double r;
                if (lq == -INFINITY) r = (lp == -INFINITY) ? 0.0 : INFINITY;
                else r = exp2_lean(lp - lq);
                acc = u0 < r;
                pf = exp2f(static_cast<float>(lp));
                qf = exp2f(static_cast<float>(lq));
            } else {
                acc = (x == rr.idx);
            }
        }
    }
    if (lane < k) {
        const bool pq = lane < kb && ok;
        if (write && P.tprob) P.tprob[static_cast<size_t>(b) * k + lane] = pq ? pf : __builtin_nanf("");
        if (write && P.dprob) P.dprob[static_cast<size_t>(b) * k + lane] = pq ? qf : __builtin_nanf("");
    }
    const bool valid = __ballot(!ok) == 0;
    const unsigned long long rej = __ballot(lane < kb && !acc);
    const int a = rej ? __ffsll(static_cast<long long>(rej)) - 1 : kb;
    const int idx_a = __shfl(rr.idx, a, 64);
    if (write && lane <= k) {
        int o;
        if (!valid) o = -1;
        else if (lane < a) o = x;
        else if (lane == a) o = sample ? -1 : idx_a;    // sampling: the draw writes it
        else o = -1;
        P.out_tok[static_cast<size_t>(b) * (k + 1) + lane] = o;
    }
    if (write && lane == 0) P.acc_len[b] = valid ? a : -1;
    const float mp = __shfl(rr.m, a, 64);
    const double lgp = __shfl(rr.lg, a, 64);
    const int ad = a < kb ? kb + 1 + a : a;
    const float mq = __shfl(rr.m, ad, 64);
    const double lgq = __shfl(rr.lg, ad, 64);
    BatchRec br;
    br.a = valid ? a : -1;
    br.kb = kb;
    br.u1 = sample ? __shfl(u1, a, 64) : 0.0f;
    br.mp = mp;
    br.mq = sample && a < kb ? mq : 0.0f;
    br.lam = 0.0;
    br.lam_hat = 0.0;
    if (sample && valid && a < kb) {
        // S_p/S_q in the exp((x - m)/T) normalisation of pass 2 (see decide_batch)
        const double c = P.c;
        const double d = (lgp - static_cast<double>(mp) * c) - (lgq - static_cast<double>(mq) * c);
        const double n = rint(d);
        br.lam = ldexp(static_cast<double>(exp2f(static_cast<float>(d - n))), static_cast<int>(n));
    }
    return br;
}

// Greedy mode: the decisions are the whole result after pass 1.
template <class E, int MODE>
__global__ __launch_bounds__(NT) void decide_kernel(Params P) {
    __shared__ Dec D;
    if (P.rpb <= 64) {                                     // uniform
        if (threadIdx.x < 64) decide_wave<E, MODE>(P, blockIdx.x, true);
    } else {
        decide_batch<E, MODE>(P, D, blockIdx.x, true);
    }
}

// The confidence gate over n rows (batch rows with k = 0, after a greedy pass
// 1), one thread per row: gap and argmax from the merged records, then
// fire = the rule holds on the float32 gap and the argmax is admissible.
template <class E>
__global__ __launch_bounds__(NT) void gate_kernel(Params P) {
    const int r = static_cast<int>(blockIdx.x) * NT + static_cast<int>(threadIdx.x);
    if (r >= P.B) return;
    const long long r0 = static_cast<long long>(r) * P.V;
    const RowRec rr = merge_row<SPEC_MODE_GREEDY>(P.tiles + r, r0 / P.L, (r0 + P.V - 1) / P.L, false);
    int a = -1, fire = 0;
    float g = __builtin_nanf("");
    if (rr.valid) {
        a = rr.idx;
        g = rr.t2 == -INFINITY ? INFINITY : rr.m - rr.t2;
        const bool adm = !P.admit || ((P.admit[a >> 5] >> (a & 31)) & 1u);
        const bool pass = P.gate_rule == SPEC_GATE_MARGIN ? g > P.gate_tau
                                                          : (g > 0.0f && 2.0f * P.gate_tau <= g);
        fire = adm && pass;
    }
    P.out_tok[r] = a;
    P.gap[r] = g;
    P.fire[r] = fire;
}

// The confidence gate with one workgroup per row (NTG threads streaming the
// whole row): no pass-1 records and no second launch. One CU streams a row at
// only ~28 GB/s whatever the load depth (measured: 4, 8 or 16 vectors in
// flight per thread give 9.9, 9.8 and 9.2 us for one row of 128256 bf16), so
// below GATE_ROW_MIN rows a greedy pass 1 splits the rows over many
// workgroups and gate_kernel merges them (8.1 us for one row); from 16 rows on
// the per-row kernel is as fast or faster (46 us for 1024 rows, against 53).
constexpr int NTG = 1024;
constexpr int GATE_U = 4;                  // vectors per thread in each load batch
constexpr int GATE_ROW_MIN = 16;

template <class E>
__global__ __launch_bounds__(NTG) void gate_row_kernel(Params P) {
    __shared__ RedT<NTG / 64> R;
    const int r = blockIdx.x;
    const char* rowp = static_cast<const char*>(P.tgt) + static_cast<size_t>(r) * P.V * E::ES;
    const TileRec t = tile_scan<E, K_GREEDY, NTG, GATE_U>(rowp, 0, P.V, nullptr, 0.0f, 0.0f, R);
    if (threadIdx.x != 0) return;
    const bool valid = !(t.flags & 1) && t.t1 > -INFINITY && t.t1 < INFINITY;
    int a = -1, fire = 0;
    float g = __builtin_nanf("");
    if (valid) {
        a = t.idx;
        g = t.t2 == -INFINITY ? INFINITY : t.t1 - t.t2;
        const bool adm = !P.admit || ((P.admit[a >> 5] >> (a & 31)) & 1u);
        const bool pass = P.gate_rule == SPEC_GATE_MARGIN ? g > P.gate_tau
                                                          : (g > 0.0f && 2.0f * P.gate_tau <= g);
        fire = adm && pass;
    }
    P.out_tok[r] = a;
    P.gap[r] = g;
    P.fire[r] = fire;
}

// ------------------------------------------------------------------ pass 2

// exp(y) for y <= 0 in double precision, table-driven (P. T. P. Tang, "Table-
// driven implementation of the exponential function in IEEE floating-point
// arithmetic", ACM TOMS 15(2), 1989) and free of branches: write
// y = (N m + j) ln2/N + r with N = 1024 and |r| <= ln2/2048, so
// exp(y) = 2^m 2^(j/N) e^r. The nearest integer to y N/ln2 comes from adding
// 1.5*2^52 (its low word is the integer); ln2/N is split into a 32-bit head
// (so its product with the integer is exact) and a tail (the fdlibm split of
// ln 2); e^r - 1 is its Taylor polynomial of degree 3 (truncation below
// r^4/24 < 6e-16); 2^m is added to the exponent field of T[j] = 2^(j/N).
// Inputs at or below -708 give 0 (also -inf): those terms lie below 1e-307
// relative to the row maximum.
constexpr double EXP_INV_L = 0x1.71547652b82fep+10;   // N / ln 2
constexpr double EXP_L1 = 0x1.62e42fee00000p-11;      // head of ln 2 / N (32 bits)
constexpr double EXP_L2 = 0x1.a39ef35793c76p-43;      // ln 2 / N - EXP_L1
constexpr double EXP_SHIFT = 0x1.8p52;
constexpr double EXP_C3 = 1.0 / 6.0;

__device__ inline double exp_fast(double y, const double* T) {
    const double t = fma(y, EXP_INV_L, EXP_SHIFT);
    const double kf = t - EXP_SHIFT;
    double r = fma(-kf, EXP_L1, y);
    r = fma(-kf, EXP_L2, r);
    const int k = __double2loint(t);
    const double p = fma(r * r, fma(r, EXP_C3, 0.5), r);
    const double tj = T[k & (EXP_N - 1)];
    // (k >> 10) << 20, in unsigned arithmetic (two's complement wrap)
    const unsigned hi = static_cast<unsigned>(__double2hiint(tj)) + (static_cast<unsigned>(k & ~(EXP_N - 1)) << 10);
    const double s = __hiloint2double(static_cast<int>(hi), __double2loint(tj));
    const double res = fma(s, p, s);
    return y > -708.0 ? res : 0.0;
}

// ------------------------------------------------------------------ pass-2 element values

// A bf16 logit takes one of 2^16 values, so for bf16 inputs pass 2 reads
// tau(v) = exp(v/T - C) from a table indexed by the value's bits for every v
// with 2^-16 <= |v| < 2^8 (positive values at entry m - TAB_BASE for
// magnitude bits m, negative ones TAB_NEG entries further). The table is used
// for a batch row only when both rows' maxima lie below 2^kmax (kmax <= 8,
// the largest with 2^kmax/T <= 700); C = 2^kmax/T - 600 keeps every entry
// such a row can read finite, and a sum of V of them from overflowing. Other values
// (zero, tiny, -inf, very negative) take the fp64 exp of the same argument. A
// batch row uses the table when its rows' maxima lie inside it; otherwise
// every element takes the fp64 exp normalised by its row maximum. Either way
// only ratios of sums enter the draw, so the common scale does not matter.

struct Pass2 {
    const void* rowT;
    const void* rowD;
    unsigned bytes;            // bytes of one row
    double invT;
    double offT, offD;         // added to x/T inside the exp: -C (table) or -m/T (row max)
    double dm;                 // (m_p - m_q)/T
    double lam;                // S_p/S_q in this batch row's units (set by the draw)
    double lam_hat;            // pass 1's estimate of it, same units
    int tab;                   // values come from the bf16 table
    bool resid;
};

// Rows, exponent offsets and table choice of the draw of batch row b at row
// br.a (lam_hat is still in pass 1's units here).
template <class E>
__device__ inline Pass2 pass2_rows(const Params& P, int b, const BatchRec& br) {
    const int k = P.k, V = P.V, a = br.a < 0 ? 0 : br.a;
    Pass2 Q;
    Q.resid = a < br.kb;
    const size_t rt = static_cast<size_t>(b) * (k + 1) + a;
    const size_t rd = static_cast<size_t>(b) * k + a;
    Q.rowT = static_cast<const char*>(P.tgt) + rt * V * E::ES;
    Q.rowD = Q.resid ? static_cast<const char*>(P.dft) + rd * V * E::ES : Q.rowT;
    Q.bytes = static_cast<unsigned>(V) * E::ES;
    Q.invT = P.invT;
    const double mp = br.mp, mq = Q.resid ? static_cast<double>(br.mq) : mp;
    Q.dm = (mp - mq) * P.invT;
    Q.tab = E::ES == 2 && P.tab_on && fabs(mp) < P.tab_lim && fabs(mq) < P.tab_lim && fabs(Q.dm) < 600.0;
    Q.offT = Q.tab ? -P.tab_c : -mp * P.invT;
    Q.offD = Q.tab ? -P.tab_c : -mq * P.invT;
    Q.lam = 0.0;
    Q.lam_hat = br.lam;
    return Q;
}

// Bits of element q of a 16-byte bf16 vector.
__device__ inline unsigned bf16_bits(const u32x4& w, int q) {
    const unsigned word = (q >> 1) == 0 ? w.x : (q >> 1) == 1 ? w.y : (q >> 1) == 2 ? w.z : w.w;
    return (q & 1) ? (word >> 16) : (word & 0xffffu);
}

// out[q] = v where q == z, every other entry kept (z is not known at compile
// time; the array stays in registers).
template <int N>
__device__ inline void put_at(double (&out)[N], int z, double v) {
#pragma unroll
    for (int q = 0; q < N; ++q) out[q] = q == z ? v : out[q];
}

// The fp64 exp of element q (0..7) of a bf16 vector, in pass 2's units.
__device__ inline double val_exp_bf16(const u32x4& w, int q, double off, const Pass2& Q, const double* TE) {
    return exp_fast(fma(static_cast<double>(__uint_as_float(bf16_bits(w, q) << 16)), Q.invT, off), TE);
}

// Values of the VE elements of one 16-byte vector. With the bf16 table every
// lane reads all eight entries first (a magnitude outside the table is clamped
// to its edge, so the read stays inside it), so the LDS reads issue back to
// back; the rare out-of-range values then take the fp64 exp in a compact
// divergent loop. TAB = false: every value by the fp64 exp, unrolled (the
// draw's few elements).
template <class E, bool TAB = true>
__device__ inline void vals_vec(const typename E::vec& w, double off, const Pass2& Q, const double* TT,
                                const double* TE, double (&out)[E::VE]) {
    if constexpr (E::ES == 2 && !TAB) {
#pragma unroll
        for (int q = 0; q < 8; ++q) out[q] = val_exp_bf16(w, q, off, Q, TE);
    } else if constexpr (E::ES == 2) {
        if (Q.tab) {
            // both halves of a word at once with 16-bit lane arithmetic:
            // key = magnitude bits - TAB_BASE, clamped to the table (a value
            // outside it reads an edge entry and is replaced below), times 8
            // for a byte offset, plus the sign bit itself as 32768 bytes =
            // TAB_NEG entries; a half never carries into the other
            typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
            static_assert(TAB_NEG * sizeof(double) == 0x8000u && TAB_RANGE * sizeof(double) <= 0x8000u,
                          "sign bit is the negative-table offset");
            const u16x2 base = {static_cast<unsigned short>(TAB_BASE), static_cast<unsigned short>(TAB_BASE)};
            const u16x2 last = {static_cast<unsigned short>(TAB_RANGE - 1), static_cast<unsigned short>(TAB_RANGE - 1)};
            const char* tb = reinterpret_cast<const char*>(TT);
            bool oor = false;
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const unsigned word = d == 0 ? w.x : d == 1 ? w.y : d == 2 ? w.z : w.w;
                const u16x2 key = __builtin_bit_cast(u16x2, word & 0x7fff7fffu) - base;   // wraps below TAB_BASE
                const u16x2 kc = __builtin_elementwise_min(key, last);
                oor |= __builtin_bit_cast(unsigned, kc) != __builtin_bit_cast(unsigned, key);
                const unsigned off2 = __builtin_bit_cast(unsigned, kc << 3) | (word & 0x80008000u);
                out[2 * d] = *reinterpret_cast<const double*>(tb + (off2 & 0xffffu));
                out[2 * d + 1] = *reinterpret_cast<const double*>(tb + (off2 >> 16));
            }
            if (oor) {                                     // rare
#pragma unroll 1
                for (int q = 0; q < 8; ++q) {
                    if ((bf16_bits(w, q) & 0x7fffu) - TAB_BASE >= TAB_RANGE)
                        put_at(out, q, val_exp_bf16(w, q, off, Q, TE));
                }
            }
        } else {                                           // rows outside the table's range
#pragma unroll 1
            for (int q = 0; q < 8; ++q) put_at(out, q, val_exp_bf16(w, q, off, Q, TE));
        }
    } else {
        const float x[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) out[q] = exp_fast(fma(static_cast<double>(x[q]), Q.invT, off), TE);
    }
}

// Elements q >= n of a vector set to -inf (weight 0): the row's last vector
// when V is not a multiple of VE.
template <class E>
__device__ inline void mask_tail(typename E::vec& x, int n) {
    if constexpr (E::ES == 2) {
        unsigned wd[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int q = 0; q < 8; ++q)
            if (q >= n) wd[q >> 1] = (q & 1) ? ((wd[q >> 1] & 0xffffu) | 0xff800000u) : ((wd[q >> 1] & 0xffff0000u) | 0xff80u);
        x.x = wd[0]; x.y = wd[1]; x.z = wd[2]; x.w = wd[3];
    } else {
        float v[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (q >= n) v[q] = -INFINITY;
        x.x = v[0]; x.y = v[1]; x.z = v[2]; x.w = v[3];
    }
}

// Vector vi (VE elements, 16 bytes) of a row: one buffer load when rows are
// 16-byte aligned (VEC), else VE element loads. A lane that is not `in` reads
// zeros without touching memory. Elements past V are not masked here.
template <class E, bool VEC>
__device__ inline typename E::vec load_vec(__amdgpu_buffer_rsrc_t rs, const void* row, unsigned bytes, int vi,
                                           int V, bool in) {
    if constexpr (VEC) {
        const unsigned voff = in ? static_cast<unsigned>(vi) * 16u : bytes;
        return __builtin_bit_cast(typename E::vec, __builtin_amdgcn_raw_buffer_load_b128(rs, static_cast<int>(voff), 0, 0));
    } else {
        (void)rs; (void)bytes;
        const int j0 = vi * E::VE;
        if constexpr (E::ES == 2) {
            const unsigned short* r = static_cast<const unsigned short*>(row);
            unsigned h[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) h[q] = (in && j0 + q < V) ? r[j0 + q] : 0u;
            u32x4 w;
            w.x = h[0] | (h[1] << 16); w.y = h[2] | (h[3] << 16);
            w.z = h[4] | (h[5] << 16); w.w = h[6] | (h[7] << 16);
            return w;
        } else {
            const float* r = static_cast<const float*>(row);
            f32x4 w;
            w.x = (in && j0 < V) ? r[j0] : 0.0f;
            w.y = (in && j0 + 1 < V) ? r[j0 + 1] : 0.0f;
            w.z = (in && j0 + 2 < V) ? r[j0 + 2] : 0.0f;
            w.w = (in && j0 + 3 < V) ? r[j0 + 3] : 0.0f;
            return w;
        }
    }
}

// Band elements of one lane's share of a segment (pass 2), grouped by their
// exact logit difference x_t - x_d: every element of a group has the same
// ratio e/f, so the group lies on one side of the exact lambda and its
// residual is max(0, sum e - lambda sum f). A lane keeps one group (its first
// band key); a second key marks the lane as conflicting, and the segment is
// then recomputed by the draw. At the end of the segment the lanes' groups
// are merged by key, in the order of the lowest lane holding each key.
struct LaneBand {
    double key, se, sf;
    int state;                 // 0: no band element, 1: one key, 2: several keys
};

template <class E>
struct SegLds {
    alignas(16) double TT[E::ES == 2 ? TAB_MAX : 2];
    alignas(16) double TE[EXP_N];
    Dec D;
};

// pass 2's tables held in registers between their loads and the LDS stores,
// so the loads overlap the decision. Threads t0 .. NTS-1 take part (the
// first wave is left out while it decides): at most one vector of the exp
// table and four of the value table per thread.
template <class E>
struct TableRegs {
    static constexpr int NTT = E::ES == 2 ? (TAB_MAX / 2 + (NTS - 64) - 1) / (NTS - 64) : 0;
    u32x4 te;
    u32x4 tt[NTT > 0 ? NTT : 1];
};

template <class E>
__device__ inline void tables_fetch(const Params& P, TableRegs<E>& R, int t0) {
    static_assert(EXP_N / 2 <= NTS - 64, "at most one exp-table vector per thread");
    const int t = static_cast<int>(threadIdx.x) - t0, nt = NTS - t0;
    if (t < 0) return;
    if (t < EXP_N / 2) R.te = reinterpret_cast<const u32x4*>(P.exptab)[t];
    if constexpr (E::ES == 2) {
        if (P.tab_on) {
#pragma unroll
            for (int q = 0; q < TableRegs<E>::NTT; ++q) {
                const int i = q * nt + t;
                if (i < TAB_MAX / 2) R.tt[q] = reinterpret_cast<const u32x4*>(P.tautab)[i];
            }
        }
    }
}

template <class E>
__device__ inline void tables_store(const Params& P, const TableRegs<E>& R, double* TT, double* TE, int t0) {
    const int t = static_cast<int>(threadIdx.x) - t0, nt = NTS - t0;
    if (t < 0) return;
    if (t < EXP_N / 2) reinterpret_cast<u32x4*>(TE)[t] = R.te;
    if constexpr (E::ES == 2) {
        if (P.tab_on) {
#pragma unroll
            for (int q = 0; q < TableRegs<E>::NTT; ++q) {
                const int i = q * nt + t;
                if (i < TAB_MAX / 2) reinterpret_cast<u32x4*>(TT)[i] = R.tt[q];
            }
        }
    }
}

// Sums of one wave's segment: S_p, S_q and, over the elements that are
// certainly positive for every lambda in the band around lam_hat, E and F;
// band elements go to the wave's list.
// Logit difference x_t - x_d of element q (exact in double).
template <class E>
__device__ inline double band_key(const typename E::vec& xt, const typename E::vec& xd, int q) {
    if constexpr (E::ES == 2) {
        return static_cast<double>(__uint_as_float(bf16_bits(xt, q) << 16)) -
               static_cast<double>(__uint_as_float(bf16_bits(xd, q) << 16));
    } else {
        const float a = q == 0 ? xt.x : q == 1 ? xt.y : q == 2 ? xt.z : xt.w;
        const float d = q == 0 ? xd.x : q == 1 ? xd.y : q == 2 ? xd.z : xd.w;
        return static_cast<double>(a) - static_cast<double>(d);
    }
}

// Sums of one vector pair: S_p, S_q and, over the elements that are
// certainly positive for every lambda in the band around lam_hat, E and F;
// band elements go to the lane's group.
template <class E, bool RESID>
__device__ inline void seg_vector(const typename E::vec& xt, const typename E::vec& xd, const Pass2& Q,
                                  double hi_b, double lo_b, const double* TT, const double* TE, LaneBand& L,
                                  double (&acc)[4]) {
    constexpr int VE = E::VE;
    double e[VE], f[VE];
    vals_vec<E>(xt, Q.offT, Q, TT, TE, e);
    if constexpr (RESID) vals_vec<E>(xd, Q.offD, Q, TT, TE, f);
#pragma unroll
    for (int q = 0; q < VE; ++q) {
        acc[0] += e[q];
        if constexpr (RESID) {
            acc[1] += f[q];
            const bool pos = e[q] > hi_b * f[q];
            const double pd = pos ? 1.0 : 0.0;
            acc[2] = fma(e[q], pd, acc[2]);
            acc[3] = fma(f[q], pd, acc[3]);
            if (!pos && e[q] > lo_b * f[q]) {              // rare: inside the band
                const double k = band_key<E>(xt, xd, q);
                if (L.state == 0) { L.key = k; L.state = 1; }
                if (k == L.key) { L.se += e[q]; L.sf += f[q]; }
                else L.state = 2;
            }
        }
    }
}

// Vectors per lane and row loaded together. Two measured best on MI355X:
// larger groups hold more registers and leave the first loads exposed longer.
template <bool VEC>
struct SegU {
    static constexpr int U = SEG_U;
};

template <class E, bool VEC, bool RESID>
__device__ inline void seg_group(const Params& P, const Pass2& Q, __amdgpu_buffer_rsrc_t rsT,
                                 __amdgpu_buffer_rsrc_t rsD, int v0, int v1, int t0, int T, double hi_b,
                                 double lo_b, const double* TT, const double* TE, LaneBand& L, double (&acc)[4],
                                 const typename E::vec (&xt)[SegU<VEC>::U], const typename E::vec (&xd)[SegU<VEC>::U]) {
    const int lane = threadIdx.x & 63;
    const int tailn = P.V - (P.nvec - 1) * E::VE;          // elements of the row's last vector
#pragma unroll
    for (int u = 0; u < SegU<VEC>::U; ++u) {
        const int vi = v0 + ((t0 + u) << 6) + lane;
        if (t0 + u < T && vi < v1) {
            typename E::vec a = xt[u], d = xd[u];
            if (vi == P.nvec - 1 && tailn < E::VE) {       // rare: the row's partial last vector
                mask_tail<E>(a, tailn);
                if constexpr (RESID) mask_tail<E>(d, tailn);
            }
            seg_vector<E, RESID>(a, d, Q, hi_b, lo_b, TT, TE, L, acc);
        }
    }
}

template <class E, bool VEC, bool RESID>
__device__ inline void seg_issue(const Pass2& Q, __amdgpu_buffer_rsrc_t rsT, __amdgpu_buffer_rsrc_t rsD, int V,
                                 int v0, int v1, int t0, int T, typename E::vec (&xt)[SegU<VEC>::U],
                                 typename E::vec (&xd)[SegU<VEC>::U]) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int u = 0; u < SegU<VEC>::U; ++u) {
        const int vi = v0 + ((t0 + u) << 6) + lane;
        const bool in = t0 + u < T && vi < v1;
        xt[u] = load_vec<E, VEC>(rsT, Q.rowT, Q.bytes, vi, V, in);
        if constexpr (RESID) xd[u] = load_vec<E, VEC>(rsD, Q.rowD, Q.bytes, vi, V, in);
    }
}

// One wave's segment of a batch row, then its record.
template <class E, bool VEC, bool RESID>
__device__ inline void seg_run(const Params& P, const Pass2& Q, int b, int s, int v0, int v1, SegLds<E>& S) {
    const int lane = threadIdx.x & 63;
    const __amdgpu_buffer_rsrc_t rsT = make_rsrc(Q.rowT, Q.bytes);
    const __amdgpu_buffer_rsrc_t rsD = make_rsrc(Q.rowD, RESID ? Q.bytes : 0u);
    const int T = (v1 - v0 + 63) >> 6;
    const double hi_b = Q.lam_hat * (1.0 + ETA), lo_b = Q.lam_hat * (1.0 - ETA);
    LaneBand L;
    L.key = 0.0; L.se = 0.0; L.sf = 0.0; L.state = 0;
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
    for (int t0 = 0; t0 < T; t0 += SegU<VEC>::U) {
        typename E::vec xt[SegU<VEC>::U], xd[SegU<VEC>::U];
        seg_issue<E, VEC, RESID>(Q, rsT, rsD, P.V, v0, v1, t0, T, xt, xd);
        seg_group<E, VEC, RESID>(P, Q, rsT, rsD, v0, v1, t0, T, hi_b, lo_b, S.TT, S.TE, L, acc, xt, xd);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] = wave_sum(acc[q]);
    // merge the lanes' band groups by key (uniform; rare)
    int n = 0;
    double se[MAX_AMB] = {0.0, 0.0, 0.0, 0.0}, sf[MAX_AMB] = {0.0, 0.0, 0.0, 0.0};
    if (__any(L.state != 0)) {
        if (__any(L.state == 2)) {
            n = MAX_AMB + 1;                               // a lane met two keys: recompute
        } else {
            bool pend = L.state == 1;
            while (__any(pend)) {                          // one round per distinct key
                const int l = __ffsll(static_cast<long long>(__ballot(pend))) - 1;
                const double k = __shfl(L.key, l, 64);
                const bool m = pend && L.key == k;
                const double a = wave_sum(m ? L.se : 0.0), c = wave_sum(m ? L.sf : 0.0);
                if (n < MAX_AMB) {
#pragma unroll
                    for (int g = 0; g < MAX_AMB; ++g) { se[g] = g == n ? a : se[g]; sf[g] = g == n ? c : sf[g]; }
                    ++n;
                } else {
                    n = MAX_AMB + 1;
                    break;
                }
                pend = pend && !m && lane != l;            // lane l always leaves
            }
        }
    }
    if (lane == 0) {
        SegRec r;
        r.sp = acc[0]; r.sq = acc[1]; r.e = acc[2]; r.f = acc[3];
        r.namb = n;
#pragma unroll
        for (int g = 0; g < MAX_AMB; ++g) {
            const bool h = g < n;
            r.ae[g] = h ? se[g] : 0.0;
            r.af[g] = h ? sf[g] : 0.0;
        }
#pragma unroll
        for (int q = 0; q < 7; ++q) r.pad[q] = 0;
        P.segs[static_cast<size_t>(b) * P.nseg + s] = r;
    }
}

// Pass 2, sampling mode. Batch row b has W = P.wpb workgroups of NTS/64 waves
// and its selected row pair (or bonus row) is split into 16W equal segments of
// whole 16-byte vectors, one per wave. Each workgroup decides b itself (the W
// copies agree; workgroup 0 writes the outputs and the batch record), issues
// its waves' loads, and then every wave streams its segment with lane-
// interleaved vectors and no workgroup barrier, ending with one record.
template <class E, bool VEC>
__global__ __launch_bounds__(NTS) __attribute__((amdgpu_waves_per_eu(4))) void seg_kernel(Params P) {
    __shared__ SegLds<E> S;
    const int tid = threadIdx.x;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, kept in an SGPR
    const int W = P.wpb;
    const int b = blockIdx.x / W, w = blockIdx.x % W;
    const int s = w * (NTS / 64) + wv;
    const int v0 = min(P.nvec, s * P.vps), v1 = min(P.nvec, v0 + P.vps);

    TableRegs<E> TR;
    BatchRec br;
    if (P.rpb <= 64) {                                     // uniform
        // wave 0 decides (its loads first in its queue) while the other
        // waves load and store the tables
        if (wv == 0) {
            br = decide_wave<E, SPEC_MODE_SAMPLE>(P, b, w == 0);
            if (tid == 0) S.D.br = br;
        } else {
            tables_fetch<E>(P, TR, 64);
            tables_store<E>(P, TR, S.TT, S.TE, 64);
        }
        lds_sync();                                        // decision and tables ready
        br = S.D.br;
    } else {
        tables_fetch<E>(P, TR, 64);                        // in flight during the decision
        br = decide_batch<E, SPEC_MODE_SAMPLE>(P, S.D, b, w == 0);
        tables_store<E>(P, TR, S.TT, S.TE, 64);
        lds_sync();                                        // tables ready
    }
    Pass2 Q = pass2_rows<E>(P, b, br);
    if (Q.tab) Q.lam_hat = br.lam * exp_fast(Q.dm, S.TE);  // into table units
    if (w == 0 && tid == 0) {
        br.lam_hat = Q.lam_hat;
        P.bat[b] = br;
    }
    if (br.a < 0) return;                                  // uniform: whole block leaves
    if (Q.resid) seg_run<E, VEC, true>(P, Q, b, s, v0, v1, S);
    else seg_run<E, VEC, false>(P, Q, b, s, v0, v1, S);
}

struct DrawLds {
    RedT<NT2 / 64> R;
    alignas(16) double TE[EXP_N];
    double mass[MAXS];
    double scan[NT2 / 64];
    double base;
    // the segment selection of the one-wave path
    double lam, tgt;
    int sstar, resid, slow;
};

// Vectors [v0, v1) of segment s.
__device__ inline void seg_range(const Params& P, int s, int& v0, int& v1) {
    v0 = min(P.nvec, s * P.vps);
    v1 = min(P.nvec, v0 + P.vps);
}

// Mass of segment s recomputed element by element with the values of the
// rescan (whole block: 16-byte vectors, thread-sequential sums, then a fixed
// block reduction).
template <class E>
__device__ double seg_exact(const Params& P, const Pass2& Q, int s, DrawLds& S) {
    constexpr int VE = E::VE;
    int v0, v1;
    seg_range(P, s, v0, v1);
    const __amdgpu_buffer_rsrc_t rsT = make_rsrc(Q.rowT, Q.bytes);
    const __amdgpu_buffer_rsrc_t rsD = make_rsrc(Q.rowD, Q.resid ? Q.bytes : 0u);
    const int tailn = P.V - (P.nvec - 1) * VE;
    double acc[1] = {0.0};
#pragma unroll 1
    for (int vb = v0; vb < v1; vb += NT2) {
        const int vi = vb + static_cast<int>(threadIdx.x);
        const bool in = vi < v1;
        typename E::vec xt, xd;
        if (P.vec_ok) {
            xt = load_vec<E, true>(rsT, Q.rowT, Q.bytes, vi, P.V, in);
            xd = load_vec<E, true>(rsD, Q.rowD, Q.bytes, vi, P.V, in && Q.resid);
        } else {
            xt = load_vec<E, false>(rsT, Q.rowT, Q.bytes, vi, P.V, in);
            xd = load_vec<E, false>(rsD, Q.rowD, Q.bytes, vi, P.V, in && Q.resid);
        }
        if (vi == P.nvec - 1 && tailn < VE) { mask_tail<E>(xt, tailn); mask_tail<E>(xd, tailn); }
        // one element at a time (few registers: this is the rare path)
#pragma unroll 1
        for (int q = 0; q < VE; ++q) {
            double e, f = 0.0;
            if constexpr (E::ES == 2) {
                e = val_exp_bf16(xt, q, Q.offT, Q, S.TE);
                if (Q.resid) f = val_exp_bf16(xd, q, Q.offD, Q, S.TE);
            } else {
                const float xs[4] = {xt.x, xt.y, xt.z, xt.w}, ds[4] = {xd.x, xd.y, xd.z, xd.w};
                e = exp_fast(fma(static_cast<double>(xs[q]), Q.invT, Q.offT), S.TE);
                if (Q.resid) f = exp_fast(fma(static_cast<double>(ds[q]), Q.invT, Q.offD), S.TE);
            }
            const double x = Q.resid ? e - Q.lam * f : e;
            if (x > 0.0 && in) acc[0] += x;
        }
    }
    block_sum<1>(S.R, acc);
    return acc[0];
}

// Mass of one segment from its record (NaN: must be recomputed exactly):
// the certain-positive sums, then each band group in the order it was met.
__device__ inline double seg_mass(const SegRec& r, const Pass2& Q, bool band_ok) {
    if (!Q.resid) return r.sp;
    if (!band_ok || r.namb > MAX_AMB) return __builtin_nan("");
    double m = r.e - Q.lam * r.f;
    if (!(m > 0.0)) m = 0.0;
#pragma unroll
    for (int g = 0; g < MAX_AMB; ++g) {
        if (g < r.namb) {
            const double w = r.ae[g] - Q.lam * r.af[g];
            m += w > 0.0 ? w : 0.0;
        }
    }
    return m;
}

// The draw of batch row b: one workgroup per batch row. Exact lambda from the
// segment sums, segment masses, ordered scan to the segment holding u*Z, and
// an fp64 rescan of that segment in vocabulary order.
template <class E>
__global__ __launch_bounds__(NT2) void draw_kernel(Params P) {
    __shared__ DrawLds S;
    constexpr int VE = E::VE;
    const int tid = threadIdx.x;
    const int b = blockIdx.x;
    const int k = P.k, V = P.V, NS = P.nseg;
    const SegRec* recs = P.segs + static_cast<size_t>(b) * NS;
    // one round of independent loads: exp table, batch record, this thread's first segment record
    const u32x4 te = reinterpret_cast<const u32x4*>(P.exptab)[tid];
    const BatchRec br = P.bat[b];
    SegRec r0;
    if (tid < NS) r0 = recs[tid];
    reinterpret_cast<u32x4*>(S.TE)[tid] = te;
    if (br.a < 0) return;                                  // uniform: whole block leaves
    const int a = br.a;
    Pass2 Q = pass2_rows<E>(P, b, br);
    Q.lam_hat = br.lam_hat;
    // The draw evaluates its few elements with the fp64 exp in the same units
    // as the segment records (for the bf16 table, exp(v/T - C) agrees with the
    // table entry to ~1e-15 relative), so it needs no copy of the table.
    Q.tab = 0;
    const double u1 = br.u1;
    const int lane = tid & 63, wv = tid >> 6;
    int sstar = 0;
    double tgt = 0.0;
    bool selected = false;
    if (NS <= 64) {
        // one segment per lane of wave 0: exact lambda, masses, inclusive
        // scan and the segment holding u*Z with wave operations only
        if (wv == 0) {
            const bool has = lane < NS;
            const double sp = wave_sum(has ? r0.sp : 0.0), sq = wave_sum(has ? r0.sq : 0.0);
            const double lh = Q.lam_hat;
            Q.lam = Q.resid ? sp / sq : 0.0;
            const bool band_ok = !Q.resid ||
                (!P.force_exact && Q.lam >= lh * (1.0 - ETA) && Q.lam <= lh * (1.0 + ETA));
            int slow = 0, ss = 0;
            double base = 0.0, t = 0.0;
            for (int attempt = 0; attempt < 2; ++attempt) {
                const double m = has ? seg_mass(r0, Q, band_ok) : 0.0;
                if (__any(m != m)) { slow = 1; break; }    // a segment needs the exact recompute
                double x = m;                              // inclusive scan over the lanes
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    const double y = __shfl_up(x, off, 64);
                    if (lane >= off) x += y;
                }
                const double Z = __shfl(x, 63, 64);
                if (Q.resid && !(Z > 0.0)) { Q.resid = false; continue; }   // residual rounded to zero: p_a
                t = u1 * Z;
                const unsigned long long hit = __ballot(has && x > t);
                if (hit) {
                    ss = __ffsll(static_cast<long long>(hit)) - 1;
                } else {                                   // rounding: last segment with mass
                    const unsigned long long pos = __ballot(has && m > 0.0);
                    ss = pos ? 63 - __clzll(static_cast<long long>(pos)) : 0;
                }
                base = __shfl(x, ss > 0 ? ss - 1 : 0, 64);
                if (ss == 0) base = 0.0;
                break;
            }
            if (lane == 0) {
                S.slow = slow; S.sstar = ss; S.base = base; S.tgt = t; S.lam = Q.lam; S.resid = Q.resid;
            }
        }
        lds_sync();                                        // also publishes the exp table
        if (!S.slow) {
            selected = true;
            sstar = S.sstar; tgt = S.tgt; Q.lam = S.lam; Q.resid = S.resid != 0;
        }
    }
    if (!selected) {
        // the block path: many segments, or a segment to recompute exactly
        double sums[2] = {tid < NS ? r0.sp : 0.0, tid < NS ? r0.sq : 0.0};
        for (int s = tid + NT2; s < NS; s += NT2) { sums[0] += recs[s].sp; sums[1] += recs[s].sq; }
        block_sum<2>(S.R, sums);                           // also publishes the exp table
        const double lh = Q.lam_hat;
        Q.resid = br.a < br.kb;
        Q.lam = Q.resid ? sums[0] / sums[1] : 0.0;
        const bool band_ok = !Q.resid ||
            (!P.force_exact && Q.lam >= lh * (1.0 - ETA) && Q.lam <= lh * (1.0 + ETA));
        double* M = S.mass;
        for (int attempt = 0; attempt < 2; ++attempt) {
            if (tid < NS) M[tid] = seg_mass(r0, Q, band_ok);
            for (int s = tid + NT2; s < NS; s += NT2) M[s] = seg_mass(recs[s], Q, band_ok);
            lds_sync();
            // contiguous segment ranges per thread -> ordered scan
            const int cpt = (NS + NT2 - 1) / NT2;
            const int c0 = min(NS, tid * cpt), c1 = min(NS, c0 + cpt);
            double mine = 0.0;
            for (int c = c0; c < c1; ++c) mine += M[c];
            double Z;
            double pre = block_exscan<NT2 / 64>(S.scan, mine, Z);
            if (Z != Z) {                                  // rare: a segment must be recomputed exactly
                for (int s = 0; s < NS; ++s) {
                    if (M[s] != M[s]) {
                        const double m = seg_exact<E>(P, Q, s, S);
                        if (tid == 0) M[s] = m;
                        lds_sync();
                    }
                }
                mine = 0.0;
                for (int c = c0; c < c1; ++c) mine += M[c];
                pre = block_exscan<NT2 / 64>(S.scan, mine, Z);
            }
            if (Q.resid && !(Z > 0.0)) {                  // residual mass rounded to zero: use p_a
                Q.resid = false;
                lds_sync();
                continue;
            }
            tgt = u1 * Z;
            // segment holding the target
            int cand = 0x7fffffff;
            {
                double run = pre;
                for (int c = c0; c < c1; ++c) {
                    const double nx = run + M[c];
                    if (nx > tgt) { cand = c; break; }
                    run = nx;
                }
            }
            sstar = block_min(S.R, cand);
            if (sstar == 0x7fffffff) {                     // rounding: last segment with mass
                int last = -1;
                for (int c = tid; c < NS; c += NT2) if (M[c] > 0.0) last = max(last, c);
                sstar = block_max(S.R, last);
                if (sstar < 0) sstar = 0;
            }
            if (c0 <= sstar && sstar < c1) {
                double run = pre;
                for (int c = c0; c < sstar; ++c) run += M[c];
                S.base = run;                               // mass before s*
            }
            lds_sync();                                    // S.base visible
            break;
        }
    }
    {
        // rescan s* in element order: round r covers vectors v0 + r*NT2 + [0, NT2)
        int v0, v1;
        seg_range(P, sstar, v0, v1);
        double run0 = S.base;
        int tok = 0x7fffffff, lastpos = -1;
        const __amdgpu_buffer_rsrc_t rsT = make_rsrc(Q.rowT, Q.bytes);
        const __amdgpu_buffer_rsrc_t rsD = make_rsrc(Q.rowD, Q.resid ? Q.bytes : 0u);
        const int tailn = V - (P.nvec - 1) * VE;
        for (int vb = v0; vb < v1; vb += NT2) {
            const int vi = vb + tid;
            const bool in = vi < v1;
            typename E::vec xt, xd;
            if (P.vec_ok) {
                xt = load_vec<E, true>(rsT, Q.rowT, Q.bytes, vi, V, in);
                xd = load_vec<E, true>(rsD, Q.rowD, Q.bytes, vi, V, in && Q.resid);
            } else {
                xt = load_vec<E, false>(rsT, Q.rowT, Q.bytes, vi, V, in);
                xd = load_vec<E, false>(rsD, Q.rowD, Q.bytes, vi, V, in && Q.resid);
            }
            if (vi == P.nvec - 1 && tailn < VE) { mask_tail<E>(xt, tailn); mask_tail<E>(xd, tailn); }
            double w[VE];
            double wsum = 0.0;
            double e[VE], f[VE];
            vals_vec<E, false>(xt, Q.offT, Q, nullptr, S.TE, e);
            if (Q.resid) vals_vec<E, false>(xd, Q.offD, Q, nullptr, S.TE, f);
#pragma unroll
            for (int q = 0; q < VE; ++q) {
                double x = Q.resid ? e[q] - Q.lam * f[q] : e[q];
                if (!(x > 0.0) || !in) x = 0.0;
                w[q] = x;
                wsum += x;
            }
            double tot;
            const double wpre = block_exscan<NT2 / 64>(S.scan, wsum, tot);
            const int jv = vi * VE;
            if (tok == 0x7fffffff) {
                double run = run0 + wpre;
#pragma unroll
                for (int q = 0; q < VE; ++q) {
                    if (w[q] > 0.0) lastpos = jv + q;
                    run += w[q];
                    if (run > tgt && tok == 0x7fffffff) tok = jv + q;
                }
            } else {
#pragma unroll
                for (int q = 0; q < VE; ++q) if (w[q] > 0.0) lastpos = jv + q;
            }
            run0 += tot;
        }
        tok = block_min(S.R, tok);
        if (tok == 0x7fffffff) {
            tok = block_max(S.R, lastpos);
            if (tok < 0) tok = v0 * VE;
        }
        if (tid == 0) P.out_tok[static_cast<size_t>(b) * (k + 1) + a] = tok;
    }
}

// ------------------------------------------------------------------ commit / rollback

// After a verify step: every batch row with a = accepted_len in [0, k] keeps
// the KV entries of the pending token and its a accepted drafts (kv_len +=
// 1 + a) and takes recurrent-state checkpoint slot a as its live state; other
// rows are left alone. The state copy is a plain stream: each workgroup moves
// one chunk of one row with 16-byte vectors (4-byte words when the buffers or
// the row size are not 16-byte multiples), every thread holding CPV loads in
// flight and writing with non-temporal stores. Measured on 64 rows of 4 MiB:
// 8, 16 and 32 loads in flight take 130, 89 and 92 us (the runtime's own
// device copy of the same bytes: 99 us); plain stores at 16: 104 us.
constexpr int NTC = 256;
constexpr int CPV = 16;
constexpr size_t COMMIT_CHUNK = static_cast<size_t>(NTC) * CPV * 16;   // bytes per workgroup

struct CommitParams {
    const int* acc;
    int* kv_len;               // may be null
    const char* slots;         // [B, k+1, row] bytes, may be null (with state)
    char* state;               // [B, row] bytes
    size_t row;                // state bytes per batch row
    int B, k;
    int chunks;                // workgroups per batch row
    int vec16;                 // 16-byte vectors usable
};

__global__ __launch_bounds__(NTC) void commit_kernel(CommitParams C) {
    const int b = static_cast<int>(blockIdx.x) / C.chunks, c = static_cast<int>(blockIdx.x) % C.chunks;
    const int a = C.acc[b];
    if (a < 0 || a > C.k) return;                          // uniform: nothing to commit
    if (c == 0 && threadIdx.x == 0 && C.kv_len) C.kv_len[b] += 1 + a;
    if (!C.state) return;
    const char* src = C.slots + (static_cast<size_t>(b) * (C.k + 1) + a) * C.row;
    char* dst = C.state + static_cast<size_t>(b) * C.row;
    const size_t lo = static_cast<size_t>(c) * COMMIT_CHUNK;
    const size_t hi = lo + COMMIT_CHUNK < C.row ? lo + COMMIT_CHUNK : C.row;
    if (C.vec16) {
        const u32x4* s4 = reinterpret_cast<const u32x4*>(src + lo);
        u32x4* d4 = reinterpret_cast<u32x4*>(dst + lo);
        const int n = static_cast<int>((hi - lo) / 16);
        u32x4 v[CPV];
#pragma unroll
        for (int u = 0; u < CPV; ++u) {
            const int i = u * NTC + static_cast<int>(threadIdx.x);
            if (i < n) v[u] = s4[i];
        }
#pragma unroll
        for (int u = 0; u < CPV; ++u) {
            const int i = u * NTC + static_cast<int>(threadIdx.x);
            if (i < n) __builtin_nontemporal_store(v[u], d4 + i);
        }
    } else {
        const unsigned* s1 = reinterpret_cast<const unsigned*>(src + lo);
        unsigned* d1 = reinterpret_cast<unsigned*>(dst + lo);
        const int n = static_cast<int>((hi - lo) / 4);
        for (int i = static_cast<int>(threadIdx.x); i < n; i += NTC) d1[i] = s1[i];
    }
}

// ------------------------------------------------------------------ int8 LM head + greedy verification
//
// The verify forward's last step, the LM-head projection of the k + 1 hidden
// states of every batch row, fused with greedy verification: with an int8
// head (per-row fp32 scales of the hidden states and of the vocabulary rows)
//     acc[m, v]   = sum_j h[m, j] * w[v, j]                       (int32, exact)
//     logit[m, v] = fl32(fl32(float(acc[m, v]) * h_scale[m]) * w_scale[v]),
// and the greedy decision needs of every row only its first argmax and its
// top-2 values. The head kernels compute the logits tile by tile on the matrix
// cores and reduce them in registers, so they never reach memory:
//   * one workgroup per 256-vocabulary x (64*MB)-hidden-row tile (MB = 4 or
//     2), 2 x 2 waves; the vocabulary rows are the MFMA's A operand, so each
//     lane's accumulators hold 16 vocabulary entries of ONE hidden row and
//     the row reduction is per lane (then one exchange with lane ^ 32 and one
//     through LDS between the two vocabulary waves);
//   * d (a multiple of 128) streams through LDS in 64-byte stages loaded
//     straight into LDS, several stages in flight (head_main);
//   * since the products are exact integers, the order of the d-sum is free:
//     the K layout of the MFMA only has to be the same for both operands;
//   * workgroups are numbered so that the hidden-row tiles of one vocabulary
//     tile run on one XCD and share its weights through that XCD's L2.
// Each workgroup writes one record (top-2, first argmax, NaN flag) per hidden
// row; head_merge_kernel merges the vocabulary tiles of every row into one
// pass-1 record (slot 2m: pass 1's slot rule with one slice per row), and
// decide_kernel makes the greedy decisions exactly as after pass 1.

constexpr int HV = 256;                 // vocabulary rows per head tile
constexpr int HK = 128;                 // d must be a multiple of this
constexpr int NTH = 256;                // threads per head workgroup

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

struct HeadRec {                        // one hidden row over one vocabulary tile
    float t1, t2;
    int idx;                            // first index of t1 (INT_MAX if none)
    int flags;                          // bit 0: a NaN logit
};

// Sampling mode: one hidden row over one vocabulary tile, in pass 1's terms
// (top-2, the sum 2^(x*c - ref) for an integer ref, a NaN flag).
struct alignas(8) HeadRecS {
    float t1, t2, ref;
    int flags;                          // bit 0: a NaN logit
    double s;
};

// The epilogue a head workgroup runs on its accumulators.
enum : int { EPI_GREEDY = 0, EPI_SAMPLE = 1 };

struct HeadParams {
    const signed char* h;               // [M, d]
    const float* hs;                    // [M]
    const signed char* w;               // [V, d]
    const float* ws;                    // [V]
    HeadRec* rec;                       // [M, nvt] (greedy)
    TileRec* tiles;                     // [2M], row m's merged record at 2m
    int M, V, d;
    int nvt, nmt;                       // vocabulary and hidden-row tiles
    // sampling: records, the exponent scale, and which draft token each row holds
    HeadRecS* recs;                     // [M, nvt]
    float ch, cl;                       // log2(e)/T = ch + cl, as pass 1's
    const int* tok;                     // draft tokens [B, k]
    int k;
    int role;                           // 0: target rows b*(k+1)+i, 1: draft rows b*k+i
    int rpb;                            // rows per batch row of the merged records (2k+1)
    float* logits;                      // [M, V] float32, every logit (sampling)
    double* exptab;                     // pass 2's exp table (sampling, target head), written by the merge
    int packed;                         // w in the tile-major layout of head_pack_kernel
};

// The draft token whose logit hidden row m carries (-1: none; the bonus row).
__device__ inline int head_row_token(const HeadParams& H, int m) {
    if (H.role == 0) {
        const int i = m % (H.k + 1);
        return i < H.k ? H.tok[static_cast<size_t>(m / (H.k + 1)) * H.k + i] : -1;
    }
    return H.tok[m];
}

// Fold logit x of vocabulary index v (ascending within a lane) into a top-2
// and first argmax; NaN never enters.
__device__ inline void head_take(float x, int v, float& t1, float& t2, int& i1) {
    const bool up = x > t1;
    t2 = up ? t1 : fmaxf(t2, x);
    i1 = up ? v : i1;
    t1 = up ? x : t1;
}

// Merge two top-2 records; the lower index wins a tie of the maxima.
__device__ inline void head_merge(float& t1, float& t2, int& i1, int& fl, float u1, float u2, int j1, int g) {
    const bool take = u1 > t1 || (u1 == t1 && j1 < i1);
    t2 = fmaxf(fmaxf(t2, u2), fminf(t1, u1));
    i1 = take ? j1 : i1;
    t1 = take ? u1 : t1;
    fl |= g;
}

// Scale the accumulators of one lane to logits and reduce them to a top-2
// per hidden row (EDGE: the tile reaches past V, so entries past it are skipped).
template <int MB, bool EDGE>
__device__ inline void head_epilogue(const HeadParams& H, const i32x16 (&acc)[4][MB], const float* WS, int v0,
                                     int mrow, int vw, int hi, float (&T1)[MB], float (&T2)[MB], int (&I1)[MB],
                                     int (&FL)[MB]) {
    float hsv[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int m = mrow + 32 * mb;
        hsv[mb] = m < H.M ? H.hs[m] : 0.0f;
        T1[mb] = -INFINITY; T2[mb] = -INFINITY; I1[mb] = 0x7fffffff; FL[mb] = 0;
    }
#pragma unroll
    for (int vb = 0; vb < 4; ++vb) {
        const int vbase = v0 + 128 * vw + 32 * vb + 4 * hi;
        float wsv[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) wsv[q] = WS[vbase - v0 + 8 * (q >> 2) + (q & 3)];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int v = vbase + 8 * (q >> 2) + (q & 3);
                float x = (static_cast<float>(acc[vb][mb][q]) * hsv[mb]) * wsv[q];
                FL[mb] |= x != x;
                if (EDGE) x = v < H.V ? x : -INFINITY;
                head_take(x, v, T1[mb], T2[mb], I1[mb]);
            }
    }
}

// Sampling mode: scale one lane's accumulators to logits and fold them, for
// each of its MB hidden rows, into pass 1's terms over the lane's 64 logits,
// eight at a time and in one pass, as pass 1's lanes do: the top-2, a NaN
// flag, and the sum 2^(x*c - ref) whose integer reference follows the running
// maximum (ref = ceil(max * ch), the sum rescaled by an exact power of two
// when it moves; eight terms summed in float32, then in double; a +inf logit
// poisons the sum). WB adds -inf past V (the tile edge) and 0 elsewhere, so
// the edge costs no per-entry compare: fmaf(a, w, 0) rounds as a * w does.
// The code has no branch, so the accumulators stay in place.
template <int MB>
__device__ inline void head_epilogue_sample(const HeadParams& H, const i32x16 (&acc)[4][MB], const float* WS,
                                            const float* WB, int mrow, int vw, int hi, HeadRecS (&o)[MB]) {
    float hsv[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int m = mrow + 32 * mb;
        hsv[mb] = m < H.M ? H.hs[m] : 0.0f;
        o[mb] = HeadRecS{-INFINITY, -INFINITY, 0.0f, 0, 0.0};
    }
#pragma unroll
    for (int vb = 0; vb < 4; ++vb) {
        const int vloc = 128 * vw + 32 * vb + 4 * hi;     // the lane's entries: vloc + 8*(q/4) + q%4
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            float wsv[8], wbv[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int q = 8 * g + j;
                wsv[j] = WS[vloc + 8 * (q >> 2) + (q & 3)];
                wbv[j] = WB[vloc + 8 * (q >> 2) + (q & 3)];
            }
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                HeadRecS& r = o[mb];
                const float before = r.t1;
                float x[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float y = fmaf(static_cast<float>(acc[vb][mb][8 * g + j]) * hsv[mb], wsv[j], wbv[j]);
                    r.flags |= y != y ? 1 : 0;
                    r.t2 = fmaxf(r.t2, fminf(r.t1, y));
                    r.t1 = fmaxf(r.t1, y);
                    x[j] = y;
                }
                // the shift is 0 unless the maximum rose
                const float nr = r.t1 > before ? ceilf(r.t1 * H.ch) : r.ref;
                const bool bad = !(nr <= 3.0e38f);                 // +inf logit or overflow: poison
                const int sh = static_cast<int>(fmaxf(r.ref - nr, -2000.0f));
                r.s = bad ? __builtin_nan("") : ldexp(r.s, sh);
                r.ref = bad ? 0.0f : nr;
                float e[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) e[j] = exp_term(x[j], H.ch, H.cl, r.ref);
#pragma unroll
                for (int w = 1; w < 8; w <<= 1) {
#pragma unroll
                    for (int j = 0; j + w < 8; j += 2 * w) e[j] += e[j + w];
                }
                r.s += static_cast<double>(e[0]);
            }
        }
    }
}

// Merge two sampling records of one hidden row (disjoint vocabulary ranges).
__device__ inline void head_recs_merge(HeadRecS& a, const HeadRecS& b) {
    top2_merge(a.t1, a.t2, b.t1, b.t2);
    sref_merge(a.ref, a.s, b.ref, b.s);
    a.flags |= b.flags;
}

// What a head workgroup needs besides its main loop: its tile (workgroup b
// runs on XCD b % 8, so tiles are dealt out in 8 contiguous runs, one per
// XCD: the hidden-row tiles of a vocabulary tile run together and share its
// weights through that XCD's L2) and the epilogue.
template <int MB, int NMW = 2>
struct HeadTile {
    static constexpr int BM = 32 * MB * NMW;               // hidden rows per tile
    static constexpr int NTHR = 128 * NMW;                 // threads: 2 x NMW waves
    int t, vw, mw, r, hi, vt, v0, m0, nv, nm;

    __device__ explicit HeadTile(const HeadParams& H) {
        t = static_cast<int>(threadIdx.x);
        const int lane = t & 63, wv = t >> 6;
        vw = wv & 1; mw = wv >> 1; r = lane & 31; hi = lane >> 5;
        const unsigned nb = gridDim.x, b = blockIdx.x, per = nb / 8;
        const unsigned tix = b < per * 8 ? (b % 8) * per + b / 8 : b;
        vt = static_cast<int>(tix) / H.nmt;
        const int mt = static_cast<int>(tix) % H.nmt;
        v0 = vt * HV; m0 = mt * BM;
        nv = min(HV, H.V - v0);
        nm = min(BM, H.M - m0);
    }
    // lane holds hidden row 32*MB*mw + 32*mb + r and, in register q of block
    // vb, vocabulary row 128*vw + 32*vb + 8*(q/4) + 4*hi + q%4; S (the LDS
    // stages, free again) carries the exchange between the vocabulary waves
    __device__ void finish(const HeadParams& H, const i32x16 (&acc)[4][MB], unsigned char* S) const {
        float T1[MB], T2[MB];
        int I1[MB], FL[MB];
        const int mrow = m0 + 32 * MB * mw + r;
        // the tile's weight scales go through LDS (one per thread), so the
        // epilogue reads them with short LDS loads instead of holding many
        // global loads in flight beside the accumulators
        float* WS = reinterpret_cast<float*>(S + 2 * BM * sizeof(HeadRec));
        for (int i = t; i < HV; i += NTHR) WS[i] = v0 + i < H.V ? H.ws[v0 + i] : 0.0f;
        __syncthreads();
        if (v0 + HV <= H.V) head_epilogue<MB, false>(H, acc, WS, v0, mrow, vw, hi, T1, T2, I1, FL);
        else head_epilogue<MB, true>(H, acc, WS, v0, mrow, vw, hi, T1, T2, I1, FL);
        HeadRec* L = reinterpret_cast<HeadRec*>(S);        // [2][BM]: per vocabulary wave
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const float u1 = __shfl_xor(T1[mb], 32, 64), u2 = __shfl_xor(T2[mb], 32, 64);
            const int j1 = __shfl_xor(I1[mb], 32, 64), g = __shfl_xor(FL[mb], 32, 64);
            head_merge(T1[mb], T2[mb], I1[mb], FL[mb], u1, u2, j1, g);
            if (hi == 0) L[vw * BM + 32 * MB * mw + 32 * mb + r] = HeadRec{T1[mb], T2[mb], I1[mb], FL[mb]};
        }
        __syncthreads();
        if (t < nm) {
            HeadRec o = L[t];
            const HeadRec p = L[BM + t];
            head_merge(o.t1, o.t2, o.idx, o.flags, p.t1, p.t2, p.idx, p.flags);
            H.rec[static_cast<size_t>(m0 + t) * H.nvt + vt] = o;
        }
    }

    // Sampling: the same exchange with pass 1's terms; one HeadRecS per row.
    __device__ void finish_sample(const HeadParams& H, const i32x16 (&acc)[4][MB], unsigned char* S) const {
        HeadRecS o[MB];
        const int mrow = m0 + 32 * MB * mw + r;
        float* WS = reinterpret_cast<float*>(S + 2 * BM * sizeof(HeadRecS));
        float* WB = WS + HV;
        for (int i = t; i < HV; i += NTHR) {
            WS[i] = v0 + i < H.V ? H.ws[v0 + i] : 0.0f;
            WB[i] = v0 + i < H.V ? 0.0f : -INFINITY;
        }
        __syncthreads();
        head_epilogue_sample<MB>(H, acc, WS, WB, mrow, vw, hi, o);
        HeadRecS* L = reinterpret_cast<HeadRecS*>(S);      // [2][BM]: per vocabulary wave
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            HeadRecS p;
            p.t1 = __shfl_xor(o[mb].t1, 32, 64); p.t2 = __shfl_xor(o[mb].t2, 32, 64);
            p.ref = __shfl_xor(o[mb].ref, 32, 64); p.flags = __shfl_xor(o[mb].flags, 32, 64);
            p.s = __shfl_xor(o[mb].s, 32, 64);
            head_recs_merge(o[mb], p);
            if (hi == 0) L[vw * BM + 32 * MB * mw + 32 * mb + r] = o[mb];
        }
        __syncthreads();
        if (t < nm) {
            HeadRecS a = L[t];
            head_recs_merge(a, L[BM + t]);
            H.recs[static_cast<size_t>(m0 + t) * H.nvt + vt] = a;
        }
    }

    // Logit store: logits[m, v] in float32 for every row m < M and v < V. One
    // hidden-row block mb at a time, the 64 rows x 256 logits of the tile go
    // through LDS (row pitch 260 floats, so the 16-byte writes of 16
    // consecutive rows hit distinct banks), and each wave then stores whole
    // rows: 64 lanes x 16 bytes = one contiguous 1 KB segment per instruction,
    // where the accumulator layout would give each store 32 rows.
    static constexpr int SR = NMW < 2 ? 32 * NMW : 64;    // rows of the logit slab
    static constexpr int NH = NMW < 2 ? 1 : NMW / 2;       // slab rounds per hidden-row block

    __device__ void finish_logits(const HeadParams& H, const i32x16 (&acc)[4][MB], unsigned char* S) const {
        constexpr int PITCH = HV + 4;
        float* R = reinterpret_cast<float*>(S);                         // [SR][PITCH]
        float* WS = R + SR * PITCH;
        for (int i = t; i < HV; i += NTHR) WS[i] = v0 + i < H.V ? H.ws[v0 + i] : 0.0f;
        const bool vec = (H.V & 3) == 0;                   // rows start 16-byte aligned
        const int lr = 32 * (mw & 1) + r;                  // the lane's row in the slab
        __syncthreads();
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int m = m0 + 32 * MB * mw + 32 * mb + r;
            const float hsv = m < H.M ? H.hs[m] : 0.0f;
#pragma unroll
            for (int h = 0; h < NH; ++h) {                 // the slab holds the rows of waves 2h, 2h+1
                if ((mw >> 1) == h) {                      // uniform per wave
#pragma unroll
                    for (int vb = 0; vb < 4; ++vb)
#pragma unroll
                        for (int c = 0; c < 4; ++c) {
                            const int col = 128 * vw + 32 * vb + 8 * c + 4 * hi;
                            f32x4 y;
#pragma unroll
                            for (int j = 0; j < 4; ++j)
                                y[j] = (static_cast<float>(acc[vb][mb][4 * c + j]) * hsv) * WS[col + j];
                            *reinterpret_cast<f32x4*>(R + lr * PITCH + col) = y;
                        }
                }
                __syncthreads();
                const int ch = t & 63, v = v0 + 4 * ch;
#pragma unroll 4
                for (int it = 0; it < SR * 64 / NTHR; ++it) {
                    const int row = (NTHR / 64) * it + (t >> 6);
                    const int mm = m0 + 32 * MB * (2 * h + (row >> 5)) + 32 * mb + (row & 31);
                    if (mm >= H.M) continue;
                    const f32x4 y = *reinterpret_cast<const f32x4*>(R + row * PITCH + 4 * ch);
                    float* dst = H.logits + static_cast<size_t>(mm) * H.V + v;
                    if (vec && v + 3 < H.V) {
                        __builtin_nontemporal_store(y, reinterpret_cast<f32x4*>(dst));
                    } else {
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            if (v + j < H.V) __builtin_nontemporal_store(y[j], dst + j);
                    }
                }
                __syncthreads();
            }
        }
    }
};

template <int MB>
__device__ inline void acc_zero(i32x16 (&acc)[4][MB]) {
#pragma unroll
    for (int vb = 0; vb < 4; ++vb)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[vb][mb][q] = 0;
}

// The main loop: 2 x NMW waves of 128 x 32*MB. The d-slices go from memory
// straight into LDS (16-byte buffer loads with the LDS as destination, no
// staging registers): 64 bytes of d per stage, NBUF stage buffers, the loads
// of NBUF - 1 stages in flight. Stage layout: row q (256 weight rows, then
// 64*MB hidden rows) at q*64, its 16-byte chunk c at c ^ ((q >> 2) & 3), so
// the operand reads of 16 consecutive lanes (rows r..r+15, one chunk) cover
// all banks. One load instruction of a wave fills 16 rows (1 KB, lane l at
// 16*l), so each lane fetches the chunk that lands at its position. Half-way
// through stage ks each wave waits for its own loads of stage ks + 1, a
// barrier makes everyone's visible (and certifies that stage ks - 1 has been
// read by all waves), the loads of stage ks + NBUF - 1 go into that free
// buffer, and the first operands of stage ks + 1 are read while the MFMAs of
// stage ks finish.
constexpr int HKW = 64;                 // bytes of d per stage

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// s_waitcnt immediate: vmcnt <= n (bits 3:0 and 15:14), expcnt and lgkmcnt unconstrained
constexpr int vm_wait(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// wait until at most `stages` later stages (LPW loads each) of this wave are in flight
template <int LPW, int MAXS>
__device__ inline void wait_stages(int stages) {
    static_assert(MAXS * LPW <= 63 && MAXS <= 4, "vmcnt range");
    if (MAXS >= 4 && stages >= 4) __builtin_amdgcn_s_waitcnt(vm_wait(4 * LPW));
    else if (MAXS >= 3 && stages >= 3) __builtin_amdgcn_s_waitcnt(vm_wait(3 * LPW));
    else if (MAXS >= 2 && stages >= 2) __builtin_amdgcn_s_waitcnt(vm_wait(2 * LPW));
    else if (stages >= 1) __builtin_amdgcn_s_waitcnt(vm_wait(LPW));
    else __builtin_amdgcn_s_waitcnt(vm_wait(0));
}

template <int MB, int NBUF, int EPI = EPI_GREEDY, int NMW = 2>
__device__ __attribute__((always_inline)) inline void head_main(const HeadParams& H) {
    constexpr int NW = 2 * NMW;                            // waves
    constexpr int BM = 32 * MB * NMW;
    constexpr int ST = (HV + BM) * HKW;                    // bytes per stage
    constexpr int WRW = HV / NW, HRW = BM / NW;            // weight and hidden rows each wave loads
    constexpr int LPW = (WRW + HRW) / 16;                  // load instructions per wave and stage
    static_assert(WRW % 16 == 0 && HRW % 16 == 0, "whole load instructions");
    constexpr int P = NBUF - 1;                            // stages in flight
    __shared__ __attribute__((aligned(16))) unsigned char S[NBUF * ST];
    const HeadTile<MB, NMW> w(H);
    const int lane = w.t & 63, wv = w.t >> 6;
    const unsigned d = static_cast<unsigned>(H.d);
    // weights row-major: the tile's nv rows; tile-major (head_pack_kernel):
    // the tile's HV rows, stage ks a contiguous 16 KB image of the stage
    // buffer's weight part, zeros past V
    const __amdgpu_buffer_rsrc_t rw =
        H.packed ? make_rsrc(H.w + static_cast<size_t>(w.vt) * HV * d, static_cast<unsigned>(HV) * d)
                 : make_rsrc(H.w + static_cast<size_t>(w.v0) * d, static_cast<unsigned>(w.nv) * d);
    const __amdgpu_buffer_rsrc_t rh = make_rsrc(H.h + static_cast<size_t>(w.m0) * d, static_cast<unsigned>(w.nm) * d);
    // loads: weight instruction j of wave wv fills rows wv*WRW + 16j .. +15,
    // hidden instruction j rows wv*HRW + 16j .. +15; lane l lands on row
    // + l/4, physical chunk l % 4, which holds logical chunk
    // (l % 4) ^ ((l >> 4) & 3); rows past the tile load zeros. In the
    // tile-major layout the image is stored as it lands: lane l at 16 l.
    const unsigned cl = static_cast<unsigned>(((lane & 3) ^ ((lane >> 4) & 3)) << 4);
    const unsigned low = H.packed ? static_cast<unsigned>(wv * WRW * HKW + 16 * lane)
                                  : static_cast<unsigned>(wv * WRW + (lane >> 2)) * d + cl;
    const unsigned wjs = H.packed ? 16u * HKW : 16u * d;  // per load instruction
    const unsigned wks = H.packed ? static_cast<unsigned>(HV * HKW) : static_cast<unsigned>(HKW); // per stage
    const unsigned loh = static_cast<unsigned>(wv * HRW + (lane >> 2)) * d + cl;
    auto issue = [&](int ks) {
        unsigned char* B = S + (ks % NBUF) * ST;
        const unsigned k0 = static_cast<unsigned>(ks * HKW);
#pragma unroll
        for (int j = 0; j < WRW / 16; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_ptr_t)(B + (wv * WRW + 16 * j) * HKW), 16,
                                                     static_cast<int>(low + static_cast<unsigned>(ks) * wks + wjs * j),
                                                     0, 0, 0);
#pragma unroll
        for (int j = 0; j < HRW / 16; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rh, (lds_ptr_t)(B + (HV + wv * HRW + 16 * j) * HKW), 16,
                                                     static_cast<int>(loh + k0 + 16u * j * d), 0, 0, 0);
    };
    // operands: A row 128*vw + 32*vb + r, B row 256 + 32*MB*mw + 32*mb + r;
    // K step s (two per stage) reads logical chunk 2s + hi
    const int ra = (128 * w.vw + w.r) * HKW, rb = (HV + 32 * MB * w.mw + w.r) * HKW, sw = (w.r >> 2) & 3;
    i32x4 fa[2][4], fb[2][MB];
    auto frag = [&](int ks, int s, int slot) {
        const unsigned char* B = S + (ks % NBUF) * ST;
        const int co = ((2 * s + w.hi) ^ sw) << 4;
#pragma unroll
        for (int vb = 0; vb < 4; ++vb) fa[slot][vb] = *reinterpret_cast<const i32x4*>(B + ra + vb * 32 * HKW + co);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) fb[slot][mb] = *reinterpret_cast<const i32x4*>(B + rb + mb * 32 * HKW + co);
    };
    i32x16 acc[4][MB];
    acc_zero<MB>(acc);
    auto mma = [&](int slot) {
#pragma unroll
        for (int vb = 0; vb < 4; ++vb)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                acc[vb][mb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[slot][vb], fb[slot][mb], acc[vb][mb], 0, 0, 0);
    };
    const int nks = H.d / HKW;                             // >= 2
    for (int q = 0; q < P && q < nks; ++q) issue(q);
    wait_stages<LPW, P - 1>(min(P, nks) - 1);              // stage 0 is in
    __syncthreads();
    frag(0, 0, 0);
    // the last stage is peeled off, so the second MFMA group of every loop
    // stage is reached only past the barrier (whose wait retired the reads of
    // its operands): no LDS wait holds it up behind the next stage's reads
    for (int ks = 0; ks < nks - 1; ++ks) {
        frag(ks, 1, 1);
        mma(0);
        wait_stages<LPW, P - 1>(min(P - 2, nks - 2 - ks)); // stage ks + 1 is in
        __syncthreads();
        if (ks + P < nks) issue(ks + P);
        frag(ks + 1, 0, 0);
        mma(1);
    }
    frag(nks - 1, 1, 1);
    mma(0);
    mma(1);
    __syncthreads();                                       // every wave is done with the stages
    // the epilogues reuse the stage buffers
    static_assert(NBUF * ST >= 2 * BM * static_cast<int>(sizeof(HeadRec)) + HV * 4, "greedy exchange");
    static_assert(NBUF * ST >= 2 * BM * static_cast<int>(sizeof(HeadRecS)) + 2 * HV * 4, "sampling exchange");
    static_assert(NBUF * ST >= (HeadTile<MB, NMW>::SR * (HV + 4) + HV) * 4, "logit slab");
    if constexpr (EPI == EPI_SAMPLE) {
        w.finish_sample(H, acc, S);
        w.finish_logits(H, acc, S);                        // after the exchange: the LDS is free again
    } else {
        w.finish(H, acc, S);
    }
}

// 32-row tiles when d is a multiple of 512. Such a call streams the head from
// HBM, and the rate of that stream depends on how much of each weight row one
// stage takes: in a probe of these loads alone, 64 bytes of 256 rows per
// stage (head_main's shape) streamed at ~4.2 TB/s and 512 bytes of 64 rows at
// ~5.0. So a stage here holds 512 bytes of d for one 32-row block of each
// wave (block ks % 4 of its four, bytes 512 * (ks / 4) on) and of the 32
// hidden rows: 48 KB, three buffers, one workgroup per CU, 16 MFMAs per wave
// and stage. Against head_main's 32-row tile the kernel measured 1-5% faster
// at V = 128256, d = 4096, and 18% at V = 151936 (594 tiles, which also fit
// one workgroup per CU better than two).
// Rows are 512 bytes in LDS; logical chunk c of stage row R sits at physical
// chunk c ^ (R % 16), so the operand reads of 16 consecutive lanes (rows
// r..r+15, one chunk) cover all banks, and each loading lane fetches the
// chunk that lands at its position. At the barrier of stage ks every wave has
// read all of stage ks, so stage ks + 3 goes into its buffer. The epilogues
// are head_main's (same accumulator layout).
template <int EPI>
__device__ __attribute__((always_inline)) inline void head_main_w512(const HeadParams& H) {
    using Tile = HeadTile<1, 1>;
    constexpr int RB = 512;                                // bytes of d per stage and row
    constexpr int ST = (64 + 32) * RB;                     // 2 x 32 weight rows, 32 hidden rows
    constexpr int NBUF = 3, P = 3;                         // stages in flight
    constexpr int LPW = (32 + 16) * RB / 1024;             // load instructions per wave and stage
    __shared__ __attribute__((aligned(16))) unsigned char S[NBUF * ST];
    const Tile w(H);
    const int lane = w.t & 63, wv = w.t >> 6;
    const unsigned d = static_cast<unsigned>(H.d);
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(H.w + static_cast<size_t>(w.v0) * d, static_cast<unsigned>(w.nv) * d);
    const __amdgpu_buffer_rsrc_t rh = make_rsrc(H.h + static_cast<size_t>(w.m0) * d, static_cast<unsigned>(w.nm) * d);
    // load j of wave wv fills stage rows 2j and 2j + 1 of its weight block
    // (rows 32*wv + ..) and of its half of the hidden rows (rows 64 + 16*wv
    // + ..); lane l lands on the first + l/32, physical chunk l % 32
    const int lr = lane >> 5, pc = lane & 31;
    auto issue = [&](int ks) {
        unsigned char* B = S + (ks % NBUF) * ST;
        const int vb = ks & 3;
        const unsigned k0 = static_cast<unsigned>(ks >> 2) * RB;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const unsigned c = static_cast<unsigned>(pc ^ ((2 * j + lr) & 15));
            const unsigned row = static_cast<unsigned>(128 * wv + 32 * vb + 2 * j + lr);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_ptr_t)(B + (32 * wv + 2 * j) * RB), 16,
                                                     static_cast<int>(row * d + k0 + 16u * c), 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const unsigned c = static_cast<unsigned>(pc ^ ((2 * j + lr) & 15));
            const unsigned row = static_cast<unsigned>(16 * wv + 2 * j + lr);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rh, (lds_ptr_t)(B + (64 + 16 * wv + 2 * j) * RB), 16,
                                                     static_cast<int>(row * d + k0 + 16u * c), 0, 0, 0);
        }
    };
    // operands of K step s (16 per stage): A row 32*vw + r, B row 64 + r,
    // logical chunk 2s + hi; both rows are r modulo 16
    const int ra = (32 * w.vw + w.r) * RB, rb = (64 + w.r) * RB, sw = w.r & 15;
    i32x4 fa[2], fb[2];
    auto frag = [&](int ks, int s, int slot) {
        const unsigned char* B = S + (ks % NBUF) * ST;
        const int co = ((2 * s + w.hi) ^ sw) << 4;
        fa[slot] = *reinterpret_cast<const i32x4*>(B + ra + co);
        fb[slot] = *reinterpret_cast<const i32x4*>(B + rb + co);
    };
    i32x16 acc[4][1];
    acc_zero<1>(acc);
    const int nks = 4 * (H.d / RB);                        // >= 4
    for (int q = 0; q < P; ++q) issue(q);
    wait_stages<LPW, P - 1>(P - 1);                        // stage 0 is in
    __syncthreads();
    frag(0, 0, 0);
    for (int kq = 0; kq < nks; kq += 4) {
#pragma unroll
        for (int vb = 0; vb < 4; ++vb) {
            const int ks = kq + vb;
#pragma unroll
            for (int s = 0; s < 15; ++s) {
                frag(ks, s + 1, (s + 1) & 1);
                acc[vb][0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[s & 1], fb[s & 1], acc[vb][0], 0, 0, 0);
            }
            if (ks + 1 < nks) {                            // uniform
                wait_stages<LPW, P - 1>(min(P - 2, nks - 2 - ks)); // stage ks + 1 is in
                __syncthreads();
                if (ks + P < nks) issue(ks + P);
                frag(ks + 1, 0, 0);
            }
            acc[vb][0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[1], fb[1], acc[vb][0], 0, 0, 0);
        }
    }
    __syncthreads();                                       // every wave is done with the stages
    static_assert(NBUF * ST >= 2 * Tile::BM * static_cast<int>(sizeof(HeadRecS)) + 2 * HV * 4, "exchange");
    static_assert(NBUF * ST >= (Tile::SR * (HV + 4) + HV) * 4, "logit slab");
    if constexpr (EPI == EPI_SAMPLE) {
        w.finish_sample(H, acc, S);
        w.finish_logits(H, acc, S);
    } else {
        w.finish(H, acc, S);
    }
}

// 256-row tiles: 2 x 4 waves of 128 x 64, two waves per SIMD (128
// accumulator registers each), four 32 KB stage buffers. Against 2 x 2 waves
// of 128 x 128 at one wave per SIMD (the sampling kernel's shape) the bytes per
// MFMA are the same and one wave's waits overlap the other's MFMAs: 5-6%
// faster at M = 1024 and 4608.
__global__ __launch_bounds__(2 * NTH) __attribute__((amdgpu_waves_per_eu(2))) void head_kernel_wide(HeadParams H) {
    head_main<2, 4, EPI_GREEDY, 4>(H);
}

// 192-row tiles: 128 x 96 per wave, one wave per SIMD, four 28 KB stage buffers.
__global__ __launch_bounds__(NTH) void head_kernel_mid(HeadParams H) { head_main<3, 4>(H); }

// 128-row tiles: 128 x 64 per wave, two waves per SIMD (two workgroups per
// CU interleave), three 24 KB stage buffers.
__global__ __launch_bounds__(NTH) __attribute__((amdgpu_waves_per_eu(2))) void head_kernel_narrow(HeadParams H) {
    head_main<2, 3>(H);
}

// 32-row tiles for a handful of hidden rows, where the call streams the head
// and the MFMAs are a small part of it: 2 waves of 128 x 32, 18 KB stages,
// four buffers (three stages of loads in flight), two workgroups per CU; a
// 128-row tile would stage and multiply 96 rows of padding.
__global__ __launch_bounds__(NTH / 2) void head_kernel_tiny(HeadParams H) { head_main<1, 4, EPI_GREEDY, 1>(H); }
__global__ __launch_bounds__(NTH / 2) void head_kernel_tiny_w(HeadParams H) { head_main_w512<EPI_GREEDY>(H); }

// Sampling mode, with the same tile sizes: pass 1's terms per row and
// vocabulary tile, and every logit stored for the draw. Its 256-row tiles keep
// 2 x 2 waves of 128 x 128 at one wave per SIMD: the 8-wave shape spilled in
// this epilogue and measured 2-4% slower.
__global__ __launch_bounds__(NTH) void head_kernel_wide_s(HeadParams H) { head_main<4, 4, EPI_SAMPLE>(H); }
__global__ __launch_bounds__(NTH) void head_kernel_mid_s(HeadParams H) { head_main<3, 4, EPI_SAMPLE>(H); }
__global__ __launch_bounds__(NTH) __attribute__((amdgpu_waves_per_eu(2))) void head_kernel_narrow_s(HeadParams H) {
    head_main<2, 3, EPI_SAMPLE>(H);
}
// The same for at most 128 rows (one hidden tile), where the call streams the
// head: without the two-waves-per-SIMD register cap this epilogue does not
// spill, and one workgroup per CU streams as fast: the call measured 5-9%
// faster at 36-64 rows. The capped kernel stays for more rows: at 640 rows
// the uncapped one made the call 10% slower.
__global__ __launch_bounds__(NTH) void head_kernel_narrow_s1(HeadParams H) { head_main<2, 3, EPI_SAMPLE>(H); }
__global__ __launch_bounds__(NTH / 2) void head_kernel_tiny_s(HeadParams H) { head_main<1, 4, EPI_SAMPLE, 1>(H); }
__global__ __launch_bounds__(NTH / 2) void head_kernel_tiny_ws(HeadParams H) { head_main_w512<EPI_SAMPLE>(H); }


// The tile-major layout of an int8 head [V, d]: for vocabulary tile vt (HV
// rows, zeros past V) and stage ks (HKW bytes of d), a contiguous HV x HKW
// block that is the stage buffer's weight part as head_main loads it: row R
// at R * HKW, its physical 16-byte chunk p holding logical chunk
// p ^ ((R >> 2) & 3). A stage's weight loads then read 16 KB in one run.
// One thread per 16-byte output chunk.
__global__ __launch_bounds__(NT) void head_pack_kernel(const signed char* w, int V, int d, signed char* out,
                                                       long long nchunks) {
    typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
    const long long per_tile = static_cast<long long>(HV) * d / 16;
    for (long long i = static_cast<long long>(blockIdx.x) * NT + threadIdx.x; i < nchunks;
         i += static_cast<long long>(gridDim.x) * NT) {
        const long long vt = i / per_tile, rem = i % per_tile;
        const int ks = static_cast<int>(rem / (HV * HKW / 16));
        const int rr = static_cast<int>(rem % (HV * HKW / 16));
        const int R = rr / (HKW / 16), c = (rr % (HKW / 16)) ^ ((R >> 2) & 3);
        const long long v = vt * HV + R;
        u32x4_t x = {0u, 0u, 0u, 0u};
        if (v < V) x = *reinterpret_cast<const u32x4_t*>(w + v * d + ks * HKW + 16 * c);
        *reinterpret_cast<u32x4_t*>(out + 16 * i) = x;
    }
}

// Sampling mode, one workgroup per hidden row: merge its vocabulary-tile
// records (a fixed order: per thread in tile order, a butterfly per wave, then
// the waves in order) into pass 1's record of its row: target row b*(k+1)+i is
// row b*rpb+i, draft row b*k+i is row b*rpb+k+1+i, at slot 2*row (pass 1's
// slot rule with one slice per row).
__device__ __attribute__((always_inline)) inline void head_merge_sample_row(const HeadParams& H, int m,
                                                                       HeadRecS (&Lr)[NWAVE], int (&Ld)[NWAVE]) {
    const int t = static_cast<int>(threadIdx.x), lane = t & 63, wv = t >> 6;
    HeadRecS a{-INFINITY, -INFINITY, 0.0f, 0, 0.0};
    const HeadRecS* R = H.recs + static_cast<size_t>(m) * H.nvt;
    for (int j = t; j < H.nvt; j += NT) head_recs_merge(a, R[j]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        HeadRecS p;
        p.t1 = __shfl_xor(a.t1, off, 64); p.t2 = __shfl_xor(a.t2, off, 64);
        p.ref = __shfl_xor(a.ref, off, 64); p.flags = __shfl_xor(a.flags, off, 64);
        p.s = __shfl_xor(a.s, off, 64);
        head_recs_merge(a, p);
    }
    // the draft token's logit, from the same int8 rows: the int32 dot product
    // is exact in any order, so it equals the tile's accumulator entry, and
    // it is scaled as the epilogue scales it
    const int tok = head_row_token(H, m);
    const bool has = tok >= 0 && tok < H.V;                // uniform per workgroup
    int dot = 0;
    if (has) {
        const u32x4* hr = reinterpret_cast<const u32x4*>(H.h + static_cast<size_t>(m) * H.d);
        // row-major: 16-byte chunk j of the row at j; tile-major: chunk c of
        // stage ks = j / 4 at physical chunk c ^ ((R >> 2) & 3) of row R
        const int R = tok % HV;
        const u32x4* wr = reinterpret_cast<const u32x4*>(
            H.packed ? H.w + static_cast<size_t>(tok / HV) * HV * H.d + R * HKW : H.w + static_cast<size_t>(tok) * H.d);
        for (int j = t; j < H.d / 16; j += NT) {
            const int wj = H.packed ? (j >> 2) * (HV * HKW / 16) + ((j & 3) ^ ((R >> 2) & 3)) : j;
            const u32x4 x = hr[j], y = wr[wj];
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int b = 0; b < 32; b += 8)
                    dot += static_cast<int>(static_cast<signed char>(x[q] >> b)) *
                           static_cast<int>(static_cast<signed char>(y[q] >> b));
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) dot += __shfl_xor(dot, off, 64);
    }
    if (lane == 0) { Lr[wv] = a; Ld[wv] = dot; }
    __syncthreads();
    if (t == 0) {
        HeadRecS r = Lr[0];
        int acc = Ld[0];
        for (int w = 1; w < NWAVE; ++w) { head_recs_merge(r, Lr[w]); acc += Ld[w]; }
        const float lx = has ? fmaf(static_cast<float>(acc) * H.hs[m], H.ws[tok], 0.0f) : 0.0f;
        const int k = H.k;
        const long long row = H.role == 0 ? static_cast<long long>(m / (k + 1)) * H.rpb + m % (k + 1)
                                          : static_cast<long long>(m / k) * H.rpb + k + 1 + m % k;
        TileRec tr;
        tr.t1 = r.t1; tr.t2 = r.t2; tr.ref = r.ref; tr.idx = 0x7fffffff; tr.s = r.s; tr.lx = lx;
        tr.flags = (r.flags & 1) | (has ? 2 : 0);
        H.tiles[2 * row] = tr;
    }
}

// Both heads' rows in one launch: workgroups 0 .. T.M-1 take the target's
// rows, the rest the draft's; the first also writes pass 2's exp table.
__global__ __launch_bounds__(NT) void head_merge_sample_kernel(HeadParams T, HeadParams D) {
    __shared__ HeadRecS Lr[NWAVE];
    __shared__ int Ld[NWAVE];
    const int b = static_cast<int>(blockIdx.x);
    if (b == 0)
        for (int j = static_cast<int>(threadIdx.x); j < EXP_N; j += NT) T.exptab[j] = exp2(static_cast<double>(j) / EXP_N);
    if (b < T.M) head_merge_sample_row(T, b, Lr, Ld);       // uniform per workgroup
    else head_merge_sample_row(D, b - T.M, Lr, Ld);
}

// One wave per hidden row: merge its vocabulary-tile records into the row's
// pass-1 record.
__global__ __launch_bounds__(NT) void head_merge_kernel(HeadParams H) {
    const int lane = static_cast<int>(threadIdx.x) & 63;
    const int m = static_cast<int>(blockIdx.x) * NWAVE + (static_cast<int>(threadIdx.x) >> 6);
    if (m >= H.M) return;                                  // uniform per wave
    float t1 = -INFINITY, t2 = -INFINITY;
    int i1 = 0x7fffffff, fl = 0;
    const HeadRec* R = H.rec + static_cast<size_t>(m) * H.nvt;
    for (int j = lane; j < H.nvt; j += 64) {
        const HeadRec o = R[j];
        head_merge(t1, t2, i1, fl, o.t1, o.t2, o.idx, o.flags);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const float u1 = __shfl_xor(t1, off, 64), u2 = __shfl_xor(t2, off, 64);
        const int j1 = __shfl_xor(i1, off, 64), g = __shfl_xor(fl, off, 64);
        head_merge(t1, t2, i1, fl, u1, u2, j1, g);
    }
    if (lane == 0) {
        TileRec tr;
        tr.t1 = t1; tr.t2 = t2; tr.ref = 0.0f; tr.idx = i1; tr.s = 0.0; tr.lx = 0.0f; tr.flags = fl & 1;
        H.tiles[2 * static_cast<size_t>(m)] = tr;
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
    int rpb;
    int nvec;                  // 16-byte vectors per row
    int wmax;                  // most pass-2 workgroups per batch row (sampling; 0 in greedy mode)
    size_t rows_total;
    // workspace offsets (bytes)
    size_t o_tiles, o_bat, o_segs, o_exp, o_tau, o_rowoff, o_rowmap, o_rhdr, total;
};

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

bool make_plan(int32_t B, int32_t k, int32_t V, int mode, int dtype, Plan& p) {
    if (B < 1 || k < 0 || k > SPEC_MAX_K || V < 1) return false;
    if (mode != SPEC_MODE_SAMPLE && mode != SPEC_MODE_GREEDY) return false;
    p.rpb = mode == SPEC_MODE_SAMPLE ? 2 * k + 1 : k + 1;
    p.rows_total = static_cast<size_t>(B) * p.rpb;
    if (p.rows_total > (1u << 26)) return false;
    if (B > (1 << 21)) return false;                       // grid sizes stay below 2^32 threads
    if (V > (1 << 29)) return false;                       // a row must fit one buffer resource
    const int ve = dtype == SPEC_DTYPE_F32 ? 4 : 8;
    p.nvec = (V + ve - 1) / ve;
    p.wmax = 0;
    if (mode == SPEC_MODE_SAMPLE) {
        if (V > MAX_V) return false;
        // pass 2: enough workgroups per batch row to fill SLOTS_CAP resident
        // slots, but at least one vector per lane
        long long w = (p.nvec + NTS - 1) / NTS;
        const long long by_slots = (SLOTS_CAP + B - 1) / B;
        if (w > by_slots) w = by_slots;
        if (w > W_CAP) w = W_CAP;
        if (w < 1) w = 1;
        p.wmax = static_cast<int>(w);
    }
    size_t o = 0;
    p.o_tiles = o; o = align256(o + (p.rows_total + G_MAX) * sizeof(TileRec));
    p.o_bat = o; o = align256(o + static_cast<size_t>(B) * sizeof(BatchRec));
    p.o_segs = o; o = align256(o + static_cast<size_t>(B) * p.wmax * (NTS / 64) * sizeof(SegRec));
    p.o_exp = o; o = align256(o + EXP_N * sizeof(double));
    p.o_tau = o; o = align256(o + TAB_MAX * sizeof(double));
    // ragged drafts (also counted for fixed-length calls: one size serves both)
    p.o_rowoff = o; o = align256(o + static_cast<size_t>(B) * sizeof(int));
    p.o_rowmap = o; o = align256(o + p.rows_total * sizeof(int));
    p.o_rhdr = o; o = align256(o + 2 * sizeof(long long));
    p.total = o;
    return true;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check(const void* tgt, const void* dft, const int32_t* tok, const float* uni, float T, int mode,
          int32_t B, int32_t k, int32_t V, int dtype, const int32_t* acc, const int32_t* out,
          const float* gap, const void* ws, size_t ws_bytes, Plan& plan, bool ragged = false,
          const int32_t* dlen = nullptr) {
    if (dtype != SPEC_DTYPE_F32 && dtype != SPEC_DTYPE_BF16)
        return fail(SPEC_ERR_DTYPE, "dtype %d is not SPEC_DTYPE_F32 or SPEC_DTYPE_BF16", dtype);
    if (mode != SPEC_MODE_SAMPLE && mode != SPEC_MODE_GREEDY)
        return fail(SPEC_ERR_MODE, "mode %d is not SPEC_MODE_SAMPLE or SPEC_MODE_GREEDY", mode);
    if (B < 1 || k < 0 || k > SPEC_MAX_K || V < 1)
        return fail(SPEC_ERR_SHAPE, "need B >= 1, 0 <= k <= %d, V >= 1 (got B=%d k=%d V=%d)", SPEC_MAX_K, B, k, V);
    if (!make_plan(B, k, V, mode, dtype, plan))
        return fail(SPEC_ERR_SHAPE, "sizes B=%d k=%d V=%d exceed the supported range", B, k, V);
    const unsigned long long elems = static_cast<unsigned long long>(B) * (k + 1) * static_cast<unsigned long long>(V);
    if (elems > (1ull << 46)) return fail(SPEC_ERR_SHAPE, "B*(k+1)*V = %llu is too large", elems);
    const bool sample = mode == SPEC_MODE_SAMPLE;
    if (!tgt) return fail(SPEC_ERR_NULL, "target_logits is NULL");
    if (k > 0 && !tok) return fail(SPEC_ERR_NULL, "draft_tokens is NULL");
    if (ragged && !dlen) return fail(SPEC_ERR_NULL, "draft_len is NULL");
    if (sample && k > 0 && !dft) return fail(SPEC_ERR_NULL, "draft_logits is NULL in sampling mode");
    if (sample && !uni) return fail(SPEC_ERR_NULL, "uniforms is NULL in sampling mode");
    if (!acc || !out || !gap) return fail(SPEC_ERR_NULL, "an output pointer is NULL");
    if (sample && !(T > 0.0f && T <= 3.0e38f))
        return fail(SPEC_ERR_TEMP, "temperature must be finite and > 0 in sampling mode (got %g)", (double)T);
    const size_t es = dtype == SPEC_DTYPE_F32 ? 4 : 2;
    if (!aligned(tgt, es) || (dft && !aligned(dft, es)) || (tok && !aligned(tok, 4)) ||
        (uni && !aligned(uni, 4)) || !aligned(acc, 4) || !aligned(out, 4) || !aligned(gap, 4) ||
        (dlen && !aligned(dlen, 4)))
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
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, scan_kernel<E, MODE>, NT, 0) != hipSuccess || n < 1)
        n = 1;
    if (dev >= 0 && dev < 64) cache[dev] = n;
    return n;
}

template <class E, bool VEC>
int seg_blocks_per_cu(int dev) {
    static int cache[64] = {0};
    if (dev >= 0 && dev < 64 && cache[dev] > 0) return cache[dev];
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, seg_kernel<E, VEC>, NTS, 0) != hipSuccess || n < 1)
        n = 1;
    if (dev >= 0 && dev < 64) cache[dev] = n;
    return n;
}

// Pass 2 and the draw of a sampling call whose pass-1 records (and pass 2's
// tables) are in place: one resident round of workgroups split evenly over
// the batch rows, then one draw workgroup per batch row. ev (or null): ev[0]
// after pass 2, ev[1] after the draw.
template <class E>
hipError_t launch_pass2(Params& P, int dev, int ncu, hipStream_t s, hipEvent_t const* ev) {
    auto mark = [&](int i) { return ev ? hipEventRecord(ev[i], s) : hipSuccess; };
    long long slots = static_cast<long long>(ncu) *
        (P.vec_ok ? seg_blocks_per_cu<E, true>(dev) : seg_blocks_per_cu<E, false>(dev));
    if (slots > SLOTS_CAP) slots = SLOTS_CAP;
    long long W = (slots + P.B - 1) / P.B;
    if (W > P.wpb) W = P.wpb;                              // the plan's bound (workspace size)
    if (W < 1) W = 1;
    P.wpb = static_cast<int>(W);
    P.nseg = P.wpb * (NTS / 64);
    P.vps = (P.nvec + P.nseg - 1) / P.nseg;
    const unsigned G2 = static_cast<unsigned>(static_cast<long long>(P.B) * W);
    if (P.vec_ok) hipLaunchKernelGGL((seg_kernel<E, true>), dim3(G2), dim3(NTS), 0, s, P);
    else hipLaunchKernelGGL((seg_kernel<E, false>), dim3(G2), dim3(NTS), 0, s, P);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess) e = mark(0);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((draw_kernel<E>), dim3(P.B), dim3(NT2), 0, s, P);
    e = hipGetLastError();
    if (e == hipSuccess) e = mark(1);
    return e;
}

// Phase events of spec_verify_timed (null otherwise): ev[0] before the first
// kernel, ev[1] after pass 1, ev[2] after the decisions and pass 2, ev[3] after
// the draw (greedy mode records ev[2] and ev[3] together).
template <class E, int MODE>
hipError_t launch_all(Params& P, int dev, int ncu, hipStream_t s, hipEvent_t const* ev = nullptr) {
    auto mark = [&](int i) { return ev ? hipEventRecord(ev[i], s) : hipSuccess; };
    long long G = static_cast<long long>(ncu) * scan_blocks_per_cu<E, MODE>(dev);
    // slices of at least MIN_SLICE elements, but at least one workgroup per
    // row while the rows fit the round: a workgroup walks its row segments
    // one after another, so small calls are bound by segments per workgroup
    long long by_size = (P.N + MIN_SLICE - 1) / MIN_SLICE;
    const long long rows = P.N / P.V;
    if (by_size < rows) by_size = rows;
    if (G > by_size) G = by_size;
    if (G > G_MAX) G = G_MAX;
    if (G < 1) G = 1;
    P.L = (P.N + G - 1) / G;
    P.G = static_cast<int>((P.N + P.L - 1) / P.L);
    hipError_t e;
    if (MODE == SPEC_MODE_GREEDY && P.fire && P.B >= GATE_ROW_MIN) {   // gate: one workgroup per row
        hipLaunchKernelGGL((gate_row_kernel<E>), dim3(P.B), dim3(NTG), 0, s, P);
        return hipGetLastError();
    }
    e = mark(0);
    if (e != hipSuccess) return e;
    if (P.dlen && P.B > RAG_INLINE) {
        // ragged drafts with many batch rows: the packed rows and pass 1's
        // slices over them (at most P.N elements, so the same G workgroups
        // suffice); fewer batch rows are packed by pass 1 itself
        hipLaunchKernelGGL(rows_kernel, dim3(1), dim3(NTR), 0, s, P);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((scan_kernel<E, MODE>), dim3(P.G), dim3(NT), 0, s, P);
    e = hipGetLastError();
    if (e == hipSuccess) e = mark(1);
    if (e != hipSuccess) return e;
    if constexpr (MODE == SPEC_MODE_GREEDY) {
        if (P.fire)
            hipLaunchKernelGGL((gate_kernel<E>), dim3((P.B + NT - 1) / NT), dim3(NT), 0, s, P);
        else
            hipLaunchKernelGGL((decide_kernel<E, MODE>), dim3(P.B), dim3(NT), 0, s, P);
        e = hipGetLastError();
        if (e == hipSuccess) e = mark(2);
        if (e == hipSuccess) e = mark(3);
        return e;
    }
    return launch_pass2<E>(P, dev, ncu, s, ev ? ev + 2 : nullptr);
}

struct GateOut {
    const uint32_t* admit;
    int32_t* fire;
    int rule;
    float tau;
};

// Fill the launch parameters of checked arguments and enqueue the kernels.
// c = ch + cl. ch: c rounded toward zero to (bf16) 16 or (fp32) 24
// significant bits, so x*ch is exact for bf16 x. cl: the rest, kept strictly
// positive so that x = -inf gives -inf (not -inf + inf) in x*ch - ref + x*cl.
void split_c(double c, int dtype, float& ch, float& cl) {
    ch = static_cast<float>(c);
    uint32_t u;
    memcpy(&u, &ch, 4);
    if (static_cast<double>(ch) > c) --u;                  // toward zero
    const uint32_t unit = dtype == SPEC_DTYPE_BF16 ? 0x100u : 0x1u;
    u &= ~(unit - 1u);
    memcpy(&ch, &u, 4);
    if (static_cast<double>(ch) == c && u >= unit) {
        u -= unit;
        memcpy(&ch, &u, 4);
    }
    cl = static_cast<float>(c - static_cast<double>(ch));
    if (!(cl > 0.0f)) cl = 1.17549435e-38f;                // smallest normal float
}

int enqueue(const Plan& plan, const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
            const int32_t* draft_len, const float* uniforms, float temperature, int mode, int32_t B, int32_t k,
            int32_t V, int dtype, int32_t* accepted_len, int32_t* out_tokens, float* gap, float* target_prob,
            float* draft_prob, const GateOut* gate, void* workspace, void* stream,
            void* const* events = nullptr) {
    char* ws = static_cast<char*>(workspace);
    Params P{};
    P.tgt = target_logits;
    P.dft = draft_logits;
    P.tok = draft_tokens;
    P.dlen = draft_len;
    P.admit = gate ? reinterpret_cast<const unsigned*>(gate->admit) : nullptr;
    P.fire = gate ? gate->fire : nullptr;
    P.gate_rule = gate ? gate->rule : 0;
    P.gate_tau = gate ? gate->tau : 0.0f;
    P.uni = uniforms;
    P.acc_len = accepted_len;
    P.out_tok = out_tokens;
    P.gap = gap;
    P.tprob = k > 0 ? target_prob : nullptr;
    P.dprob = k > 0 ? draft_prob : nullptr;
    P.B = B; P.k = k; P.V = V;
    P.rpb = plan.rpb;
    P.nvec = plan.nvec;
    P.wpb = plan.wmax;                                     // launch_all picks the count (<= this)
    P.nseg = 0;
    P.vps = 0;
    P.N = static_cast<long long>(plan.rows_total) * V;
    P.G = 0; P.L = 0;
    P.mode = mode;
    const char* fe = getenv("SPEC_VERIFY_FORCE_EXACT_PATH");
    P.force_exact = (fe && fe[0] == '1') ? 1 : 0;
    const double Td = mode == SPEC_MODE_SAMPLE ? static_cast<double>(temperature) : 1.0;
    const double c = 1.4426950408889634 / Td;
    float ch, cl;
    split_c(c, dtype, ch, cl);
    P.ch = ch;
    P.cl = cl;
    P.c = static_cast<double>(P.ch) + static_cast<double>(P.cl);
    P.invT = 1.0 / Td;
    P.vec_ok = aligned(target_logits, 16) && (draft_logits == nullptr || aligned(draft_logits, 16)) &&
               (static_cast<size_t>(V) * (dtype == SPEC_DTYPE_F32 ? 4 : 2)) % 16 == 0;
    P.tiles = reinterpret_cast<TileRec*>(ws + plan.o_tiles);
    P.bat = reinterpret_cast<BatchRec*>(ws + plan.o_bat);
    P.segs = reinterpret_cast<SegRec*>(ws + plan.o_segs);
    P.exptab = reinterpret_cast<double*>(ws + plan.o_exp);
    P.tautab = reinterpret_cast<double*>(ws + plan.o_tau);
    P.rowoff = reinterpret_cast<int*>(ws + plan.o_rowoff);
    P.rowmap = reinterpret_cast<int*>(ws + plan.o_rowmap);
    P.rhdr = reinterpret_cast<long long*>(ws + plan.o_rhdr);
    // bf16 value table: |v| in [2^-16, 2^8), usable for rows whose maxima lie
    // below 2^kmax, kmax <= 8 the largest with 2^kmax / T <= 700, centred by
    // C = 2^kmax/T - 600
    P.tab_on = 0;
    P.tab_lim = 0.0;
    P.tab_c = 0.0;
    if (dtype == SPEC_DTYPE_BF16 && mode == SPEC_MODE_SAMPLE) {
        int kmax = static_cast<int>(floor(log2(700.0 * Td)));
        if (kmax > 8) kmax = 8;
        if (kmax > -12) {
            P.tab_on = 1;
            P.tab_lim = ldexp(1.0, kmax);
            P.tab_c = P.tab_lim / Td - 600.0;
        }
    }

    int dev = 0, ncu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu < 1)
        return fail(SPEC_ERR_HIP, "cannot query the current HIP device");
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipEvent_t const* ev = reinterpret_cast<hipEvent_t const*>(events);
    hipError_t e;
    if (dtype == SPEC_DTYPE_BF16)
        e = mode == SPEC_MODE_SAMPLE ? launch_all<Bf16, SPEC_MODE_SAMPLE>(P, dev, ncu, s, ev)
                                     : launch_all<Bf16, SPEC_MODE_GREEDY>(P, dev, ncu, s, ev);
    else
        e = mode == SPEC_MODE_SAMPLE ? launch_all<F32, SPEC_MODE_SAMPLE>(P, dev, ncu, s, ev)
                                     : launch_all<F32, SPEC_MODE_GREEDY>(P, dev, ncu, s, ev);
    if (e != hipSuccess) return fail(SPEC_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return SPEC_OK;
}

int run(const void* target_logits, const void* draft_logits, const int32_t* draft_tokens, const int32_t* draft_len,
        bool ragged, const float* uniforms, float temperature, int mode, int32_t B, int32_t k, int32_t V, int dtype,
        int32_t* accepted_len, int32_t* out_tokens, float* gap, float* target_prob, float* draft_prob,
        void* workspace, size_t workspace_bytes, void* stream, void* const* events = nullptr) {
    Plan plan;
    const int rc = check(target_logits, draft_logits, draft_tokens, uniforms, temperature, mode, B, k, V,
                         dtype, accepted_len, out_tokens, gap, workspace, workspace_bytes, plan, ragged, draft_len);
    if (rc != SPEC_OK) return rc;
    return enqueue(plan, target_logits, draft_logits, draft_tokens, ragged ? draft_len : nullptr, uniforms,
                   temperature, mode, B, k, V, dtype, accepted_len, out_tokens, gap, target_prob, draft_prob,
                   nullptr, workspace, stream, events);
}

int check_gate(const void* logits, int32_t n, int32_t V, int dtype, int rule, float tau, const uint32_t* admit,
               const int32_t* argmax, const float* gap, const int32_t* fire, const void* ws, size_t ws_bytes,
               Plan& plan) {
    if (dtype != SPEC_DTYPE_F32 && dtype != SPEC_DTYPE_BF16)
        return fail(SPEC_ERR_DTYPE, "dtype %d is not SPEC_DTYPE_F32 or SPEC_DTYPE_BF16", dtype);
    if (rule != SPEC_GATE_MARGIN && rule != SPEC_GATE_CERTIFIED)
        return fail(SPEC_ERR_MODE, "rule %d is not SPEC_GATE_MARGIN or SPEC_GATE_CERTIFIED", rule);
    if (n < 1 || V < 1) return fail(SPEC_ERR_SHAPE, "need n >= 1 and V >= 1 (got n=%d V=%d)", n, V);
    if (!make_plan(n, 0, V, SPEC_MODE_GREEDY, dtype, plan))
        return fail(SPEC_ERR_SHAPE, "sizes n=%d V=%d exceed the supported range", n, V);
    if (tau != tau || (rule == SPEC_GATE_CERTIFIED && tau < 0.0f))
        return fail(SPEC_ERR_VALUE, "tau must not be NaN, and must be >= 0 for the certified rule (got %g)",
                    (double)tau);
    if (!logits) return fail(SPEC_ERR_NULL, "logits is NULL");
    if (!argmax || !gap || !fire) return fail(SPEC_ERR_NULL, "an output pointer is NULL");
    const size_t es = dtype == SPEC_DTYPE_F32 ? 4 : 2;
    if (!aligned(logits, es) || (admit && !aligned(admit, 4)) || !aligned(argmax, 4) || !aligned(gap, 4) ||
        !aligned(fire, 4))
        return fail(SPEC_ERR_ALIGN, "a pointer is not aligned to its element size");
    if (!ws || ws_bytes < plan.total)
        return fail(SPEC_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu%s)", plan.total, ws_bytes,
                    ws ? "" : ", NULL");
    if (!aligned(ws, 256)) return fail(SPEC_ERR_ALIGN, "workspace must be 256-byte aligned");
    return SPEC_OK;
}

// ---- int8 LM head + greedy verification

constexpr int HEAD_MAX_D = 65536;       // |acc| <= 2^14 * d stays inside int32

struct HeadPlan {
    int M, nvt;
    int bm;                             // hidden rows per tile: 256, 192, 128 or 32
    size_t o_rec, o_tiles, total;
};

// Hidden rows per tile for M rows: wider tiles reuse each staged operand
// more; a narrower one when it pads the hidden rows clearly less (e.g. 384
// rows: 2 x 192, not 2 x 256); 32-row tiles for at most 32 rows.
int head_bm(long long M) {
    if (M <= 32) return 32;
    const long long pad4 = (M + 255) / 256 * 256, pad3 = (M + 191) / 192 * 192, pad2 = (M + 127) / 128 * 128;
    if (pad4 * 10 <= (pad3 < pad2 ? pad3 : pad2) * 11) return 256;
    if (pad3 * 10 <= pad2 * 11) return 192;
    return 128;
}

bool make_head_plan(int32_t B, int32_t k, int32_t V, int32_t d, HeadPlan& p) {
    if (B < 1 || B > (1 << 21) || k < 0 || k > SPEC_MAX_K || V < 1 || V > (1 << 29)) return false;
    if (d < HK || d > HEAD_MAX_D || d % HK != 0) return false;
    const long long M = static_cast<long long>(B) * (k + 1);
    if (M > (1 << 26)) return false;
    const long long nvt = (V + HV - 1) / HV;
    p.bm = head_bm(M);
    const long long nmt = (M + p.bm - 1) / p.bm;
    if (nvt * nmt >= (1ll << 31)) return false;
    p.M = static_cast<int>(M);
    p.nvt = static_cast<int>(nvt);
    size_t o = 0;
    p.o_rec = o; o = align256(o + static_cast<size_t>(M) * nvt * sizeof(HeadRec));
    p.o_tiles = o; o = align256(o + 2 * static_cast<size_t>(M) * sizeof(TileRec));
    p.total = o;
    return true;
}

int run_head(const int8_t* hidden, const float* hidden_scale, const int8_t* weight, const float* weight_scale,
             const int32_t* draft_tokens, int32_t B, int32_t k, int32_t V, int32_t d, int32_t* accepted_len,
             int32_t* out_tokens, float* gap, void* workspace, size_t workspace_bytes, void* stream,
             void* const* events, int packed = 0) {
    if (B < 1 || B > (1 << 21) || k < 0 || k > SPEC_MAX_K || V < 1 || V > (1 << 29))
        return fail(SPEC_ERR_SHAPE, "need 1 <= B <= 2^21, 0 <= k <= %d, 1 <= V <= 2^29 (got B=%d k=%d V=%d)",
                    SPEC_MAX_K, B, k, V);
    if (d < HK || d > HEAD_MAX_D || d % HK != 0)
        return fail(SPEC_ERR_SHAPE, "d must be a multiple of %d in [%d, %d] (got %d)", HK, HK, HEAD_MAX_D, d);
    HeadPlan plan;
    if (!make_head_plan(B, k, V, d, plan))
        return fail(SPEC_ERR_SHAPE, "sizes B=%d k=%d V=%d d=%d exceed the supported range", B, k, V, d);
    if (!hidden || !hidden_scale || !weight || !weight_scale)
        return fail(SPEC_ERR_NULL, "hidden, hidden_scale, weight and weight_scale are required");
    if (k > 0 && !draft_tokens) return fail(SPEC_ERR_NULL, "draft_tokens is NULL");
    if (!accepted_len || !out_tokens || !gap) return fail(SPEC_ERR_NULL, "an output pointer is NULL");
    if (!aligned(hidden, 16) || !aligned(weight, 16))
        return fail(SPEC_ERR_ALIGN, "hidden and weight must be 16-byte aligned");
    if (!aligned(hidden_scale, 4) || !aligned(weight_scale, 4) || (draft_tokens && !aligned(draft_tokens, 4)) ||
        !aligned(accepted_len, 4) || !aligned(out_tokens, 4) || !aligned(gap, 4))
        return fail(SPEC_ERR_ALIGN, "a pointer is not aligned to its element size");
    if (!workspace || workspace_bytes < plan.total)
        return fail(SPEC_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu%s)", plan.total, workspace_bytes,
                    workspace ? "" : ", NULL");
    if (!aligned(workspace, 256)) return fail(SPEC_ERR_ALIGN, "workspace must be 256-byte aligned");
    if (events && (!events[0] || !events[1] || !events[2]))
        return fail(SPEC_ERR_NULL, "spec_verify_lmhead_timed needs three events");

    char* ws = static_cast<char*>(workspace);
    HeadParams H{};
    H.h = reinterpret_cast<const signed char*>(hidden);
    H.hs = hidden_scale;
    H.w = reinterpret_cast<const signed char*>(weight);
    H.packed = packed;
    H.ws = weight_scale;
    H.rec = reinterpret_cast<HeadRec*>(ws + plan.o_rec);
    H.tiles = reinterpret_cast<TileRec*>(ws + plan.o_tiles);
    H.M = plan.M; H.V = V; H.d = d;
    H.nvt = plan.nvt;
    H.nmt = (plan.M + plan.bm - 1) / plan.bm;
    // the greedy decisions read the merged records as pass 1's, one slice per row
    Params P;
    memset(&P, 0, sizeof P);
    P.tok = draft_tokens;
    P.acc_len = accepted_len;
    P.out_tok = out_tokens;
    P.gap = gap;
    P.B = B; P.k = k; P.V = V;
    P.rpb = k + 1;
    P.N = static_cast<long long>(plan.M) * V;
    P.L = V;
    P.G = plan.M;
    P.mode = SPEC_MODE_GREEDY;
    P.c = 1.4426950408889634;
    P.tiles = H.tiles;

    hipStream_t s = static_cast<hipStream_t>(stream);
    hipEvent_t const* ev = reinterpret_cast<hipEvent_t const*>(events);
    hipError_t e = ev ? hipEventRecord(ev[0], s) : hipSuccess;
    if (e == hipSuccess) {
        const dim3 grid(static_cast<unsigned>(plan.nvt) * static_cast<unsigned>(H.nmt));
        if (plan.bm == 256) hipLaunchKernelGGL(head_kernel_wide, grid, dim3(2 * NTH), 0, s, H);
        else if (plan.bm == 192) hipLaunchKernelGGL(head_kernel_mid, grid, dim3(NTH), 0, s, H);
        else if (plan.bm == 128) hipLaunchKernelGGL(head_kernel_narrow, grid, dim3(NTH), 0, s, H);
        else if (d % 512 == 0 && !packed) hipLaunchKernelGGL(head_kernel_tiny_w, grid, dim3(NTH / 2), 0, s, H);
        else hipLaunchKernelGGL(head_kernel_tiny, grid, dim3(NTH / 2), 0, s, H);
        e = hipGetLastError();
    }
    if (e == hipSuccess && ev) e = hipEventRecord(ev[1], s);
    if (e == hipSuccess) {
        hipLaunchKernelGGL(head_merge_kernel, dim3(static_cast<unsigned>((plan.M + NWAVE - 1) / NWAVE)), dim3(NT),
                           0, s, H);
        e = hipGetLastError();
    }
    if (e == hipSuccess) {
        hipLaunchKernelGGL((decide_kernel<F32, SPEC_MODE_GREEDY>), dim3(B), dim3(NT), 0, s, P);
        e = hipGetLastError();
    }
    if (e == hipSuccess && ev) e = hipEventRecord(ev[2], s);
    if (e != hipSuccess) return fail(SPEC_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return SPEC_OK;
}

}  // namespace

// Device scratch of spec_verify_noalloc, in place of a caller workspace: one
// copy on every GPU the library runs on, held until the process ends. Host
// code never uses this name as an address (on the host it is only a stand-in
// for the symbol); it uses the device address that hipGetSymbolAddress
// returned for the current device.
static __device__ __align__(256) unsigned char scratch[SPEC_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES];

// The device address of `scratch` on device dev (the current device), looked
// up once per device.
int scratch_ptr(int dev, void** out) {
    if (dev < 0 || dev >= MAX_DEVICES) return fail(SPEC_ERR_HIP, "device %d is out of range", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(SPEC_ERR_HIP, "cannot resolve the scratch buffer on device %d: %s", dev,
                        hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return SPEC_OK;
}

}  // namespace

// ------------------------------------------------------------------ LM head, sampling mode

// A shared head: the target's hidden rows, then the draft's, copied into one
// matrix (with their scales) for a single pass over the head, which then
// streams its weights once instead of once per set of rows. One workgroup per
// row; d is a multiple of 128, so rows are whole 16-byte vectors.
struct ConcatParams {
    const signed char* a;
    const signed char* b;
    const float* as;
    const float* bs;
    signed char* out;
    float* outs;
    int na, d;
};

__global__ __launch_bounds__(NT) void head_concat_kernel(ConcatParams C) {
    const int m = static_cast<int>(blockIdx.x), t = static_cast<int>(threadIdx.x);
    const bool first = m < C.na;
    const int row = first ? m : m - C.na;
    const u32x4* src = reinterpret_cast<const u32x4*>((first ? C.a : C.b) + static_cast<size_t>(row) * C.d);
    u32x4* dst = reinterpret_cast<u32x4*>(C.out + static_cast<size_t>(m) * C.d);
    for (int i = t; i < C.d / 16; i += NT) dst[i] = src[i];
    if (t == 0) C.outs[m] = first ? C.as[row] : C.bs[row];
}

struct HeadSamplePlan {
    Plan pv;                            // pass 2's part of the verify plan (batch records, segments)
    int nvt, bmT, bmD, bmC;
    size_t o_recT, o_recD, o_tiles, o_bat, o_segs, o_exp, o_lt, o_ld, o_hc, o_hsc, total;
};

bool make_head_sample_plan(int32_t B, int32_t k, int32_t V, int32_t d, HeadSamplePlan& p) {
    if (B < 1 || B > (1 << 21) || k < 0 || k > SPEC_MAX_K || V < 1 || V > (1 << 29)) return false;
    if (d < HK || d > HEAD_MAX_D || d % HK != 0) return false;
    const long long MT = static_cast<long long>(B) * (k + 1), MD = static_cast<long long>(B) * k;
    if (MT > (1 << 26)) return false;
    if (!make_plan(B, k, V, SPEC_MODE_SAMPLE, SPEC_DTYPE_F32, p.pv)) return false;
    const long long nvt = (V + HV - 1) / HV;
    p.bmT = head_bm(MT);
    p.bmD = head_bm(MD > 0 ? MD : 1);
    p.bmC = head_bm(MT + MD);
    if (nvt * ((MT + MD + 31) / 32) >= (1ll << 31)) return false;
    p.nvt = static_cast<int>(nvt);
    const size_t rows = static_cast<size_t>(B) * (2 * k + 1);
    size_t o = 0;
    // the draft's records and logits follow the target's without a gap, so
    // one launch over both sets of rows (a shared head) fills them in order
    p.o_recT = o; p.o_recD = o + static_cast<size_t>(MT) * nvt * sizeof(HeadRecS);
    o = align256(p.o_recD + static_cast<size_t>(MD) * nvt * sizeof(HeadRecS));
    p.o_tiles = o; o = align256(o + 2 * rows * sizeof(TileRec));
    p.o_bat = o; o = align256(o + static_cast<size_t>(B) * sizeof(BatchRec));
    p.o_segs = o; o = align256(o + static_cast<size_t>(B) * p.pv.wmax * (NTS / 64) * sizeof(SegRec));
    p.o_exp = o; o = align256(o + EXP_N * sizeof(double));
    p.o_lt = o; p.o_ld = o + static_cast<size_t>(MT) * V * sizeof(float);
    o = align256(p.o_ld + static_cast<size_t>(MD) * V * sizeof(float));
    p.o_hc = o; o = align256(o + static_cast<size_t>(MT + MD) * d);
    p.o_hsc = o; o = align256(o + static_cast<size_t>(MT + MD) * sizeof(float));
    p.total = o;
    return true;
}

hipError_t launch_head_sample(HeadParams& H, int bm, hipStream_t s) {
    H.nmt = (H.M + bm - 1) / bm;
    const dim3 grid(static_cast<unsigned>(H.nvt) * static_cast<unsigned>(H.nmt));
    if (bm == 256) hipLaunchKernelGGL(head_kernel_wide_s, grid, dim3(NTH), 0, s, H);
    else if (bm == 192) hipLaunchKernelGGL(head_kernel_mid_s, grid, dim3(NTH), 0, s, H);
    else if (bm == 128 && H.nmt == 1) hipLaunchKernelGGL(head_kernel_narrow_s1, grid, dim3(NTH), 0, s, H);
    else if (bm == 128) hipLaunchKernelGGL(head_kernel_narrow_s, grid, dim3(NTH), 0, s, H);
    else if (H.d % 512 == 0 && !H.packed) hipLaunchKernelGGL(head_kernel_tiny_ws, grid, dim3(NTH / 2), 0, s, H);
    else hipLaunchKernelGGL(head_kernel_tiny_s, grid, dim3(NTH / 2), 0, s, H);
    return hipGetLastError();
}

int run_head_sample(const int8_t* th, const float* ths, const int8_t* tw, const float* tws, const int8_t* dh,
                    const float* dhs, const int8_t* dw, const float* dws, const int32_t* draft_tokens,
                    const float* uniforms, float temperature, int32_t B, int32_t k, int32_t V, int32_t d,
                    int32_t* accepted_len, int32_t* out_tokens, float* gap, float* target_prob,
                    float* draft_prob, void* workspace, size_t workspace_bytes, void* stream,
                    void* const* events, int packed = 0) {
    if (B < 1 || B > (1 << 21) || k < 0 || k > SPEC_MAX_K || V < 1 || V > (1 << 29))
        return fail(SPEC_ERR_SHAPE, "need 1 <= B <= 2^21, 0 <= k <= %d, 1 <= V <= 2^29 (got B=%d k=%d V=%d)",
                    SPEC_MAX_K, B, k, V);
    if (d < HK || d > HEAD_MAX_D || d % HK != 0)
        return fail(SPEC_ERR_SHAPE, "d must be a multiple of %d in [%d, %d] (got %d)", HK, HK, HEAD_MAX_D, d);
    if (V > SPEC_MAX_V_SAMPLE)
        return fail(SPEC_ERR_SHAPE, "sampling mode supports V <= %d (got %d)", SPEC_MAX_V_SAMPLE, V);
    HeadSamplePlan plan;
    if (!make_head_sample_plan(B, k, V, d, plan))
        return fail(SPEC_ERR_SHAPE, "sizes B=%d k=%d V=%d d=%d exceed the supported range", B, k, V, d);
    if (!(temperature > 0.0f) || !(temperature < INFINITY))
        return fail(SPEC_ERR_TEMP, "temperature must be finite and > 0 (got %g)", static_cast<double>(temperature));
    if (!th || !ths || !tw || !tws || !uniforms)
        return fail(SPEC_ERR_NULL, "the target head, its hidden rows, their scales and the uniforms are required");
    if (k > 0 && (!draft_tokens || !dh || !dhs))
        return fail(SPEC_ERR_NULL, "draft_tokens and the draft hidden rows and scales are required when k > 0");
    if ((dw == nullptr) != (dws == nullptr))
        return fail(SPEC_ERR_NULL, "draft_weight and draft_weight_scale must both be given or both be NULL");
    if (!accepted_len || !out_tokens || !gap) return fail(SPEC_ERR_NULL, "an output pointer is NULL");
    if (!aligned(th, 16) || !aligned(tw, 16) || (dh && !aligned(dh, 16)) || (dw && !aligned(dw, 16)))
        return fail(SPEC_ERR_ALIGN, "hidden rows and weights must be 16-byte aligned");
    if (!aligned(ths, 4) || !aligned(tws, 4) || (dhs && !aligned(dhs, 4)) || (dws && !aligned(dws, 4)) ||
        (draft_tokens && !aligned(draft_tokens, 4)) || !aligned(uniforms, 4) || !aligned(accepted_len, 4) ||
        !aligned(out_tokens, 4) || !aligned(gap, 4) || (target_prob && !aligned(target_prob, 4)) ||
        (draft_prob && !aligned(draft_prob, 4)))
        return fail(SPEC_ERR_ALIGN, "a pointer is not aligned to its element size");
    if (!workspace || workspace_bytes < plan.total)
        return fail(SPEC_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu%s)", plan.total, workspace_bytes,
                    workspace ? "" : ", NULL");
    if (!aligned(workspace, 256)) return fail(SPEC_ERR_ALIGN, "workspace must be 256-byte aligned");
    if (events && (!events[0] || !events[1] || !events[2] || !events[3]))
        return fail(SPEC_ERR_NULL, "spec_verify_lmhead_sample_timed needs four events");
    const bool shared = dw == nullptr || (dw == tw && dws == tws);
    if (!dw) { dw = tw; dws = tws; }                       // the draft shares the target's head

    char* ws = static_cast<char*>(workspace);
    const double c = 1.4426950408889634 / static_cast<double>(temperature);
    float ch, cl;
    split_c(c, SPEC_DTYPE_F32, ch, cl);
    TileRec* tiles = reinterpret_cast<TileRec*>(ws + plan.o_tiles);
    const int rpb = 2 * k + 1;

    HeadParams HT{};
    HT.h = reinterpret_cast<const signed char*>(th); HT.hs = ths;
    HT.w = reinterpret_cast<const signed char*>(tw); HT.ws = tws;
    HT.packed = packed;
    HT.recs = reinterpret_cast<HeadRecS*>(ws + plan.o_recT);
    HT.tiles = tiles;
    HT.M = B * (k + 1); HT.V = V; HT.d = d; HT.nvt = plan.nvt;
    HT.ch = ch; HT.cl = cl; HT.tok = draft_tokens; HT.k = k; HT.role = 0; HT.rpb = rpb;
    HT.logits = reinterpret_cast<float*>(ws + plan.o_lt);
    HT.exptab = reinterpret_cast<double*>(ws + plan.o_exp);
    HeadParams HD = HT;
    HD.h = reinterpret_cast<const signed char*>(dh); HD.hs = dhs;
    HD.w = reinterpret_cast<const signed char*>(dw); HD.ws = dws;
    HD.recs = reinterpret_cast<HeadRecS*>(ws + plan.o_recD);
    HD.M = B * k; HD.role = 1;
    HD.logits = reinterpret_cast<float*>(ws + plan.o_ld);
    HD.exptab = nullptr;

    // decisions and pass 2: the verify parameters over the stored logits
    // ([B, k+1, V] and [B, k, V], as spec_verify takes them)
    Params P{};
    P.tgt = ws + plan.o_lt;
    P.dft = ws + plan.o_ld;
    P.tok = draft_tokens;
    P.uni = uniforms;
    P.acc_len = accepted_len; P.out_tok = out_tokens; P.gap = gap;
    P.tprob = k > 0 ? target_prob : nullptr;
    P.dprob = k > 0 ? draft_prob : nullptr;
    P.B = B; P.k = k; P.V = V;
    P.rpb = rpb;
    P.nvec = plan.pv.nvec;
    P.wpb = plan.pv.wmax;
    P.N = static_cast<long long>(B) * rpb * V;
    P.L = V;                                               // one slice per row: row r's record at 2r
    P.G = B * rpb;
    P.mode = SPEC_MODE_SAMPLE;
    const char* fe = getenv("SPEC_VERIFY_FORCE_EXACT_PATH");
    P.force_exact = (fe && fe[0] == '1') ? 1 : 0;
    P.ch = ch; P.cl = cl;
    P.c = static_cast<double>(ch) + static_cast<double>(cl);
    P.invT = 1.0 / static_cast<double>(temperature);
    P.vec_ok = (static_cast<size_t>(V) * 4) % 16 == 0;
    P.tiles = tiles;
    P.bat = reinterpret_cast<BatchRec*>(ws + plan.o_bat);
    P.segs = reinterpret_cast<SegRec*>(ws + plan.o_segs);
    P.exptab = reinterpret_cast<double*>(ws + plan.o_exp);
    P.tab_on = 0;

    int dev = 0, ncu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu < 1)
        return fail(SPEC_ERR_HIP, "cannot query the current HIP device");
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipEvent_t const* ev = reinterpret_cast<hipEvent_t const*>(events);
    hipError_t e = ev ? hipEventRecord(ev[0], s) : hipSuccess;
    if (shared && k > 0) {
        // one pass over the shared head for both sets of rows: records and
        // logits land in the target's then the draft's (contiguous) slots
        ConcatParams C;
        C.a = HT.h; C.b = HD.h; C.as = ths; C.bs = dhs;
        C.out = reinterpret_cast<signed char*>(ws + plan.o_hc);
        C.outs = reinterpret_cast<float*>(ws + plan.o_hsc);
        C.na = HT.M; C.d = d;
        if (e == hipSuccess) {
            hipLaunchKernelGGL(head_concat_kernel, dim3(static_cast<unsigned>(HT.M + HD.M)), dim3(NT), 0, s, C);
            e = hipGetLastError();
        }
        HeadParams HC = HT;
        HC.h = C.out; HC.hs = C.outs; HC.M = HT.M + HD.M;
        if (e == hipSuccess) e = launch_head_sample(HC, plan.bmC, s);
    } else {
        if (e == hipSuccess) e = launch_head_sample(HT, plan.bmT, s);
        if (e == hipSuccess && k > 0) e = launch_head_sample(HD, plan.bmD, s);
    }
    if (e == hipSuccess && ev) e = hipEventRecord(ev[1], s);
    if (e == hipSuccess) {
        hipLaunchKernelGGL(head_merge_sample_kernel, dim3(static_cast<unsigned>(HT.M + HD.M)), dim3(NT), 0, s, HT, HD);
        e = hipGetLastError();
    }
    if (e == hipSuccess && ev) e = hipEventRecord(ev[2], s);
    if (e == hipSuccess) e = launch_pass2<F32>(P, dev, ncu, s, nullptr);
    if (e == hipSuccess && ev) e = hipEventRecord(ev[3], s);
    if (e != hipSuccess) return fail(SPEC_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return SPEC_OK;
}

extern "C" {

size_t spec_verify_workspace_size(int32_t B, int32_t k, int32_t V, int dtype, int mode) {
    if (dtype != SPEC_DTYPE_F32 && dtype != SPEC_DTYPE_BF16) return 0;
    Plan p;
    if (!make_plan(B, k, V, mode, dtype, p)) return 0;
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
    return run(target_logits, draft_logits, draft_tokens, nullptr, false, uniforms, temperature, mode, B, k, V,
               dtype, accepted_len, out_tokens, gap, target_prob, draft_prob, workspace, workspace_bytes, stream);
}

int spec_verify_ragged(const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                       const int32_t* draft_len, const float* uniforms, float temperature, int mode, int32_t B,
                       int32_t k, int32_t V, int dtype, int32_t* accepted_len, int32_t* out_tokens, float* gap,
                       float* target_prob, float* draft_prob, void* workspace, size_t workspace_bytes,
                       void* stream) {
    return run(target_logits, draft_logits, draft_tokens, draft_len, true, uniforms, temperature, mode, B, k, V,
               dtype, accepted_len, out_tokens, gap, target_prob, draft_prob, workspace, workspace_bytes, stream);
}

int spec_verify_timed(const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                      const int32_t* draft_len, const float* uniforms, float temperature, int mode, int32_t B,
                      int32_t k, int32_t V, int dtype, int32_t* accepted_len, int32_t* out_tokens, float* gap,
                      float* target_prob, float* draft_prob, void* workspace, size_t workspace_bytes, void* stream,
                      void* const* events) {
    if (!events || !events[0] || !events[1] || !events[2] || !events[3])
        return fail(SPEC_ERR_NULL, "spec_verify_timed needs four events");
    return run(target_logits, draft_logits, draft_tokens, draft_len, draft_len != nullptr, uniforms, temperature,
               mode, B, k, V, dtype, accepted_len, out_tokens, gap, target_prob, draft_prob, workspace,
               workspace_bytes, stream, events);
}

int spec_verify_noalloc(const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                        const float* uniforms, float temperature, int mode, int32_t B, int32_t k, int32_t V,
                        int dtype, int32_t* accepted_len, int32_t* out_tokens, float* gap, float* target_prob,
                        float* draft_prob, void* stream) {
    Plan plan;
    if ((dtype == SPEC_DTYPE_F32 || dtype == SPEC_DTYPE_BF16) && make_plan(B, k, V, mode, dtype, plan) &&
        plan.total > SPEC_NOALLOC_SCRATCH_BYTES)
        return fail(SPEC_ERR_WORKSPACE,
                    "spec_verify_noalloc: B=%d k=%d V=%d need %zu bytes of scratch, more than its %u-byte "
                    "maximum (use spec_verify with a caller workspace)", B, k, V, plan.total,
                    static_cast<unsigned>(SPEC_NOALLOC_SCRATCH_BYTES));
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(SPEC_ERR_HIP, "cannot query the current HIP device");
    void* ws = nullptr;
    const int rc = scratch_ptr(dev, &ws);
    if (rc != SPEC_OK) return rc;
    return run(target_logits, draft_logits, draft_tokens, nullptr, false, uniforms, temperature, mode, B, k, V,
               dtype, accepted_len, out_tokens, gap, target_prob, draft_prob, ws, SPEC_NOALLOC_SCRATCH_BYTES,
               stream);
}

size_t spec_gate_workspace_size(int32_t n, int32_t V, int dtype) {
    return spec_verify_workspace_size(n, 0, V, dtype, SPEC_MODE_GREEDY);
}

int spec_gate(const void* logits, int32_t n, int32_t V, int dtype, int rule, float tau, const uint32_t* admit,
              int32_t* argmax, float* gap, int32_t* fire, void* workspace, size_t workspace_bytes, void* stream) {
    Plan plan;
    const int rc = check_gate(logits, n, V, dtype, rule, tau, admit, argmax, gap, fire, workspace,
                              workspace_bytes, plan);
    if (rc != SPEC_OK) return rc;
    const GateOut g{admit, fire, rule, tau};
    return enqueue(plan, logits, nullptr, nullptr, nullptr, nullptr, 1.0f, SPEC_MODE_GREEDY, n, 0, V, dtype,
                   nullptr, argmax, gap, nullptr, nullptr, &g, workspace, stream);
}

int spec_commit(const int32_t* accepted_len, int32_t B, int32_t k, int32_t* kv_len, const void* slots,
                void* state, size_t state_bytes, void* stream) {
    if (B < 1 || B > (1 << 21) || k < 0 || k > SPEC_MAX_K)
        return fail(SPEC_ERR_SHAPE, "need 1 <= B <= 2^21 and 0 <= k <= %d (got B=%d k=%d)", SPEC_MAX_K, B, k);
    if (!accepted_len) return fail(SPEC_ERR_NULL, "accepted_len is NULL");
    const bool has_state = state_bytes > 0;
    if (has_state && (!slots || !state))
        return fail(SPEC_ERR_NULL, "slots and state are required when state_bytes > 0");
    if (state_bytes % 4 != 0 || !aligned(accepted_len, 4) || (kv_len && !aligned(kv_len, 4)) ||
        (has_state && (!aligned(slots, 4) || !aligned(state, 4))))
        return fail(SPEC_ERR_ALIGN, "pointers must be 4-byte aligned and state_bytes a multiple of 4");
    if (has_state && state_bytes > (static_cast<size_t>(1) << 40))
        return fail(SPEC_ERR_SHAPE, "state_bytes %zu is too large", state_bytes);
    CommitParams C{};
    C.acc = accepted_len;
    C.kv_len = kv_len;
    C.slots = static_cast<const char*>(has_state ? slots : nullptr);
    C.state = static_cast<char*>(has_state ? state : nullptr);
    C.row = state_bytes;
    C.B = B;
    C.k = k;
    const size_t chunks = has_state ? (state_bytes + COMMIT_CHUNK - 1) / COMMIT_CHUNK : 1;
    if (static_cast<double>(chunks) * B >= 2147483647.0)
        return fail(SPEC_ERR_SHAPE, "B * state_bytes is too large");
    C.chunks = static_cast<int>(chunks);
    C.vec16 = has_state && state_bytes % 16 == 0 && aligned(slots, 16) && aligned(state, 16);
    if (!kv_len && !has_state) return SPEC_OK;             // nothing to do
    hipLaunchKernelGGL(commit_kernel, dim3(static_cast<unsigned>(chunks * B)), dim3(NTC), 0,
                       static_cast<hipStream_t>(stream), C);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(SPEC_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return SPEC_OK;
}

size_t spec_lmhead_workspace_size(int32_t B, int32_t k, int32_t V, int32_t d) {
    HeadPlan p;
    if (!make_head_plan(B, k, V, d, p)) return 0;
    return p.total;
}

int spec_verify_lmhead(const int8_t* hidden, const float* hidden_scale, const int8_t* weight,
                       const float* weight_scale, const int32_t* draft_tokens, int32_t B, int32_t k, int32_t V,
                       int32_t d, int32_t* accepted_len, int32_t* out_tokens, float* gap, void* workspace,
                       size_t workspace_bytes, void* stream) {
    return run_head(hidden, hidden_scale, weight, weight_scale, draft_tokens, B, k, V, d, accepted_len,
                    out_tokens, gap, workspace, workspace_bytes, stream, nullptr);
}

int spec_verify_lmhead_timed(const int8_t* hidden, const float* hidden_scale, const int8_t* weight,
                             const float* weight_scale, const int32_t* draft_tokens, int32_t B, int32_t k,
                             int32_t V, int32_t d, int32_t* accepted_len, int32_t* out_tokens, float* gap,
                             void* workspace, size_t workspace_bytes, void* stream, void* const* events) {
    if (!events) return fail(SPEC_ERR_NULL, "spec_verify_lmhead_timed needs three events");
    return run_head(hidden, hidden_scale, weight, weight_scale, draft_tokens, B, k, V, d, accepted_len,
                    out_tokens, gap, workspace, workspace_bytes, stream, events);
}

size_t spec_lmhead_packed_size(int32_t V, int32_t d) {
    if (V < 1 || V > (1 << 29) || d < HK || d > HEAD_MAX_D || d % HK != 0) return 0;
    return static_cast<size_t>((V + HV - 1) / HV) * HV * static_cast<size_t>(d);
}

int spec_lmhead_pack(const int8_t* weight, int32_t V, int32_t d, int8_t* packed, size_t packed_bytes, void* stream) {
    const size_t need = spec_lmhead_packed_size(V, d);
    if (need == 0) return fail(SPEC_ERR_SHAPE, "need 1 <= V <= 2^29 and d a multiple of %d in [%d, %d] (got V=%d d=%d)",
                               HK, HK, HEAD_MAX_D, V, d);
    if (!weight || !packed) return fail(SPEC_ERR_NULL, "weight and packed are required");
    if (!aligned(weight, 16) || !aligned(packed, 16)) return fail(SPEC_ERR_ALIGN, "weight and packed must be 16-byte aligned");
    if (packed_bytes < need) return fail(SPEC_ERR_WORKSPACE, "packed needs %zu bytes (got %zu)", need, packed_bytes);
    const long long nchunks = static_cast<long long>(need / 16);
    const unsigned grid = static_cast<unsigned>(std::min<long long>((nchunks + NT - 1) / NT, 1 << 16));
    hipLaunchKernelGGL(head_pack_kernel, dim3(grid), dim3(NT), 0, static_cast<hipStream_t>(stream),
                       reinterpret_cast<const signed char*>(weight), V, d, reinterpret_cast<signed char*>(packed),
                       nchunks);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? 0 : fail(SPEC_ERR_HIP, "HIP error: %s", hipGetErrorString(e));
}

int spec_verify_lmhead_packed(const int8_t* hidden, const float* hidden_scale, const int8_t* packed_weight,
                              const float* weight_scale, const int32_t* draft_tokens, int32_t B, int32_t k,
                              int32_t V, int32_t d, int32_t* accepted_len, int32_t* out_tokens, float* gap,
                              void* workspace, size_t workspace_bytes, void* stream, void* const* events) {
    return run_head(hidden, hidden_scale, packed_weight, weight_scale, draft_tokens, B, k, V, d, accepted_len,
                    out_tokens, gap, workspace, workspace_bytes, stream, events, 1);
}

size_t spec_lmhead_sample_workspace_size(int32_t B, int32_t k, int32_t V, int32_t d) {
    HeadSamplePlan p;
    if (V > SPEC_MAX_V_SAMPLE || !make_head_sample_plan(B, k, V, d, p)) return 0;
    return p.total;
}

int spec_verify_lmhead_sample(const int8_t* target_hidden, const float* target_hidden_scale,
                              const int8_t* target_weight, const float* target_weight_scale,
                              const int8_t* draft_hidden, const float* draft_hidden_scale,
                              const int8_t* draft_weight, const float* draft_weight_scale,
                              const int32_t* draft_tokens, const float* uniforms, float temperature, int32_t B,
                              int32_t k, int32_t V, int32_t d, int32_t* accepted_len, int32_t* out_tokens,
                              float* gap, float* target_prob, float* draft_prob, void* workspace,
                              size_t workspace_bytes, void* stream) {
    return run_head_sample(target_hidden, target_hidden_scale, target_weight, target_weight_scale, draft_hidden,
                           draft_hidden_scale, draft_weight, draft_weight_scale, draft_tokens, uniforms,
                           temperature, B, k, V, d, accepted_len, out_tokens, gap, target_prob, draft_prob,
                           workspace, workspace_bytes, stream, nullptr);
}

int spec_verify_lmhead_sample_timed(const int8_t* target_hidden, const float* target_hidden_scale,
                                    const int8_t* target_weight, const float* target_weight_scale,
                                    const int8_t* draft_hidden, const float* draft_hidden_scale,
                                    const int8_t* draft_weight, const float* draft_weight_scale,
                                    const int32_t* draft_tokens, const float* uniforms, float temperature,
                                    int32_t B, int32_t k, int32_t V, int32_t d, int32_t* accepted_len,
                                    int32_t* out_tokens, float* gap, float* target_prob, float* draft_prob,
                                    void* workspace, size_t workspace_bytes, void* stream, void* const* events) {
    if (!events) return fail(SPEC_ERR_NULL, "spec_verify_lmhead_sample_timed needs four events");
    return run_head_sample(target_hidden, target_hidden_scale, target_weight, target_weight_scale, draft_hidden,
                           draft_hidden_scale, draft_weight, draft_weight_scale, draft_tokens, uniforms,
                           temperature, B, k, V, d, accepted_len, out_tokens, gap, target_prob, draft_prob,
                           workspace, workspace_bytes, stream, events);
}

int spec_verify_lmhead_sample_packed(const int8_t* target_hidden, const float* target_hidden_scale,
                                     const int8_t* target_packed_weight, const float* target_weight_scale,
                                     const int8_t* draft_hidden, const float* draft_hidden_scale,
                                     const int8_t* draft_packed_weight, const float* draft_weight_scale,
                                     const int32_t* draft_tokens, const float* uniforms, float temperature,
                                     int32_t B, int32_t k, int32_t V, int32_t d, int32_t* accepted_len,
                                     int32_t* out_tokens, float* gap, float* target_prob, float* draft_prob,
                                     void* workspace, size_t workspace_bytes, void* stream, void* const* events) {
    return run_head_sample(target_hidden, target_hidden_scale, target_packed_weight, target_weight_scale,
                           draft_hidden, draft_hidden_scale, draft_packed_weight, draft_weight_scale, draft_tokens,
                           uniforms, temperature, B, k, V, d, accepted_len, out_tokens, gap, target_prob, draft_prob,
                           workspace, workspace_bytes, stream, events, 1);
}

const char* spec_verify_last_error(void) { return g_err; }

const char* spec_verify_version(void) { return "specverify 0.5.0 (gfx950)"; }

}  // extern "C"
