/*
 * spec_verify_ref.c -- plain fp64 CPU oracle of the speculative-decoding verify step.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may link, load or call
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline
 * leg use it. It shares no code, header or table with the HIP library.
 *
 * What it computes (per batch row b, positions 0-based: drafts i = 0..k-1,
 * bonus row i = k):
 *
 *  Sampling mode ("Speculative Decoding: The Physics of Stolen Time", section 2,
 *  the modified rejection sampling rule and its losslessness proof; the
 *  speculative-decoding design note, "The acceptance math"):
 *    p_i = softmax(target_logits[b,i,:] / T) for i <= k,
 *    q_i = softmax(draft_logits[b,i,:]  / T) for i <  k,
 *    for i = 0..k-1: r_i = p_i(x_i) / q_i(x_i), accept iff u[b,i,0] < r_i;
 *    at the first rejection a: sample from norm(max(0, p_a - q_a));
 *    if all k accepted (a = k): sample a bonus token from p_k.
 *    Sampling from a weight vector w uses the inverse CDF in vocabulary order:
 *    the smallest j with C_j > u*Z, C_j = sum_{x<=j} w_x, Z = C_{V-1},
 *    with u = u[b,a,1].
 *
 *  Greedy mode ("The Inference Wall" part 7, "How speculative decoding works":
 *  accept while the guess equals the target's own token, at the first mismatch
 *  take the target's token; all matched gives k+1 tokens):
 *    g_i = argmax target_logits[b,i,:] (lowest index on ties),
 *    a = first i < k with x_i != g_i, else k; the emitted token is g_a.
 *
 *  Gap ("Speculative Pre-Positioning", Eq. 11): top-1 minus top-2 of the raw
 *  target logits of every row i <= k (0 on ties at the top; +inf when fewer
 *  than two finite entries exist).
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *  - temperature divides target and draft logits alike; the gap and greedy
 *    use raw logits; T is the float argument widened exactly to double;
 *  - uniform channel 0 is the acceptance test, channel 1 the inverse-CDF draw;
 *  - accept iff u < r (strict), so r >= 1 always accepts and p(x) = 0 always
 *    rejects; q(x) = 0 gives r = +inf if p(x) > 0 and r = 0 otherwise;
 *  - if a rejection leaves Z = 0 (only possible through rounding), the token
 *    is drawn from p_a instead and the row is flagged;
 *  - a row pair with NaN or +inf anywhere, a row with no finite entry, or a
 *    draft token outside [0, V) makes batch row b invalid: accepted_len = -1
 *    and every out_token = -1. (Greedy mode reads no draft logits.)
 *
 * Every sum is a Neumaier-compensated sum in vocabulary order.
 *
 * Ragged drafts (the speculative-decoding design note and "Speculative
 * Decoding: The Physics of Stolen Time" allow each sequence its own number of
 * guesses): with draft_len[b] = kb in [0, k], batch row b verifies only
 * positions 0..kb-1, as the rule above with k = kb: the target rows 0..kb,
 * the draft rows and tokens 0..kb-1 are read, nothing else of the row; the
 * bonus comes from target row kb. Outputs keep the [.., k+1] / [.., k] layout:
 * gap of rows past kb and p/q of positions past kb-1 are NaN (not read), and
 * out_tokens past the emitted token are -1. A draft_len outside [0, k] makes
 * the row invalid (gap all NaN). draft_len = NULL means kb = k everywhere.
 *
 * Margins (for the flagged near-tie policy): margin_acc[b] is the smallest
 * |u - r_i| over the decisions actually taken, margin_cdf[b] the distance of u
 * to the nearest edge of the chosen token's normalized CDF interval
 * min(u - C_{j-1}/Z, C_j/Z - u). Both are +inf where no such decision exists.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { REF_F32 = 0, REF_BF16 = 1 };
enum { REF_SAMPLE = 0, REF_GREEDY = 1 };

/* Exact widening of one stored logit to double. */
static double ref_load(const void* base, int dtype, size_t idx)
{
    if (dtype == REF_F32) {
        return (double)((const float*)base)[idx];
    }
    uint32_t bits = (uint32_t)((const uint16_t*)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* Neumaier compensated accumulator. */
typedef struct { double s, c; } ref_sum_t;

static void ref_sum_add(ref_sum_t* a, double x)
{
    double t = a->s + x;
    if (fabs(a->s) >= fabs(x)) a->c += (a->s - t) + x;
    else                       a->c += (x - t) + a->s;
    a->s = t;
}

static double ref_sum_value(const ref_sum_t* a) { return a->s + a->c; }

/* Row check: 1 if the row has no NaN, no +inf and at least one finite entry. */
static int ref_row_ok(const void* base, int dtype, size_t off, int V)
{
    int finite = 0;
    for (int x = 0; x < V; ++x) {
        double v = ref_load(base, dtype, off + (size_t)x);
        if (isnan(v) || (isinf(v) && v > 0)) return 0;
        if (isfinite(v)) finite = 1;
    }
    return finite;
}

/* p[x] = exp(z_x - max z) / sum, z_x = logit_x / T. Requires ref_row_ok. */
static void ref_softmax(const void* base, int dtype, size_t off, int V, double T, double* p)
{
    double m = -INFINITY;
    for (int x = 0; x < V; ++x) {
        double z = ref_load(base, dtype, off + (size_t)x) / T;
        if (z > m) m = z;
    }
    ref_sum_t S = {0.0, 0.0};
    for (int x = 0; x < V; ++x) {
        double z = ref_load(base, dtype, off + (size_t)x) / T;
        double e = isinf(z) ? 0.0 : exp(z - m);
        p[x] = e;
        ref_sum_add(&S, e);
    }
    double s = ref_sum_value(&S);
    for (int x = 0; x < V; ++x) p[x] /= s;
}

/* Top-1 minus top-2 of the raw row (multiset, so ties give 0). */
static double ref_gap(const void* base, int dtype, size_t off, int V)
{
    double t1 = -INFINITY, t2 = -INFINITY;
    int finite = 0;
    for (int x = 0; x < V; ++x) {
        double v = ref_load(base, dtype, off + (size_t)x);
        if (isnan(v)) continue;
        if (isfinite(v)) ++finite;
        if (v > t1) { t2 = t1; t1 = v; }
        else if (v > t2) { t2 = v; }
    }
    if (finite < 2) return INFINITY;
    return t1 - t2;
}

/* Lowest index of the maximum of the raw row (NaN entries never win). */
static int ref_argmax(const void* base, int dtype, size_t off, int V)
{
    int best = 0;
    double bv = -INFINITY;
    int seen = 0;
    for (int x = 0; x < V; ++x) {
        double v = ref_load(base, dtype, off + (size_t)x);
        if (isnan(v)) continue;
        if (!seen || v > bv) { bv = v; best = x; seen = 1; }
    }
    return best;
}

/*
 * Inverse-CDF draw from the non-negative weights w[0..V-1] with uniform u:
 * the smallest j with C_j > u*Z. Returns -1 when Z <= 0. *margin receives the
 * normalized distance of u to the chosen interval's nearest edge, *alt the
 * token on the other side of that edge (the nearest index with positive
 * weight below j when the lower edge is nearer, above j otherwise; j itself
 * when there is none): what the draw gives when u moves across that edge.
 */
static int ref_inverse_cdf(const double* w, int V, double u, double* margin, double* Zout, int* alt)
{
    ref_sum_t acc = {0.0, 0.0};
    for (int x = 0; x < V; ++x) ref_sum_add(&acc, w[x]);
    double Z = ref_sum_value(&acc);
    *Zout = Z;
    *alt = -1;
    if (!(Z > 0.0)) return -1;
    double t = u * Z;
    ref_sum_t C = {0.0, 0.0};
    double prev = 0.0;
    for (int j = 0; j < V; ++j) {
        ref_sum_add(&C, w[j]);
        double cj = ref_sum_value(&C);
        if (j == V - 1) cj = Z;               /* C_{V-1} is Z by definition */
        if (cj > t) {
            double lo = u - prev / Z, hi = cj / Z - u;
            *margin = lo < hi ? lo : hi;
            int nb = j;
            if (lo < hi) {
                for (int x = j - 1; x >= 0; --x) if (w[x] > 0.0) { nb = x; break; }
            } else {
                for (int x = j + 1; x < V; ++x) if (w[x] > 0.0) { nb = x; break; }
            }
            *alt = nb;
            return j;
        }
        prev = cj;
    }
    *margin = 0.0;                           /* unreachable for u < 1 */
    *alt = V - 1;
    return V - 1;
}

static void ref_fill_invalid(int k, int32_t* acc_len, int32_t* out)
{
    *acc_len = -1;
    for (int i = 0; i <= k; ++i) out[i] = -1;
}


/*
 * Smallest distance, in units of the target distribution's total mass, between
 * the residual draw's point u*Z and a CDF boundary that fp64 can resolve. The
 * residual weights max(0, p - q) are differences of two probability vectors,
 * so any double-precision evaluation of them (this one included) carries
 * absolute errors of order 1e-15 of the total mass; a draw closer than this to
 * a boundary is flagged (bit 2), whatever its distance relative to Z.
 */
#define REF_RESID_ABS_MARGIN 1e-13

/*
 * The draw at position a of batch row b (0-based, a <= k): a < k samples the
 * residual norm(max(0, p_a - q_a)), a = k the bonus from p_k, both with the
 * uniform u[b,a,1]. Sets *tok, *alt (the token across the nearest CDF edge,
 * see ref_inverse_cdf) and *m_cdf; returns the flag bits (1: the residual mass
 * was zero and p_a was used; 2: the residual draw lies within
 * REF_RESID_ABS_MARGIN of a boundary). work holds 3*V doubles.
 */
static int ref_draw(const void* target, const void* draft, const float* uniforms, double T,
                    int kmax, int k, int a, int V, int dtype, size_t b, int32_t* tok, int32_t* alt,
                    double* m_cdf, double* work)
{
    const size_t rowsT = (size_t)(kmax + 1), rowsD = (size_t)kmax;
    double* p = work;
    double* q = work + V;
    double* w = work + 2 * (size_t)V;
    int flags = 0, t, nb;
    double Z;
    double u1 = (double)uniforms[(b * rowsT + (size_t)a) * 2 + 1];
    ref_softmax(target, dtype, (b * rowsT + (size_t)a) * (size_t)V, V, T, p);
    if (a < k) {
        ref_softmax(draft, dtype, (b * rowsD + (size_t)a) * (size_t)V, V, T, q);
        for (int x = 0; x < V; ++x) {
            double d = p[x] - q[x];
            w[x] = d > 0.0 ? d : 0.0;
        }
        t = ref_inverse_cdf(w, V, u1, m_cdf, &Z, &nb);
        if (t < 0) {                          /* Z = 0: draw from p_a, flag */
            flags |= 1;
            t = ref_inverse_cdf(p, V, u1, m_cdf, &Z, &nb);
            *m_cdf = 0.0;
        } else if (*m_cdf * Z < REF_RESID_ABS_MARGIN) {
            flags |= 2;
        }
    } else {
        t = ref_inverse_cdf(p, V, u1, m_cdf, &Z, &nb);
    }
    *tok = t;
    *alt = nb;
    return flags;
}

/*
 * One batch row. work must hold 3*V doubles.
 * Returns a bit set: 1 = Z fell back to p_a, 2 = the residual draw is within
 * REF_RESID_ABS_MARGIN of a CDF boundary (both are flags).
 *
 * Alternatives (sampling mode; NULL pointers skip them): alt_tok receives the
 * token the final draw gives with its uniform moved across the nearest CDF
 * edge. When the smallest acceptance margin |u - r_i| of the tests taken is
 * below flip_delta, alt_acc/alt_out receive the whole outcome with that one
 * test decided the other way (an accept becomes the first rejection, a
 * rejection an accept, after which the later tests run as usual); otherwise
 * they repeat acc_len/out.
 */
static int ref_one_row(const void* target, const void* draft, const int32_t* tokens,
                       const float* uniforms, double T, int mode, int kmax, int kb, int V,
                       int dtype, size_t b, int32_t* acc_len, int32_t* out, double* gap,
                       double* p_tok, double* q_tok, double* m_acc, double* m_cdf,
                       double flip_delta, int32_t* alt_acc, int32_t* alt_out, int32_t* alt_tok,
                       double* work)
{
    const size_t rowsT = (size_t)(kmax + 1), rowsD = (size_t)kmax;
    int flags = 0;
    *m_acc = INFINITY;
    *m_cdf = INFINITY;
    for (int i = 0; i <= kmax; ++i) gap[i] = NAN;
    for (int i = 0; i < kmax; ++i) { p_tok[i] = NAN; q_tok[i] = NAN; }
    if (alt_acc) { *alt_acc = -1; for (int i = 0; i <= kmax; ++i) alt_out[i] = -1; }
    if (alt_tok) *alt_tok = -1;
    if (kb < 0 || kb > kmax) { ref_fill_invalid(kmax, acc_len, out); return 0; }
    const int k = kb;                         /* this row's draft length */
    for (int i = 0; i <= k; ++i) {
        gap[i] = ref_gap(target, dtype, (b * rowsT + (size_t)i) * (size_t)V, V);
    }

    /* validity of the whole batch row */
    int ok = 1;
    for (int i = 0; i < k && ok; ++i) {
        int32_t x = tokens[b * rowsD + (size_t)i];
        if (x < 0 || x >= V) ok = 0;
    }
    for (int i = 0; i <= k && ok; ++i) {
        ok = ref_row_ok(target, dtype, (b * rowsT + (size_t)i) * (size_t)V, V);
    }
    if (mode == REF_SAMPLE) {
        for (int i = 0; i < k && ok; ++i) {
            ok = ref_row_ok(draft, dtype, (b * rowsD + (size_t)i) * (size_t)V, V);
        }
    }
    if (!ok) { ref_fill_invalid(kmax, acc_len, out); return 0; }

    if (mode == REF_GREEDY) {
        int a = k;
        for (int i = 0; i < k; ++i) {
            int g = ref_argmax(target, dtype, (b * rowsT + (size_t)i) * (size_t)V, V);
            if (tokens[b * rowsD + (size_t)i] != g) { a = i; break; }
        }
        *acc_len = a;
        for (int i = 0; i < a; ++i) out[i] = tokens[b * rowsD + (size_t)i];
        out[a] = ref_argmax(target, dtype, (b * rowsT + (size_t)a) * (size_t)V, V);
        for (int i = a + 1; i <= kmax; ++i) out[i] = -1;
        return 0;
    }

    double* p = work;
    double* q = work + V;

    /* p_i(x_i) and q_i(x_i) for every position */
    for (int i = 0; i < k; ++i) {
        ref_softmax(target, dtype, (b * rowsT + (size_t)i) * (size_t)V, V, T, p);
        ref_softmax(draft, dtype, (b * rowsD + (size_t)i) * (size_t)V, V, T, q);
        int32_t x = tokens[b * rowsD + (size_t)i];
        p_tok[i] = p[x];
        q_tok[i] = q[x];
    }
    /* acceptance tests, in order, up to the first rejection; `flip` decides
       the test at that position the other way (-1: none) */
    int a = k, amin = -1;
    for (int pass = 0; pass < 2; ++pass) {
        const int flip = pass == 0 ? -1 : amin;
        if (pass == 1 && !(alt_acc && amin >= 0 && *m_acc < flip_delta)) break;
        int aa = k;
        for (int i = 0; i < k; ++i) {
            double P = p_tok[i], Q = q_tok[i];
            double r = (Q > 0.0) ? P / Q : (P > 0.0 ? INFINITY : 0.0);
            double u0 = (double)uniforms[(b * rowsT + (size_t)i) * 2 + 0];
            int accept = u0 < r;
            if (pass == 0) {
                double mg = fabs(u0 - r);
                if (mg < *m_acc) { *m_acc = mg; amin = i; }
            }
            if (i == flip) accept = !accept;
            if (!accept) { aa = i; break; }
        }
        if (pass == 0) {
            a = aa;
            *acc_len = a;
            for (int i = 0; i < a; ++i) out[i] = tokens[b * rowsD + (size_t)i];
            for (int i = a + 1; i <= kmax; ++i) out[i] = -1;
            int32_t tok, nb;
            flags = ref_draw(target, draft, uniforms, T, kmax, k, a, V, dtype, b, &tok, &nb, m_cdf, work);
            out[a] = tok;
            if (alt_tok) *alt_tok = nb;
            if (alt_acc) { *alt_acc = a; for (int i = 0; i <= kmax; ++i) alt_out[i] = out[i]; }
        } else {
            int32_t tok, nb;
            double mc;
            *alt_acc = aa;
            for (int i = 0; i < aa; ++i) alt_out[i] = tokens[b * rowsD + (size_t)i];
            for (int i = aa + 1; i <= kmax; ++i) alt_out[i] = -1;
            ref_draw(target, draft, uniforms, T, kmax, k, aa, V, dtype, b, &tok, &nb, &mc, work);
            alt_out[aa] = tok;
        }
    }
    return flags;
}

/*
 * Public entry. All buffers are host memory.
 *  target  [B,k+1,V] (float32 or bfloat16 bits), draft [B,k,V] (may be NULL in
 *  greedy mode), tokens [B,k] int32, draft_len [B] int32 (may be NULL: all k),
 *  uniforms [B,k+1,2] float32 (may be NULL in greedy mode).
 *  Outputs: acc_len [B], out_tokens [B,k+1], gap [B,k+1], p_tok/q_tok [B,k]
 *  (NaN where not computed), margin_acc [B], margin_cdf [B], flags [B].
 *  Optional alternatives (sampling mode; all three NULL to skip): alt_acc [B],
 *  alt_out [B,k+1] and alt_tok [B], see ref_one_row; flip_delta chooses the
 *  rows whose nearest acceptance test is flipped.
 *  threads <= 0 uses the OpenMP default. Returns 0, or -1 on bad arguments.
 */
int spec_verify_ref_full(const void* target, const void* draft, const int32_t* tokens,
                         const int32_t* draft_len, const float* uniforms, float temperature,
                         int mode, int B, int k, int V, int dtype,
                         int32_t* acc_len, int32_t* out_tokens, double* gap,
                         double* p_tok, double* q_tok, double* margin_acc,
                         double* margin_cdf, int32_t* flags, double flip_delta,
                         int32_t* alt_acc, int32_t* alt_out, int32_t* alt_tok, int threads)
{
    if (B < 0 || k < 0 || V < 1) return -1;
    if (dtype != REF_F32 && dtype != REF_BF16) return -1;
    if (mode != REF_SAMPLE && mode != REF_GREEDY) return -1;
    if (!target || (k > 0 && !tokens)) return -1;
    if (mode == REF_SAMPLE && (!uniforms || (k > 0 && !draft))) return -1;
    if ((alt_acc == NULL) != (alt_out == NULL)) return -1;
    double T = (double)temperature;
    if (mode == REF_SAMPLE && !(T > 0.0 && isfinite(T))) return -1;

    int nt = threads;
#ifdef _OPENMP
    if (nt <= 0) nt = omp_get_max_threads();
#else
    nt = 1;
#endif
    int failed = 0;
#ifdef _OPENMP
#pragma omp parallel num_threads(nt)
#endif
    {
        double* work = (double*)malloc(sizeof(double) * 3 * (size_t)V);
        if (!work) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            failed = 1;
        }
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (int b = 0; b < B; ++b) {
            if (!work) continue;
            const int kb = draft_len ? draft_len[b] : k;
            flags[b] = ref_one_row(target, draft, tokens, uniforms, T, mode, k, kb, V, dtype,
                                   (size_t)b, &acc_len[b], &out_tokens[(size_t)b * (k + 1)],
                                   &gap[(size_t)b * (k + 1)], &p_tok[(size_t)b * k],
                                   &q_tok[(size_t)b * k], &margin_acc[b], &margin_cdf[b],
                                   flip_delta, alt_acc ? &alt_acc[b] : NULL,
                                   alt_out ? &alt_out[(size_t)b * (k + 1)] : NULL,
                                   alt_tok ? &alt_tok[b] : NULL, work);
        }
        free(work);
    }
    return failed ? -2 : 0;
}

/* Per-row draft lengths, no alternatives. */
int spec_verify_ref_ragged(const void* target, const void* draft, const int32_t* tokens,
                           const int32_t* draft_len, const float* uniforms, float temperature,
                           int mode, int B, int k, int V, int dtype,
                           int32_t* acc_len, int32_t* out_tokens, double* gap,
                           double* p_tok, double* q_tok, double* margin_acc,
                           double* margin_cdf, int32_t* flags, int threads)
{
    return spec_verify_ref_full(target, draft, tokens, draft_len, uniforms, temperature, mode, B, k,
                                V, dtype, acc_len, out_tokens, gap, p_tok, q_tok, margin_acc,
                                margin_cdf, flags, 0.0, NULL, NULL, NULL, threads);
}

/* Fixed-length drafts: every batch row verifies all k positions. */
int spec_verify_ref(const void* target, const void* draft, const int32_t* tokens,
                    const float* uniforms, float temperature, int mode,
                    int B, int k, int V, int dtype,
                    int32_t* acc_len, int32_t* out_tokens, double* gap,
                    double* p_tok, double* q_tok, double* margin_acc,
                    double* margin_cdf, int32_t* flags, int threads)
{
    return spec_verify_ref_ragged(target, draft, tokens, NULL, uniforms, temperature, mode, B, k, V,
                                  dtype, acc_len, out_tokens, gap, p_tok, q_tok, margin_acc,
                                  margin_cdf, flags, threads);
}

/* Number of threads the OpenMP runtime would use by default. */
int spec_verify_ref_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Confidence gate over n ready distributions logits[n, V] ("Speculative
 * Pre-Positioning", section 2.4, Eqs. 11-12, and the gated serve of
 * Algorithm 2): gamma = l(1) - l(2), the two largest raw logits counted as a
 * multiset (so a tie at the top gives 0; +inf when the row has fewer than two
 * finite entries), a = the lowest index of the maximum, and
 *   rule 0 (margin):    fire iff gamma > tau and a is admissible;
 *   rule 1 (certified): fire iff gamma > 0, 2*tau <= gamma and a is admissible
 * (the speculative-decoding design note, "Axis 1 reuses the gate we already
 * have": with a strict argmax and every logit moved by less than tau in
 * sup-norm, 2*tau <= gamma keeps the argmax; tau is then the residual bound Q).
 * The comparison is made on the gap rounded to float32 (the difference of the
 * two float logits in single precision) against the float32 tau, the
 * precision the gap is stored in. admit is a V-bit mask, bit (j & 31) of word
 * j >> 5 marking token j admissible; NULL admits every token. A row with NaN
 * or +inf anywhere or with no finite entry is invalid: argmax -1, gap NaN,
 * fire 0. Returns 0, or -1 on bad arguments (tau NaN; rule 1 with tau < 0).
 */
int spec_gate_ref(const void* logits, int n, int V, int dtype, int rule, float tau,
                  const uint32_t* admit, int32_t* argmax, double* gap, int32_t* fire)
{
    if (n < 0 || V < 1 || (dtype != REF_F32 && dtype != REF_BF16)) return -1;
    if (rule != 0 && rule != 1) return -1;
    if (isnan(tau) || (rule == 1 && tau < 0.0f)) return -1;
    for (int r = 0; r < n; ++r) {
        const size_t off = (size_t)r * (size_t)V;
        if (!ref_row_ok(logits, dtype, off, V)) {
            argmax[r] = -1;
            gap[r] = NAN;
            fire[r] = 0;
            continue;
        }
        double t1 = -INFINITY, t2 = -INFINITY;
        int finite = 0;
        for (int x = 0; x < V; ++x) {
            const double v = ref_load(logits, dtype, off + (size_t)x);
            if (isfinite(v)) ++finite;
            if (v > t1) { t2 = t1; t1 = v; }
            else if (v > t2) { t2 = v; }
        }
        const int a = ref_argmax(logits, dtype, off, V);
        volatile float g32 = finite < 2 ? INFINITY : (float)t1 - (float)t2;
        const int ok_a = admit == NULL || ((admit[a >> 5] >> (a & 31)) & 1u);
        int f;
        if (rule == 0) f = g32 > tau;
        else f = g32 > 0.0f && 2.0f * tau <= g32;
        argmax[r] = a;
        gap[r] = finite < 2 ? INFINITY : t1 - t2;
        fire[r] = f && ok_a;
    }
    return 0;
}
