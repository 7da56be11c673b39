/*
 * CPU oracle for the routing half of the one-GPU MoE layer.  TEST INFRASTRUCTURE
 * ONLY: tests, the smoke check and the benchmark's CPU-baseline leg may call it;
 * the product path never does.
 *
 * What it follows.  "MoE Parallel Folding" (arXiv 2504.14960), knowledge-base
 * notes page, method paragraph and the Section 3.3 Token Dispatcher quote: the
 * router assigns each token to its Top-K experts, a permutation makes the tokens
 * of one expert contiguous, and assignments beyond an expert's capacity are
 * dropped per sub-sequence (the default drop strategy).  The pages name Top-K
 * gating and a capacity factor but give no formula for either; the readings fixed here
 * (softmax over all experts, top-K, gates renormalised over the K chosen,
 * capacity ceil(cf*S*K/E), drop key (p desc, t asc), expert-major then
 * token-ascending row order) are the plainest ones the rest supports.
 *
 * Precision.  Integer decisions (top-K, drops) are taken from fp32 values, the
 * precision of the kernel, so everything here is fp32 with every operation
 * rounded on its own.  Build with -ffp-contract=off and without fast-math; on
 * x86-64 float arithmetic is SSE, so there is no excess precision.
 *
 * exp.  Cody & Waite range reduction (W. J. Cody and W. Waite, "Software Manual
 * for the Elementary Functions", 1980): n = rint(r / ln 2), r' = (r - n*C1) - n*C2
 * with C1 + C2 = ln 2 and C1 short enough that n*C1 is exact, then the degree-7
 * Taylor polynomial of exp on [-ln2/2, ln2/2] in Horner form, scaled by 2^n.
 * Inputs are r <= 0 (a logit minus the row maximum).  Results that would fall
 * below 2^-125 are returned as +0, so no denormal is ever produced.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_BAD_ARG (-1)

static float from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* ln 2 split: C1 = ln 2 truncated to a multiple of 2^-16 (16 significant bits, so
 * n*C1 is exact for |n| < 2^8), C2 = the rest, rounded to fp32.  Both are derived
 * from the double-precision ln 2 at first use. */
static float g_c1, g_c2, g_inv_ln2;
static float g_coef[8];
static int g_init = 0;

static void init_consts(void) {
    if (g_init) return;
    const double ln2 = 0.69314718055994530942;
    double c1 = floor(ln2 * 65536.0) / 65536.0;
    g_c1 = (float)c1;
    g_c2 = (float)(ln2 - c1);
    g_inv_ln2 = (float)(1.0 / ln2);
    double fact = 1.0;
    for (int i = 0; i < 8; ++i) {
        if (i > 0) fact *= (double)i;
        g_coef[i] = (float)(1.0 / fact);
    }
    g_init = 1;
}

float oracle_exp(float r) {
    init_consts();
    float t = r * g_inv_ln2;
    float n = rintf(t);
    if (n < -125.0f) return 0.0f;
    float nc1 = n * g_c1;
    float rr = r - nc1;
    float nc2 = n * g_c2;
    rr = rr - nc2;
    /* Horner: ((((((c7 r + c6) r + c5) r + c4) r + c3) r + c2) r + c1) r + c0 */
    float q = g_coef[7];
    for (int i = 6; i >= 0; --i) {
        q = q * rr;
        q = q + g_coef[i];
    }
    uint32_t eb = (uint32_t)((int)n + 127) << 23;
    return q * from_bits(eb);
}

/* Pairwise sum of v[0..n): pad to the next power of two with +0.0, then add
 * neighbours level by level ((v0+v1), (v2+v3), ... then pairs of those). */
static float pairwise_sum(const float* v, int n) {
    float buf[256];
    int p = 1;
    while (p < n) p <<= 1;
    for (int i = 0; i < p; ++i) buf[i] = (i < n) ? v[i] : 0.0f;
    while (p > 1) {
        for (int i = 0; i < p / 2; ++i) buf[i] = buf[2 * i] + buf[2 * i + 1];
        p >>= 1;
    }
    return buf[0];
}

float oracle_pairwise_sum(const float* v, int n) {
    if (n < 1 || n > 256) return 0.0f;
    return pairwise_sum(v, n);
}

/* Softmax of one row of E logits, in the rounding described above. */
void oracle_softmax_row(const float* logit, int E, float* p) {
    float m = logit[0];
    for (int e = 1; e < E; ++e) if (logit[e] > m) m = logit[e];
    float u[256];
    for (int e = 0; e < E; ++e) {
        float r = logit[e] - m;
        u[e] = oracle_exp(r);
    }
    float Z = pairwise_sum(u, E);
    for (int e = 0; e < E; ++e) p[e] = u[e] / Z;
}

/* "a before b" in the top-K order: larger probability first, lower index on ties. */
static int topk_before(float pa, int ea, float pb, int eb) {
    if (pa != pb) return pa > pb;
    return ea < eb;
}

/* Capacity per (sub-sequence, expert): ceil(cf * S * K / E) in double; cf < 0
 * means dropless (-1). */
int oracle_capacity(int S, int K, int E, double cf) {
    if (cf < 0.0) return -1;
    double c = ceil(cf * (double)S * (double)K / (double)E);
    return (int)c;
}

/*
 * Full routing of T tokens.
 *   logits        [T,E] fp32 input
 *   topk_idx      [T,K] expert of slot k (slot 0 = most probable)
 *   topk_prob     [T,K] softmax probability of that expert (over all E)
 *   topk_gate     [T,K] renormalised gate p / (pairwise sum of the K chosen p)
 *   keep          [T,K] 1 if the assignment survives the capacity drop
 *   row_of        [T,K] row in the permuted buffer, -1 if dropped
 *   src_of        [T*K] (only the first n_kept are written) t*K + k of each row
 *   routed_counts [T/S,E] assignments per (sub-sequence, expert) before dropping
 *   kept_counts   [E]   kept assignments per expert
 *   offsets       [E+1] exclusive scan of kept_counts
 *   n_kept        [1]
 * capacity < 0: dropless.  Returns 0, or -1 on a bad argument.
 */
int oracle_route(int T, int E, int K, int S, int capacity, const float* logits,
                 int32_t* topk_idx, float* topk_prob, float* topk_gate, uint8_t* keep,
                 int32_t* row_of, int32_t* src_of, int32_t* routed_counts,
                 int32_t* kept_counts, int32_t* offsets, int32_t* n_kept) {
    if (T < 0 || E < 1 || E > 256 || K < 1 || K > E || S < 1 || (T % S) != 0)
        return ORACLE_BAD_ARG;
    int n_sub = T / S;

    /* Softmax, top-K and gates, token by token. */
    float p[256];
    int order[256];
    for (int t = 0; t < T; ++t) {
        oracle_softmax_row(logits + (size_t)t * E, E, p);
        /* insertion sort of expert ids by (p desc, e asc); E <= 256 */
        for (int e = 0; e < E; ++e) {
            int j = e;
            while (j > 0 && topk_before(p[e], e, p[order[j - 1]], order[j - 1])) {
                order[j] = order[j - 1];
                --j;
            }
            order[j] = e;
        }
        float sel[256];
        for (int k = 0; k < K; ++k) {
            topk_idx[(size_t)t * K + k] = order[k];
            topk_prob[(size_t)t * K + k] = p[order[k]];
            sel[k] = p[order[k]];
        }
        float P = pairwise_sum(sel, K);
        for (int k = 0; k < K; ++k) topk_gate[(size_t)t * K + k] = sel[k] / P;
    }

    /* Routed counts per (sub-sequence, expert). */
    memset(routed_counts, 0, sizeof(int32_t) * (size_t)n_sub * E);
    for (int t = 0; t < T; ++t)
        for (int k = 0; k < K; ++k)
            routed_counts[(size_t)(t / S) * E + topk_idx[(size_t)t * K + k]] += 1;

    /* Capacity drop: in each (sub-sequence, expert), keep the `capacity` candidates
     * that come first under (p desc, t asc).  Candidate a beats b iff
     * p_a > p_b, or p_a == p_b and t_a < t_b.  A candidate is kept iff fewer than
     * `capacity` candidates of its group beat it. */
    for (size_t i = 0; i < (size_t)T * K; ++i) keep[i] = 1;
    if (capacity >= 0) {
        int32_t* cand = (int32_t*)malloc(sizeof(int32_t) * (size_t)S);
        if (!cand) return ORACLE_BAD_ARG;
        for (int s = 0; s < n_sub; ++s) {
            for (int e = 0; e < E; ++e) {
                int n = 0;
                for (int t = s * S; t < (s + 1) * S; ++t)
                    for (int k = 0; k < K; ++k)
                        if (topk_idx[(size_t)t * K + k] == e) cand[n++] = t * K + k;
                if (n <= capacity) continue;
                for (int i = 0; i < n; ++i) {
                    float pi = topk_prob[cand[i]];
                    int ti = cand[i] / K;
                    int beaten_by = 0;
                    for (int j = 0; j < n; ++j) {
                        float pj = topk_prob[cand[j]];
                        int tj = cand[j] / K;
                        if (pj > pi || (pj == pi && tj < ti)) ++beaten_by;
                    }
                    if (beaten_by >= capacity) keep[cand[i]] = 0;
                }
            }
        }
        free(cand);
    }

    /* Maps: experts in ascending order; inside an expert, tokens in ascending
     * order over the whole T (a stable counting sort of the kept assignments). */
    int r = 0;
    for (size_t i = 0; i < (size_t)T * K; ++i) row_of[i] = -1;
    for (int e = 0; e < E; ++e) {
        offsets[e] = r;
        for (int t = 0; t < T; ++t)
            for (int k = 0; k < K; ++k) {
                size_t i = (size_t)t * K + k;
                if (topk_idx[i] == e && keep[i]) {
                    row_of[i] = r;
                    src_of[r] = (int32_t)i;
                    ++r;
                }
            }
        kept_counts[e] = r - offsets[e];
    }
    offsets[E] = r;
    *n_kept = r;
    return ORACLE_OK;
}

/*
 * Exhaustive check helper for the exp pin: walks every fp32 r in [lo, -0] (lo < 0)
 * and returns the largest distance, in units in the last place of the fp32 result,
 * between oracle_exp(r) and the double-precision libm exp(r) over the r whose
 * result is not flushed; counts flushed results whose exact value is >= 2^-125 in
 * *bad_flush and nonzero results below 2^-125 (or denormal) in *bad_tiny.
 */
double oracle_exp_scan(float lo, int64_t* n_checked, int64_t* bad_flush,
                       int64_t* bad_tiny) {
    init_consts();
    double worst = 0.0;
    int64_t cnt = 0, bf = 0, bt = 0;
    const int64_t first = 0x80000000LL, last = (int64_t)to_bits(lo);
    const double tiny = ldexp(1.0, -125);
#pragma omp parallel for schedule(static, 1 << 20) reduction(max : worst) reduction(+ : cnt, bf, bt)
    for (int64_t b = first; b <= last; ++b) {
        float r = from_bits((uint32_t)b);
        float y = oracle_exp(r);
        double ex = exp((double)r);
        if (y == 0.0f) {
            if (ex >= tiny) ++bf;
        } else {
            if ((double)y < 0.70710678 * tiny) ++bt;
            int ee;
            frexp(ex, &ee);                    /* ex = m * 2^ee, m in [0.5, 1) */
            double ulp = ldexp(1.0, ee - 24);  /* spacing of fp32 numbers near ex */
            double err = fabs((double)y - ex) / ulp;
            if (err > worst) worst = err;
        }
        ++cnt;
    }
    {   /* and +0 */
        float y = oracle_exp(0.0f);
        double err = fabs((double)y - 1.0) / ldexp(1.0, -23);
        if (err > worst) worst = err;
        ++cnt;
    }
    *n_checked = cnt;
    *bad_flush = bf;
    *bad_tiny = bt;
    return worst;
}
