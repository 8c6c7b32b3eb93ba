/*
 * Reference oracle for causal attention with per-RoPE-wavelength distance
 * windows (the ATFlash idea).  TEST INFRASTRUCTURE ONLY: the test suite, the
 * smoke check and the CPU-baseline leg of the benchmark call it; the product
 * path never does.  It shares no code with the HIP library.
 *
 * Everything is plain fp64 loops, in the order the definition states, so a
 * reader can check it against the source page by eye:
 *   Source page: "ATFlash: RoPE-Frequenzen kuerzen Attention-Arbeit um bis zu
 *   57 Prozent" (sudo-ai.de), section "Was ATFlash anders macht":
 *     - RoPE encodes position with 2-D rotations at several frequencies;
 *     - every frequency pair gets its own distance window derived from its
 *       wavelength, and beyond a distance proportional to that wavelength the
 *       pair's part of the query-key product is left out;
 *     - a distant key never vanishes, because slow (low-frequency) pairs still
 *       see it.
 *   Same page, section "Die Zahlen - und ihre Grenze": the online-softmax
 *   recurrence is not changed, so the windowed score feeds a plain softmax.
 *
 * Readings taken where the page is silent (each is listed in the design notes):
 *   theta_p  = base^(-2p/d), p = 0 .. P-1, P = d/2   (p = 0 is the fastest pair)
 *   lambda_p = 2*pi / theta_p                          (wavelength)
 *   W_p      = ceil(alpha * lambda_p) for p < P-1, W_{P-1} = infinity
 *              ("proportional distance"; the slowest pair is never cut, which
 *              is what keeps every causal key reachable); alpha = +inf turns
 *              every window off.
 *   pair p   = dims (lo, hi) = (p, p + P) in the NeoX half-split layout
 *              (layout 0), or (2p, 2p + 1) in the GPT-J interleaved layout
 *              (layout 1); the frequency theta_p is the same in both
 *   rotation by +angle: x'_lo = x_lo cos a - x_hi sin a,
 *                       x'_hi = x_hi cos a + x_lo sin a, a = pos*theta_p
 *   pair p contributes q'_lo k'_lo + q'_hi k'_hi to score(i,j) iff
 *   delta = pos_q - pos_k <= W_p (|delta| when not causal); dropped terms
 *   add 0 (they are not -inf); logits = score / sqrt(d).
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -shared -fPIC (no fused
 * multiply-add, so every product and sum is rounded exactly as written).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_W_INF INT64_MAX

static const double ORC_TWO_PI = 6.283185307179586476925286766559;

/* Window table W[0..d/2-1].  Returns 0 on success, -1 on bad arguments. */
int orc_window_table(int d, double base, double alpha, int64_t *W)
{
    if (d <= 0 || (d % 2) != 0 || !(base > 1.0) || !(alpha > 0.0) || W == NULL)
        return -1;
    const int P = d / 2;
    for (int p = 0; p < P; ++p) {
        if (p == P - 1 || isinf(alpha)) {
            W[p] = ORC_W_INF;
            continue;
        }
        double theta = pow(base, -2.0 * (double)p / (double)d);
        double lambda = ORC_TWO_PI / theta;
        double w = ceil(alpha * lambda);
        W[p] = (w >= 9.0e18) ? ORC_W_INF : (int64_t)w;
    }
    return 0;
}

/* Is pair p's term kept at signed distance delta? */
static int orc_kept(int64_t delta, int causal, int64_t Wp)
{
    int64_t dist = delta;
    if (!causal && dist < 0)
        dist = -dist;
    return Wp == ORC_W_INF || dist <= Wp;
}

/* The two dims of pair p: (p, p + P) half-split, (2p, 2p + 1) interleaved. */
static int orc_dim_lo(int p, int P, int layout) { return layout ? 2 * p : p; }
static int orc_dim_hi(int p, int P, int layout) { return layout ? 2 * p + 1 : p + P; }

/* Rotate one row x[0..d) at position pos into y (fp64). */
static void orc_rotate(const float *x, int d, int layout, double pos, const double *theta, double *y)
{
    const int P = d / 2;
    for (int p = 0; p < P; ++p) {
        const int il = orc_dim_lo(p, P, layout), ih = orc_dim_hi(p, P, layout);
        double a = pos * theta[p];
        double c = cos(a);
        double s = sin(a);
        double lo = (double)x[il];
        double hi = (double)x[ih];
        y[il] = lo * c - hi * s;
        y[ih] = hi * c + lo * s;
    }
}

/*
 * Attention for a list of query rows.
 *   q   [B][Hq][Sq][d], k, v [B][Hkv][Sk][d]  (float32; bf16 inputs are exact
 *       in float32, and float32 is exact in fp64)
 *   query i sits at position q_pos0 + i, key j at k_pos0 + j,
 *   delta = (q_pos0 + i) - (k_pos0 + j).  causal: only keys with delta >= 0.
 *   rows: n_rows triples (b, h_q, i); out: [n_rows][d] fp64.
 *   q_rows (nullable): if given, row r's query vector is q_rows[r][0..d)
 *       instead of q[b][h_q][i] (lets a caller pass only sampled rows);
 *       q may then be NULL.
 *   GQA: query head h reads key/value head h / (Hq / Hkv).
 *   layout: 0 = NeoX half-split pairs, 1 = GPT-J interleaved pairs.
 *   skipped (nullable): number of (row, key, pair) terms left out, summed
 *   over the listed rows (causal keys only when causal != 0).
 * Returns 0, or -1 on bad arguments.
 */
int orc_attention_rows(const float *q, const float *k, const float *v,
                       int B, int Hq, int Hkv, int64_t Sq, int64_t Sk, int d, int layout,
                       double base, double alpha, int causal,
                       int64_t q_pos0, int64_t k_pos0,
                       const int64_t *rows, int64_t n_rows, const float *q_rows,
                       double *out, uint64_t *skipped)
{
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || (Hq % Hkv) != 0 || Sq <= 0 || Sk <= 0)
        return -1;
    if (d <= 0 || (d % 2) != 0 || rows == NULL || out == NULL || n_rows < 0)
        return -1;
    if (layout != 0 && layout != 1)
        return -1;
    if (q == NULL && q_rows == NULL)
        return -1;
    const int P = d / 2;
    const int group = Hq / Hkv;
    int64_t *W = (int64_t *)malloc(sizeof(int64_t) * (size_t)P);
    double *theta = (double *)malloc(sizeof(double) * (size_t)P);
    if (!W || !theta || orc_window_table(d, base, alpha, W) != 0) {
        free(W);
        free(theta);
        return -1;
    }
    for (int p = 0; p < P; ++p)
        theta[p] = pow(base, -2.0 * (double)p / (double)d);

    for (int64_t r = 0; r < n_rows; ++r) {
        int64_t b = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
        if (b < 0 || b >= B || h < 0 || h >= Hq || i < 0 || i >= Sq) {
            free(W);
            free(theta);
            return -1;
        }
    }

    /* Rotated keys of one (b, h_kv) at a time, reused by every listed row of
     * that head (the same values the definition asks for, computed once). */
    double *krot = (double *)malloc(sizeof(double) * (size_t)Sk * (size_t)d);
    if (!krot) {
        free(W);
        free(theta);
        return -1;
    }
    uint64_t total_skipped = 0;

    for (int b = 0; b < B; ++b) {
        for (int hk = 0; hk < Hkv; ++hk) {
            int64_t n_here = 0;
            for (int64_t r = 0; r < n_rows; ++r)
                if (rows[3 * r] == b && rows[3 * r + 1] / group == hk)
                    ++n_here;
            if (n_here == 0)
                continue;
            const float *kh = k + ((size_t)b * Hkv + hk) * (size_t)Sk * d;
            const float *vh = v + ((size_t)b * Hkv + hk) * (size_t)Sk * d;

#pragma omp parallel for schedule(static)
            for (int64_t j = 0; j < Sk; ++j)
                orc_rotate(kh + (size_t)j * d, d, layout, (double)(k_pos0 + j), theta,
                           krot + (size_t)j * d);

            uint64_t skipped_here = 0;
#pragma omp parallel reduction(+ : skipped_here)
            {
                double *qrot = (double *)malloc(sizeof(double) * (size_t)d);
                double *logit = (double *)malloc(sizeof(double) * (size_t)Sk);
                double *acc = (double *)malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(dynamic, 1)
                for (int64_t r = 0; r < n_rows; ++r) {
                    if (rows[3 * r] != b || rows[3 * r + 1] / group != hk)
                        continue;
                    int64_t h = rows[3 * r + 1], i = rows[3 * r + 2];
                    const float *qrow = q_rows ? q_rows + (size_t)r * d
                                               : q + (((size_t)b * Hq + h) * (size_t)Sq + i) * d;
                    int64_t qpos = q_pos0 + i;
                    orc_rotate(qrow, d, layout, (double)qpos, theta, qrot);

                    /* pass 1: windowed scores and their maximum */
                    double m = -INFINITY;
                    for (int64_t j = 0; j < Sk; ++j) {
                        int64_t delta = qpos - (k_pos0 + j);
                        if (causal && delta < 0) {
                            logit[j] = -INFINITY;
                            continue;
                        }
                        const double *kr = krot + (size_t)j * d;
                        double s = 0.0;
                        for (int p = 0; p < P; ++p) {
                            if (orc_kept(delta, causal, W[p])) {
                                const int il = orc_dim_lo(p, P, layout), ih = orc_dim_hi(p, P, layout);
                                double term = qrot[il] * kr[il] + qrot[ih] * kr[ih];
                                s += term;
                            } else {
                                skipped_here += 1;
                            }
                        }
                        logit[j] = s / sqrt((double)d);
                        if (logit[j] > m)
                            m = logit[j];
                    }
                    /* pass 2: softmax weights and the weighted sum of values */
                    double den = 0.0;
                    for (int c = 0; c < d; ++c)
                        acc[c] = 0.0;
                    for (int64_t j = 0; j < Sk; ++j) {
                        if (logit[j] == -INFINITY)
                            continue;
                        double w = exp(logit[j] - m);
                        den += w;
                        const float *vr = vh + (size_t)j * d;
                        for (int c = 0; c < d; ++c)
                            acc[c] += w * (double)vr[c];
                    }
                    double *o = out + (size_t)r * d;
                    for (int c = 0; c < d; ++c)
                        o[c] = (den > 0.0) ? acc[c] / den : 0.0;
                }
                free(qrot);
                free(logit);
                free(acc);
            }
            total_skipped += skipped_here;
        }
    }
    free(krot);
    free(W);
    free(theta);
    if (skipped)
        *skipped = total_skipped;
    return 0;
}

/*
 * Closed form of the skipped count for ONE (b, h_q), from the window table:
 *   mode 0, causal prefill of S tokens: pair p loses the (i, j) with
 *     i - j in [W_p + 1, S - 1]; distance t occurs S - t times, so the count
 *     is n_p (n_p + 1) / 2 with n_p = max(0, S - 1 - W_p).
 *   mode 1, decode (one query at position S after S cached keys): distances
 *     are 1 .. S, so pair p loses max(0, S - W_p) keys.
 * Returns 0, or -1 on bad arguments.
 */
int orc_skipped_closed_form(int64_t S, int d, double base, double alpha, int mode,
                            uint64_t *per_head)
{
    if (S <= 0 || per_head == NULL || (mode != 0 && mode != 1))
        return -1;
    const int P = d / 2;
    int64_t *W = (int64_t *)malloc(sizeof(int64_t) * (size_t)(P > 0 ? P : 1));
    if (!W || orc_window_table(d, base, alpha, W) != 0) {
        free(W);
        return -1;
    }
    uint64_t total = 0;
    for (int p = 0; p < P; ++p) {
        if (W[p] == ORC_W_INF)
            continue;
        if (mode == 0) {
            int64_t n = S - 1 - W[p];
            if (n > 0)
                total += (uint64_t)n * (uint64_t)(n + 1) / 2u;
        } else {
            int64_t n = S - W[p];
            if (n > 0)
                total += (uint64_t)n;
        }
    }
    free(W);
    *per_head = total;
    return 0;
}

/* Threads the OpenMP runtime will use (1 without OpenMP). */
int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
