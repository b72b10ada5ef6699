/*
 * SATA oracle: TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, double-precision CPU implementation of what symmetry-aware
 * Taylor approximation (SATA) attention computes.  Only the tests, the smoke
 * check and the CPU-baseline leg of the benchmark load this library; the
 * product path (the HIP library under constant_cost_attention_amd/) never
 * does, and the two share no code, headers or tables.
 *
 * Sources (cited by page and section):
 *   [hotdry] blog.hotdry.top, "Symmetry-aware Taylor approximation attention:
 *            engineering a constant per-token cost" (2026-02-05).
 *            Sections: "Scale bottleneck of conventional self-attention",
 *            "Core insight of symmetric tensor decomposition",
 *            "Engineering realisation of the constant compute cost".
 *   [mokono] www.mokono.cn survey of attention variants, section on standard
 *            scaled dot-product attention: layout (batch, heads, seq, dim).
 *
 * What the method computes (plain reading, see the function comments):
 *   x_ij = q_i . k_j / sqrt(d_K)
 *   w(x) = sum_{p<P} x^p / p!          (exp kernel truncated after P orders)
 *   o_i  = sum_{j<=i} w(x_ij) v_j / sum_{j<=i} w(x_ij)
 *
 * Inputs are float32 arrays holding exactly the values the GPU consumes
 * (bf16 inputs are widened to fp32 exactly before they get here); every
 * operation below is carried out in double (or, for the diagnostic
 * orc_recurrent_attention_f32, deliberately in float).
 *
 * Build: gcc -O2 -ffp-contract=off -fPIC -shared -pthread (no fast-math).
 */
#define _GNU_SOURCE
#include <math.h>
#include <pthread.h>
#include <sched.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

/* ------------------------------------------------------------------ */
/* threads                                                             */
/* ------------------------------------------------------------------ */

int orc_num_cpus(void) {
    cpu_set_t set;
    CPU_ZERO(&set);
    if (sched_getaffinity(0, sizeof(set), &set) == 0) {
        int c = CPU_COUNT(&set);
        if (c > 0) return c;
    }
    long n = sysconf(_SC_NPROCESSORS_ONLN);
    return n > 0 ? (int)n : 1;
}

typedef struct {
    const float *q, *k, *v;
    double *out;
    int64_t bh, n;
    int dk, dv, P;
    const int64_t *rows;
    int64_t nrows;
    int64_t next;   /* shared work counter */
    int softmax;    /* 0: Taylor weight, 1: exact softmax */
} row_job;

/* One output row of causal attention, by the definition.
 *
 * Taylor weight [hotdry, "Core insight of symmetric tensor decomposition"]:
 * the softmax kernel exp(x) is replaced by its Taylor series kept up to the
 * order P-1 (P orders including the constant one), and the result is
 * normalised by the sum of the weights, which is what the extra "+1" column
 * of the state carries [hotdry, "Engineering realisation of the constant
 * compute cost"].  The scale 1/sqrt(d_K) on q.k is the usual one of scaled
 * dot-product attention [mokono, standard attention].
 *
 * Causality includes the diagonal: row i sees keys 0..i.
 * Softmax variant: max-subtracted exp, same normalisation. */
static void one_row(const row_job *J, int64_t h, int64_t i, double *dst, double *num) {
    const int dk = J->dk, dv = J->dv;
    const float *qi = J->q + (h * J->n + i) * dk;
    const float *kh = J->k + h * J->n * dk;
    const float *vh = J->v + h * J->n * dv;
    const double scale = 1.0 / sqrt((double)dk);

    /* 1/p! for p = 0..P-1 */
    double inv_fact[64];
    if (!J->softmax) {
        inv_fact[0] = 1.0;
        for (int p = 1; p < J->P; ++p) inv_fact[p] = inv_fact[p - 1] / (double)p;
    }
    double mx = 0.0;
    if (J->softmax) {
        mx = -INFINITY;
        for (int64_t j = 0; j <= i; ++j) {
            double s = 0.0;
            for (int c = 0; c < dk; ++c) s += (double)qi[c] * (double)kh[j * dk + c];
            s *= scale;
            if (s > mx) mx = s;
        }
    }
    for (int c = 0; c < dv; ++c) num[c] = 0.0;
    double den = 0.0;
    for (int64_t j = 0; j <= i; ++j) {
        double s = 0.0;
        for (int c = 0; c < dk; ++c) s += (double)qi[c] * (double)kh[j * dk + c];
        const double x = s * scale;
        double w;
        if (J->softmax) {
            w = exp(x - mx);
        } else {
            /* Horner: sum_{p<P} x^p/p! */
            w = inv_fact[J->P - 1];
            for (int p = J->P - 2; p >= 0; --p) w = w * x + inv_fact[p];
        }
        const float *vj = vh + j * dv;
        for (int c = 0; c < dv; ++c) num[c] += w * (double)vj[c];
        den += w;
    }
    for (int c = 0; c < dv; ++c) dst[c] = num[c] / den;
}

static void *row_worker(void *arg) {
    row_job *J = (row_job *)arg;
    double *num = (double *)malloc(sizeof(double) * (size_t)(J->dv > 0 ? J->dv : 1));
    const int64_t total = J->bh * J->nrows;
    for (;;) {
        /* rows are handed out interleaved: item t -> row t / bh, head t % bh,
         * so that cheap early rows and costly late rows mix across threads */
        int64_t t = __atomic_fetch_add(&J->next, 1, __ATOMIC_RELAXED);
        if (t >= total) break;
        int64_t r = t / J->bh, h = t % J->bh;
        int64_t i = J->rows ? J->rows[r] : r;
        one_row(J, h, i, J->out + (h * J->nrows + r) * J->dv, num);
    }
    free(num);
    return NULL;
}

static int run_rows(row_job *J, int nthreads) {
    if (J->bh < 0 || J->n < 0 || J->dk <= 0 || J->dv <= 0) return 1;
    if (!J->softmax && (J->P < 1 || J->P > 60)) return 1;
    if (J->rows) {
        for (int64_t r = 0; r < J->nrows; ++r)
            if (J->rows[r] < 0 || J->rows[r] >= J->n) return 2;
    } else {
        J->nrows = J->n;
    }
    if (nthreads <= 0) nthreads = orc_num_cpus();
    if (nthreads > 512) nthreads = 512;
    J->next = 0;
    pthread_t th[512];
    int started = 0;
    for (int t = 1; t < nthreads; ++t) {
        if (pthread_create(&th[started], NULL, row_worker, J) == 0) ++started;
    }
    row_worker(J);
    for (int t = 0; t < started; ++t) pthread_join(th[t], NULL);
    return 0;
}

/* O1: quadratic causal Taylor-weighted attention (the oracle proper).
 * q,k: [bh][n][dk]; v: [bh][n][dv]; out: [bh][nrows][dv] (double).
 * rows: NULL for every row, else nrows row indices applied to every head.
 * Returns 0 on success, nonzero on bad arguments. */
int orc_taylor_attention(const float *q, const float *k, const float *v, double *out,
                         int64_t bh, int64_t n, int dk, int dv, int P,
                         const int64_t *rows, int64_t nrows, int nthreads) {
    row_job J = {q, k, v, out, bh, n, dk, dv, P, rows, nrows, 0, 0};
    return run_rows(&J, nthreads);
}

/* O2: exact causal softmax attention, same layout; used only to report the
 * gap between SATA and the attention it truncates [hotdry, "Scale bottleneck
 * of conventional self-attention"]. */
int orc_softmax_attention(const float *q, const float *k, const float *v, double *out,
                          int64_t bh, int64_t n, int dk, int dv,
                          const int64_t *rows, int64_t nrows, int nthreads) {
    row_job J = {q, k, v, out, bh, n, dk, dv, 1, rows, nrows, 0, 1};
    return run_rows(&J, nthreads);
}

/* ------------------------------------------------------------------ */
/* O3: brute-force symmetric basis                                     */
/* ------------------------------------------------------------------ */

/* Every one of the d^p ordered index tuples of (q^T k)^p is visited; each is
 * sorted and the sorted tuples are counted.  The distinct sorted tuples are
 * the minimal basis of the symmetric tensor of order p [hotdry, "Core insight
 * of symmetric tensor decomposition"]; the count of a group is how many
 * ordered monomials collapse onto it.  Groups are returned in lexicographic
 * order of the sorted tuple (first index most significant).
 *
 * tuples_out: [cap][p] int32 (may be NULL), counts_out: [cap] (may be NULL).
 * Returns the number of groups, or -1 when d^p exceeds the brute-force limit
 * or the arguments are bad. */
int64_t orc_basis_bruteforce(int d, int p, int32_t *tuples_out, int64_t *counts_out, int64_t cap) {
    if (d <= 0 || p < 0 || p > 8) return -1;
    int64_t total = 1;
    for (int r = 0; r < p; ++r) {
        total *= d;
        if (total > ((int64_t)1 << 27)) return -1;
    }
    int32_t *hits = (int32_t *)calloc((size_t)total, sizeof(int32_t));
    if (!hits) return -1;
    int idx[8] = {0}, srt[8];
    for (int64_t o = 0; o < total; ++o) {
        /* decode ordered tuple o (base d, first index most significant) */
        int64_t rem = o;
        for (int r = p - 1; r >= 0; --r) { idx[r] = (int)(rem % d); rem /= d; }
        for (int r = 0; r < p; ++r) srt[r] = idx[r];
        for (int a = 1; a < p; ++a) {           /* insertion sort */
            int key = srt[a], b = a - 1;
            while (b >= 0 && srt[b] > key) { srt[b + 1] = srt[b]; --b; }
            srt[b + 1] = key;
        }
        int64_t key = 0;
        for (int r = 0; r < p; ++r) key = key * d + srt[r];
        hits[key] += 1;
    }
    int64_t ng = 0;
    for (int64_t key = 0; key < total; ++key) {
        if (!hits[key]) continue;
        if (ng < cap) {
            if (tuples_out) {
                int64_t rem = key;
                for (int r = p - 1; r >= 0; --r) { tuples_out[ng * p + r] = (int32_t)(rem % d); rem /= d; }
            }
            if (counts_out) counts_out[ng] = hits[key];
        }
        ++ng;
    }
    free(hits);
    return ng;
}

/* O4: symmetric feature map of one vector x for one order p, from the
 * brute-force groups: phi_p(x)_t = sqrt(count_t) * prod_r x[t_r], so that
 * phi_p(q) . phi_p(k) = (q . k)^p [hotdry, "Core insight of symmetric tensor
 * decomposition"].  out: [ng] double.  Returns ng or -1. */
int64_t orc_phi(const double *x, int d, int p, double *out, int64_t cap) {
    int64_t ng = orc_basis_bruteforce(d, p, NULL, NULL, 0);
    if (ng < 0 || ng > cap) return -1;
    int32_t *tup = (int32_t *)malloc(sizeof(int32_t) * (size_t)(ng * (p > 0 ? p : 1)));
    int64_t *cnt = (int64_t *)malloc(sizeof(int64_t) * (size_t)ng);
    orc_basis_bruteforce(d, p, tup, cnt, ng);
    for (int64_t t = 0; t < ng; ++t) {
        double prod = 1.0;
        for (int r = 0; r < p; ++r) prod *= x[tup[t * p + r]];
        out[t] = sqrt((double)cnt[t]) * prod;
    }
    free(tup);
    free(cnt);
    return ng;
}

/* ------------------------------------------------------------------ */
/* O5 / O7: the recurrent constant-size state form                      */
/* ------------------------------------------------------------------ */

/* Recurrent form [hotdry, "Engineering realisation of the constant compute
 * cost"]: for every order p a state S_p = sum_s phi_p(k_s) (x) [v_s, 1] of
 * size C(d+p-1,p) x (d_V+1) is accumulated token by token (the orders are
 * independent scans); each token is first added, then read out as
 * y = sum_p phi_p(q) . S_p / (p! d^(p/2)) and normalised by the last column.
 * The feature map is the brute-force one above.  Tiny inputs only.
 *
 * REAL selects double (O5, exact form) or float (O7, a diagnostic emulation
 * of fp32 state accumulation). */
#define DEFINE_RECURRENT(NAME, REAL)                                                     \
int NAME(const float *q, const float *k, const float *v, double *out,                    \
         int64_t bh, int64_t n, int dk, int dv, int P) {                                \
    if (bh < 0 || n < 0 || dk <= 0 || dv <= 0 || P < 1 || P > 8) return 1;               \
    int64_t ng[8], off[8], m = 0;                                                        \
    for (int p = 0; p < P; ++p) {                                                        \
        ng[p] = orc_basis_bruteforce(dk, p, NULL, NULL, 0);                              \
        if (ng[p] < 0) return 1;                                                         \
        off[p] = m; m += ng[p];                                                          \
    }                                                                                    \
    int32_t *tup[8]; int64_t *cnt[8];                                                    \
    for (int p = 0; p < P; ++p) {                                                        \
        tup[p] = (int32_t *)malloc(sizeof(int32_t) * (size_t)(ng[p] * (p ? p : 1)));     \
        cnt[p] = (int64_t *)malloc(sizeof(int64_t) * (size_t)ng[p]);                     \
        orc_basis_bruteforce(dk, p, tup[p], cnt[p], ng[p]);                              \
    }                                                                                    \
    REAL *S = (REAL *)malloc(sizeof(REAL) * (size_t)(m * (dv + 1)));                     \
    REAL *fk = (REAL *)malloc(sizeof(REAL) * (size_t)m);                                 \
    REAL *fq = (REAL *)malloc(sizeof(REAL) * (size_t)m);                                 \
    REAL *y = (REAL *)malloc(sizeof(REAL) * (size_t)(dv + 1));                           \
    double readw[8];                                                                     \
    { double fact = 1.0;                                                                 \
      for (int p = 0; p < P; ++p) {                                                      \
        if (p) fact *= p;                                                                \
        readw[p] = 1.0 / (fact * pow(sqrt((double)dk), (double)p));                      \
      } }                                                                                \
    for (int64_t h = 0; h < bh; ++h) {                                                   \
        memset(S, 0, sizeof(REAL) * (size_t)(m * (dv + 1)));                             \
        for (int64_t s = 0; s < n; ++s) {                                                \
            const float *qs = q + (h * n + s) * dk, *ks = k + (h * n + s) * dk;          \
            const float *vs = v + (h * n + s) * dv;                                      \
            for (int p = 0; p < P; ++p)                                                  \
                for (int64_t t = 0; t < ng[p]; ++t) {                                    \
                    REAL a = (REAL)sqrt((double)cnt[p][t]), b = a;                       \
                    for (int r = 0; r < p; ++r) {                                        \
                        a *= (REAL)ks[tup[p][t * p + r]];                                \
                        b *= (REAL)qs[tup[p][t * p + r]];                                \
                    }                                                                    \
                    fk[off[p] + t] = a; fq[off[p] + t] = b;                              \
                }                                                                        \
            for (int64_t f = 0; f < m; ++f) {                                            \
                for (int c = 0; c < dv; ++c) S[f * (dv + 1) + c] += fk[f] * (REAL)vs[c]; \
                S[f * (dv + 1) + dv] += fk[f];                                           \
            }                                                                            \
            for (int c = 0; c <= dv; ++c) y[c] = 0;                                      \
            for (int p = 0; p < P; ++p) {                                                \
                for (int c = 0; c <= dv; ++c) {                                          \
                    REAL acc = 0;                                                        \
                    for (int64_t t = 0; t < ng[p]; ++t)                                  \
                        acc += fq[off[p] + t] * S[(off[p] + t) * (dv + 1) + c];          \
                    y[c] += acc * (REAL)readw[p];                                        \
                }                                                                        \
            }                                                                            \
            for (int c = 0; c < dv; ++c)                                                 \
                out[(h * n + s) * dv + c] = (double)y[c] / (double)y[dv];                \
        }                                                                                \
    }                                                                                    \
    for (int p = 0; p < P; ++p) { free(tup[p]); free(cnt[p]); }                          \
    free(S); free(fk); free(fq); free(y);                                                \
    return 0;                                                                            \
}

DEFINE_RECURRENT(orc_recurrent_attention, double)
DEFINE_RECURRENT(orc_recurrent_attention_f32, float)

/* ------------------------------------------------------------------ */
/* O8: decode on a state stored in bf16                                */
/* ------------------------------------------------------------------ */

/* Rounds x to the nearest bfloat16 value, ties to even: 8 significant bits
 * (7 stored plus the implicit one) and the exponent range of binary32, with
 * gradual underflow below 2^-126.  Inputs here are finite and far below
 * bf16's largest value; a result beyond it becomes +-inf.  nearbyint() in the
 * default rounding mode rounds half-way cases to even. */
double orc_round_bf16(double x) {
    if (x == 0.0 || !isfinite(x)) return x;
    int e;
    (void)frexp(x, &e);              /* x = f * 2^e, 0.5 <= |f| < 1 */
    if (e < -125) e = -125;          /* subnormal range: fixed quantum 2^-133 */
    const double r = ldexp(nearbyint(ldexp(x, 8 - e)), e - 8);
    return fabs(r) > 0x1.fep127 ? copysign(INFINITY, r) : r;
}

void orc_round_bf16_array(const double *x, double *out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_round_bf16(x[i]);
}

/* Rounds x to the nearest IEEE binary16 value, ties to even: 11 significant
 * bits (10 stored plus the implicit one), normal numbers from 2^-14 up to
 * 65504, gradual underflow below 2^-14 (fixed quantum 2^-24), and anything
 * that rounds past 65504 becomes +-inf. */
double orc_round_f16(double x) {
    if (x == 0.0 || !isfinite(x)) return x;
    int e;
    (void)frexp(x, &e);              /* x = f * 2^e, 0.5 <= |f| < 1 */
    if (e < -13) e = -13;            /* subnormal range: fixed quantum 2^-24 */
    const double r = ldexp(nearbyint(ldexp(x, 11 - e)), e - 11);
    return fabs(r) > 65504.0 ? copysign(INFINITY, r) : r;
}

void orc_round_f16_array(const double *x, double *out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_round_f16(x[i]);
}

/* The value a 16-bit state stores for feature f: round_mode 0 keeps it exact,
 * 1 rounds to bf16, 2 rounds to binary32 for the first m_low features (the
 * lowest orders) and to binary16 for the rest. */
static double store_round(int round_mode, int64_t f, int64_t m_low, double x) {
    if (round_mode == 0) return x;
    if (round_mode == 1) return orc_round_bf16(x);
    return f < m_low ? (double)(float)x : orc_round_f16(x);
}

/* Decode steps on a state whose stored elements are 16-bit (bfloat16, or
 * binary16 with the lowest orders in binary32: see store_round).
 *
 * The state is the one of the recurrent form [hotdry, "Engineering
 * realisation of the constant compute cost"] kept in the layout the library
 * documents: for every sorted index tuple t of order p < P (the minimal basis
 * [hotdry, "Core insight of symmetric tensor decomposition"]) the key side
 * carries the plain monomial prod_r k[t_r], so element (t, c) holds
 * sum_s prod_r k_s[t_r] * [v_s, 1][c]; the query side carries
 * prod_r q[t_r] * (p!/alpha_t!) / (p! d^(p/2)), where p!/alpha_t! is the
 * number of ordered tuples sorting to t.
 *
 * Storing the elements in a 16-bit format is the page's suggestion for
 * halving the state's bandwidth [hotdry, "Hardware optimisation paths and
 * current limits"]; the reading taken here: the tokens 0..n0-1 are summed
 * exactly and rounded once (a prefill in full precision, then converted);
 * every later token s is added to the stored values exactly, read out from
 * those unrounded sums, and the sums are rounded to bf16 when stored back.
 * Rows n0..n-1 are written to out: [bh][n - n0][dv].
 *
 * window W >= 1 defers the stores: W - 1 steps in a row read out the stored
 * values plus, exactly, the terms of the tokens not yet stored and of the
 * step's own token; every W-th step adds all of them to the stored values,
 * reads out from those sums and stores them rounded.  W = 1 stores every
 * step.
 *
 * round_mode 0 skips every rounding: the exact one-sided recurrent form.
 * Tiny to moderate inputs; returns nonzero on bad arguments. */
/* The summed prefix of one head, features [f_lo, f_hi) per thread. */
typedef struct {
    const float *k, *v;
    const int32_t *tup;
    const int *ord;
    double *S;
    int64_t n0, f_lo, f_hi, m_low;
    int dk, dv, W, round_mode;
} prefix_job;

static void *prefix_worker(void *arg) {
    const prefix_job *J = (const prefix_job *)arg;
    const int dv = J->dv;
    double *a = (double *)malloc(sizeof(double) * (size_t)(J->n0 > 0 ? J->n0 : 1));
    if (!a) return (void *)1;
    for (int64_t f = J->f_lo; f < J->f_hi; ++f) {
        for (int64_t s = 0; s < J->n0; ++s) {
            double mono = 1.0;
            for (int r = 0; r < J->ord[f]; ++r) mono *= (double)J->k[s * J->dk + J->tup[f * J->W + r]];
            a[s] = mono;
        }
        for (int c = 0; c <= dv; ++c) {
            double acc = 0.0;
            for (int64_t s = 0; s < J->n0; ++s) acc += a[s] * (c < dv ? (double)J->v[s * dv + c] : 1.0);
            J->S[f * (dv + 1) + c] = store_round(J->round_mode, f, J->m_low, acc);
        }
    }
    free(a);
    return NULL;
}

static int state16_decode(const float *q, const float *k, const float *v, double *out, int64_t bh, int64_t n0,
                          int64_t n, int dk, int dv, int P, int round_mode, int64_t m_low, int window) {
    if (bh < 0 || n0 < 0 || n < n0 || dk <= 0 || dv <= 0 || P < 1 || P > 8 || window < 1 || m_low < 0)
        return 1;
    int64_t ng[8], off[8], m = 0;
    for (int p = 0; p < P; ++p) {
        ng[p] = orc_basis_bruteforce(dk, p, NULL, NULL, 0);
        if (ng[p] < 0) return 1;
        off[p] = m;
        m += ng[p];
    }
    int32_t *tup = (int32_t *)malloc(sizeof(int32_t) * (size_t)(m * (P > 1 ? P - 1 : 1)));
    double *qw = (double *)malloc(sizeof(double) * (size_t)m);     /* query-side weight per feature */
    int *ord = (int *)malloc(sizeof(int) * (size_t)m);
    double *S = (double *)malloc(sizeof(double) * (size_t)(m * (dv + 1)));
    double *y = (double *)malloc(sizeof(double) * (size_t)(dv + 1));
    if (!tup || !qw || !ord || !S || !y) {
        free(tup); free(qw); free(ord); free(S); free(y);
        return 1;
    }
    const int W = P > 1 ? P - 1 : 1;   /* tuple slots per feature */
    {
        double fact = 1.0;
        for (int p = 0; p < P; ++p) {
            if (p) fact *= p;
            int32_t *tp = (int32_t *)malloc(sizeof(int32_t) * (size_t)(ng[p] * (p ? p : 1)));
            int64_t *cp = (int64_t *)malloc(sizeof(int64_t) * (size_t)ng[p]);
            orc_basis_bruteforce(dk, p, tp, cp, ng[p]);
            for (int64_t t = 0; t < ng[p]; ++t) {
                const int64_t f = off[p] + t;
                ord[f] = p;
                for (int r = 0; r < p; ++r) tup[f * W + r] = tp[t * p + r];
                qw[f] = (double)cp[t] / (fact * pow(sqrt((double)dk), (double)p));
            }
            free(tp);
            free(cp);
        }
    }
    for (int64_t h = 0; h < bh; ++h) {
        const float *qh = q + h * n * dk, *kh = k + h * n * dk, *vh = v + h * n * dv;
        /* tokens 0..n0-1: exact sums, then one rounding (features split over threads) */
        {
            int nt = orc_num_cpus();
            if (nt > 64) nt = 64;
            if ((int64_t)nt > m) nt = (int)m;
            prefix_job jobs[64];
            pthread_t th[64];
            int started[64] = {0};
            for (int t = 0; t < nt; ++t) {
                jobs[t] = (prefix_job){kh, vh, tup, ord, S, n0, m * t / nt, m * (t + 1) / nt, m_low, dk, dv, W,
                                       round_mode};
                started[t] = t > 0 && pthread_create(&th[t], NULL, prefix_worker, &jobs[t]) == 0;
                if (t > 0 && !started[t]) prefix_worker(&jobs[t]);
            }
            prefix_worker(&jobs[0]);
            for (int t = 1; t < nt; ++t)
                if (started[t]) pthread_join(th[t], NULL);
        }
        /* decode steps; tokens first..s are not yet in the stored values */
        int64_t first = n0;
        for (int64_t s = n0; s < n; ++s) {
            const int store = (s - first + 1) >= window;
            for (int c = 0; c <= dv; ++c) y[c] = 0.0;
            for (int64_t f = 0; f < m; ++f) {
                double mq = qw[f];
                for (int r = 0; r < ord[f]; ++r) mq *= (double)qh[s * dk + tup[f * W + r]];
                for (int c = 0; c <= dv; ++c) {
                    double x = S[f * (dv + 1) + c];
                    for (int64_t t = first; t <= s; ++t) {
                        double mk = 1.0;
                        for (int r = 0; r < ord[f]; ++r) mk *= (double)kh[t * dk + tup[f * W + r]];
                        x += mk * (c < dv ? (double)vh[t * dv + c] : 1.0);
                    }
                    y[c] += mq * x;
                    if (store) S[f * (dv + 1) + c] = store_round(round_mode, f, m_low, x);
                }
            }
            if (store) first = s + 1;
            for (int c = 0; c < dv; ++c) out[(h * (n - n0) + (s - n0)) * dv + c] = y[c] / y[dv];
        }
    }
    free(tup); free(qw); free(ord); free(S); free(y);
    return 0;
}

int orc_bf16_state_decode(const float *q, const float *k, const float *v, double *out,
                          int64_t bh, int64_t n0, int64_t n, int dk, int dv, int P, int round_mode, int window) {
    return state16_decode(q, k, v, out, bh, n0, n, dk, dv, P, round_mode ? 1 : 0, 0, window);
}

/* O8 with the fp16 state: the first low_features features (numbered order by
 * order, so the lowest orders) stored in binary32, the rest in binary16 (the
 * same reading of the 16-bit storage otherwise: exact prefix rounded once,
 * exact adds, rounding on every store). */
int orc_f16_state_decode(const float *q, const float *k, const float *v, double *out, int64_t bh, int64_t n0,
                         int64_t n, int dk, int dv, int P, int64_t low_features, int window) {
    return state16_decode(q, k, v, out, bh, n0, n, dk, dv, P, 2, low_features, window);
}
