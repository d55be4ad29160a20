/*
 * oracle_sanitize_main.c -- drives every function of oracle/attn_oracle.c on
 * small seeded inputs, for a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_oracle_sanitize.py compiles and runs
 * it on the CPU).  The sanitizers catch out-of-bounds accesses, leaks and
 * undefined behaviour; the cross-checks below make sure the calls did real
 * work: the tiled online-softmax forward and the key-outer backward against
 * the plain definitions, and the selected-row functions against the whole
 * problem.  Exit status 0 when every check holds.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

void orc_attn_fwd(const double*, const double*, const double*, long, long, long, double, int,
                  double*, double*);
void orc_attn_bwd(const double*, const double*, const double*, const double*, long, long, long,
                  double, int, double*, double*, double*, double*);
void orc_row_stats(const double*, const double*, const double*, const double*, long, long,
                   double, int, double*, double*);
void orc_fwd_rows(const double*, const double*, const double*, long, long, double, int,
                  const long*, long, double*, double*);
void orc_dq_rows(const double*, const double*, const double*, const double*, long, long, double,
                 int, const long*, long, double*);
void orc_dkdv_rows(const double*, const double*, const double*, const double*, const double*,
                   const double*, long, long, double, int, const long*, long, double*, double*);
void orc_flash_fwd_tiled(const double*, const double*, const double*, long, long, long, double,
                         int, long, long, int, double*, double*);
void orc_flash_bwd_tiled(const double*, const double*, const double*, const double*,
                         const double*, const double*, long, long, long, double, int, long, long,
                         double*, double*, double*);
int orc_max_threads(void);
void orc_set_threads(int);

static uint64_t rng_state;

/* splitmix64 step mapped to a value in [-2, 2) */
static double draw(void) {
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    return 4.0 * ((double)(z >> 11) / 9007199254740992.0) - 2.0;
}

static double* alloc_fill(long n) {
    double* p = (double*)malloc(sizeof(double) * (size_t)n);
    for (long i = 0; i < n; ++i) p[i] = draw();
    return p;
}

static double max_diff(const double* a, const double* b, long n) {
    double m = 0.0;
    for (long i = 0; i < n; ++i) {
        const double e = fabs(a[i] - b[i]);
        if (!(e <= m)) m = e; /* also propagates NaN */
    }
    return m;
}

static int failures = 0;

static void check(const char* what, double err, double bound) {
    if (!(err <= bound)) {
        fprintf(stderr, "FAIL %s: %.3e > %.1e\n", what, err, bound);
        ++failures;
    }
}

/* one problem shape through every function, both causal modes */
static void run_case(long BH, long N, long d, long Br, long Bc) {
    const long n4 = BH * N * d, n3 = BH * N;
    const double scale = 1.0 / sqrt((double)d);
    double *Q = alloc_fill(n4), *K = alloc_fill(n4), *V = alloc_fill(n4), *G = alloc_fill(n4);
    double *O = malloc(sizeof(double) * n4), *L = malloc(sizeof(double) * n3);
    double *Ot = malloc(sizeof(double) * n4), *Lt = malloc(sizeof(double) * n3);
    double *dQ = malloc(sizeof(double) * n4), *dK = malloc(sizeof(double) * n4);
    double *dV = malloc(sizeof(double) * n4), *Dd = malloc(sizeof(double) * n3);
    double *tQ = malloc(sizeof(double) * n4), *tK = malloc(sizeof(double) * n4);
    double *tV = malloc(sizeof(double) * n4);
    double *Lr = malloc(sizeof(double) * N), *Dr = malloc(sizeof(double) * N);
    long rows[4] = {0, N / 3, N / 2, N - 1};
    const long nr = N >= 4 ? 4 : 1;
    double *ro = malloc(sizeof(double) * nr * d), *rl = malloc(sizeof(double) * nr);
    double *rq = malloc(sizeof(double) * nr * d), *rk = malloc(sizeof(double) * nr * d);
    double *rv = malloc(sizeof(double) * nr * d);
    char what[128];
    for (int causal = 0; causal < 2; ++causal) {
        orc_attn_fwd(Q, K, V, BH, N, d, scale, causal, O, L);
        orc_attn_bwd(Q, K, V, G, BH, N, d, scale, causal, dQ, dK, dV, Dd);
        orc_attn_bwd(Q, K, V, G, BH, N, d, scale, causal, tQ, tK, tV, NULL);
        /* threads take rows dynamically, so partial sums may be added in
         * another order: equal up to rounding */
        snprintf(what, sizeof what, "bwd with and without D, N=%ld causal=%d", N, causal);
        check(what, max_diff(dQ, tQ, n4) + max_diff(dK, tK, n4) + max_diff(dV, tV, n4), 1e-13);

        orc_flash_fwd_tiled(Q, K, V, BH, N, d, scale, causal, Br, Bc, 0, Ot, Lt);
        snprintf(what, sizeof what, "tiled forward, N=%ld causal=%d", N, causal);
        check(what, max_diff(O, Ot, n4) + max_diff(L, Lt, n3), 1e-12);
        /* the negative-control flag must run cleanly (its values may differ) */
        orc_flash_fwd_tiled(Q, K, V, BH, N, d, scale, causal, Br, Bc, 1, Ot, Lt);

        orc_flash_bwd_tiled(Q, K, V, O, G, L, BH, N, d, scale, causal, Br, Bc, tQ, tK, tV);
        snprintf(what, sizeof what, "tiled backward, N=%ld causal=%d", N, causal);
        check(what, max_diff(dQ, tQ, n4) + max_diff(dK, tK, n4) + max_diff(dV, tV, n4), 1e-11);

        /* selected rows of the last head against the whole problem */
        const long h = BH - 1;
        const double *q = Q + h * N * d, *k = K + h * N * d, *v = V + h * N * d,
                     *g = G + h * N * d;
        orc_row_stats(q, k, v, g, N, d, scale, causal, Lr, Dr);
        snprintf(what, sizeof what, "row stats, N=%ld causal=%d", N, causal);
        check(what, max_diff(Lr, L + h * N, N) + max_diff(Dr, Dd + h * N, N), 1e-12);
        orc_fwd_rows(q, k, v, N, d, scale, causal, rows, nr, ro, rl);
        orc_dq_rows(q, k, v, g, N, d, scale, causal, rows, nr, rq);
        orc_dkdv_rows(q, k, v, g, Lr, Dr, N, d, scale, causal, rows, nr, rk, rv);
        double e = 0.0;
        for (long r = 0; r < nr; ++r) {
            const long i = rows[r];
            e += max_diff(ro + r * d, O + (h * N + i) * d, d) + fabs(rl[r] - L[h * N + i]);
            e += max_diff(rq + r * d, dQ + (h * N + i) * d, d);
            e += max_diff(rk + r * d, dK + (h * N + i) * d, d);
            e += max_diff(rv + r * d, dV + (h * N + i) * d, d);
        }
        snprintf(what, sizeof what, "selected rows, N=%ld causal=%d", N, causal);
        check(what, e, 1e-11);
    }
    free(Q); free(K); free(V); free(G); free(O); free(L); free(Ot); free(Lt);
    free(dQ); free(dK); free(dV); free(Dd); free(tQ); free(tK); free(tV);
    free(Lr); free(Dr); free(ro); free(rl); free(rq); free(rk); free(rv);
}

int main(void) {
    rng_state = 12345;
    if (orc_max_threads() < 1) return 2;
    orc_set_threads(3);
    run_case(2, 48, 16, 16, 12); /* the pages' tiles, whole tiles */
    run_case(3, 37, 5, 16, 12);  /* ragged last tiles */
    run_case(1, 1, 4, 16, 12);   /* a single row */
    run_case(2, 7, 1, 2, 3);     /* d = 1, tiles smaller than N */
    if (failures) return 1;
    printf("oracle sanitizer driver: all checks passed\n");
    return 0;
}
