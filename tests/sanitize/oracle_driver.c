/* Runs the fp64 oracle's entry points on small random inputs under the
 * address and undefined-behaviour sanitizers: chain, tree (random trees, per
 * sequence), chunked prefill for several chunk lengths and ragged lengths,
 * with one and several threads.  Checks the identities the oracle is pinned
 * by (a tree of chain parents is the chain; chunked equals stepwise), so a
 * run that touches memory out of bounds or overflows also fails them.
 * Exit status 0 on success. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_gdn_chain(int B, int N, int Hqk, int Hv, int dk, int dv, double scale, const double *q,
                     const double *k, const double *v, const double *alpha, const double *beta,
                     const double *state0, double *out, double *nodes, double *final_state, int nthreads);
int oracle_gdn_tree(int B, int N, int Hqk, int Hv, int dk, int dv, double scale, const double *q, const double *k,
                    const double *v, const double *alpha, const double *beta, const double *state0,
                    const int32_t *parent, double *out, double *nodes, int nthreads);
int oracle_gdn_chunked(int B, int T, int Hqk, int Hv, int dk, int dv, double scale, int chunk, const double *q,
                       const double *k, const double *v, const double *alpha, const double *beta,
                       const double *state0, double *out, double *final_state, int nthreads);

static double urand(unsigned *s) { *s = *s * 1103515245u + 12345u; return ((*s >> 8) & 0xffffff) / 16777216.0; }

static double *filled(size_t n, unsigned *s, double lo, double hi) {
    double *x = malloc(n * sizeof(double));
    for (size_t i = 0; i < n; ++i) x[i] = lo + (hi - lo) * urand(s);
    return x;
}

static double maxdiff(const double *a, const double *b, size_t n) {
    double m = 0;
    for (size_t i = 0; i < n; ++i) m = fmax(m, fabs(a[i] - b[i]));
    return m;
}

int main(void) {
    unsigned seed = 7;
    int bad = 0;
    for (int it = 0; it < 40; ++it) {
        const int B = 1 + it % 3, N = 1 + it % 20, Hqk = 1 + it % 2, Hv = Hqk * (1 + it % 3);
        const int dk = 2 + it % 7, dv = 1 + it % 5, th = 1 + it % 4;
        const size_t nq = (size_t)B * N * Hqk * dk, nv = (size_t)B * N * Hv * dv, ng = (size_t)B * N * Hv;
        const size_t ns = (size_t)B * Hv * dv * dk;
        double *q = filled(nq, &seed, -1, 1), *k = filled(nq, &seed, -0.5, 0.5), *v = filled(nv, &seed, -1, 1);
        double *al = filled(ng, &seed, 0.3, 1), *be = filled(ng, &seed, 0, 1), *s0 = filled(ns, &seed, -0.1, 0.1);
        double *out = malloc(nv * sizeof(double)), *nodes = malloc(nv * dk * sizeof(double));
        double *fin = malloc(ns * sizeof(double));
        double *tout = malloc(nv * sizeof(double)), *tnodes = malloc(nv * dk * sizeof(double));
        double *cout = malloc(nv * sizeof(double)), *cfin = malloc(ns * sizeof(double));
        int32_t *par = malloc((size_t)B * N * sizeof(int32_t));
        bad |= oracle_gdn_chain(B, N, Hqk, Hv, dk, dv, 1.0, q, k, v, al, be, s0, out, nodes, fin, th) != 0;
        for (int b = 0; b < B; ++b)
            for (int n = 0; n < N; ++n) par[b * N + n] = n - 1;
        bad |= oracle_gdn_tree(B, N, Hqk, Hv, dk, dv, 1.0, q, k, v, al, be, s0, par, tout, tnodes, th) != 0;
        bad |= maxdiff(out, tout, nv) != 0.0 || maxdiff(nodes, tnodes, nv * dk) != 0.0;
        for (int chunk = 1; chunk <= 9; chunk += 4) {
            bad |= oracle_gdn_chunked(B, N, Hqk, Hv, dk, dv, 1.0, chunk, q, k, v, al, be, s0, cout, cfin, th) != 0;
            bad |= maxdiff(out, cout, nv) > 1e-10 || maxdiff(fin, cfin, ns) > 1e-10;
        }
        for (int b = 0; b < B; ++b)  /* random trees, one per sequence */
            for (int n = 0; n < N; ++n) par[b * N + n] = n == 0 ? -1 : (int)(urand(&seed) * n);
        bad |= oracle_gdn_tree(B, N, Hqk, Hv, dk, dv, 0.5, q, k, v, al, be, s0, par, tout, tnodes, th) != 0;
        if (N >= 2) {  /* a parent that is not earlier is refused */
            par[1] = 1;
            bad |= oracle_gdn_tree(B, N, Hqk, Hv, dk, dv, 1.0, q, k, v, al, be, s0, par, tout, tnodes, th) == 0;
        }
        free(q); free(k); free(v); free(al); free(be); free(s0); free(out); free(nodes); free(fin);
        free(tout); free(tnodes); free(cout); free(cfin); free(par);
        if (bad) { fprintf(stderr, "oracle identity failed at iteration %d\n", it); return 1; }
    }
    printf("oracle driver ok\n");
    return 0;
}
