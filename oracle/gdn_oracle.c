/*
 * gdn_oracle.c -- fp64 CPU oracle for the Gated DeltaNet recurrent-state path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
 * the CPU-baseline leg of the benchmark may load this library.  It shares no
 * code, header, table or helper with the HIP library; nothing in the product
 * path may call it.
 *
 * What it computes (all arithmetic in IEEE double, no fast-math):
 *
 *   One step of the gated delta rule for one (sequence, value head):
 *       S_t = alpha_t * S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *       o_t = scale * S_t q_t
 *   S is d_v x d_k, stored row-major (row j = value channel j, d_k contiguous
 *   key channels).  This is the gated delta rule of a Gated DeltaNet layer,
 *   which the pages describe in words only: page "LightSeek's TokenSpeed Hits
 *   580 Tokens per Second on Qwen3.5's 400B Model", section "Why Qwen3.5 is
 *   hard to serve fast": a fixed state whose size is the head dimension
 *   squared, updated incrementally per token, and each output is read by
 *   querying the current (already updated) state.  The formula above is the
 *   statement of that rule this oracle follows.
 *
 *   Chain: nodes 0..N-1, node t starts from node t-1 (node 0 from the cached
 *   state).  Tree: node t starts from node parent[t] (parent[0] = -1 = the
 *   cached state, parent[t] < t).  Page "Qwen3.6 27B: From 20 t/s to 184 t/s",
 *   section "Diffusion applied to text" (a best-first tree of up to 22 nodes
 *   verified in one target pass); page "We got 207 tok/s with Qwen3.5-27B on
 *   an RTX 3090", section "Key wins" (per-node intermediate states kept).
 *
 *   Chunked form (WY / UT transform) of the same recurrence, for prefill: see
 *   oracle_gdn_chunked() below for the derivation it follows.
 *
 * Parity status: every function here is pinned by the CPU tests (closed
 * forms, special cases, exact-rational brute force, tree-vs-chain and
 * chunked-vs-stepwise identities).  Nothing is compared against an external
 * implementation: the pages print no numerical example.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

/* ------------------------------------------------------------------------ */
/* Shapes shared by every entry point.                                      */
/*   q, k       [B][N][Hqk][dk]                                              */
/*   v          [B][N][Hv][dv]                                               */
/*   alpha,beta [B][N][Hv]                                                   */
/*   state0     [B][Hv][dv][dk]   (S, row-major, one matrix per head)        */
/*   out        [B][N][Hv][dv]                                               */
/*   nodes      [B][N][Hv][dv][dk] (state after each node; nullable)         */
/*   final      [B][Hv][dv][dk]   (state after the last chain step; nullable)*/
/* Value head h reads q/k head h / (Hv / Hqk) (contiguous groups).          */
/* ------------------------------------------------------------------------ */
typedef struct {
    int B, N, Hqk, Hv, dk, dv;
    double scale;
    const double *q, *k, *v, *alpha, *beta, *state0;
    const int32_t *parent; /* [B][N] for trees, NULL for a chain */
    int chunk;             /* chunk length for the chunked form */
    double *out, *nodes, *final_state;
} job_t;

static const double *q_at(const job_t *j, int b, int n, int h)
{
    int g = h / (j->Hv / j->Hqk);
    return j->q + (((size_t)b * j->N + n) * j->Hqk + g) * j->dk;
}
static const double *k_at(const job_t *j, int b, int n, int h)
{
    int g = h / (j->Hv / j->Hqk);
    return j->k + (((size_t)b * j->N + n) * j->Hqk + g) * j->dk;
}
static const double *v_at(const job_t *j, int b, int n, int h)
{
    return j->v + (((size_t)b * j->N + n) * j->Hv + h) * j->dv;
}
static double gate_at(const double *g, const job_t *j, int b, int n, int h)
{
    return g[((size_t)b * j->N + n) * j->Hv + h];
}

/*
 * One application of the rule to a single head:
 *   S_out = alpha * S_in (I - beta k k^T) + beta v k^T,   o = scale * S_out q.
 * S_in (I - beta k k^T) is formed as S_in - beta (S_in k) k^T, the same
 * product with the (k k^T) factor associated to the right.
 * S_in and S_out may alias.
 */
void oracle_gdn_step(int dk, int dv, double scale, const double *S_in,
                     const double *q, const double *k, const double *v,
                     double alpha, double beta, double *S_out, double *o)
{
    for (int j = 0; j < dv; ++j) {
        const double *row = S_in + (size_t)j * dk;
        double sk = 0.0; /* (S_in k)_j */
        for (int i = 0; i < dk; ++i) sk += row[i] * k[i];
        double *orow = S_out + (size_t)j * dk;
        for (int i = 0; i < dk; ++i)
            orow[i] = alpha * (row[i] - beta * sk * k[i]) + beta * v[j] * k[i];
    }
    if (o) {
        for (int j = 0; j < dv; ++j) {
            const double *row = S_out + (size_t)j * dk;
            double acc = 0.0;
            for (int i = 0; i < dk; ++i) acc += row[i] * q[i];
            o[j] = scale * acc;
        }
    }
}

/* ---------------------------- chain ------------------------------------ */
static void chain_unit(const job_t *j, int b, int h, double *S)
{
    const size_t hs = (size_t)j->dv * j->dk;
    memcpy(S, j->state0 + ((size_t)b * j->Hv + h) * hs, hs * sizeof(double));
    for (int n = 0; n < j->N; ++n) {
        double *o = j->out ? j->out + (((size_t)b * j->N + n) * j->Hv + h) * j->dv : NULL;
        oracle_gdn_step(j->dk, j->dv, j->scale, S, q_at(j, b, n, h), k_at(j, b, n, h),
                        v_at(j, b, n, h), gate_at(j->alpha, j, b, n, h),
                        gate_at(j->beta, j, b, n, h), S, o);
        if (j->nodes)
            memcpy(j->nodes + (((size_t)b * j->N + n) * j->Hv + h) * hs, S, hs * sizeof(double));
    }
    if (j->final_state)
        memcpy(j->final_state + ((size_t)b * j->Hv + h) * hs, S, hs * sizeof(double));
}

/* ---------------------------- tree ------------------------------------- */
/* Node n starts from node parent[n]'s state (the cached state for -1).     */
/* All node states of the unit are kept, so any parent can be read.         */
static int tree_unit(const job_t *j, int b, int h, double *scratch /* N*hs */)
{
    const size_t hs = (size_t)j->dv * j->dk;
    const double *S0 = j->state0 + ((size_t)b * j->Hv + h) * hs;
    const int32_t *par = j->parent + (size_t)b * j->N;
    for (int n = 0; n < j->N; ++n) {
        int p = par[n];
        if (p < -1 || p >= n) return -1;
        const double *Sp = (p < 0) ? S0 : scratch + (size_t)p * hs;
        double *Sn = scratch + (size_t)n * hs;
        double *o = j->out ? j->out + (((size_t)b * j->N + n) * j->Hv + h) * j->dv : NULL;
        oracle_gdn_step(j->dk, j->dv, j->scale, Sp, q_at(j, b, n, h), k_at(j, b, n, h),
                        v_at(j, b, n, h), gate_at(j->alpha, j, b, n, h),
                        gate_at(j->beta, j, b, n, h), Sn, o);
        if (j->nodes)
            memcpy(j->nodes + (((size_t)b * j->N + n) * j->Hv + h) * hs, Sn, hs * sizeof(double));
    }
    return 0;
}

/* --------------------------- chunked ----------------------------------- */
/*
 * Chunked (WY / UT) form of the chain recurrence, one head.  Derived from
 * the rule; the pages only name chunked linear-attention prefill (page
 * "We got 207 tok/s with Qwen3.5-27B on an RTX 3090", section "Prefill").
 * Written with H = S^T (d_k x d_v) as in the derivation; the storage is S.
 *
 * Inside a chunk of C tokens t = 1..C starting from H_0:
 *   u_t = beta_t (v_t - alpha_t H_{t-1}^T k_t),   H_t = alpha_t H_{t-1} + k_t u_t^T
 *   Gamma_{t,i} = prod_{s=i+1..t} alpha_s,  gamma_t = prod_{s=1..t} alpha_s
 *   H_t = gamma_t H_0 + sum_{i<=t} Gamma_{t,i} k_i u_i^T
 * so the residuals solve a unit lower-triangular system
 *   (I + A) U = diag(beta) V - diag(beta gamma) K H_0,
 *   A_{t,i} = beta_t Gamma_{t,i} (k_t . k_i)   for i < t.
 * With T = (I + A)^{-1} (the UT transform, by forward substitution):
 *   W = T diag(beta gamma) K,   U' = T diag(beta) V,   U = U' - W H_0
 *   O = scale [ diag(gamma) Q H_0 + (Gamma o tril(Q K^T)) U ]   (diagonal kept)
 *   H_C = gamma_C H_0 + K^T diag(Gamma_{C,.}) U
 * The products of alphas are formed directly (no division, no logs), so a
 * zero gate is handled exactly.
 */
static void chunked_unit(const job_t *j, int b, int h, double *work)
{
    const int dk = j->dk, dv = j->dv, Cmax = j->chunk;
    const size_t hs = (size_t)dv * dk;
    double *S = work;                              /* dv*dk  (S = H^T)      */
    double *Gam = S + hs;                          /* C*C    Gamma_{t,i}     */
    double *gam = Gam + (size_t)Cmax * Cmax;       /* C      gamma_t         */
    double *Tm = gam + Cmax;                       /* C*C    T = (I+A)^-1    */
    double *A = Tm + (size_t)Cmax * Cmax;          /* C*C                    */
    double *W = A + (size_t)Cmax * Cmax;           /* C*dk                   */
    double *U = W + (size_t)Cmax * dk;             /* C*dv                   */
    double *Snew = U + (size_t)Cmax * dv;          /* dv*dk                  */

    memcpy(S, j->state0 + ((size_t)b * j->Hv + h) * hs, hs * sizeof(double));
    for (int t0 = 0; t0 < j->N; t0 += Cmax) {
        const int C = (j->N - t0 < Cmax) ? (j->N - t0) : Cmax;
        /* gates: Gamma_{t,i} for i <= t, gamma_t (0-based t, i) */
        for (int t = 0; t < C; ++t) {
            Gam[(size_t)t * Cmax + t] = 1.0;
            for (int i = t - 1; i >= 0; --i)
                Gam[(size_t)t * Cmax + i] =
                    Gam[(size_t)t * Cmax + i + 1] * gate_at(j->alpha, j, b, t0 + i + 1, h);
            double g = 1.0;
            for (int s = 0; s <= t; ++s) g *= gate_at(j->alpha, j, b, t0 + s, h);
            gam[t] = g;
        }
        /* A (strictly lower) */
        for (int t = 0; t < C; ++t) {
            const double *kt = k_at(j, b, t0 + t, h);
            double bt = gate_at(j->beta, j, b, t0 + t, h);
            for (int i = 0; i < C; ++i) {
                double a = 0.0;
                if (i < t) {
                    const double *ki = k_at(j, b, t0 + i, h);
                    double kk = 0.0;
                    for (int c = 0; c < dk; ++c) kk += kt[c] * ki[c];
                    a = bt * Gam[(size_t)t * Cmax + i] * kk;
                }
                A[(size_t)t * Cmax + i] = a;
            }
        }
        /* T = (I + A)^{-1}, unit lower triangular, by forward substitution:
           row t of T: T_{t,t} = 1, T_{t,i} = -sum_{m=i}^{t-1} A_{t,m} T_{m,i}. */
        for (int t = 0; t < C; ++t) {
            for (int i = 0; i < C; ++i) {
                double x;
                if (i > t) x = 0.0;
                else if (i == t) x = 1.0;
                else {
                    x = 0.0;
                    for (int m = i; m < t; ++m) x -= A[(size_t)t * Cmax + m] * Tm[(size_t)m * Cmax + i];
                }
                Tm[(size_t)t * Cmax + i] = x;
            }
        }
        /* W = T diag(beta gamma) K ;  U' = T diag(beta) V ;  U = U' - W H_0 */
        for (int t = 0; t < C; ++t) {
            for (int c = 0; c < dk; ++c) {
                double acc = 0.0;
                for (int i = 0; i <= t; ++i)
                    acc += Tm[(size_t)t * Cmax + i] * gate_at(j->beta, j, b, t0 + i, h) * gam[i] *
                           k_at(j, b, t0 + i, h)[c];
                W[(size_t)t * dk + c] = acc;
            }
            for (int c = 0; c < dv; ++c) {
                double acc = 0.0;
                for (int i = 0; i <= t; ++i)
                    acc += Tm[(size_t)t * Cmax + i] * gate_at(j->beta, j, b, t0 + i, h) *
                           v_at(j, b, t0 + i, h)[c];
                /* (W H_0)_{t,c} = sum_i W_{t,i} H_0[i][c] = sum_i W_{t,i} S[c][i] */
                double wh = 0.0;
                for (int i = 0; i < dk; ++i) wh += W[(size_t)t * dk + i] * S[(size_t)c * dk + i];
                U[(size_t)t * dv + c] = acc - wh;
            }
        }
        /* outputs */
        if (j->out) {
            for (int t = 0; t < C; ++t) {
                const double *qt = q_at(j, b, t0 + t, h);
                double *o = j->out + (((size_t)b * j->N + t0 + t) * j->Hv + h) * dv;
                for (int c = 0; c < dv; ++c) {
                    double qh = 0.0; /* (H_0^T q_t)_c = (S q_t)_c */
                    for (int i = 0; i < dk; ++i) qh += S[(size_t)c * dk + i] * qt[i];
                    double acc = gam[t] * qh;
                    for (int i = 0; i <= t; ++i) {
                        const double *ki = k_at(j, b, t0 + i, h);
                        double qk = 0.0;
                        for (int m = 0; m < dk; ++m) qk += qt[m] * ki[m];
                        acc += Gam[(size_t)t * Cmax + i] * qk * U[(size_t)i * dv + c];
                    }
                    o[c] = j->scale * acc;
                }
            }
        }
        /* H_C = gamma_C H_0 + K^T diag(Gamma_{C,.}) U, stored as S = H^T */
        for (int c = 0; c < dv; ++c) {
            for (int i = 0; i < dk; ++i) {
                double acc = gam[C - 1] * S[(size_t)c * dk + i];
                for (int t = 0; t < C; ++t)
                    acc += k_at(j, b, t0 + t, h)[i] * Gam[(size_t)(C - 1) * Cmax + t] * U[(size_t)t * dv + c];
                Snew[(size_t)c * dk + i] = acc;
            }
        }
        memcpy(S, Snew, hs * sizeof(double));
    }
    if (j->final_state)
        memcpy(j->final_state + ((size_t)b * j->Hv + h) * hs, S, hs * sizeof(double));
}

/* ------------------------- threading ----------------------------------- */
/* Independent (sequence, head) units are spread over threads; each unit's */
/* arithmetic is the same whatever the thread count.                       */
enum { KIND_CHAIN = 0, KIND_TREE = 1, KIND_CHUNKED = 2 };

typedef struct {
    const job_t *job;
    int kind, tid, nthreads, err, started;
} worker_t;

static size_t scratch_doubles(const job_t *j, int kind)
{
    const size_t hs = (size_t)j->dv * j->dk;
    if (kind == KIND_CHAIN) return hs;
    if (kind == KIND_TREE) return (size_t)j->N * hs;
    const size_t C = (size_t)j->chunk;
    return 2 * hs + 3 * C * C + C + C * j->dk + C * j->dv;
}

static void *worker(void *arg)
{
    worker_t *w = (worker_t *)arg;
    const job_t *j = w->job;
    double *scratch = (double *)malloc(scratch_doubles(j, w->kind) * sizeof(double));
    if (!scratch) { w->err = -2; return NULL; }
    const int units = j->B * j->Hv;
    for (int u = w->tid; u < units; u += w->nthreads) {
        int b = u / j->Hv, h = u % j->Hv;
        if (w->kind == KIND_CHAIN) chain_unit(j, b, h, scratch);
        else if (w->kind == KIND_TREE) { if (tree_unit(j, b, h, scratch)) w->err = -1; }
        else chunked_unit(j, b, h, scratch);
    }
    free(scratch);
    return NULL;
}

static int run(const job_t *j, int kind, int nthreads)
{
    if (j->B < 0 || j->N < 0 || j->Hqk <= 0 || j->Hv <= 0 || j->dk <= 0 || j->dv <= 0) return -3;
    if (j->Hv % j->Hqk) return -3;
    if (kind == KIND_CHUNKED && j->chunk <= 0) return -3;
    if (j->B == 0 || j->N == 0) {
        /* nothing to do; a chain of zero steps leaves the state as it is */
        if (j->final_state && j->B > 0)
            memcpy(j->final_state, j->state0, (size_t)j->B * j->Hv * j->dv * j->dk * sizeof(double));
        return 0;
    }
    const int units = j->B * j->Hv;
    if (nthreads <= 0) {
        long n = sysconf(_SC_NPROCESSORS_ONLN);
        nthreads = n > 0 ? (int)n : 1;
    }
    if (nthreads > units) nthreads = units;
    worker_t *ws = (worker_t *)calloc((size_t)nthreads, sizeof(worker_t));
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!ws || !th) { free(ws); free(th); return -2; }
    for (int t = 0; t < nthreads; ++t) {
        ws[t].job = j; ws[t].kind = kind; ws[t].tid = t; ws[t].nthreads = nthreads; ws[t].err = 0;
    }
    for (int t = 1; t < nthreads; ++t)
        ws[t].started = (pthread_create(&th[t], NULL, worker, &ws[t]) == 0);
    worker(&ws[0]);
    int err = ws[0].err;
    for (int t = 1; t < nthreads; ++t) {
        if (ws[t].started) pthread_join(th[t], NULL);
        else ws[t].err = -2; /* its units were not computed */
        if (ws[t].err) err = ws[t].err;
    }
    free(ws); free(th);
    return err;
}

/* ---------------------------- API -------------------------------------- */
/* Returns 0 on success, -1 bad parent array, -2 out of memory, -3 bad shape. */

int oracle_gdn_chain(int B, int N, int Hqk, int Hv, int dk, int dv, double scale,
                     const double *q, const double *k, const double *v,
                     const double *alpha, const double *beta, const double *state0,
                     double *out, double *nodes, double *final_state, int nthreads)
{
    job_t j = {B, N, Hqk, Hv, dk, dv, scale, q, k, v, alpha, beta, state0, NULL, 0,
               out, nodes, final_state};
    return run(&j, KIND_CHAIN, nthreads);
}

int oracle_gdn_tree(int B, int N, int Hqk, int Hv, int dk, int dv, double scale,
                    const double *q, const double *k, const double *v,
                    const double *alpha, const double *beta, const double *state0,
                    const int32_t *parent, double *out, double *nodes, int nthreads)
{
    job_t j = {B, N, Hqk, Hv, dk, dv, scale, q, k, v, alpha, beta, state0, parent, 0,
               out, nodes, NULL};
    return run(&j, KIND_TREE, nthreads);
}

int oracle_gdn_chunked(int B, int T, int Hqk, int Hv, int dk, int dv, double scale, int chunk,
                       const double *q, const double *k, const double *v,
                       const double *alpha, const double *beta, const double *state0,
                       double *out, double *final_state, int nthreads)
{
    job_t j = {B, T, Hqk, Hv, dk, dv, scale, q, k, v, alpha, beta, state0, NULL, chunk,
               out, NULL, final_state};
    return run(&j, KIND_CHUNKED, nthreads);
}
