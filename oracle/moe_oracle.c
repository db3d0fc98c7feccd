/*
 * moe_oracle.c -- plain fp64 CPU oracle of the single-token routed-expert MoE
 * decode layer (router GEMV, softmax + top-k, expert-indexed gate/up GEMV,
 * SiLU*mul, down GEMV with the top-k weighted combine, shared-expert add).
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the checker, not the product: only
 * the test suite, the smoke check and the benchmark's CPU-baseline leg may
 * load it.  It shares no code, header, table or helper with the HIP path and
 * must never be reached from it.
 *
 * Sources (the method as described on the web pages):
 *   [W]  "如何在天垓 BI-V100 上优化大模型推理：一份工作日志" (BI-V100 inference
 *        worklog), part 3 (why the PyTorch MoE fallback is slow: gather,
 *        F.linear, SiluAndMul, bmm, weighted sum), part 8 (topk + softmax
 *        launches of the MoE layer), part 10 (W13 kernel: input(1,H) x
 *        W13[expert_ids[k], row, :] -> gate_up(K, 2I); W2 kernel:
 *        activated(K, I) x W2[expert_ids[k], h, :] -> expert_out(H) with the
 *        weighted sum), part 2 (shared expert = gate_up + SiluAndMul + down).
 *   [R]  "decode analysis report 2026-07-14", section on code-level profiling
 *        (MoE = gate / routing topk / routed experts / shared expert).
 *
 * Every function evaluates the plain definition in double precision with
 * plain loops, in index order, no blocking, no fusion, no BLAS, no fast-math
 * (built with -O2 -ffp-contract=off).  Inputs are doubles holding the exact
 * values of the fp16 tensors (fp16 -> fp64 conversion is exact).
 *
 * Readings taken where the pages are silent (each is listed in the design
 * notes as well):
 *   - selection compares logits (softmax is monotone); equal logits order by
 *     the lower expert id first; expert_ids are emitted in that order;
 *   - weights: softmax over all E logits, then (renormalize=1) divided by the
 *     sum over the K selected -- equal to a softmax over the selected logits;
 *   - W13 rows [0, I) are the gate half, rows [I, 2I) the up half;
 *     silu(g) = g / (1 + exp(-g)); activated = silu(gate) * up;
 *   - W2 is [E, H, I], contiguous along I;
 *   - the shared expert is added with weight 1, no gate.
 *
 * Threading: optional OpenMP over independent output rows only; every row's
 * sum stays serial, so results are bitwise identical for any thread count.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_ABI 1

int oracle_abi_version(void) { return ORACLE_ABI; }

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

static int nthreads_or_one(int n) { return n > 0 ? n : 1; }

/* [W] part 8 / [R]: the router ("gate") of the MoE layer.
 * logits[e] = sum_h wr[e, h] * x[h], for one token. */
void oracle_router_logits(const double *x, const double *wr, int H, int E,
                          int nthreads, double *logits)
{
    int nt = nthreads_or_one(nthreads);
    (void)nt;
#pragma omp parallel for num_threads(nt) schedule(static)
    for (int e = 0; e < E; ++e) {
        double acc = 0.0;
        for (int h = 0; h < H; ++h)
            acc += wr[(size_t)e * H + h] * x[h];
        logits[e] = acc;
    }
}

typedef struct {
    double v;
    int id;
} scored_t;

/* larger logit first; equal logits: lower id first */
static int cmp_scored(const void *pa, const void *pb)
{
    const scored_t *a = (const scored_t *)pa, *b = (const scored_t *)pb;
    if (a->v > b->v) return -1;
    if (a->v < b->v) return 1;
    return (a->id < b->id) ? -1 : (a->id > b->id) ? 1 : 0;
}

/* [W] part 8 (topk + softmax of the routing step).
 * Orders all E experts by (logit descending, id ascending), keeps the first K
 * as expert_ids (in that order), and gives each its routing weight.
 * margin = smallest gap between neighbours among the first min(K+1, E)
 * sorted logits (how far the selection is from a tie).
 * Returns 0, or -1 on bad sizes / allocation failure. */
int oracle_topk_softmax(const double *logits, int E, int K, int renormalize,
                        int32_t *expert_ids, double *weights, double *margin)
{
    if (E <= 0 || K <= 0 || K > E) return -1;
    scored_t *s = (scored_t *)malloc(sizeof(scored_t) * (size_t)E);
    if (!s) return -1;
    for (int e = 0; e < E; ++e) {
        s[e].v = logits[e];
        s[e].id = e;
    }
    qsort(s, (size_t)E, sizeof(scored_t), cmp_scored);

    double lmax = s[0].v;
    double z = 0.0; /* softmax denominator over all E experts */
    for (int e = 0; e < E; ++e) z += exp(logits[e] - lmax);

    double sel = 0.0; /* sum of the selected probabilities */
    for (int k = 0; k < K; ++k) {
        expert_ids[k] = s[k].id;
        weights[k] = exp(s[k].v - lmax) / z;
        sel += weights[k];
    }
    if (renormalize)
        for (int k = 0; k < K; ++k) weights[k] = weights[k] / sel;

    if (margin) {
        double m = INFINITY;
        int last = (K < E) ? K : E - 1;
        for (int i = 0; i < last; ++i) {
            double gap = s[i].v - s[i + 1].v;
            if (gap < m) m = gap;
        }
        *margin = m;
    }
    free(s);
    return 0;
}

/* [W] part 8: the routing weights of a given selection.  For expert ids
 * ids[0..K) (each in [0, E)), weights[k] = softmax over all E logits taken at
 * ids[k], divided by their sum over the K entries when renormalize != 0.
 * Used where the selection itself is not unique (logits closer than their
 * rounding error): any top-K order of the computed logits is a correct
 * routing, and this gives the exact weights that routing carries.
 * Returns 0, or -1 on bad sizes or an id outside [0, E). */
int oracle_route_weights(const double *logits, int E, int K, const int32_t *ids,
                         int renormalize, double *weights)
{
    if (E <= 0 || K <= 0 || K > E) return -1;
    for (int k = 0; k < K; ++k)
        if (ids[k] < 0 || ids[k] >= E) return -1;
    double lmax = logits[0];
    for (int e = 1; e < E; ++e)
        if (logits[e] > lmax) lmax = logits[e];
    double z = 0.0;
    for (int e = 0; e < E; ++e) z += exp(logits[e] - lmax);
    double picked = 0.0; /* sum of the given ids' probabilities */
    for (int k = 0; k < K; ++k) {
        weights[k] = exp(logits[ids[k]] - lmax) / z;
        picked += weights[k];
    }
    if (renormalize != 0)
        for (int k = 0; k < K; ++k) weights[k] /= picked;
    return 0;
}

static double silu(double g) { return g / (1.0 + exp(-g)); }

/* [W] part 10 (W13 kernel) + part 3 (SiluAndMul), for one expert and one token.
 * gate_up rows of this expert: w13e[r, h], r < 2I (gate = rows [0,I), up = rows [I,2I)).
 * activated[j] = silu(sum_h w13e[j,h] x[h]) * (sum_h w13e[I+j,h] x[h]). */
void oracle_expert_activated(const double *x, const double *w13e, int H, int I,
                             int nthreads, double *activated)
{
    int nt = nthreads_or_one(nthreads);
    (void)nt;
#pragma omp parallel for num_threads(nt) schedule(static)
    for (int j = 0; j < I; ++j) {
        const double *grow = w13e + (size_t)j * H;
        const double *urow = w13e + (size_t)(I + j) * H;
        double g = 0.0, u = 0.0;
        for (int h = 0; h < H; ++h) g += grow[h] * x[h];
        for (int h = 0; h < H; ++h) u += urow[h] * x[h];
        activated[j] = silu(g) * u;
    }
}

/* [W] part 10 (W2 kernel with the weighted sum), for one token.
 * out[h] = sum_k weights[k] * (sum_j w2k[k][h, j] * activated[k][j]),
 * k in routing order.  w2k[k] points at W2[expert_ids[k]] ([H, I]),
 * activated is [K, I]. */
void oracle_weighted_down(const double *const *w2k, const double *activated,
                          const double *weights, int H, int I, int K,
                          int nthreads, double *out)
{
    int nt = nthreads_or_one(nthreads);
    (void)nt;
#pragma omp parallel for num_threads(nt) schedule(static)
    for (int h = 0; h < H; ++h) {
        double acc = 0.0;
        for (int k = 0; k < K; ++k) {
            const double *row = w2k[k] + (size_t)h * I;
            const double *a = activated + (size_t)k * I;
            double d = 0.0;
            for (int j = 0; j < I; ++j) d += row[j] * a[j];
            acc += weights[k] * d;
        }
        out[h] = acc;
    }
}

/* [W] part 2 (shared expert: gate_up + SiluAndMul + down), one token.
 * wsgu: [2Is, H] (gate rows [0,Is), up rows [Is,2Is)); wsd: [H, Is].
 * s[h] = sum_j wsd[h, j] * silu(gate_j) * up_j.  scratch: Is doubles. */
void oracle_shared_expert(const double *x, const double *wsgu, const double *wsd,
                          int H, int Is, int nthreads, double *scratch, double *s)
{
    oracle_expert_activated(x, wsgu, H, Is, nthreads, scratch);
    const double *rows[1] = {wsd};
    const double one[1] = {1.0};
    oracle_weighted_down(rows, scratch, one, H, Is, 1, nthreads, s);
}

/* Routed + shared output of one token, given the selected experts' slices.
 * w13sel: [K, 2I, H] = W13[expert_ids[k]] for k = 0..K-1 (routing order);
 * w2sel:  [K, H, I]  = W2[expert_ids[k]];  weights: [K].
 * wsgu/wsd may be NULL (no shared expert; Is ignored).
 * scratch: at least K*I + Is doubles.  y: [H]. */
void oracle_token_output(const double *x, const double *w13sel, const double *w2sel,
                         const double *weights, const double *wsgu, const double *wsd,
                         int H, int I, int K, int Is, int nthreads,
                         double *scratch, double *y)
{
    double *act = scratch;
    for (int k = 0; k < K; ++k)
        oracle_expert_activated(x, w13sel + (size_t)k * 2 * I * H, H, I, nthreads,
                                act + (size_t)k * I);
    const double **rows = (const double **)malloc(sizeof(double *) * (size_t)K);
    for (int k = 0; k < K; ++k) rows[k] = w2sel + (size_t)k * H * I;
    oracle_weighted_down(rows, act, weights, H, I, K, nthreads, y);
    free(rows);
    if (wsgu && wsd) {
        double *s = (double *)malloc(sizeof(double) * (size_t)H);
        oracle_shared_expert(x, wsgu, wsd, H, Is, nthreads, act + (size_t)K * I, s);
        for (int h = 0; h < H; ++h) y[h] = y[h] + s[h];
        free(s);
    }
}

/* The whole layer for M tokens with the full expert tensors resident in host
 * memory (small configurations).  Each token is routed independently.
 *   x [M,H], wr [E,H], w13 [E,2I,H], w2 [E,H,I], wsgu [2Is,H] | NULL, wsd [H,Is] | NULL
 * Outputs: expert_ids [M,K], weights [M,K], y [M,H], logits [M,E], margin [M].
 * Returns 0, or -1 on bad sizes / allocation failure. */
int oracle_moe_layer(const double *x, const double *wr, const double *w13, const double *w2,
                     const double *wsgu, const double *wsd,
                     int M, int H, int E, int I, int K, int Is, int renormalize, int nthreads,
                     int32_t *expert_ids, double *weights, double *y, double *logits,
                     double *margin)
{
    if (M <= 0 || H <= 0 || E <= 0 || I <= 0 || K <= 0 || K > E) return -1;
    size_t nscr = (size_t)K * I + (size_t)(Is > 0 ? Is : 0);
    double *scratch = (double *)malloc(sizeof(double) * nscr);
    double *w13sel = (double *)malloc(sizeof(double) * (size_t)K * 2 * I * H);
    double *w2sel = (double *)malloc(sizeof(double) * (size_t)K * H * I);
    if (!scratch || !w13sel || !w2sel) {
        free(scratch); free(w13sel); free(w2sel);
        return -1;
    }
    int rc = 0;
    for (int m = 0; m < M && rc == 0; ++m) {
        const double *xm = x + (size_t)m * H;
        double *lm = logits + (size_t)m * E;
        oracle_router_logits(xm, wr, H, E, nthreads, lm);
        rc = oracle_topk_softmax(lm, E, K, renormalize, expert_ids + (size_t)m * K,
                                 weights + (size_t)m * K, margin ? margin + m : NULL);
        if (rc) break;
        /* index the expert tensors by expert id (a copy here only because the
         * slice form is the oracle's single code path; values are unchanged) */
        for (int k = 0; k < K; ++k) {
            int e = expert_ids[(size_t)m * K + k];
            const double *src13 = w13 + (size_t)e * 2 * I * H;
            const double *src2 = w2 + (size_t)e * H * I;
            for (size_t i = 0; i < (size_t)2 * I * H; ++i) w13sel[(size_t)k * 2 * I * H + i] = src13[i];
            for (size_t i = 0; i < (size_t)H * I; ++i) w2sel[(size_t)k * H * I + i] = src2[i];
        }
        oracle_token_output(xm, w13sel, w2sel, weights + (size_t)m * K, wsgu, wsd, H, I, K, Is,
                            nthreads, scratch, y + (size_t)m * H);
    }
    free(scratch); free(w13sel); free(w2sel);
    return rc;
}
