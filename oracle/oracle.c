/*
 * Plain fp64 CPU oracle of the dropless sparse-MoE forward pass.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may call, link or
 * load this file: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it. It shares no code, header or table with the HIP
 * library, and it is deliberately slow and obvious: straight loops, fp64
 * arithmetic, no blocking, no fusion, no reordering of any sum.
 *
 * Sources (web pages on ScatterMoE and related kernels):
 *  - ScatterMoE Guide (aifetchly blog), section "1. The Dynamic Routing
 *    Imbalance Dilemma", equation H(X) = Softmax(TopK(X W_gate, k)).
 *  - same page, section "2. Grouped Coordinate Indexing Without Padding",
 *    the Histogram(e) and Offsets(e) equations, and section "2. The Complete
 *    ParallelLinear PyTorch Layer" (sort of the flattened routes by expert).
 *  - same page, section "1. The Anatomy of ParallelLinear" (gather rows of X
 *    by index, multiply by the expert's W, scale by the router coefficient,
 *    accumulate into the token's output row) and section "2. The Hidden Cost
 *    of Activation Materialization" (SwiGLU experts, scatter-add of gated
 *    expert outputs back to token order).
 *  - Fast-LLM pull request "Add scalable sparse map kernel", section
 *    "Testing / Correctness Validation" (unique rows inside disjoint expert
 *    ranges, histogram counts, deterministic results).
 *
 * Readings where the pages leave a step open (each is also listed with the
 * design notes):
 *  - top-k order is descending logit, ties go to the lower expert id;
 *  - softmax is taken over the k selected logits (equal to softmax over all
 *    E followed by top-k and renormalisation);
 *  - h = SiLU(x W1[e]) * (x W3[e]), y = h W2[e], with W stored
 *    [E, D_in, D_out] row-major; the router coefficient multiplies y once,
 *    after the nonlinearity;
 *  - the sparse map is the stable (flat route index order) sort by expert.
 *
 * Inputs are raw bf16 bit patterns (uint16); each one is widened exactly to
 * fp64 before use. Every dot product is summed in ascending index order.
 *
 * Parity pins: every function here is pinned by the CPU test suite (brute
 * force, library sort, closed forms and invariants); none is unpinned.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static double bf16_to_double(uint16_t b) {
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* ---------------------------------------------------------------- route -- */

/* Router logits of one token: l[e] = sum_d x[d] * W_gate[d, e]. */
static void token_logits(const uint16_t *x_row, const uint16_t *wg, int64_t D, int64_t E, double *l) {
    for (int64_t e = 0; e < E; ++e) l[e] = 0.0;
    for (int64_t d = 0; d < D; ++d) {
        double xv = bf16_to_double(x_row[d]);
        const uint16_t *wrow = wg + d * E;
        for (int64_t e = 0; e < E; ++e) l[e] += xv * bf16_to_double(wrow[e]);
    }
}

/* Top-k by repeated arg-max: descending logit, ties to the lower id. */
static void token_topk(const double *l, int64_t E, int64_t k, int32_t *ids, unsigned char *taken) {
    memset(taken, 0, (size_t)E);
    for (int64_t j = 0; j < k; ++j) {
        int64_t best = -1;
        for (int64_t e = 0; e < E; ++e) {
            if (taken[e]) continue;
            if (best < 0 || l[e] > l[best]) best = e;
        }
        taken[best] = 1;
        ids[j] = (int32_t)best;
    }
}

/* Softmax over the k selected logits (max subtracted). */
static void token_softmax(const double *l, const int32_t *ids, int64_t k, double *w) {
    double m = l[ids[0]];
    for (int64_t j = 1; j < k; ++j)
        if (l[ids[j]] > m) m = l[ids[j]];
    double z = 0.0;
    for (int64_t j = 0; j < k; ++j) {
        w[j] = exp(l[ids[j]] - m);
        z += w[j];
    }
    for (int64_t j = 0; j < k; ++j) w[j] /= z;
}

/*
 * Router: H(X) = Softmax(TopK(X W_gate, k)).
 * x [S, D], wg [D, E] (bf16 bits) -> ids [S, k], weights [S, k] fp64,
 * and, when logits != NULL, the fp64 logits [S, E].
 * If ids_in != NULL the top-k step is skipped and those ids are used
 * (the weights are then the softmax over the given experts' logits).
 */
int oracle_route(const uint16_t *x, const uint16_t *wg, int64_t S, int64_t D, int64_t E, int64_t k,
                 const int32_t *ids_in, int32_t *ids, double *weights, double *logits) {
    if (S < 0 || D < 1 || E < 1 || k < 1 || k > E) return 1;
    double *l = (double *)malloc(sizeof(double) * (size_t)E);
    unsigned char *taken = (unsigned char *)malloc((size_t)E);
    if (!l || !taken) { free(l); free(taken); return 2; }
    for (int64_t s = 0; s < S; ++s) {
        token_logits(x + s * D, wg, D, E, l);
        if (logits) memcpy(logits + s * E, l, sizeof(double) * (size_t)E);
        if (ids_in) {
            memcpy(ids + s * k, ids_in + s * k, sizeof(int32_t) * (size_t)k);
        } else {
            token_topk(l, E, k, ids + s * k, taken);
        }
        token_softmax(l, ids + s * k, k, weights + s * k);
    }
    free(l);
    free(taken);
    return 0;
}

/* ----------------------------------------------------------- sparse map -- */

/*
 * Stable counting sort of the flat routes f = s*k + j by expert id.
 *   counts[e]  = Histogram(e) = #{f : ids[f] = e}
 *   offsets[e] = Offsets(e) = sum_{e' < e} counts[e'], offsets[E] = S*k
 *   slot(f)    = offsets[ids[f]] + #{f' < f : ids[f'] = ids[f]}
 *   sparse_rows[f] = slot(f), slot_src[slot(f)] = f
 * Returns 1 if an id is out of range.
 */
int oracle_sparse_map(const int32_t *ids, int64_t S, int64_t k, int64_t E, int32_t *counts,
                      int32_t *offsets, int32_t *sparse_rows, int32_t *slot_src) {
    int64_t n = S * k;
    for (int64_t e = 0; e < E; ++e) counts[e] = 0;
    for (int64_t f = 0; f < n; ++f) {
        if (ids[f] < 0 || ids[f] >= E) return 1;
        counts[ids[f]] += 1;
    }
    offsets[0] = 0;
    for (int64_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    int32_t *next = (int32_t *)malloc(sizeof(int32_t) * (size_t)(E > 0 ? E : 1));
    if (!next) return 2;
    for (int64_t e = 0; e < E; ++e) next[e] = offsets[e];
    for (int64_t f = 0; f < n; ++f) {
        int32_t slot = next[ids[f]]++;
        sparse_rows[f] = slot;
        slot_src[slot] = (int32_t)f;
    }
    free(next);
    return 0;
}

/* ------------------------------------------------------------------ ffn -- */

static double silu(double z) { return z / (1.0 + exp(-z)); }

/*
 * One SwiGLU expert on one token row:
 *   a = x W1[e], b = x W3[e]  (length F), h = SiLU(a) * b, y = h W2[e] (length D)
 * w1e, w3e [D, F], w2e [F, D]; a, b, y are caller scratch.
 */
static void expert_row(const uint16_t *x_row, const uint16_t *w1e, const uint16_t *w3e,
                       const uint16_t *w2e, int64_t D, int64_t F, double *a, double *b, double *y) {
    for (int64_t f = 0; f < F; ++f) { a[f] = 0.0; b[f] = 0.0; }
    for (int64_t d = 0; d < D; ++d) {
        double xv = bf16_to_double(x_row[d]);
        const uint16_t *r1 = w1e + d * F, *r3 = w3e + d * F;
        for (int64_t f = 0; f < F; ++f) {
            a[f] += xv * bf16_to_double(r1[f]);
            b[f] += xv * bf16_to_double(r3[f]);
        }
    }
    for (int64_t f = 0; f < F; ++f) a[f] = silu(a[f]) * b[f]; /* a now holds h */
    for (int64_t n = 0; n < D; ++n) y[n] = 0.0;
    for (int64_t f = 0; f < F; ++f) {
        double hv = a[f];
        const uint16_t *r2 = w2e + f * D;
        for (int64_t n = 0; n < D; ++n) y[n] += hv * bf16_to_double(r2[n]);
    }
}

typedef struct {
    const uint16_t *x, *w1, *w3, *w2;
    const int32_t *ids;
    const double *weights;
    int64_t D, F, E, k;
    const int64_t *tokens;
    int64_t t_begin, t_end;
    double *out;
    int status;
} ffn_job;

static void *ffn_worker(void *arg) {
    ffn_job *jb = (ffn_job *)arg;
    int64_t D = jb->D, F = jb->F, k = jb->k;
    double *a = (double *)malloc(sizeof(double) * (size_t)F);
    double *b = (double *)malloc(sizeof(double) * (size_t)F);
    double *y = (double *)malloc(sizeof(double) * (size_t)D);
    if (!a || !b || !y) { jb->status = 2; free(a); free(b); free(y); return NULL; }
    for (int64_t i = jb->t_begin; i < jb->t_end; ++i) {
        int64_t s = jb->tokens[i];
        double *o = jb->out + i * D;
        for (int64_t n = 0; n < D; ++n) o[n] = 0.0;
        for (int64_t j = 0; j < k; ++j) {
            int64_t e = jb->ids[s * k + j];
            if (e < 0 || e >= jb->E) { jb->status = 1; continue; }
            expert_row(jb->x + s * D, jb->w1 + e * D * F, jb->w3 + e * D * F, jb->w2 + e * F * D, D, F, a, b, y);
            double g = jb->weights[s * k + j];
            for (int64_t n = 0; n < D; ++n) o[n] += g * y[n];
        }
    }
    free(a); free(b); free(y);
    return NULL;
}

/*
 * Dropless MoE FFN with weighted combine, for a list of tokens:
 *   out[i, :] = sum_{j=0..k-1} weights[s, j] * SwiGLU_{ids[s, j]}(x[s, :]),  s = tokens[i]
 * summed in j order. x [S, D]; w1, w3 [E, D, F]; w2 [E, F, D] (bf16 bits);
 * ids [S, k]; weights [S, k] fp64; out [ntok, D] fp64.
 * Work is split over `nthreads` POSIX threads by token; each output element
 * is still summed in the order above.
 */
int oracle_ffn_tokens(const uint16_t *x, const uint16_t *w1, const uint16_t *w3, const uint16_t *w2,
                      const int32_t *ids, const double *weights, int64_t D, int64_t F, int64_t E,
                      int64_t k, const int64_t *tokens, int64_t ntok, double *out, int nthreads) {
    if (D < 1 || F < 1 || E < 1 || k < 1 || ntok < 0) return 1;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > ntok) nthreads = ntok > 0 ? (int)ntok : 1;
    ffn_job *jobs = (ffn_job *)calloc((size_t)nthreads, sizeof(ffn_job));
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !th) { free(jobs); free(th); return 2; }
    int64_t per = (ntok + nthreads - 1) / nthreads;
    for (int t = 0; t < nthreads; ++t) {
        ffn_job *jb = &jobs[t];
        jb->x = x; jb->w1 = w1; jb->w3 = w3; jb->w2 = w2; jb->ids = ids; jb->weights = weights;
        jb->D = D; jb->F = F; jb->E = E; jb->k = k; jb->tokens = tokens; jb->out = out;
        jb->t_begin = t * per;
        jb->t_end = jb->t_begin + per < ntok ? jb->t_begin + per : ntok;
        if (jb->t_begin > jb->t_end) jb->t_begin = jb->t_end;
    }
    for (int t = 1; t < nthreads; ++t) pthread_create(&th[t], NULL, ffn_worker, &jobs[t]);
    ffn_worker(&jobs[0]);
    for (int t = 1; t < nthreads; ++t) pthread_join(th[t], NULL);
    int st = 0;
    for (int t = 0; t < nthreads; ++t)
        if (jobs[t].status) st = jobs[t].status;
    free(jobs); free(th);
    return st;
}

/* ------------------------------------------------------ parallel linear -- */

/*
 * ParallelLinear(X, W, I, G) (ScatterMoE Guide, "1. The Anatomy of
 * ParallelLinear" and the figure "The ParallelLinear Core Abstraction"):
 * the routes f = t*k + j (token t, expert e = ids[f], gate g_f) are sorted
 * by expert into slots r (the map above). For every route
 *     z_f = g_f * in(f) W[e]                          (length D_out)
 * where in(f) = x[r] (grouped input: x holds S*k rows in slot order) or
 * x[t] (scattered input: x holds S token rows). The output is
 *     y[r] = z_f          (grouped output, S*k rows in slot order) or
 *     y[t] = sum_j z_f    (scattered output, S token rows, summed j = 0..k-1).
 * gates == NULL means g_f = 1. W is [E, D_in, D_out] (bf16 bits); y is fp64.
 */
static int pl_map(const int32_t *ids, int64_t S, int64_t k, int64_t E, int32_t **rows_out) {
    int64_t n = S * k;
    int32_t *counts = (int32_t *)malloc(sizeof(int32_t) * (size_t)(E > 0 ? E : 1));
    int32_t *offsets = (int32_t *)malloc(sizeof(int32_t) * (size_t)(E + 1));
    int32_t *rows = (int32_t *)malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
    int32_t *src = (int32_t *)malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
    if (!counts || !offsets || !rows || !src) { free(counts); free(offsets); free(rows); free(src); return 2; }
    int st = oracle_sparse_map(ids, S, k, E, counts, offsets, rows, src);
    free(counts); free(offsets); free(src);
    if (st) { free(rows); return st; }
    *rows_out = rows;
    return 0;
}

/* z = in W[e]: in [D_in] bf16 bits, we [D_in, D_out] bf16 bits, z [D_out] fp64 */
static void row_times_w(const uint16_t *in, const uint16_t *we, int64_t D_in, int64_t D_out, double *z) {
    for (int64_t n = 0; n < D_out; ++n) z[n] = 0.0;
    for (int64_t d = 0; d < D_in; ++d) {
        double v = bf16_to_double(in[d]);
        const uint16_t *wr = we + d * D_out;
        for (int64_t n = 0; n < D_out; ++n) z[n] += v * bf16_to_double(wr[n]);
    }
}

/* c = dy W[e]^T: dy [D_out] bf16 bits, c [D_in] fp64 (c[d] = sum_n dy[n] W[e][d, n]) */
static void row_times_wt(const uint16_t *dy, const uint16_t *we, int64_t D_in, int64_t D_out, double *c) {
    for (int64_t d = 0; d < D_in; ++d) {
        const uint16_t *wr = we + d * D_out;
        double s = 0.0;
        for (int64_t n = 0; n < D_out; ++n) s += bf16_to_double(dy[n]) * bf16_to_double(wr[n]);
        c[d] = s;
    }
}

int oracle_parallel_linear(const uint16_t *x, const uint16_t *w, const double *gates, const int32_t *ids,
                           int64_t S, int64_t k, int64_t D_in, int64_t D_out, int64_t E, int grouped_in,
                           int grouped_out, double *y) {
    if (S < 0 || k < 1 || D_in < 1 || D_out < 1 || E < 1) return 1;
    int32_t *rows = NULL;
    int st = pl_map(ids, S, k, E, &rows);
    if (st) return st;
    double *z = (double *)malloc(sizeof(double) * (size_t)D_out);
    if (!z) { free(rows); return 2; }
    int64_t n_out = grouped_out ? S * k : S;
    for (int64_t i = 0; i < n_out * D_out; ++i) y[i] = 0.0;
    for (int64_t t = 0; t < S; ++t) {
        for (int64_t j = 0; j < k; ++j) {
            int64_t f = t * k + j, r = rows[f], e = ids[f];
            const uint16_t *in = grouped_in ? x + r * D_in : x + t * D_in;
            row_times_w(in, w + e * D_in * D_out, D_in, D_out, z);
            double g = gates ? gates[f] : 1.0;
            double *o = grouped_out ? y + r * D_out : y + t * D_out;
            for (int64_t n = 0; n < D_out; ++n) o[n] += g * z[n];
        }
    }
    free(z); free(rows);
    return 0;
}

/*
 * Backward of ParallelLinear (ScatterMoE Guide, "3. Fused Backward Pass
 * Dynamics"): with dy_f = dy[r] (grouped output) or dy[t] (scattered output),
 *     dx:  c_f = g_f * dy_f W[e]^T;  dx[r] = c_f (grouped input) or
 *          dx[t] = sum_j c_f (scattered input, j = 0..k-1)
 *     dw:  dw[e] = sum over the slots r of expert e, ascending, of
 *          g_f * in(f)^T dy_f                        ([D_in, D_out])
 *     dg:  dg[f] = <dy_f, in(f) W[e]>               (the router coefficient's
 *          gradient; needs no gates)
 * Any of dx, dw, dg may be NULL. All outputs fp64; dw is [E, D_in, D_out]
 * and is zero for an expert with no routes.
 */
int oracle_parallel_linear_bwd(const uint16_t *x, const uint16_t *w, const double *gates, const int32_t *ids,
                               const uint16_t *dy, int64_t S, int64_t k, int64_t D_in, int64_t D_out, int64_t E,
                               int grouped_in, int grouped_out, double *dx, double *dw, double *dg) {
    if (S < 0 || k < 1 || D_in < 1 || D_out < 1 || E < 1) return 1;
    int32_t *rows = NULL;
    int st = pl_map(ids, S, k, E, &rows);
    if (st) return st;
    int64_t n = S * k;
    int32_t *src = (int32_t *)calloc((size_t)(n > 0 ? n : 1), sizeof(int32_t));
    double *c = (double *)malloc(sizeof(double) * (size_t)(D_in > D_out ? D_in : D_out));
    if (!src || !c) { free(rows); free(src); free(c); return 2; }
    for (int64_t f = 0; f < n; ++f) src[rows[f]] = (int32_t)f;
    if (dx) {
        int64_t n_in = grouped_in ? n : S;
        for (int64_t i = 0; i < n_in * D_in; ++i) dx[i] = 0.0;
        for (int64_t t = 0; t < S; ++t) {
            for (int64_t j = 0; j < k; ++j) {
                int64_t f = t * k + j, r = rows[f], e = ids[f];
                const uint16_t *d = grouped_out ? dy + r * D_out : dy + t * D_out;
                row_times_wt(d, w + e * D_in * D_out, D_in, D_out, c);
                double g = gates ? gates[f] : 1.0;
                double *o = grouped_in ? dx + r * D_in : dx + t * D_in;
                for (int64_t i = 0; i < D_in; ++i) o[i] += g * c[i];
            }
        }
    }
    if (dw) {
        for (int64_t i = 0; i < E * D_in * D_out; ++i) dw[i] = 0.0;
        for (int64_t r = 0; r < n; ++r) {
            int64_t f = src[r], t = f / k, e = ids[f];
            const uint16_t *in = grouped_in ? x + r * D_in : x + t * D_in;
            const uint16_t *d = grouped_out ? dy + r * D_out : dy + t * D_out;
            double g = gates ? gates[f] : 1.0;
            double *we = dw + e * D_in * D_out;
            for (int64_t a = 0; a < D_in; ++a) {
                double xa = g * bf16_to_double(in[a]);
                for (int64_t b = 0; b < D_out; ++b) we[a * D_out + b] += xa * bf16_to_double(d[b]);
            }
        }
    }
    if (dg) {
        for (int64_t f = 0; f < n; ++f) {
            int64_t r = rows[f], t = f / k, e = ids[f];
            const uint16_t *in = grouped_in ? x + r * D_in : x + t * D_in;
            const uint16_t *d = grouped_out ? dy + r * D_out : dy + t * D_out;
            row_times_w(in, w + e * D_in * D_out, D_in, D_out, c);
            double s = 0.0;
            for (int64_t b = 0; b < D_out; ++b) s += bf16_to_double(d[b]) * c[b];
            dg[f] = s;
        }
    }
    free(rows); free(src); free(c);
    return 0;
}

/* ------------------------------------------------------------ ffn bwd -- */

/*
 * Backward of the SwiGLU expert FFN with weighted combine (ScatterMoE Guide,
 * "3. Fused Backward Pass Dynamics" applied to both linears of the expert
 * and to the SwiGLU between them). For route f = t*k + j, expert e, gate g:
 *   a = x W1[e], b = x W3[e], h = SiLU(a) b, y_f = h W2[e]   (forward, fp64)
 *   dy     = g * dout[t]
 *   dg[f]  = <dout[t], y_f>
 *   dh     = dy W2[e]^T
 *   da     = dh * b * SiLU'(a),  SiLU'(a) = s (1 + a (1 - s)),  s = sigma(a)
 *   db     = dh * SiLU(a)
 *   dx[t] += da W1[e]^T + db W3[e]^T          (routes j = 0..k-1 in order)
 *   dW1[e] += x^T da,  dW3[e] += x^T db,  dW2[e] += h^T dy
 *                                             (routes in flat order f)
 * Inputs bf16 bits (dout too); outputs fp64: dx [S, D], dw1 and dw3
 * [E, D, F], dw2 [E, F, D], dg [S, k]. Any output may be NULL.
 */
int oracle_ffn_bwd(const uint16_t *x, const uint16_t *w1, const uint16_t *w3, const uint16_t *w2,
                   const int32_t *ids, const double *weights, const uint16_t *dout, int64_t S, int64_t D,
                   int64_t F, int64_t E, int64_t k, double *dx, double *dw1, double *dw3, double *dw2,
                   double *dg) {
    if (S < 0 || D < 1 || F < 1 || E < 1 || k < 1) return 1;
    double *a = (double *)malloc(sizeof(double) * (size_t)F);
    double *b = (double *)malloc(sizeof(double) * (size_t)F);
    double *h = (double *)malloc(sizeof(double) * (size_t)F);
    double *dh = (double *)malloc(sizeof(double) * (size_t)F);
    double *da = (double *)malloc(sizeof(double) * (size_t)F);
    double *db = (double *)malloc(sizeof(double) * (size_t)F);
    double *y = (double *)malloc(sizeof(double) * (size_t)D);
    double *go = (double *)malloc(sizeof(double) * (size_t)D);
    if (!a || !b || !h || !dh || !da || !db || !y || !go) {
        free(a); free(b); free(h); free(dh); free(da); free(db); free(y); free(go);
        return 2;
    }
    if (dx) for (int64_t i = 0; i < S * D; ++i) dx[i] = 0.0;
    if (dw1) for (int64_t i = 0; i < E * D * F; ++i) dw1[i] = 0.0;
    if (dw3) for (int64_t i = 0; i < E * D * F; ++i) dw3[i] = 0.0;
    if (dw2) for (int64_t i = 0; i < E * F * D; ++i) dw2[i] = 0.0;
    int st = 0;
    for (int64_t t = 0; t < S; ++t) {
        const uint16_t *xr = x + t * D;
        for (int64_t n = 0; n < D; ++n) go[n] = bf16_to_double(dout[t * D + n]);
        for (int64_t j = 0; j < k; ++j) {
            int64_t f = t * k + j, e = ids[f];
            if (e < 0 || e >= E) { st = 1; continue; }
            const uint16_t *w1e = w1 + e * D * F, *w3e = w3 + e * D * F, *w2e = w2 + e * F * D;
            double g = weights[f];
            /* forward of this route */
            for (int64_t c = 0; c < F; ++c) { a[c] = 0.0; b[c] = 0.0; }
            for (int64_t d = 0; d < D; ++d) {
                double xv = bf16_to_double(xr[d]);
                for (int64_t c = 0; c < F; ++c) {
                    a[c] += xv * bf16_to_double(w1e[d * F + c]);
                    b[c] += xv * bf16_to_double(w3e[d * F + c]);
                }
            }
            for (int64_t c = 0; c < F; ++c) h[c] = silu(a[c]) * b[c];
            if (dg) {
                for (int64_t n = 0; n < D; ++n) y[n] = 0.0;
                for (int64_t c = 0; c < F; ++c)
                    for (int64_t n = 0; n < D; ++n) y[n] += h[c] * bf16_to_double(w2e[c * D + n]);
                double s = 0.0;
                for (int64_t n = 0; n < D; ++n) s += go[n] * y[n];
                dg[f] = s;
            }
            /* dh = (g dout) W2^T, then through the SwiGLU */
            for (int64_t c = 0; c < F; ++c) {
                double s = 0.0;
                for (int64_t n = 0; n < D; ++n) s += g * go[n] * bf16_to_double(w2e[c * D + n]);
                dh[c] = s;
            }
            for (int64_t c = 0; c < F; ++c) {
                double sg = 1.0 / (1.0 + exp(-a[c]));
                da[c] = dh[c] * b[c] * sg * (1.0 + a[c] * (1.0 - sg));
                db[c] = dh[c] * silu(a[c]);
            }
            if (dx) {
                for (int64_t d = 0; d < D; ++d) {
                    double s = 0.0;
                    for (int64_t c = 0; c < F; ++c)
                        s += da[c] * bf16_to_double(w1e[d * F + c]) + db[c] * bf16_to_double(w3e[d * F + c]);
                    dx[t * D + d] += s;
                }
            }
            if (dw1 || dw3) {
                for (int64_t d = 0; d < D; ++d) {
                    double xv = bf16_to_double(xr[d]);
                    for (int64_t c = 0; c < F; ++c) {
                        if (dw1) dw1[e * D * F + d * F + c] += xv * da[c];
                        if (dw3) dw3[e * D * F + d * F + c] += xv * db[c];
                    }
                }
            }
            if (dw2) {
                for (int64_t c = 0; c < F; ++c)
                    for (int64_t n = 0; n < D; ++n) dw2[e * F * D + c * D + n] += h[c] * g * go[n];
            }
        }
    }
    free(a); free(b); free(h); free(dh); free(da); free(db); free(y); free(go);
    return st;
}
