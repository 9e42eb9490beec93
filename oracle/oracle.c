/*
 * Diffuser CPU oracle -- TEST INFRASTRUCTURE ONLY (see oracle.h).
 *
 * Every function follows a definition on the pages directly, in double
 * precision, with no blocking, fusion or reordering beyond what the
 * definition states. Row loops may be split over threads; each row's sums
 * are taken by one thread in ascending column order, so the result does not
 * depend on the thread count.
 */
#include "oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Random draws: SplitMix64 (Steele, Lea & Flood 2014).                     */
/* ------------------------------------------------------------------------ */

uint64_t oracle_mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

/* The counter (b*n + i, t) is packed as ((b*n + i) << 20) | t; the draw is
 * the (counter + 1)-th SplitMix64 output of a generator seeded with seed. */
uint64_t oracle_draw(uint64_t seed, int64_t b, int64_t n, int64_t i, int64_t t) {
    uint64_t ctr = (((uint64_t)(b * n + i)) << 20) | (uint64_t)t;
    return oracle_mix64(seed + 0x9E3779B97F4A7C15ull * (ctr + 1ull));
}

#define ORACLE_MAX_DRAWS (1ll << 20)

/* ------------------------------------------------------------------------ */
/* Graph: N(i) = W(i) u G u Rnd(i) for i not global; N(i) = all for i in G. */
/* ------------------------------------------------------------------------ */

typedef struct {
    int64_t n;
    int32_t radius;
    int32_t num_global;
    const int32_t* global_idx;
    const unsigned char* is_global; /* [n] */
    int32_t num_random;
    int32_t causal;
    uint64_t seed;
    int32_t layout;   /* 0: seeded random extras; 1: evenly spaced extras */
} graph_spec;

/* Marks N(i) of graph gr in member[0..n) (1 = window or global, 2 = random)
 * and returns 0, or -2 when the draw budget is exhausted. member must be all
 * zero on entry. */
static int mark_row(const graph_spec* s, int64_t gr, int64_t i, unsigned char* member) {
    const int64_t n = s->n;
    if (s->is_global[i]) {
        /* A global position reads every position (page "1.2.1", eq. 12). */
        memset(member, 1, (size_t)n);
        return 0;
    }
    /* Local window |i - j| <= r (page "1.2.1", eq. 5). */
    int64_t lo = i - s->radius < 0 ? 0 : i - s->radius;
    int64_t hi = i + s->radius > n - 1 ? n - 1 : i + s->radius;
    for (int64_t j = lo; j <= hi; ++j) member[j] = 1;
    /* Every position reads every global position (eq. 12). */
    for (int32_t k = 0; k < s->num_global; ++k) member[s->global_idx[k]] = 1;
    /* Random edges: num_random distinct positions outside window and globals. */
    int64_t pool = 0;
    for (int64_t j = 0; j < n; ++j) pool += member[j] == 0;
    if (pool <= s->num_random) {
        for (int64_t j = 0; j < n; ++j)
            if (member[j] == 0) member[j] = 2;
        return 0;
    }
    if (s->layout == 1) {
        /* Evenly spaced extras ("w uni."): pool members number q * pool / R
         * (q = 0 .. R - 1) in ascending order of the pool. */
        int64_t q = 0, rank = 0;
        for (int64_t j = 0; j < n && q < s->num_random; ++j) {
            if (member[j] != 0) continue;
            if (rank == q * pool / s->num_random) {
                member[j] = 2;
                ++q;
            }
            ++rank;
        }
        return 0;
    }
    int32_t taken = 0;
    int64_t t = 0;
    while (taken < s->num_random) {
        if (t >= ORACLE_MAX_DRAWS) return -2;
        uint64_t u = oracle_draw(s->seed, gr, n, i, t);
        ++t;
        uint64_t j = ((u >> 32) * (uint64_t)n) >> 32;
        if (member[j] == 0) {
            member[j] = 2;
            ++taken;
        }
    }
    return 0;
}

/* Number of members of N(i), after the causal filter j <= i when enabled. */
static int64_t count_row(const graph_spec* s, int64_t i, const unsigned char* member) {
    int64_t last = s->causal ? i : s->n - 1;
    int64_t c = 0;
    for (int64_t j = 0; j <= last; ++j) c += member[j] != 0;
    return c;
}

typedef struct {
    const graph_spec* spec;
    int64_t gr;
    int64_t row_begin, row_end;
    int64_t* counts;          /* [n] out (count pass) */
    const int64_t* row_ptr;   /* [n+1] in (fill pass) or NULL */
    int32_t* cols;            /* fill pass output (this graph's columns) */
    int status;
} graph_task;

static void* graph_worker(void* arg) {
    graph_task* tk = (graph_task*)arg;
    const graph_spec* s = tk->spec;
    unsigned char* member = (unsigned char*)calloc((size_t)s->n, 1);
    if (!member) {
        tk->status = -1;
        return NULL;
    }
    for (int64_t i = tk->row_begin; i < tk->row_end; ++i) {
        int st = mark_row(s, tk->gr, i, member);
        if (st) {
            tk->status = st;
            break;
        }
        if (tk->row_ptr == NULL) {
            tk->counts[i] = count_row(s, i, member);
        } else {
            int64_t last = s->causal ? i : s->n - 1;
            int64_t e = tk->row_ptr[i];
            for (int64_t j = 0; j <= last; ++j)
                if (member[j]) tk->cols[e++] = (int32_t)j;
        }
        memset(member, 0, (size_t)s->n);
    }
    free(member);
    return NULL;
}

#define ORACLE_GRAPH_THREADS 8

static int run_graph_pass(const graph_spec* s, int64_t gr, int64_t* counts,
                          const int64_t* row_ptr, int32_t* cols) {
    int nt = ORACLE_GRAPH_THREADS;
    if (s->n < 64) nt = 1;
    pthread_t th[ORACLE_GRAPH_THREADS];
    graph_task tk[ORACLE_GRAPH_THREADS];
    for (int t = 0; t < nt; ++t) {
        tk[t].spec = s;
        tk[t].gr = gr;
        tk[t].row_begin = s->n * t / nt;
        tk[t].row_end = s->n * (t + 1) / nt;
        tk[t].counts = counts;
        tk[t].row_ptr = row_ptr;
        tk[t].cols = cols;
        tk[t].status = 0;
    }
    if (nt == 1) {
        graph_worker(&tk[0]);
    } else {
        for (int t = 0; t < nt; ++t) pthread_create(&th[t], NULL, graph_worker, &tk[t]);
        for (int t = 0; t < nt; ++t) pthread_join(th[t], NULL);
    }
    for (int t = 0; t < nt; ++t)
        if (tk[t].status) return tk[t].status;
    return 0;
}

static int make_spec(graph_spec* s, unsigned char** is_global, int64_t n, int32_t radius,
                     int32_t num_global, const int32_t* global_idx, int32_t num_random,
                     int32_t num_graphs, int32_t causal, uint64_t seed, int32_t layout) {
    if (n < 1 || n > (1ll << 31) - 1 || radius < 0 || num_global < 0 || num_global > n ||
        num_random < 0 || num_graphs < 1 || (num_global > 0 && global_idx == NULL) ||
        layout < 0 || layout > 1)
        return -1;
    for (int32_t k = 0; k < num_global; ++k) {
        if (global_idx[k] < 0 || global_idx[k] >= n) return -1;
        if (k > 0 && global_idx[k] <= global_idx[k - 1]) return -1;
    }
    unsigned char* ig = (unsigned char*)calloc((size_t)n, 1);
    if (!ig) return -1;
    for (int32_t k = 0; k < num_global; ++k) ig[global_idx[k]] = 1;
    s->n = n;
    s->radius = radius;
    s->num_global = num_global;
    s->global_idx = global_idx;
    s->is_global = ig;
    s->num_random = num_random;
    s->causal = causal != 0;
    s->seed = seed;
    s->layout = layout;
    *is_global = ig;
    return 0;
}

int oracle_graph_nnz_layout(int64_t n, int32_t radius, int32_t num_global,
                            const int32_t* global_idx, int32_t num_random, int32_t num_graphs,
                            int32_t causal, uint64_t seed, int32_t layout, int64_t* nnz_out) {
    graph_spec s;
    unsigned char* ig = NULL;
    int st = make_spec(&s, &ig, n, radius, num_global, global_idx, num_random, num_graphs,
                       causal, seed, layout);
    if (st) return st;
    int64_t* counts = (int64_t*)malloc(sizeof(int64_t) * (size_t)n);
    if (!counts) {
        free(ig);
        return -1;
    }
    for (int32_t gr = 0; gr < num_graphs && st == 0; ++gr) {
        st = run_graph_pass(&s, gr, counts, NULL, NULL);
        int64_t total = 0;
        for (int64_t i = 0; i < n; ++i) total += counts[i];
        nnz_out[gr] = total;
    }
    free(counts);
    free(ig);
    return st;
}

int oracle_graph_build_layout(int64_t n, int32_t radius, int32_t num_global,
                              const int32_t* global_idx, int32_t num_random, int32_t num_graphs,
                              int32_t causal, uint64_t seed, int32_t layout, int64_t* row_ptr,
                              int32_t* col_idx) {
    graph_spec s;
    unsigned char* ig = NULL;
    int st = make_spec(&s, &ig, n, radius, num_global, global_idx, num_random, num_graphs,
                       causal, seed, layout);
    if (st) return st;
    int64_t* counts = (int64_t*)malloc(sizeof(int64_t) * (size_t)n);
    if (!counts) {
        free(ig);
        return -1;
    }
    int64_t col_base = 0;
    for (int32_t gr = 0; gr < num_graphs && st == 0; ++gr) {
        int64_t* rp = row_ptr + (int64_t)gr * (n + 1);
        st = run_graph_pass(&s, gr, counts, NULL, NULL);
        if (st) break;
        rp[0] = 0;
        for (int64_t i = 0; i < n; ++i) rp[i + 1] = rp[i] + counts[i];
        st = run_graph_pass(&s, gr, NULL, rp, col_idx + col_base);
        col_base += rp[n];
    }
    free(counts);
    free(ig);
    return st;
}

int oracle_graph_nnz(int64_t n, int32_t radius, int32_t num_global, const int32_t* global_idx,
                     int32_t num_random, int32_t num_graphs, int32_t causal, uint64_t seed,
                     int64_t* nnz_out) {
    return oracle_graph_nnz_layout(n, radius, num_global, global_idx, num_random, num_graphs,
                                   causal, seed, 0, nnz_out);
}

int oracle_graph_build(int64_t n, int32_t radius, int32_t num_global, const int32_t* global_idx,
                       int32_t num_random, int32_t num_graphs, int32_t causal, uint64_t seed,
                       int64_t* row_ptr, int32_t* col_idx) {
    return oracle_graph_build_layout(n, radius, num_global, global_idx, num_random, num_graphs,
                                     causal, seed, 0, row_ptr, col_idx);
}

/* ------------------------------------------------------------------------ */
/* Row-parallel helper.                                                     */
/* ------------------------------------------------------------------------ */

typedef void (*row_fn)(void* ctx, int64_t i);

typedef struct {
    row_fn fn;
    void* ctx;
    int64_t begin, end;
} row_task;

static void* row_worker(void* arg) {
    row_task* tk = (row_task*)arg;
    for (int64_t i = tk->begin; i < tk->end; ++i) tk->fn(tk->ctx, i);
    return NULL;
}

static void parallel_rows(row_fn fn, void* ctx, int64_t n, int32_t threads) {
    if (threads <= 1 || n < 2) {
        for (int64_t i = 0; i < n; ++i) fn(ctx, i);
        return;
    }
    if (threads > 256) threads = 256;
    if (threads > n) threads = (int32_t)n;
    pthread_t th[256];
    row_task tk[256];
    for (int32_t t = 0; t < threads; ++t) {
        tk[t].fn = fn;
        tk[t].ctx = ctx;
        tk[t].begin = n * t / threads;
        tk[t].end = n * (t + 1) / threads;
        pthread_create(&th[t], NULL, row_worker, &tk[t]);
    }
    for (int32_t t = 0; t < threads; ++t) pthread_join(th[t], NULL);
}

/* ------------------------------------------------------------------------ */
/* Scores and edge softmax (Diffuser notes section 2.1, eqs. S.1-S.5;      */
/* page "1.2.1" eqs. 1 and 3).                                              */
/* ------------------------------------------------------------------------ */

typedef struct {
    const double* Q;
    const double* K;
    int32_t d;
    const int64_t* row_ptr;
    const int32_t* col_idx;
    double* out;
    int softmax;
} score_ctx;

static void score_row(void* vctx, int64_t i) {
    score_ctx* c = (score_ctx*)vctx;
    const double scale = 1.0 / sqrt((double)c->d);
    const double* q = c->Q + i * c->d;
    int64_t e0 = c->row_ptr[i], e1 = c->row_ptr[i + 1];
    for (int64_t e = e0; e < e1; ++e) {
        const double* k = c->K + (int64_t)c->col_idx[e] * c->d;
        double dot = 0.0;
        for (int32_t ch = 0; ch < c->d; ++ch) dot += q[ch] * k[ch];
        c->out[e] = dot * scale;
    }
    if (!c->softmax || e1 == e0) return;
    /* Normalise over exactly the neighbour set N(i); subtracting the row
     * maximum leaves the exact result unchanged. */
    double m = c->out[e0];
    for (int64_t e = e0 + 1; e < e1; ++e)
        if (c->out[e] > m) m = c->out[e];
    double sum = 0.0;
    for (int64_t e = e0; e < e1; ++e) {
        c->out[e] = exp(c->out[e] - m);
        sum += c->out[e];
    }
    for (int64_t e = e0; e < e1; ++e) c->out[e] /= sum;
}

static int check_csr(int64_t n, int32_t d, const int64_t* row_ptr, const int32_t* col_idx) {
    if (n < 1 || d < 1 || !row_ptr || (!col_idx && row_ptr[n] > 0)) return -1;
    return 0;
}

int oracle_scores_softmax(const double* Q, const double* K, int64_t n, int32_t d,
                          const int64_t* row_ptr, const int32_t* col_idx, double* A_out,
                          int32_t threads) {
    if (check_csr(n, d, row_ptr, col_idx) || !Q || !K || !A_out) return -1;
    score_ctx c = {Q, K, d, row_ptr, col_idx, A_out, 1};
    parallel_rows(score_row, &c, n, threads);
    return 0;
}

int oracle_scores(const double* Q, const double* K, int64_t n, int32_t d,
                  const int64_t* row_ptr, const int32_t* col_idx, double* S_out,
                  int32_t threads) {
    if (check_csr(n, d, row_ptr, col_idx) || !Q || !K || !S_out) return -1;
    score_ctx c = {Q, K, d, row_ptr, col_idx, S_out, 0};
    parallel_rows(score_row, &c, n, threads);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Diffusion: Z_0 = V, Z_{k+1} = (1 - alpha) A Z_k + alpha V, 0 <= k < K    */
/* (Diffuser notes section 2.4, eq. S.7).                                   */
/* ------------------------------------------------------------------------ */

typedef struct {
    const double* A;
    const double* V;
    const double* Zk;
    double* Zn;
    int32_t d;
    double alpha;
    const int64_t* row_ptr;
    const int32_t* col_idx;
} diffuse_ctx;

static void diffuse_row(void* vctx, int64_t i) {
    diffuse_ctx* c = (diffuse_ctx*)vctx;
    double* out = c->Zn + i * c->d;
    for (int32_t ch = 0; ch < c->d; ++ch) out[ch] = 0.0;
    for (int64_t e = c->row_ptr[i]; e < c->row_ptr[i + 1]; ++e) {
        const double a = c->A[e];
        const double* z = c->Zk + (int64_t)c->col_idx[e] * c->d;
        for (int32_t ch = 0; ch < c->d; ++ch) out[ch] += a * z[ch];
    }
    const double* v = c->V + i * c->d;
    for (int32_t ch = 0; ch < c->d; ++ch)
        out[ch] = (1.0 - c->alpha) * out[ch] + c->alpha * v[ch];
}

int oracle_diffuse(const double* A, const double* V, int64_t n, int32_t d,
                   const int64_t* row_ptr, const int32_t* col_idx, int32_t K_steps,
                   double alpha, double* Z_out, int32_t threads) {
    if (check_csr(n, d, row_ptr, col_idx) || !A || !V || !Z_out || K_steps < 0 ||
        !(alpha >= 0.0 && alpha <= 1.0))
        return -1;
    size_t bytes = sizeof(double) * (size_t)n * (size_t)d;
    memcpy(Z_out, V, bytes);
    if (K_steps == 0) return 0;
    double* tmp = (double*)malloc(bytes);
    if (!tmp) return -1;
    for (int32_t k = 0; k < K_steps; ++k) {
        diffuse_ctx c = {A, V, Z_out, tmp, d, alpha, row_ptr, col_idx};
        parallel_rows(diffuse_row, &c, n, threads);
        memcpy(Z_out, tmp, bytes);
    }
    free(tmp);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* General diffusion coefficients: Z = sum_{k=0..K} theta_k A^k V           */
/* (Diffuser notes section 2.3, eq. S.6, the series taken through A^K).     */
/* The powers are applied one at a time: Y_0 = V, Y_{k+1} = A Y_k.          */
/* ------------------------------------------------------------------------ */

int oracle_diffuse_theta(const double* A, const double* V, int64_t n, int32_t d,
                         const int64_t* row_ptr, const int32_t* col_idx, int32_t K_steps,
                         const double* theta, double* Z_out, int32_t threads) {
    if (check_csr(n, d, row_ptr, col_idx) || !A || !V || !Z_out || !theta || K_steps < 0)
        return -1;
    const size_t count = (size_t)n * (size_t)d;
    const size_t bytes = sizeof(double) * count;
    double* y = (double*)malloc(bytes);
    double* next = (double*)malloc(bytes);
    if (!y || !next) {
        free(y);
        free(next);
        return -1;
    }
    memcpy(y, V, bytes);
    for (size_t e = 0; e < count; ++e) Z_out[e] = theta[0] * V[e];
    for (int32_t k = 1; k <= K_steps; ++k) {
        /* next = A y: the step of eq. S.7 with no restart term */
        diffuse_ctx c = {A, V, y, next, d, 0.0, row_ptr, col_idx};
        parallel_rows(diffuse_row, &c, n, threads);
        memcpy(y, next, bytes);
        for (size_t e = 0; e < count; ++e) Z_out[e] += theta[k] * y[e];
    }
    free(y);
    free(next);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Backward of the whole path for one (batch, head): the chain rule through  */
/* the recurrence (eq. S.7), the edge softmax (eqs. S.1-S.5) and the scores. */
/* With G_K = dZ, for k = K-1 .. 0:                                          */
/*   dA_ij += (1 - alpha) G_{k+1}[i] . Z_k[j]   (edges),                     */
/*   dV    += alpha G_{k+1},                                                 */
/*   G_k    = (1 - alpha) A^T G_{k+1};                                       */
/* then dV += G_0 (Z_0 = V), dS_ij = A_ij (dA_ij - sum_u A_iu dA_iu),       */
/* dQ_i = sum_j dS_ij k_j / sqrt(d), dK_j = sum_i dS_ij q_i / sqrt(d).     */
/* Serial; column sums run over edges in CSR order (ascending rows).        */
/* ------------------------------------------------------------------------ */

int oracle_attn_backward(const double* Q, const double* K, const double* V, const double* dZ,
                         int64_t n, int32_t d, const int64_t* row_ptr, const int32_t* col_idx,
                         int32_t K_steps, double alpha, double* dQ, double* dK, double* dV) {
    if (check_csr(n, d, row_ptr, col_idx) || !Q || !K || !V || !dZ || !dQ || !dK || !dV ||
        K_steps < 0 || !(alpha >= 0.0 && alpha <= 1.0))
        return -1;
    const int64_t nnz = row_ptr[n];
    const size_t cnt = (size_t)n * (size_t)d;
    double* A = (double*)malloc(sizeof(double) * (size_t)(nnz > 0 ? nnz : 1));
    double* dA = (double*)calloc((size_t)(nnz > 0 ? nnz : 1), sizeof(double));
    double* Zs = (double*)malloc(sizeof(double) * cnt * (size_t)(K_steps > 0 ? K_steps : 1));
    double* G = (double*)malloc(sizeof(double) * cnt);
    double* Gn = (double*)malloc(sizeof(double) * cnt);
    int st = (A && dA && Zs && G && Gn) ? 0 : -1;
    if (st == 0) st = oracle_scores_softmax(Q, K, n, d, row_ptr, col_idx, A, 1);
    if (st == 0) {
        /* Forward states Z_0 .. Z_{K-1}. */
        if (K_steps > 0) memcpy(Zs, V, sizeof(double) * cnt);
        for (int32_t k = 1; k < K_steps; ++k) {
            diffuse_ctx c = {A, V, Zs + (size_t)(k - 1) * cnt, Zs + (size_t)k * cnt, d, alpha,
                             row_ptr, col_idx};
            parallel_rows(diffuse_row, &c, n, 1);
        }
        memcpy(G, dZ, sizeof(double) * cnt);
        for (size_t e = 0; e < cnt; ++e) dV[e] = 0.0;
        for (int32_t k = K_steps - 1; k >= 0; --k) {
            const double* Zk = Zs + (size_t)k * cnt;
            for (size_t e = 0; e < cnt; ++e) Gn[e] = 0.0;
            for (int64_t i = 0; i < n; ++i) {
                const double* gi = G + i * d;
                for (int64_t e = row_ptr[i]; e < row_ptr[i + 1]; ++e) {
                    const int64_t j = col_idx[e];
                    const double* zj = Zk + j * d;
                    double dot = 0.0;
                    for (int32_t ch = 0; ch < d; ++ch) dot += gi[ch] * zj[ch];
                    dA[e] += (1.0 - alpha) * dot;
                    double* gj = Gn + j * d;
                    for (int32_t ch = 0; ch < d; ++ch) gj[ch] += (1.0 - alpha) * A[e] * gi[ch];
                }
            }
            for (size_t e = 0; e < cnt; ++e) dV[e] += alpha * G[e];
            memcpy(G, Gn, sizeof(double) * cnt);
        }
        for (size_t e = 0; e < cnt; ++e) dV[e] += G[e];
        /* Softmax and score backward. */
        const double scale = 1.0 / sqrt((double)d);
        for (size_t e = 0; e < cnt; ++e) dQ[e] = dK[e] = 0.0;
        for (int64_t i = 0; i < n; ++i) {
            double s = 0.0;
            for (int64_t e = row_ptr[i]; e < row_ptr[i + 1]; ++e) s += A[e] * dA[e];
            for (int64_t e = row_ptr[i]; e < row_ptr[i + 1]; ++e) {
                const double ds = A[e] * (dA[e] - s) * scale;
                const int64_t j = col_idx[e];
                for (int32_t ch = 0; ch < d; ++ch) {
                    dQ[i * d + ch] += ds * K[j * d + ch];
                    dK[j * d + ch] += ds * Q[i * d + ch];
                }
            }
        }
    }
    free(A);
    free(dA);
    free(Zs);
    free(G);
    free(Gn);
    return st;
}
