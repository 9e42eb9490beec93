/*
 * Diffuser CPU oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, double-precision CPU implementation of what the Diffuser
 * attention-diffusion path computes. Only the test suite, the smoke check and
 * the CPU-baseline leg of the benchmark may load it; the product path never
 * does. It shares no code, header, table or helper with the HIP library.
 *
 * Sources (cited by page title and section):
 *  - "Diffuser: modelling long sequences with multi-hop attention diffusion"
 *    reading notes, section 2.1 (edge-restricted softmax, eqs. S.1-S.5),
 *    section 2.2 (local window / global / random connection table),
 *    section 2.3 (diffusion operator with general coefficients, eq. S.6),
 *    section 2.4 (PPR recurrence, eq. S.7), section 2.5 (finite-K expansion),
 *    section 4.5 / table S.7 (the "w uni." evenly spaced extras).
 *  - "1.2.1 Static sparsity: Longformer, BigBird and sliding windows",
 *    section 1 (score eq. 1, mask eq. 2, normalisation eqs. 3-4),
 *    section 1.1 (window eq. 5), section 1.2 (global neighbourhood eq. 12).
 *  - "038 BigBird", section 2 (union neighbourhood S_i = W_i u R_i u G).
 *  - Random draws: SplitMix64 (Steele, Lea & Flood, OOPSLA 2014) with the
 *    multiply-shift range map (Lemire 2019); the draw schedule is this
 *    project's own (the pages fix no generator).
 *
 * Conventions: all indices 0-based; Q, K are [n][d] row-major, V and Z are
 * [n][d] row-major; A is in CSR order (row_ptr/col_idx). Every function
 * returns 0 on success and a negative code on bad arguments:
 *   -1 invalid argument, -2 random draw budget (2^20 draws per row) exhausted.
 */
#ifndef DIFFUSER_ORACLE_H
#define DIFFUSER_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* SplitMix64 output function (finaliser) applied to z. */
uint64_t oracle_mix64(uint64_t z);

/* The t-th random draw for row i of graph b:
 * mix64(seed + 0x9E3779B97F4A7C15 * ((((b*n + i) << 20) | t) + 1)). */
uint64_t oracle_draw(uint64_t seed, int64_t b, int64_t n, int64_t i, int64_t t);

/* Number of edges of each graph (nnz_out[num_graphs]).
 * global_idx: strictly increasing positions in [0, n). */
int oracle_graph_nnz(int64_t n, int32_t radius, int32_t num_global,
                     const int32_t* global_idx, int32_t num_random,
                     int32_t num_graphs, int32_t causal, uint64_t seed,
                     int64_t* nnz_out);

/* Builds all graphs: row_ptr[num_graphs][n+1] (each graph's row_ptr starts
 * at 0) and col_idx = concatenation of each graph's columns (graph gr starts
 * at the sum of the nnz of graphs < gr). */
int oracle_graph_build(int64_t n, int32_t radius, int32_t num_global,
                       const int32_t* global_idx, int32_t num_random,
                       int32_t num_graphs, int32_t causal, uint64_t seed,
                       int64_t* row_ptr, int32_t* col_idx);

/* The same two with the extras' layout: 0 = seeded random draws (above),
 * 1 = evenly spaced ("w uni.", "Diffuser" notes section 4.5, table S.7):
 * row i takes the pool members of rank floor(q * P / R), q = 0 .. R - 1,
 * P = |pool(i)| (all of the pool when P <= R); the seed is not used. */
int oracle_graph_nnz_layout(int64_t n, int32_t radius, int32_t num_global,
                            const int32_t* global_idx, int32_t num_random, int32_t num_graphs,
                            int32_t causal, uint64_t seed, int32_t layout, int64_t* nnz_out);
int oracle_graph_build_layout(int64_t n, int32_t radius, int32_t num_global,
                              const int32_t* global_idx, int32_t num_random, int32_t num_graphs,
                              int32_t causal, uint64_t seed, int32_t layout, int64_t* row_ptr,
                              int32_t* col_idx);

/* Edge scores and edge softmax for one (batch, head):
 * A[e] = exp(s_e - m_i) / sum_u exp(s_u - m_i), s_e = q_i . k_j / sqrt(d). */
int oracle_scores_softmax(const double* Q, const double* K, int64_t n, int32_t d,
                          const int64_t* row_ptr, const int32_t* col_idx,
                          double* A_out, int32_t threads);

/* Raw edge scores s_e = q_i . k_j / sqrt(d) (stage diagnostic). */
int oracle_scores(const double* Q, const double* K, int64_t n, int32_t d,
                  const int64_t* row_ptr, const int32_t* col_idx,
                  double* S_out, int32_t threads);

/* K steps of Z_{k+1} = (1 - alpha) A Z_k + alpha V from Z_0 = V. */
int oracle_diffuse(const double* A, const double* V, int64_t n, int32_t d,
                   const int64_t* row_ptr, const int32_t* col_idx,
                   int32_t K_steps, double alpha, double* Z_out, int32_t threads);

/* Z = sum_{k=0..K} theta[k] A^k V (theta has K_steps + 1 entries). */
int oracle_diffuse_theta(const double* A, const double* V, int64_t n, int32_t d,
                         const int64_t* row_ptr, const int32_t* col_idx,
                         int32_t K_steps, const double* theta, double* Z_out,
                         int32_t threads);

/* Gradients of sum(dZ * Z) for the whole path of one (batch, head) (scores,
 * edge softmax, K_steps PPR steps): dQ, dK [n][d], dV [n][d]. */
int oracle_attn_backward(const double* Q, const double* K, const double* V, const double* dZ,
                         int64_t n, int32_t d, const int64_t* row_ptr, const int32_t* col_idx,
                         int32_t K_steps, double alpha, double* dQ, double* dK, double* dV);

#ifdef __cplusplus
}
#endif

#endif
