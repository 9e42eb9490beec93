/*
 * diffuser.h -- C ABI of the MI355X (gfx950) Diffuser attention-diffusion
 * library.
 *
 * The library computes, on one GPU, the Diffuser hot path:
 *   1. a static sparse token graph: a local window of radius r, g global
 *      positions with full rows and columns, and up to R random extra keys
 *      per token ("Diffuser" reading notes, section 2.2 connection table;
 *      "1.2.1 Static sparsity", section 1.1 eq. 5 and section 1.2 eq. 12;
 *      "038 BigBird", section 2, union neighbourhood S_i = W_i u R_i u G);
 *   2. edge scores s_ij = q_i . k_j / sqrt(d_h) on graph edges only and a
 *      softmax over each row's neighbour set into A ("Diffuser" notes,
 *      section 2.1, eqs. S.1-S.5; "1.2.1", section 1, eqs. 1-3);
 *   3. K personalized-PageRank steps Z_0 = V,
 *      Z_{k+1} = (1 - alpha) A Z_k + alpha V, 0 <= k < K, reusing the same
 *      A in every step ("Diffuser" notes, section 2.4, eq. S.7).
 *
 * General conventions
 *  - Every entry point returns a diffuser_status. Nothing is thrown, no
 *    entry point aborts or exits. On a non-OK status,
 *    diffuser_last_error() returns a thread-local message.
 *  - Arguments are validated synchronously, before any GPU work is
 *    enqueued; an invalid call has no side effects.
 *  - "stream" is a hipStream_t passed as void* (NULL = the null stream).
 *    Compute entry points only enqueue work on it; kernel faults surface at
 *    the caller's next synchronisation. Launch failures are reported as
 *    DIFFUSER_ERR_HIP.
 *  - Device pointers are plain device addresses owned by the caller unless
 *    stated otherwise; tensors are dense and row-major.
 *  - Floating-point storage is fp32 or bf16 (round-to-nearest-even); all
 *    accumulation is fp32.
 */
#ifndef DIFFUSER_H
#define DIFFUSER_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define DIFFUSER_API __attribute__((visibility("default")))
#else
#define DIFFUSER_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DIFFUSER_OK = 0,
    DIFFUSER_ERR_INVALID_ARG = 1,   /* bad size, pointer, alignment, range */
    DIFFUSER_ERR_UNSUPPORTED = 2,   /* valid but not implemented (d, dtype) */
    DIFFUSER_ERR_OUT_OF_MEMORY = 3, /* device allocation failed (build only) */
    DIFFUSER_ERR_HIP = 4,           /* a HIP runtime call or launch failed */
    DIFFUSER_ERR_INTERNAL = 5       /* e.g. random-draw budget exhausted */
} diffuser_status;

typedef enum { DIFFUSER_F32 = 0, DIFFUSER_BF16 = 1 } diffuser_dtype;

/*
 * Graph descriptor ("Diffuser" notes, section 2.2; "1.2.1", eqs. 5 and 12;
 * "038 BigBird", section 2). For each graph b < num_graphs and row i < n:
 *  - i global:   N(i) = {0, ..., n-1};
 *  - otherwise:  N(i) = W(i) u G u Rnd(i), W(i) = [max(0, i-r), min(n-1, i+r)],
 *    Rnd(i) = min(R, P) distinct positions drawn uniformly from the pool
 *    {0..n-1} minus (W(i) u G) of size P (the whole pool when P <= R);
 *  - causal:     afterwards keep only j <= i (the draws are made on the
 *    bidirectional pool, so the causal graph is a subgraph of it).
 * The draws: u_t = SplitMix64 output number (c + 1) of a generator seeded
 * with `seed`, where c = ((b*n + i) << 20) | t; the candidate is
 * j = ((u_t >> 32) * n) >> 32; a candidate is accepted when it is in the
 * pool and not yet taken; t runs 0, 1, ... below 2^20 (else
 * DIFFUSER_ERR_INTERNAL).
 * Rows are stored in CSR with strictly ascending columns; every row holds
 * its own index (self edge).
 */
typedef struct {
    int64_t n;                 /* tokens, 1 <= n <= 2^24 */
    int32_t window_radius;     /* r >= 0 */
    int32_t num_global;        /* g, 0 <= g <= n */
    const int32_t* global_idx; /* HOST pointer, g strictly increasing in [0, n) */
    int32_t num_random;        /* R >= 0; R <= 1024 unless every pool <= R */
    int32_t num_graphs;        /* >= 1; graph of batch element b is b when
                                  num_graphs == B, else graph 0 */
    int32_t causal;            /* 0 or 1 */
    uint64_t seed;
} diffuser_graph_desc;

/* Opaque, library-owned, immutable after build. Holds device CSR
 * (row_ptr int64[num_graphs][n+1], col_idx int32[sum of nnz]) and per-row
 * metadata. */
typedef struct diffuser_graph diffuser_graph;

/* Builds the graphs on the current HIP device. The call synchronises
 * `stream` before returning; the graph may then be used on any stream of
 * that device. *out receives the handle (unchanged on error). */
DIFFUSER_API diffuser_status diffuser_build_graph(const diffuser_graph_desc* desc, void* stream,
                                     diffuser_graph** out);

/* Layouts of the extras Rnd(i). */
enum {
    DIFFUSER_EXTRAS_RANDOM = 0,   /* the seeded uniform draws above */
    DIFFUSER_EXTRAS_EVEN = 1      /* evenly spaced ("w uni.", "Diffuser" notes section 4.5,
                                     table S.7): the pool members of rank
                                     floor(q * P / R), q = 0 .. R - 1, in ascending order;
                                     the whole pool when P <= R; seed unused */
};

/* As diffuser_build_graph, with the extras in `layout`
 * (DIFFUSER_EXTRAS_RANDOM or DIFFUSER_EXTRAS_EVEN; anything else gives
 * DIFFUSER_ERR_INVALID_ARG). diffuser_build_graph is layout RANDOM. */
DIFFUSER_API diffuser_status diffuser_build_graph_layout(const diffuser_graph_desc* desc,
                                            int32_t layout, void* stream,
                                            diffuser_graph** out);

/* Imports caller-given CSR graphs (HOST arrays): row_ptr int64
 * [num_graphs][n+1] with each graph's row_ptr starting at 0, col_idx int32
 * = the graphs' columns concatenated. Each row must be strictly ascending,
 * in [0, n), and contain its own index. Used for arbitrary layouts (no
 * window metadata); synchronous like diffuser_build_graph. */
DIFFUSER_API diffuser_status diffuser_graph_from_csr(int64_t n, int32_t num_graphs, const int64_t* row_ptr_host,
                                        const int32_t* col_idx_host, void* stream,
                                        diffuser_graph** out);

/* BigBird block graph ("1.2.1 Static sparsity", section 2, eq. 13): the
 * sequence splits into N = n / block blocks. Query block I < num_global_blocks
 * reads every key block; any other reads the local blocks I - h .. I + h
 * (h = (local_blocks - 1) / 2, clipped to [0, N)), the global blocks
 * 0 .. num_global_blocks - 1, and num_random_blocks random blocks drawn
 * from the others (draw t of block I of graph b: SplitMix64 at counter
 * ((b N + I) << 20 | t), block (u >> 32) N >> 32, kept if new; all others
 * when at most num_random_blocks remain). Every token of a query block reads
 * every token of its key blocks; rows are ascending, so each row's weight
 * slots are its key blocks' columns in order. Constraints: block >= 1
 * divides n, local_blocks odd >= 1, 0 <= num_global_blocks <= N,
 * num_random_blocks >= 0, num_graphs >= 1 (graph of batch element b as in
 * diffuser_graph_desc). Built on the host, then imported as by
 * diffuser_graph_from_csr (synchronous). With block == 64 the bf16, d = 64
 * score and diffusion entry points run block-tile kernels on it. */
typedef struct {
    int64_t n;
    int32_t block;
    int32_t local_blocks;
    int32_t num_random_blocks;
    int32_t num_global_blocks;
    int32_t num_graphs;
    uint64_t seed;
} diffuser_block_graph_desc;

DIFFUSER_API diffuser_status diffuser_build_block_graph(const diffuser_block_graph_desc* desc,
                                                        void* stream, diffuser_graph** out);

/* Longformer dilated window with global positions ("1.2.1 Static sparsity",
 * section 1.2, eqs. 11 and 12): row i not in G reads {i + k dilation :
 * -radius <= k <= radius} within [0, n) plus G; a row in G reads every
 * position. global_idx is a HOST array of num_global strictly increasing
 * positions in [0, n); radius >= 0, dilation >= 1. One graph; built on the
 * host and imported as by diffuser_graph_from_csr (synchronous). */
DIFFUSER_API diffuser_status diffuser_build_dilated_graph(int64_t n, int32_t radius,
                                                          int32_t dilation, int32_t num_global,
                                                          const int32_t* global_idx, void* stream,
                                                          diffuser_graph** out);

/* n, num_graphs, nnz[num_graphs] edges per graph and slots[num_graphs]
 * weight slots per graph (see diffuser_graph_copy_slots). Any output
 * pointer may be NULL. */
DIFFUSER_API diffuser_status diffuser_graph_info(const diffuser_graph* g, int64_t* n,
                                                 int32_t* num_graphs, int64_t* nnz,
                                                 int64_t* slots);

/* Copies graph `graph` to HOST arrays row_ptr[n+1] and col_idx[nnz];
 * synchronous on return. */
DIFFUSER_API diffuser_status diffuser_graph_copy_csr(const diffuser_graph* g, int32_t graph,
                                        int64_t* row_ptr_host, int32_t* col_idx_host,
                                        void* stream);

/* Copies the weight-slot layout of graph `graph` (where A holds its edge
 * weights) to HOST arrays slot_row[slots] and slot_col[slots]: slot s holds
 * the weight of edge (slot_row[s], slot_col[s]); both are -1 for a padding
 * slot, whose weight is always 0. Every edge of the graph owns exactly one
 * slot. An imported graph's slots are its CSR entries. A built graph's
 * slots are, first, one segment per row, each a multiple of 8 slots: a
 * global row's columns in order; for any other row the window as 8-column
 * blocks from (lo & ~7), then the g globals in order (padding where a
 * global lies in the window or, when causal, above the row), then, for
 * n > 65536 only, its random columns in ascending order. The random edges
 * of shorter sequences follow all row segments:
 *  - n <= 4576: one area per block of 16 rows, in block order, of
 *    8 * 16 * noct slots, noct = ceil(most random edges of the block's
 *    rows / 8): random edge e (ascending column) of row m of the block at
 *    ((e / 8) * 16 + m) * 8 + e % 8; the rest is padding;
 *  - 4576 < n <= 65536: in schedule order: for each block of 16 rows and
 *    each 512-key chunk, the block's random edges into the chunk, by row and
 *    then column, two of one row per pair, 16 pairs per 32-slot group.
 * Synchronous on return. */
DIFFUSER_API diffuser_status diffuser_graph_copy_slots(const diffuser_graph* g, int32_t graph,
                                                       int32_t* slot_row_host,
                                                       int32_t* slot_col_host, void* stream);

/* Frees the graph (waits for the device first). Accepts NULL. */
DIFFUSER_API void diffuser_graph_destroy(diffuser_graph* g);

/* Size in bytes of the workspace diffuser_attn needs (A, one Z buffer, the
 * row scales and, on block graphs, the block step's partial sums, each
 * 256-byte aligned). diffuser_scores_softmax needs none and
 * diffuser_diffuse(_theta) what diffuser_diffuse_workspace_size returns;
 * this size is accepted by all of them. */
DIFFUSER_API diffuser_status diffuser_attn_workspace_size(const diffuser_graph* g, int32_t B, int32_t H,
                                             int32_t d_h, int32_t d_v, diffuser_dtype dtype,
                                             size_t* bytes);

/*
 * Layouts shared by the compute entry points:
 *  Q, K : [B][H][n][d_h];  V, Z : [B][H][n][d_v];  all of `dtype`.
 *  A    : edge weights in the graph's weight-slot layout
 *         (diffuser_graph_copy_slots), concatenated over (b, h) in row-major
 *         (b, h) order; the block of (b, h) holds slots(graph(b)) values
 *         and starts at sum_{b' < b} H * slots(graph(b')) +
 *         h * slots(graph(b)). Padding slots hold 0.
 * Supported: d_h, d_v in {16, 32, 64, 128}; pointers 16-byte aligned
 * (A: element aligned); Z must not overlap Q, K, V, A or the workspace.
 */

/* Whole path: scores and edge softmax into A (in the workspace), then
 * K_steps diffusion steps; writes Z = Z_K. K_steps >= 0 (0 copies V),
 * 0 <= alpha <= 1. No allocation is made. The call enqueues only kernel
 * launches (and, at K_steps = 0, one device-to-device copy) on `stream`,
 * with no memset and no host synchronisation, so it may be captured into
 * a HIP graph and replayed; diffuser_attn_theta is the same. */
DIFFUSER_API diffuser_status diffuser_attn(const void* Q, const void* K, const void* V, diffuser_dtype dtype,
                              int32_t B, int32_t H, int32_t d_h, int32_t d_v,
                              const diffuser_graph* g, int32_t K_steps, float alpha, void* Z,
                              void* workspace, size_t ws_bytes, void* stream);

/* Stage 1 alone ("Diffuser" notes, section 2.1, eqs. S.1-S.5): A_out gets
 * the edge-softmax weights in the A layout above. */
DIFFUSER_API diffuser_status diffuser_scores_softmax(const void* Q, const void* K, diffuser_dtype dtype,
                                        int32_t B, int32_t H, int32_t d_h,
                                        const diffuser_graph* g, void* A_out, void* workspace,
                                        size_t ws_bytes, void* stream);

/* Stage 2 alone ("Diffuser" notes, section 2.4, eq. S.7): K_steps
 * diffusion steps with caller-given edge weights A (A layout above; rows
 * need not sum to one). */
DIFFUSER_API diffuser_status diffuser_diffuse(const void* A, const void* V, diffuser_dtype dtype, int32_t B,
                                 int32_t H, int32_t d_v, const diffuser_graph* g,
                                 int32_t K_steps, float alpha, void* Z, void* workspace,
                                 size_t ws_bytes, void* stream);

/* Size in bytes of the workspace diffuser_diffuse and diffuser_diffuse_theta
 * need for K_steps steps on g: one Z buffer when K_steps >= 2, plus, on
 * block graphs ("1.2.1 Static sparsity", section 2, eq. 13) whose global
 * query blocks are split over workgroups, the fp32 partial sums of the block
 * step. 0 means workspace may be NULL. The figure covers both entry points
 * (diffuser_diffuse_theta launches one step even at K_steps = 0); a smaller
 * ws_bytes gives DIFFUSER_ERR_INVALID_ARG before any launch. */
DIFFUSER_API diffuser_status diffuser_diffuse_workspace_size(const diffuser_graph* g, int32_t B,
                                                             int32_t H, int32_t d_v,
                                                             int32_t K_steps,
                                                             diffuser_dtype dtype, size_t* bytes);

/* diffuser_diffuse without a workspace argument, for callers that cannot
 * allocate device memory or pass one in (code under HIP graph capture,
 * tight serving loops). Arguments, layouts and results as for
 * diffuser_diffuse. The Z ping-pong buffer and the block step's partial
 * sums live in a 64 MiB device array inside the library, one per GPU,
 * held until the process ends; none of it needs to start at zero. A call
 * whose diffuser_diffuse_workspace_size exceeds 64 MiB (K_steps >= 2 with
 * B * H * n * d_v * element size above it) gets DIFFUSER_ERR_INVALID_ARG
 * before any launch. The call allocates nothing. Calls that overlap on one
 * GPU (on different streams, or from several threads) share that array
 * and race; serialise them. */
DIFFUSER_API diffuser_status diffuser_diffuse_noalloc(const void* A, const void* V,
                                                      diffuser_dtype dtype, int32_t B, int32_t H,
                                                      int32_t d_v, const diffuser_graph* g,
                                                      int32_t K_steps, float alpha, void* Z,
                                                      void* stream);

/*
 * General diffusion coefficients ("Diffuser" notes, section 2.3, eq. S.6,
 * the series taken through A^K): Z = sum_{k=0..K_steps} theta[k] A^k V.
 * theta: host array of K_steps + 1 floats, each finite and >= 0, summing to
 * 1 within 1e-5 (otherwise DIFFUSER_ERR_INVALID_ARG); it is read before the
 * call returns. PPR is the case theta[k] = alpha (1 - alpha)^k for k < K,
 * theta[K] = (1 - alpha)^K. Evaluated in nested form, U_K = theta[K] V,
 * U_k = theta[k] V + A U_{k+1}, Z = U_0: K_steps launches of the diffusion
 * step (one for K_steps = 0), rounding U_k to `dtype` after each.
 * Arguments, layouts, workspace, ownership and errors as for diffuser_attn
 * and diffuser_diffuse.
 */
DIFFUSER_API diffuser_status diffuser_attn_theta(const void* Q, const void* K, const void* V,
                                    diffuser_dtype dtype, int32_t B, int32_t H, int32_t d_h,
                                    int32_t d_v, const diffuser_graph* g, int32_t K_steps,
                                    const float* theta, void* Z, void* workspace,
                                    size_t ws_bytes, void* stream);
DIFFUSER_API diffuser_status diffuser_diffuse_theta(const void* A, const void* V, diffuser_dtype dtype,
                                       int32_t B, int32_t H, int32_t d_v,
                                       const diffuser_graph* g, int32_t K_steps,
                                       const float* theta, void* Z, void* workspace,
                                       size_t ws_bytes, void* stream);

/*
 * Edge weights in CSR order. A_csr holds, for each (b, h) in row-major
 * order, the weights of graph(b)'s edges in the order of its CSR
 * (diffuser_graph_copy_csr: rows ascending, each row's columns ascending),
 * nnz(graph(b)) values, the block of (b, h) starting at
 * sum_{b' < b} H * nnz(graph(b')) + h * nnz(graph(b)); `dtype` elements,
 * element aligned. This is the order in which the "Diffuser" notes write
 * each row's neighbourhood: the softmax over N(i) (section 2.1,
 * eqs. S.1-S.5) and the sum over N(i) of one diffusion step (section 2.4,
 * eq. S.7). The entry points below compute exactly what
 * diffuser_scores_softmax and diffuser_diffuse compute, with A moved
 * between CSR order and the weight-slot layout by a permutation kernel
 * (bits moved, no arithmetic).
 *
 * The first call on a graph builds its slot -> CSR map (4 bytes per slot,
 * device memory owned by the graph, freed with it; built once, under a
 * lock, synchronising `stream`); later calls enqueue only kernel launches.
 * Graphs must have fewer than 2^31 edges each.
 *
 * diffuser_csr_workspace_size: bytes of workspace that both entry points
 * accept for K_steps steps at width d: the weights in the slot layout
 * (256-byte aligned), then what diffuser_diffuse needs.
 * diffuser_scores_softmax_csr: scores and edge softmax into A_csr; the
 * workspace (at least the slot-layout weights) receives the slot layout.
 * A_csr must not overlap Q, K or the workspace.
 * diffuser_diffuse_csr: K_steps diffusion steps with caller-given weights
 * A_csr (rows need not sum to one); writes Z as diffuser_diffuse does.
 * A_csr, V and Z must not overlap the workspace; Z not A_csr or V.
 * Errors as for diffuser_diffuse; a smaller ws_bytes gives
 * DIFFUSER_ERR_INVALID_ARG before any launch.
 */
DIFFUSER_API diffuser_status diffuser_csr_workspace_size(const diffuser_graph* g, int32_t B,
                                                         int32_t H, int32_t d, int32_t K_steps,
                                                         diffuser_dtype dtype, size_t* bytes);
DIFFUSER_API diffuser_status diffuser_scores_softmax_csr(const void* Q, const void* K,
                                                         diffuser_dtype dtype, int32_t B,
                                                         int32_t H, int32_t d_h,
                                                         const diffuser_graph* g, void* A_csr,
                                                         void* workspace, size_t ws_bytes,
                                                         void* stream);
DIFFUSER_API diffuser_status diffuser_diffuse_csr(const void* A_csr, const void* V,
                                                  diffuser_dtype dtype, int32_t B, int32_t H,
                                                  int32_t d_v, const diffuser_graph* g,
                                                  int32_t K_steps, float alpha, void* Z,
                                                  void* workspace, size_t ws_bytes, void* stream);

/*
 * Backward of diffuser_attn (the chain rule through the recurrence of
 * "Diffuser" notes section 2.4, eq. S.7, the edge softmax of section 2.1,
 * eqs. S.1-S.5, and the scores): given dZ = dL/dZ, writes dQ, dK, dV (the
 * gradients of L through Z). Q, K, V, dZ, dQ, dK, dV: [B][H][n][d] of
 * `dtype` (d_h = d_v = d); accumulation and every intermediate are fp32.
 * The workspace (size from diffuser_attn_backward_workspace_size, about
 * (3 slots + (2 K_steps + 2) n d) * 4 bytes per (b, h)) holds A, dA, the
 * weights in column order, the states Z_0 .. Z_{K-1}, the backward states
 * G_0 .. G_K and dV. The first call on a
 * graph builds its column index (device memory owned by the graph, freed
 * with it; built once, under a lock, synchronising `stream`). Later calls
 * enqueue only kernel launches, with no memset and no host synchronisation,
 * so they may be captured into a HIP graph. Outputs must not overlap
 * inputs, each other or the workspace. Errors as for diffuser_attn.
 */
DIFFUSER_API diffuser_status diffuser_attn_backward_workspace_size(const diffuser_graph* g, int32_t B,
                                                      int32_t H, int32_t d, int32_t K_steps,
                                                      diffuser_dtype dtype, size_t* bytes);
DIFFUSER_API diffuser_status diffuser_attn_backward(const void* Q, const void* K, const void* V,
                                        const void* dZ, diffuser_dtype dtype, int32_t B,
                                        int32_t H, int32_t d, const diffuser_graph* g,
                                        int32_t K_steps, float alpha, void* dQ, void* dK,
                                        void* dV, void* workspace, size_t ws_bytes,
                                        void* stream);

/*
 * One attention layer around the path ("Diffuser" notes section 2.1: the
 * per-head Q, K, V of the input; section 2.4: head concatenation and the
 * output projection outside the diffusion module):
 *   [Q | K | V] = X W_qkv, Z = diffuser_attn(Q, K, V), Y = concat_h(Z) W_o.
 * X: [B][n][d_model]; W_qkv: [d_model][3 H d], columns p H d + h d + c give
 * channel c of head h of Q (p = 0), K (1), V (2); W_o: [H d][d_model];
 * Y: [B][n][d_model]; all of `dtype`, row-major, 16-byte aligned. The two
 * products are dense GEMMs with fp32 accumulation (rocBLAS, on a handle the
 * library creates once per device; calls sharing a device are serialised
 * through it). The workspace (size from diffuser_layer_workspace_size)
 * holds the projections, Q, K, V, Z, the path's own workspace and the GEMM
 * library's workspace; no other memory is allocated by the call after the
 * handle exists. Y must not overlap the inputs or the workspace. Errors as
 * for diffuser_attn; a GEMM failure gives DIFFUSER_ERR_INTERNAL.
 */
DIFFUSER_API diffuser_status diffuser_layer_workspace_size(const diffuser_graph* g, int32_t B,
                                              int32_t H, int32_t d, int32_t d_model,
                                              diffuser_dtype dtype, size_t* bytes);
DIFFUSER_API diffuser_status diffuser_layer_forward(const void* X, const void* W_qkv,
                                       const void* W_o, diffuser_dtype dtype, int32_t B,
                                       int32_t H, int32_t d, int32_t d_model,
                                       const diffuser_graph* g, int32_t K_steps, float alpha,
                                       void* Y, void* workspace, size_t ws_bytes,
                                       void* stream);

/* Static string for a status code. */
DIFFUSER_API const char* diffuser_status_string(diffuser_status s);

/* Thread-local message describing the last non-OK status returned on this
 * thread ("" if none). */
DIFFUSER_API const char* diffuser_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DIFFUSER_H */
