// Internal declarations shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/diffuser.h"

namespace diffuser {
constexpr int32_t kRowBlock = 16;     // rows per block of the random schedule
constexpr int32_t kChunkRows = 512;   // key rows per chunk of the random schedule
constexpr int32_t kGroupSlots = 32;   // weight slots per schedule group
constexpr uint32_t kZeroRow = kChunkRows;  // key row index of a dummy slot
constexpr int64_t kMaxScheduledN = 1 << 16;
// Largest n whose built graphs keep their random weights in per-row-block
// octet areas (the resident-slice diffusion step's layout): a 16-channel
// slice of every key row (32 bytes each, a zero row after the last) then
// fits in LDS beside the 16 KB of global-row partial sums.
constexpr int64_t kMaxResidentN = 4576;
static_assert(kMaxResidentN < 65535, "resident key-row slots fit 16 bits");
// Rows with more weight slots than this (a global row's n, say) are split
// over the waves of one workgroup by the generic kernels' long-row
// companions instead of walked by one wave.
constexpr int64_t kLongRow = 1024;
// Random octets per batch of the resident-slice step's key table (one
// 16-byte load per lane covers a batch).
constexpr int32_t kOctBatch = 4;
// Bytes of device scratch that diffuser_diffuse_noalloc holds per GPU.
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;

// n rounded up to a multiple of 32: the slot of the zero row of the
// resident-slice layout (every 32-key step of a row block stays below it).
__host__ __device__ constexpr int64_t res_npad(int64_t n) { return (n + 31) & ~31ll; }

// LDS placement of key row `row` (0..kChunkRows) in the score kernel's
// layout, in 16-byte units: unit u of the row sits at unit (code ^ u) with
// code = 8 row + ((row >> 1) & 7), so the 16 rows of one 16-byte-per-lane
// operand read fall in distinct LDS bank groups.
__host__ __device__ constexpr uint32_t score_row_code(uint32_t row) {
    return (row << 3) | ((row >> 1) & 7u);
}

// LDS placement of key row `row` (0..kChunkRows) of a chunk, in 32-byte
// units: the row's 128 bytes start at unit 4 * row, and the 32-byte quarter
// of channel block nb sits at quarter nb ^ sw(row), sw taken from row bits 1
// and 3, so the 16 rows 8k + q (k, q < 4) of one transposed read fall in
// distinct LDS bank groups. The schedule stores this code for every slot.
__host__ __device__ constexpr uint32_t key_row_code(uint32_t row) {
    return (row << 2) | ((row >> 1) & 1u) | (((row >> 3) & 1u) << 1);
}
}  // namespace diffuser

struct diffuser_graph {
    int64_t n = 0;
    int32_t num_graphs = 0;
    // Generator parameters (meaningful when structured).
    bool structured = false;  // built from a descriptor: window metadata valid
    int32_t radius = 0;
    int32_t num_global = 0;
    int32_t num_random = 0;
    int32_t rnd_width = 0;    // ELL width of the random-column table
    int32_t causal = 0;
    uint64_t seed = 0;
    int32_t random_layout = 0;   // DIFFUSER_EXTRAS_RANDOM or DIFFUSER_EXTRAS_EVEN
    int device = 0;

    // Ascending CSR (what the graph is).
    std::vector<int64_t> nnz;       // [num_graphs]
    std::vector<int64_t> col_off;   // [num_graphs + 1] prefix sums of nnz
    int64_t max_row_len = 0;
    int64_t* d_row_ptr = nullptr;   // [num_graphs][n + 1]
    int32_t* d_col_idx = nullptr;   // [col_off[num_graphs]]
    int64_t* d_col_off = nullptr;   // [num_graphs + 1]

    // Weight-slot layout (where the edge weights live in A), per graph:
    //  * row segments: seg_ptr [n + 1] row offsets (a global row: its
    //    columns; any other row: window blocks then global columns, then,
    //    for n > kMaxScheduledN, its random columns);
    //  * random area (built graphs with n <= kMaxScheduledN): from
    //    seg_ptr[n], laid out as the random layout below says.
    // slot_col / slot_row [slots] give each slot's edge, or -1 for padding
    // (weight 0). Imported graphs use their CSR as is (no random area).
    std::vector<int64_t> slots;     // [num_graphs]
    std::vector<int64_t> slot_off;  // [num_graphs + 1] prefix sums of slots
    int64_t max_row_slots = 0;      // longest row segment
    int64_t* d_seg_ptr = nullptr;   // [num_graphs][n + 1]
    int32_t* d_slot_col = nullptr;  // [slot_off[num_graphs]]
    int32_t* d_slot_row = nullptr;  // [slot_off[num_graphs]]
    int64_t* d_slot_off = nullptr;  // [num_graphs + 1]

    // Generator metadata (structured graphs).
    int32_t* d_global = nullptr;    // [num_global]
    int32_t* d_gchunk = nullptr;    // [nchunks + 1] globals below key row kChunkRows * c
    int32_t* d_rnd = nullptr;       // [num_graphs][n][rnd_width] ascending
    int32_t* d_rnd_cnt = nullptr;   // [num_graphs][n] random columns kept per row
    int32_t* d_rslot = nullptr;     // [num_graphs][n][rnd_width] slot of each kept random edge
    // Per-row segment geometry, int4 {segment start, window block start
    // column (lo & ~7), window slots (-1 for a global row), global slots}.
    int32_t* d_row_info = nullptr;  // [num_graphs][n][4]

    // Random schedule (built graphs with n <= kMaxScheduledN). Rows form
    // blocks of kRowBlock, key rows chunks of kChunkRows. For each (row
    // block, chunk) the block's random edges with keys in the chunk are
    // listed by row, two edges of one row per pair (a lone edge is paired
    // with a dummy), 16 pairs per group in that order.
    // Where the random weights live (rand_layout):
    //  * kRow (graphs with n > kMaxScheduledN): in each row's segment, after
    //    its global slots, ascending, padded to a multiple of 8;
    //  * kGroup (kMaxResidentN < n <= kMaxScheduledN): after all row
    //    segments, a group's 32 weights in 32 consecutive slots, pair p
    //    owning slots 2p and 2p + 1;
    //  * kOctet (n <= kMaxResidentN): after all row segments, one area per
    //    row block of noct = ceil(max random edges of its rows / 8) octets,
    //    starting at slot seg_ptr[n] + 128 * rb_roff[rb]: random edge e of
    //    row m of the block at ((e / 8) * 16 + m) * 8 + e % 8, positions
    //    past a row's edges (and rows past n) padding. A pair of the
    //    schedule covers an even position e and e + 1 of one row (a dummy
    //    slot is another edge's, or padding); sched_off gives its first slot.
    enum class RandLayout { kRow, kGroup, kOctet };
    bool scheduled = false;
    RandLayout rand_layout = RandLayout::kRow;
    bool grouped() const { return rand_layout == RandLayout::kGroup; }
    bool octet() const { return rand_layout == RandLayout::kOctet; }
    // Random weights outside the row segments (found through d_rslot).
    bool rand_apart() const { return rand_layout != RandLayout::kRow; }
    std::vector<int64_t> groups;    // [num_graphs]
    std::vector<int64_t> grp_off;   // [num_graphs + 1] prefix sums of groups
    int64_t* d_grp_off = nullptr;   // [num_graphs + 1]
    int64_t* d_grp_ptr = nullptr;   // [num_graphs][nrb + 1] groups of each row block
    int32_t* d_grp_cptr = nullptr;  // [num_graphs][nrb][nchunks + 1] first group (in the
                                    //   graph) of each key chunk of each row block
    uint32_t* d_sched_row = nullptr;// [groups][4]: byte p of word k = row (within the
                                    //   block) of pair 4k + p, plus 0x40 when the
                                    //   pair's first slot is a dummy and 0x80 when
                                    //   its second is; 0xFF for a dummy pair
    uint16_t* d_sched_off = nullptr;// [groups][16] (kOctet): slot of pair p's first slot
                                    //   within its row block's octet area
    uint32_t* d_sched_j = nullptr;  // [groups][16]: word 4k + a = key_row_code of the
                                    //   key row (within the chunk) of slot 8k + a (low
                                    //   half) and of slot 8k + 4 + a (high half);
                                    //   kZeroRow's code for a dummy
    uint16_t* d_sched_k = nullptr;  // [groups][32]: score_row_code of the key row of
                                    //   each slot, in slot order
    // kOctet graphs (n <= kMaxResidentN):
    int32_t* d_rb_oct = nullptr;    // [graphs][nrb]: random octets of each row block
    int64_t* d_rb_roff = nullptr;   // [graphs][nrb + 1]: prefix sums of d_rb_oct
    std::vector<int64_t> octets;    // [num_graphs]: random octets of each graph
    // Resident-slice diffusion step's key table: for row block rb, batch
    // b of kOctBatch octets, lane l = 16 kg + 4 q + j (64 lanes), 8 uint16
    // entries t * 2 + h: the res_unit slot of the key of random edge
    // 8 o + 4 h + q of row 4 t + ((kg + o) & 3) of the block, o = 4 b + j,
    // or the zero row res_npad(n) where there is none (the key row's slot
    // in an LDS plane of 32-byte slots). A batch is one contiguous
    // kilobyte, 16 bytes per lane.
    int32_t key_batches = 0;        // batches per row block: ceil(ceil(rnd_width / 8) / 4)
    uint16_t* d_rkey = nullptr;     // [graphs][nrb][key_batches][64][8]
    int64_t* d_rb_cost = nullptr;   // [graphs][nrb + 1]: prefix sums of row-block costs
    int64_t* d_rb_cost_max = nullptr;  // [graphs]: largest row-block cost

    // Column index of the weight slots (built on first use by the backward
    // pass, under bw_mutex): for each graph, col_ptr [n + 1] and, from
    // col_off_slots[gr], the slot numbers (within the graph) of each column
    // by ascending row.
    std::mutex bw_mutex;
    // Long rows (more than kLongRow weight slots, random slots included),
    // ascending, per graph from long_off[gr]; the generic kernels' main
    // pass skips them and a companion splits each over a workgroup.
    std::vector<int64_t> long_off;  // [num_graphs + 1]
    int64_t max_long = 0;           // most long rows in one graph
    int32_t* d_long_rows = nullptr; // [long_off[num_graphs]]
    int64_t* d_long_off = nullptr;  // [num_graphs + 1]
    // CSR position (within its graph) of each slot's edge, -1 for padding
    // (built on first use by the CSR-order entry points, under bw_mutex).
    int32_t* d_slot_csr = nullptr;  // [slot_off[num_graphs]]

    // Block layout (graphs from diffuser_build_block_graph): every row of
    // query block I reads whole key blocks, listed (ascending, absolute
    // indices into d_bcol) at d_bptr[gr][I] .. d_bptr[gr][I + 1].
    bool blocked = false;
    int32_t block = 0;              // tokens per block
    int64_t nblocks = 0;            // n / block
    int32_t max_key_blocks = 0;     // longest key-block list
    int32_t global_blocks = 0;      // query blocks 0 .. global_blocks - 1 read every block
    int32_t* d_bptr = nullptr;      // [num_graphs][nblocks + 1]
    int32_t* d_bcol = nullptr;      // [key blocks of all graphs]
    int64_t* d_col_ptr = nullptr;        // [num_graphs][n + 1]
    int64_t* d_col_off_slots = nullptr;  // [num_graphs + 1]
    int32_t* d_col_slot = nullptr;       // [valid slots of all graphs]
    int32_t* d_col_row = nullptr;        // row of each d_col_slot entry
    // Columns with more than kLongRow entries (built with the column index),
    // ascending, per graph from d_long_col_off.
    int64_t max_long_col = 0;
    int32_t* d_long_cols = nullptr;      // [long columns of all graphs]
    int64_t* d_long_col_off = nullptr;   // [num_graphs + 1]
    // Random edges by column (built with the column index on bidirectional
    // graphs whose random weights lie outside the row segments): for graph
    // gr and column j, entries d_trand_ptr[gr (n + 1) + j] .. + 1 hold the
    // weight slot (within the graph) and the row of each random edge (i, j),
    // rows ascending.
    int64_t* d_trand_ptr = nullptr;      // [num_graphs][n + 1]
    int32_t* d_trand_slot = nullptr;
    int32_t* d_trand_row = nullptr;
};

namespace diffuser {

// Thread-local error message helpers (api.cpp).
diffuser_status fail(diffuser_status s, const std::string& msg);

// --- graph builder (graph_build.hip) ---------------------------------------
// Enqueues the per-row random draw kernel: deg and slots ([num_graphs][n])
// receive each row's edge and weight-slot counts.
hipError_t launch_draw(const diffuser_graph& g, int32_t* deg, int32_t* slots, int32_t* status,
                       hipStream_t st);
// Exclusive scan of counts [num_graphs][n] into offsets [num_graphs][n + 1]
// (each graph from 0); max_count[gr] receives each graph's largest count.
hipError_t launch_scan(int64_t n, int32_t num_graphs, const int32_t* counts, int64_t* offsets,
                       int64_t* max_count, hipStream_t st);
// Fills d_col_idx and the row segments' d_slot_col / d_slot_row.
hipError_t launch_fill(const diffuser_graph& g, hipStream_t st);
// Counts the schedule groups of every row block into counts [graphs][nrb].
hipError_t launch_sched_count(const diffuser_graph& g, int32_t* counts, hipStream_t st);
// Writes the random schedule, the random area's slot_col / slot_row and
// d_rslot (needs d_grp_ptr, d_grp_off and the allocated schedule arrays).
hipError_t launch_sched_fill(const diffuser_graph& g, hipStream_t st);
// kOctet graphs: the random octets of every row block into d_rb_oct and
// their prefix sums into d_rb_roff (max_count: [graphs] int64 scratch).
hipError_t launch_rb_octets(const diffuser_graph& g, int64_t* max_count, hipStream_t st);
// kOctet graphs: writes d_rkey and d_rb_cost (cost_tmp: [graphs][nrb]
// int32 scratch).
hipError_t launch_res_tables(const diffuser_graph& g, int32_t* cost_tmp, hipStream_t st);

// Marks the long rows of every graph (flags [graphs][n] int32, 1 for a row
// with more than kLongRow slots), then, once long_off and d_long_rows are
// allocated from the flags' scan (offsets [graphs][n + 1]), lists them.
hipError_t launch_long_flags(const diffuser_graph& g, int32_t* flags, hipStream_t st);
hipError_t launch_long_fill(const diffuser_graph& g, const int32_t* flags,
                            const int64_t* offsets, hipStream_t st);

// --- CSR order of A (csr_order.hip) ----------------------------------------
// Writes map [slot_off[num_graphs]]: each slot's CSR position within its
// graph, -1 for padding (graph CSR and slot arrays must be on the device).
hipError_t launch_slot_csr(const diffuser_graph& g, int32_t* map, hipStream_t st);
// Moves B * H blocks of es-byte weights (es = 2 or 4) between the slot
// layout and CSR order through g.d_slot_csr: to_csr reads the slot layout
// (padding ignored), otherwise writes it (padding 0).
hipError_t launch_slots_csr_permute(const diffuser_graph& g, int32_t B, int32_t H, size_t es,
                                    const void* src, void* dst, bool to_csr, hipStream_t st);

// --- compute (scores.hip, diffuse.hip) --------------------------------------
// Graph arrays of the generic kernels (defined in vec.h).
struct GenericGraph;
GenericGraph generic_graph(const diffuser_graph& g);

struct attn_shape {
    int32_t B, H, d;          // d = d_h for scores, d_v for diffusion
    diffuser_dtype dtype;
};

// Writes A; when row_scale != nullptr also 1 / (sum of each row's stored
// weights) per (b, h, row).
// `part`: the block-tile kernels' scratch (block_part_bytes), or null.
hipError_t launch_scores_softmax(const diffuser_graph& g, const attn_shape& s, const void* Q,
                                 const void* K, void* A, float* row_scale, float scale_log2,
                                 hipStream_t st, float* part = nullptr);

// The same on scheduled graphs (bf16, d_h = 64), LDS-streamed with MFMA.
// normalized: A holds the softmax weights; otherwise A holds exp(s - m)
// unnormalised and row_scale (required) 1 / (sum of each row's stored
// weights), the form the diffusion step applies.
bool fast_scores_supported(const diffuser_graph& g, const attn_shape& s);
hipError_t launch_scores_fast(const diffuser_graph& g, const attn_shape& s, const void* Q,
                              const void* K, void* A, float* row_scale, float scale_log2,
                              bool normalized, hipStream_t st);

// Coefficients of one diffusion step Zn = keep * c_i * (A Zk)_i + restart * V_i:
// (1 - alpha, alpha) for the PPR recurrence, (theta_{k+1} or 1, theta_k)
// for the nested evaluation of general coefficients.
struct step_coefs {
    float keep, restart;
};

// One step with c_i = row_scale[(b, h, i)], or 1 when row_scale == nullptr.
// Generic kernel.
hipError_t launch_diffuse_step(const diffuser_graph& g, const attn_shape& s, const void* A,
                               const void* Zk, const void* V, void* Zn, const float* row_scale,
                               step_coefs k, hipStream_t st);
// The same step on built graphs with fp32 storage (d = 64), one wave per
// row, the window and global-column key rows of each 64-row group in LDS;
// the global rows several at a time, each key row read once.
bool rows_diffuse_supported(const diffuser_graph& g, const attn_shape& s);
hipError_t launch_diffuse_rows(const diffuser_graph& g, const attn_shape& s, const void* A,
                               const void* Zk, const void* V, void* Zn, const float* row_scale,
                               step_coefs k, hipStream_t st);
// The same kernels for fp32 states of a B x H batch whose restart rows V
// are fp32 or bf16 (d = 64, no row scale): the backward's recomputed states.
bool rows_states_supported(const diffuser_graph& g, int32_t B, int32_t H, int32_t d);
hipError_t launch_states_rows(const diffuser_graph& g, int32_t B, int32_t H, const float* A,
                              const float* Zk, const void* V, diffuser_dtype v_dtype, float* Zn,
                              step_coefs k, hipStream_t st);
// The transposed product Y = scale * A^T X on the same kernels for
// bidirectional built graphs once the column index (and with it the random
// edges by column) exists: At = A^T in the graph's slot geometry
// (launch_transpose_struct), the random weights read from A.
bool rows_transposed_supported(const diffuser_graph& g, int32_t B, int32_t H, int32_t d);
hipError_t launch_transpose_struct(const diffuser_graph& g, int32_t B, int32_t H, const float* A,
                                   float* At, hipStream_t st);
hipError_t launch_transposed_rows(const diffuser_graph& g, int32_t B, int32_t H, const float* At,
                                  const float* A, const float* X, float* Y, float scale,
                                  hipStream_t st);
// Y = scale * W X with X and Y of storage type dtype (the backward's dQ =
// dS K and, transposed, dK = dS^T Q): W the weights in the graph's slot
// geometry (A^T's when transposed), WR the weights the random edges' slots
// name.
hipError_t launch_grad_rows(const diffuser_graph& g, int32_t B, int32_t H, const float* W,
                            const float* WR, bool transposed, const void* X, void* Y,
                            diffuser_dtype dtype, float scale, hipStream_t st);
// The same step on built graphs with a whole channel slice of Z_k resident
// in LDS (bf16, d = 32 or 64, n up to about 4.5 K keys).
bool res_diffuse_supported(const diffuser_graph& g, const attn_shape& s);
hipError_t launch_diffuse_res(const diffuser_graph& g, const attn_shape& s, const void* A,
                              const void* Zk, const void* V, void* Zn, const float* row_scale,
                              step_coefs k, hipStream_t st);
// The same step on built graphs (bf16, d = 64), LDS-streamed with MFMA.
bool fast_diffuse_supported(const diffuser_graph& g, const attn_shape& s);
hipError_t launch_diffuse_fast(const diffuser_graph& g, const attn_shape& s, const void* A,
                               const void* Zk, const void* V, void* Zn, const float* row_scale,
                               step_coefs k, hipStream_t st);

// Block-tile kernels for block graphs (block_fast.hip; block == 64, bf16,
// d = 64): the score pass (as launch_scores_fast: normalised, or exp(s - m)
// with row_scale) and one diffusion step.
bool fast_block_supported(const diffuser_graph& g, const attn_shape& s);
hipError_t launch_block_scores(const diffuser_graph& g, const attn_shape& s, const void* Q,
                               const void* K, void* A, float* row_scale, float scale_log2,
                               bool normalized, float* part, hipStream_t st);
// The diffusion step splits each global query block's key blocks over
// several workgroups, whose fp32 partial sums (block_part_bytes of scratch
// at `part`) a second kernel adds in a fixed order.
size_t block_part_bytes(const diffuser_graph& g, const attn_shape& s);
hipError_t launch_block_diffuse(const diffuser_graph& g, const attn_shape& s, const void* A,
                                const void* Zk, const void* V, void* Zn, const float* row_scale,
                                step_coefs k, float* part, hipStream_t st);

// Host construction of the block and dilated layouts (block_graph.cpp).
// build_block_lists: keys[gr * nblocks + I] = ascending key blocks of query
// block I; false when a row's draws exceed their budget.
bool build_block_lists(int64_t nblocks, int32_t local_blocks, int32_t num_random,
                       int32_t num_global, int32_t num_graphs, uint64_t seed,
                       std::vector<std::vector<int32_t>>& keys);
void block_lists_to_csr(int64_t n, int32_t block, int32_t num_graphs,
                        const std::vector<std::vector<int32_t>>& keys,
                        std::vector<int64_t>& row_ptr, std::vector<int32_t>& cols);
void dilated_csr(int64_t n, int32_t radius, int32_t dilation, const int32_t* G, int32_t g,
                 std::vector<int64_t>& row_ptr, std::vector<int32_t>& cols);

// Backward of the whole path (backward.hip). Workspace pointers are fp32:
// A and dA [a_count] in the A layout, Zs [K_steps][B*H*n*d], G0, G1, dV
// [B*H*n*d]. d_h == d_v == d.
struct BackwardArgs {
    int32_t B, H, d;
    diffuser_dtype dtype;
    int32_t K_steps;
    float alpha, scale;                    // scale = 1 / sqrt(d)
    const void *Q, *K, *V, *dZ;
    void *dQ, *dK, *dVout;
    int64_t a_count;
    // A, dA and At (the weights in column order) are [a_count]; Zs holds
    // Z_0 .. Z_{K-1}, Gs G_0 .. G_K, each [B][H][n][d].
    float *A, *dA, *At, *Zs, *Gs, *dV;
};
hipError_t launch_backward(const diffuser_graph& g, const BackwardArgs& p, hipStream_t st);

// Projections around the path (layer.hip): head split of [B*n][3 H d] into
// Q, K, V [B][H][n][d]; head merge of Z into [B*n][H d]; a row-major GEMM
// C[M][N] = A[M][K] B[K][N] on the device's library-owned rocBLAS handle.
hipError_t launch_split_heads(diffuser_dtype t, int64_t B, int32_t n, int32_t H, int32_t d,
                              const void* in, void* q, void* k, void* v, hipStream_t st);
hipError_t launch_merge_heads(diffuser_dtype t, int64_t B, int32_t n, int32_t H, int32_t d,
                              const void* z, void* out, hipStream_t st);
diffuser_status blas_gemm(int device, diffuser_dtype t, int64_t M, int64_t N, int64_t K,
                          const void* A, const void* B, void* C, void* blas_ws,
                          size_t blas_ws_bytes, hipStream_t st);

// The fused fp32 score pass on built graphs (d = 64, n > kLongRow, every
// long row a global row): one wave per row with the window and global-column
// key rows of each 64-row group in LDS, the long global rows four at a
// time; then the zeroing of the random area's dummy slots
// (launch_zero_dummies_f32).
bool rows_scores_supported(const diffuser_graph& g, const attn_shape& s);
// The same for fp32 or bf16 queries and keys (the weights are fp32).
bool rows_scores_any_supported(const diffuser_graph& g, const attn_shape& s);
hipError_t launch_scores_rows(const diffuser_graph& g, const attn_shape& s, const void* Q,
                              const void* K, void* A, float* row_scale, float scale_log2,
                              hipStream_t st);
// dA_ij = f sum_{k < K} Gs_{k+1}[i] . Zs_k[j] on the segment slots of a
// built graph (window bands, global columns, global rows) on MFMA, d = 64;
// the random slots are left to the caller. K >= 1.
bool mfma_dots_supported(const diffuser_graph& g, int32_t d);
hipError_t launch_dots_dense(const diffuser_graph& g, int32_t B, int32_t H, const float* Gs,
                             const float* Zs, int64_t stride, int32_t K, float f, float* dA,
                             hipStream_t st);
hipError_t launch_zero_dummies_f32(const diffuser_graph& g, const attn_shape& s, void* A,
                                  hipStream_t st);
// Normalised edge softmax into fp32 A (any graph). With row_scale (B*H*n
// floats of scratch) built d = 64 graphs take the fused LDS-window pass and
// a normalisation; otherwise the generic kernel.
hipError_t launch_scores_softmax_f32(const diffuser_graph& g, const attn_shape& s, const void* Q,
                                     const void* K, float* A, float scale_log2, hipStream_t st,
                                     float* row_scale);

}  // namespace diffuser
