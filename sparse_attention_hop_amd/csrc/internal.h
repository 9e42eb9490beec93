// Internal declarations shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>
#include <vector>

#include "../../include/diffuser.h"

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
    int device = 0;

    // Ascending CSR (what the graph is).
    std::vector<int64_t> nnz;       // [num_graphs]
    std::vector<int64_t> col_off;   // [num_graphs + 1] prefix sums of nnz
    int64_t max_row_len = 0;
    int64_t* d_row_ptr = nullptr;   // [num_graphs][n + 1]
    int32_t* d_col_idx = nullptr;   // [col_off[num_graphs]]
    int64_t* d_col_off = nullptr;   // [num_graphs + 1]

    // Weight-slot layout (where the edge weights live in A): per graph,
    // slot_ptr [n + 1] row offsets and slot_col [slots] the column of each
    // slot (-1 = padding, weight 0). Imported graphs use their CSR as is.
    std::vector<int64_t> slots;     // [num_graphs]
    std::vector<int64_t> slot_off;  // [num_graphs + 1] prefix sums of slots
    int64_t max_row_slots = 0;
    int64_t* d_slot_ptr = nullptr;  // [num_graphs][n + 1]
    int32_t* d_slot_col = nullptr;  // [slot_off[num_graphs]]
    int64_t* d_slot_off = nullptr;  // [num_graphs + 1]

    // Generator metadata (structured graphs).
    int32_t* d_global = nullptr;    // [num_global]
    int32_t* d_rnd = nullptr;       // [num_graphs][n][rnd_width] ascending
    int32_t* d_rnd_cnt = nullptr;   // [num_graphs][n] random columns kept per row
    // Key-row chunking of the LDS-streamed kernels: bnd[gr][i][c] = number of
    // row i's kept random columns below c * chunk, c = 0 .. ceil(n / chunk).
    int32_t chunk = 512;
    int32_t* d_bnd = nullptr;
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
// Fills d_col_idx and d_slot_col from the draws.
hipError_t launch_fill(const diffuser_graph& g, hipStream_t st);
// Fills d_bnd from the draws.
hipError_t launch_bounds(const diffuser_graph& g, hipStream_t st);

// --- compute (scores.hip, diffuse.hip) --------------------------------------
struct attn_shape {
    int32_t B, H, d;          // d = d_h for scores, d_v for diffusion
    diffuser_dtype dtype;
};

// Writes A; when row_scale != nullptr also 1 / (sum of each row's stored
// weights) per (b, h, row).
hipError_t launch_scores_softmax(const diffuser_graph& g, const attn_shape& s, const void* Q,
                                 const void* K, void* A, float* row_scale, float scale_log2,
                                 hipStream_t st);

// One step: Zn = (1 - alpha) * c_i * (A Zk)_i + alpha * V_i with c_i =
// row_scale[(b, h, i)] or 1 when row_scale == nullptr. Generic kernel.
hipError_t launch_diffuse_step(const diffuser_graph& g, const attn_shape& s, const void* A,
                               const void* Zk, const void* V, void* Zn, const float* row_scale,
                               float alpha, hipStream_t st);
// The same step on built graphs (bf16, d = 64), LDS-streamed with MFMA.
bool fast_diffuse_supported(const diffuser_graph& g, const attn_shape& s);
hipError_t launch_diffuse_fast(const diffuser_graph& g, const attn_shape& s, const void* A,
                               const void* Zk, const void* V, void* Zn, const float* row_scale,
                               float alpha, hipStream_t st);

}  // namespace diffuser
