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

    std::vector<int64_t> nnz;      // [num_graphs]
    std::vector<int64_t> col_off;  // [num_graphs + 1] prefix sums of nnz
    int64_t max_row_len = 0;

    int64_t* d_row_ptr = nullptr;  // [num_graphs][n + 1]
    int32_t* d_col_idx = nullptr;  // [col_off[num_graphs]]
    int64_t* d_col_off = nullptr;  // [num_graphs + 1]
    int32_t* d_global = nullptr;   // [num_global] (structured)
    int32_t* d_rnd = nullptr;      // [num_graphs][n][rnd_width] sorted (structured)
    int32_t* d_rnd_cnt = nullptr;  // [num_graphs][n] (structured)
    int32_t* d_win_off = nullptr;  // [num_graphs][n] CSR offset of the window run (structured)
};

namespace diffuser {

// Thread-local error message helpers (api.cpp).
diffuser_status fail(diffuser_status s, const std::string& msg);

// --- graph builder (graph_build.hip) ---------------------------------------
// Enqueues the per-row random draw + degree kernel. deg: [num_graphs][n].
hipError_t launch_draw(const diffuser_graph& g, int32_t* deg, int32_t* status, hipStream_t st);
// Exclusive scan of deg into d_row_ptr (each graph from 0); max_deg[gr]
// receives the longest row of each graph.
hipError_t launch_scan(const diffuser_graph& g, const int32_t* deg, int64_t* max_deg,
                       hipStream_t st);
// Fills d_col_idx and d_win_off from the draws.
hipError_t launch_fill(const diffuser_graph& g, hipStream_t st);

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
// row_scale[(b, h, i)] or 1 when row_scale == nullptr.
hipError_t launch_diffuse_step(const diffuser_graph& g, const attn_shape& s, const void* A,
                               const void* Zk, const void* V, void* Zn, const float* row_scale,
                               float alpha, hipStream_t st);

}  // namespace diffuser
