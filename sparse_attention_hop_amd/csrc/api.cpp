// C ABI of the Diffuser library: argument validation, graph handles,
// workspace layout and stage dispatch. Every entry point validates its
// arguments before enqueuing anything and reports failures as a status code
// plus a thread-local message.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "internal.h"

namespace diffuser {

namespace {
thread_local std::string g_last_error;

constexpr int64_t kMaxN = 1ll << 24;
constexpr int32_t kMaxSampledRandom = 1024;
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

size_t elem_size(diffuser_dtype t) { return t == DIFFUSER_F32 ? 4 : 2; }

bool supported_width(int32_t d) { return d == 16 || d == 32 || d == 64 || d == 128; }

diffuser_status hip_fail(hipError_t e, const char* what) {
    return fail(DIFFUSER_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

template <typename P>
hipError_t dev_alloc(P** p, size_t count) {
    *p = nullptr;
    if (count == 0) count = 1;
    return hipMalloc(reinterpret_cast<void**>(p), sizeof(P) * count);
}

void free_graph_memory(diffuser_graph* g) {
    hipFree(g->d_row_ptr);
    hipFree(g->d_col_idx);
    hipFree(g->d_col_off);
    hipFree(g->d_global);
    hipFree(g->d_gchunk);
    hipFree(g->d_rnd);
    hipFree(g->d_rnd_cnt);
    hipFree(g->d_seg_ptr);
    hipFree(g->d_slot_col);
    hipFree(g->d_slot_row);
    hipFree(g->d_slot_off);
    hipFree(g->d_rslot);
    hipFree(g->d_row_info);
    hipFree(g->d_grp_off);
    hipFree(g->d_grp_ptr);
    hipFree(g->d_grp_cptr);
    hipFree(g->d_sched_row);
    hipFree(g->d_sched_j);
    hipFree(g->d_sched_k);
    hipFree(g->d_sched_off);
    hipFree(g->d_rkey);
    hipFree(g->d_rb_oct);
    hipFree(g->d_rb_roff);
    hipFree(g->d_rb_cost);
    hipFree(g->d_rb_cost_max);
    hipFree(g->d_col_ptr);
    hipFree(g->d_col_off_slots);
    hipFree(g->d_col_slot);
    hipFree(g->d_col_row);
    hipFree(g->d_long_cols);
    hipFree(g->d_long_col_off);
    hipFree(g->d_trand_ptr);
    hipFree(g->d_trand_slot);
    hipFree(g->d_trand_row);
    hipFree(g->d_slot_csr);
    hipFree(g->d_long_rows);
    hipFree(g->d_long_off);
    hipFree(g->d_bptr);
    hipFree(g->d_bcol);
    g->d_bptr = nullptr;
    g->d_bcol = nullptr;
    g->d_row_ptr = nullptr;
    g->d_col_idx = nullptr;
    g->d_col_off = nullptr;
    g->d_global = nullptr;
    g->d_gchunk = nullptr;
    g->d_rnd = nullptr;
    g->d_rnd_cnt = nullptr;
    g->d_seg_ptr = nullptr;
    g->d_slot_col = nullptr;
    g->d_slot_row = nullptr;
    g->d_slot_off = nullptr;
    g->d_rslot = nullptr;
    g->d_row_info = nullptr;
    g->d_grp_off = nullptr;
    g->d_grp_ptr = nullptr;
    g->d_grp_cptr = nullptr;
    g->d_sched_row = nullptr;
    g->d_sched_j = nullptr;
    g->d_sched_k = nullptr;
    g->d_sched_off = nullptr;
    g->d_rkey = nullptr;
    g->d_rb_oct = nullptr;
    g->d_rb_roff = nullptr;
    g->d_rb_cost = nullptr;
    g->d_rb_cost_max = nullptr;
    g->d_col_ptr = nullptr;
    g->d_col_off_slots = nullptr;
    g->d_col_slot = nullptr;
    g->d_col_row = nullptr;
    g->d_long_cols = nullptr;
    g->d_long_col_off = nullptr;
    g->d_trand_ptr = nullptr;
    g->d_trand_slot = nullptr;
    g->d_trand_row = nullptr;
    g->d_slot_csr = nullptr;
    g->d_long_rows = nullptr;
    g->d_long_off = nullptr;
}

diffuser_status alloc_status(hipError_t e, const char* what) {
    if (e == hipErrorOutOfMemory) return fail(DIFFUSER_ERR_OUT_OF_MEMORY, what);
    return hip_fail(e, what);
}

// Largest random pool of a non-global row: n minus |window u globals|.
int64_t max_pool(int64_t n, int32_t r, const int32_t* G, int32_t g) {
    int64_t best = 0;
    for (int64_t i = 0; i < n; ++i) {
        if (g > 0 && std::binary_search(G, G + g, (int32_t)i)) continue;
        const int64_t lo = std::max<int64_t>(0, i - r), hi = std::min<int64_t>(n - 1, i + r);
        const int64_t in_w = std::upper_bound(G, G + g, (int32_t)hi) - std::lower_bound(G, G + g, (int32_t)lo);
        best = std::max(best, n - (hi - lo + 1) - (g - in_w));
    }
    return best;
}

struct graph_guard {
    diffuser_graph* g;
    ~graph_guard() {
        if (g) {
            free_graph_memory(g);
            delete g;
        }
    }
};

diffuser_status check_graph(const diffuser_graph* g) {
    if (!g) return fail(DIFFUSER_ERR_INVALID_ARG, "graph handle is NULL");
    return DIFFUSER_OK;
}

// Shared validation of (B, H, width, dtype) against a graph.
diffuser_status check_shape(const diffuser_graph* g, int32_t B, int32_t H, int32_t d,
                            diffuser_dtype dtype, const char* dname) {
    if (auto s = check_graph(g)) return s;
    if (B < 1 || H < 1) return fail(DIFFUSER_ERR_INVALID_ARG, "B and H must be >= 1");
    if (g->num_graphs != 1 && g->num_graphs != B)
        return fail(DIFFUSER_ERR_INVALID_ARG, "graph has num_graphs not in {1, B}");
    if (dtype != DIFFUSER_F32 && dtype != DIFFUSER_BF16)
        return fail(DIFFUSER_ERR_UNSUPPORTED, "dtype must be DIFFUSER_F32 or DIFFUSER_BF16");
    if (d < 1) return fail(DIFFUSER_ERR_INVALID_ARG, std::string(dname) + " must be >= 1");
    if (!supported_width(d))
        return fail(DIFFUSER_ERR_UNSUPPORTED, std::string(dname) + " must be 16, 32, 64 or 128");
    if ((int64_t)B * H > 65535)
        return fail(DIFFUSER_ERR_UNSUPPORTED, "B * H above 65535");
    return DIFFUSER_OK;
}

// Elements of A: every (b, h) holds the weight slots of its graph.
int64_t total_a_elems(const diffuser_graph* g, int32_t B, int32_t H) {
    if (g->num_graphs == 1) return (int64_t)B * H * g->slots[0];
    return (int64_t)H * g->slot_off[g->num_graphs];
}

// Workspace of diffuser_attn: [A][Z ping-pong buffer][row scales (fp32)].
struct ws_layout {
    size_t a_bytes, z_bytes, s_bytes, p_bytes, total;
};

// Scratch of the block-tile diffusion step (0 unless it runs on g).
size_t part_bytes(const diffuser_graph* g, int32_t B, int32_t H, int32_t d_v, diffuser_dtype t) {
    const attn_shape s{B, H, d_v, t};
    return fast_block_supported(*g, s) ? align_up(block_part_bytes(*g, s)) : 0;
}

ws_layout layout(const diffuser_graph* g, int32_t B, int32_t H, int32_t d_v, diffuser_dtype t) {
    ws_layout w;
    w.a_bytes = align_up((size_t)total_a_elems(g, B, H) * elem_size(t));
    w.z_bytes = align_up((size_t)B * H * (size_t)g->n * d_v * elem_size(t));
    w.s_bytes = align_up((size_t)B * H * (size_t)g->n * sizeof(float));
    w.p_bytes = part_bytes(g, B, H, d_v, t);
    w.total = w.a_bytes + w.z_bytes + w.s_bytes + w.p_bytes;
    return w;
}

diffuser_status check_alpha_k(int32_t K_steps, float alpha) {
    if (K_steps < 0) return fail(DIFFUSER_ERR_INVALID_ARG, "K_steps must be >= 0");
    if (!(alpha >= 0.0f && alpha <= 1.0f))
        return fail(DIFFUSER_ERR_INVALID_ARG, "alpha must lie in [0, 1]");
    return DIFFUSER_OK;
}

diffuser_status check_ptr(const void* p, const char* name, bool need16 = true) {
    if (!p) return fail(DIFFUSER_ERR_INVALID_ARG, std::string(name) + " is NULL");
    if (need16 && !aligned16(p))
        return fail(DIFFUSER_ERR_INVALID_ARG, std::string(name) + " is not 16-byte aligned");
    return DIFFUSER_OK;
}

// One diffusion step Zn = keep * c_i * (A Zk)_i + restart * V_i on the
// fastest kernel that takes the graph and shape: block tiles (block graphs),
// the resident channel slice, the LDS-streamed tiles (scheduled graphs up
// to 2^16 keys), else the generic kernel.
struct step_launcher {
    enum kind_t { kBlock, kResident, kStreamed, kRows, kGeneric } kind;
    const diffuser_graph* g;
    attn_shape s;
    const void* A;
    const void* V;
    float* part;
    hipError_t operator()(const void* cur, void* dst, const float* row_scale, step_coefs kc,
                          hipStream_t st) const {
        switch (kind) {
            case kBlock: return launch_block_diffuse(*g, s, A, cur, V, dst, row_scale, kc, part, st);
            case kResident: return launch_diffuse_res(*g, s, A, cur, V, dst, row_scale, kc, st);
            case kStreamed: return launch_diffuse_fast(*g, s, A, cur, V, dst, row_scale, kc, st);
            case kRows: return launch_diffuse_rows(*g, s, A, cur, V, dst, row_scale, kc, st);
            default: return launch_diffuse_step(*g, s, A, cur, V, dst, row_scale, kc, st);
        }
    }
};

step_launcher pick_step(const diffuser_graph* g, const attn_shape& s, const void* A, const void* V,
                        float* part) {
    step_launcher l{step_launcher::kGeneric, g, s, A, V, part};
    if (aligned16(A)) {
        if (fast_block_supported(*g, s)) l.kind = step_launcher::kBlock;
        else if (res_diffuse_supported(*g, s)) l.kind = step_launcher::kResident;
        else if (fast_diffuse_supported(*g, s)) l.kind = step_launcher::kStreamed;
        else if (rows_diffuse_supported(*g, s)) l.kind = step_launcher::kRows;
    }
    return l;
}

// K diffusion steps from V into Z, ping-ponging with `tmp` so that the last
// step writes Z.
diffuser_status run_diffusion(const diffuser_graph* g, const attn_shape& s, const void* A,
                              const float* row_scale, const void* V, void* Z, void* tmp,
                              float* part, int32_t K_steps, float alpha, hipStream_t st) {
    const size_t zbytes = (size_t)s.B * s.H * (size_t)g->n * s.d * elem_size(s.dtype);
    if (K_steps == 0) {
        hipError_t e = hipMemcpyAsync(Z, V, zbytes, hipMemcpyDeviceToDevice, st);
        if (e != hipSuccess) return hip_fail(e, "copy of V into Z");
        return DIFFUSER_OK;
    }
    const step_launcher step = pick_step(g, s, A, V, part);
    const void* cur = V;
    for (int32_t k = 0; k < K_steps; ++k) {
        // Steps K-1, K-3, ... write Z; the others write tmp.
        void* dst = ((K_steps - 1 - k) % 2 == 0) ? Z : tmp;
        const step_coefs kc{1.0f - alpha, alpha};
        hipError_t e = step(cur, dst, row_scale, kc, st);
        if (e != hipSuccess) return hip_fail(e, "diffusion step launch");
        cur = dst;
    }
    return DIFFUSER_OK;
}

// Z = sum_{k=0..K} theta_k A^k V (eq. S.6 through A^K) in nested form:
// U_K = theta_K V, U_k = theta_k V + A U_{k+1}, Z = U_0. The first launch
// computes U_{K-1} = theta_K (A V) + theta_{K-1} V straight from V, the
// others U_k = (A U_{k+1}) + theta_k V; each is one diffusion step with
// coefficients (keep, restart). K = 0 is one launch with keep = 0.
diffuser_status run_diffusion_theta(const diffuser_graph* g, const attn_shape& s, const void* A,
                                    const float* row_scale, const void* V, void* Z, void* tmp,
                                    float* part, int32_t K_steps, const float* theta,
                                    hipStream_t st) {
    const step_launcher step = pick_step(g, s, A, V, part);
    const int32_t launches = K_steps == 0 ? 1 : K_steps;
    const void* cur = V;
    for (int32_t j = 0; j < launches; ++j) {
        void* dst = ((launches - 1 - j) % 2 == 0) ? Z : tmp;
        const int32_t k = K_steps - 1 - j;   // U_k is written
        const step_coefs kc = K_steps == 0 ? step_coefs{0.0f, theta[0]}
                              : j == 0     ? step_coefs{theta[K_steps], theta[k]}
                                           : step_coefs{1.0f, theta[k]};
        hipError_t e = step(cur, dst, row_scale, kc, st);
        if (e != hipSuccess) return hip_fail(e, "diffusion step launch");
        cur = dst;
    }
    return DIFFUSER_OK;
}

// theta: K + 1 finite, non-negative host floats summing to 1 (eq. S.6).
diffuser_status check_theta(int32_t K_steps, const float* theta) {
    if (K_steps < 0) return fail(DIFFUSER_ERR_INVALID_ARG, "K_steps must be >= 0");
    if (!theta) return fail(DIFFUSER_ERR_INVALID_ARG, "theta is NULL");
    double sum = 0.0;
    for (int32_t k = 0; k <= K_steps; ++k) {
        if (!(theta[k] >= 0.0f) || !std::isfinite(theta[k]))
            return fail(DIFFUSER_ERR_INVALID_ARG, "theta must be finite and non-negative");
        sum += theta[k];
    }
    if (std::fabs(sum - 1.0) > 1e-5)
        return fail(DIFFUSER_ERR_INVALID_ARG, "theta must sum to 1");
    return DIFFUSER_OK;
}

// Workspace of diffuser_attn_backward (fp32 intermediates): A, dA in the A
// layout, the states Z_0 .. Z_{K-1}, two G buffers and dV.
struct bw_layout {
    size_t a, zs, gs, v, total;
};

bw_layout backward_layout(const diffuser_graph* g, int32_t B, int32_t H, int32_t d,
                          int32_t K_steps) {
    bw_layout w;
    const size_t cnt = (size_t)B * H * (size_t)g->n * d;
    w.a = align_up((size_t)total_a_elems(g, B, H) * sizeof(float));
    w.zs = align_up(cnt * sizeof(float) * (size_t)K_steps);
    w.gs = align_up(cnt * sizeof(float) * ((size_t)K_steps + 1));
    w.v = align_up(cnt * sizeof(float));
    w.total = 3 * w.a + w.zs + w.gs + w.v;
    return w;
}

// Builds the graph's column index (once, under bw_mutex): the valid slots
// of each graph ordered by column, then by row (two stable counting sorts
// on the host), with the row of each entry, uploaded with per-graph column
// offsets. On bidirectional built graphs whose random weights lie past the
// row segments it also lists each column's random edges (the entries whose
// slot lies in that area), for the transposed products' row kernels.
diffuser_status ensure_col_index(diffuser_graph* g, hipStream_t st) {
    std::lock_guard<std::mutex> lock(g->bw_mutex);
    if (g->d_col_ptr != nullptr) return DIFFUSER_OK;
    const int64_t n = g->n;
    std::vector<int64_t> col_ptr((size_t)g->num_graphs * (n + 1));
    std::vector<int64_t> col_off(g->num_graphs + 1, 0);
    std::vector<int32_t> col_slot, col_row;
    std::vector<int32_t> long_cols;
    std::vector<int64_t> long_col_off(g->num_graphs + 1, 0);
    int64_t max_long_col = 0;
    std::vector<int32_t> srow, scol, by_row;
    std::vector<int64_t> cnt;
    const bool trand = g->structured && g->rand_apart() && !g->causal;
    std::vector<int64_t> trand_ptr(trand ? (size_t)g->num_graphs * (n + 1) : 0);
    std::vector<int32_t> trand_slot, trand_row;
    hipError_t e;
    for (int32_t gr = 0; gr < g->num_graphs; ++gr) {
        const int64_t slots = g->slots[gr];
        srow.resize(slots);
        scol.resize(slots);
        if ((e = hipMemcpyAsync(srow.data(), g->d_slot_row + g->slot_off[gr],
                                sizeof(int32_t) * slots, hipMemcpyDeviceToHost, st)) != hipSuccess ||
            (e = hipMemcpyAsync(scol.data(), g->d_slot_col + g->slot_off[gr],
                                sizeof(int32_t) * slots, hipMemcpyDeviceToHost, st)) != hipSuccess ||
            (e = hipStreamSynchronize(st)) != hipSuccess)
            return hip_fail(e, "copy of the slot layout for the column index");
        // Stable counting sort of the valid slots by row ...
        cnt.assign(n + 1, 0);
        for (int64_t s = 0; s < slots; ++s)
            if (scol[s] >= 0) ++cnt[srow[s] + 1];
        for (int64_t i = 0; i < n; ++i) cnt[i + 1] += cnt[i];
        const int64_t valid = cnt[n];
        by_row.resize(valid);
        for (int64_t s = 0; s < slots; ++s)
            if (scol[s] >= 0) by_row[cnt[srow[s]]++] = (int32_t)s;
        // ... then by column, which keeps rows ascending within a column.
        int64_t* cp = col_ptr.data() + (size_t)gr * (n + 1);
        for (int64_t j = 0; j <= n; ++j) cp[j] = 0;
        for (int64_t k = 0; k < valid; ++k) ++cp[scol[by_row[k]] + 1];
        for (int64_t j = 0; j < n; ++j) cp[j + 1] += cp[j];
        cnt.assign(cp, cp + n + 1);
        const size_t base = col_slot.size();
        col_slot.resize(base + valid);
        col_row.resize(base + valid);
        for (int64_t k = 0; k < valid; ++k) {
            const int32_t s = by_row[k];
            const int64_t at = cnt[scol[s]]++;
            col_slot[base + at] = s;
            col_row[base + at] = srow[s];
        }
        col_off[gr + 1] = (int64_t)col_slot.size();
        if (trand) {
            int64_t seg_end = 0;
            if ((e = hipMemcpyAsync(&seg_end, g->d_seg_ptr + (int64_t)gr * (n + 1) + n,
                                    sizeof(int64_t), hipMemcpyDeviceToHost, st)) != hipSuccess ||
                (e = hipStreamSynchronize(st)) != hipSuccess)
                return hip_fail(e, "copy of the segment end for the random column lists");
            int64_t* tp = trand_ptr.data() + (size_t)gr * (n + 1);
            for (int64_t j = 0; j < n; ++j) {
                tp[j] = (int64_t)trand_slot.size();
                for (int64_t k = cp[j]; k < cp[j + 1]; ++k)
                    if (col_slot[base + k] >= seg_end) {
                        trand_slot.push_back(col_slot[base + k]);
                        trand_row.push_back(col_row[base + k]);
                    }
            }
            tp[n] = (int64_t)trand_slot.size();
        }
        // Long columns (more than kLongRow entries), for the transposed
        // products' long-column companion.
        for (int64_t j = 0; j < n; ++j)
            if (cp[j + 1] - cp[j] > kLongRow) long_cols.push_back((int32_t)j);
        long_col_off[gr + 1] = (int64_t)long_cols.size();
        max_long_col = std::max(max_long_col, long_col_off[gr + 1] - long_col_off[gr]);
    }
    int64_t *d_ptr = nullptr, *d_off = nullptr, *d_loff = nullptr, *d_tptr = nullptr;
    int32_t *d_slot = nullptr, *d_row = nullptr, *d_lcols = nullptr, *d_tslot = nullptr,
            *d_trow = nullptr;
    if ((e = dev_alloc(&d_ptr, col_ptr.size())) != hipSuccess ||
        (e = dev_alloc(&d_off, col_off.size())) != hipSuccess ||
        (e = dev_alloc(&d_slot, col_slot.size())) != hipSuccess ||
        (e = dev_alloc(&d_row, col_row.size())) != hipSuccess ||
        (e = dev_alloc(&d_lcols, long_cols.size())) != hipSuccess ||
        (e = dev_alloc(&d_loff, long_col_off.size())) != hipSuccess ||
        (trand && ((e = dev_alloc(&d_tptr, trand_ptr.size())) != hipSuccess ||
                   (e = dev_alloc(&d_tslot, std::max<size_t>(trand_slot.size(), 1))) !=
                       hipSuccess ||
                   (e = dev_alloc(&d_trow, std::max<size_t>(trand_row.size(), 1))) !=
                       hipSuccess))) {
        hipFree(d_ptr);
        hipFree(d_off);
        hipFree(d_slot);
        hipFree(d_row);
        hipFree(d_lcols);
        hipFree(d_loff);
        hipFree(d_tptr);
        hipFree(d_tslot);
        hipFree(d_trow);
        return alloc_status(e, "device allocation of the column index");
    }
    if ((e = hipMemcpyAsync(d_ptr, col_ptr.data(), sizeof(int64_t) * col_ptr.size(),
                            hipMemcpyHostToDevice, st)) != hipSuccess ||
        (e = hipMemcpyAsync(d_off, col_off.data(), sizeof(int64_t) * col_off.size(),
                            hipMemcpyHostToDevice, st)) != hipSuccess ||
        (col_slot.size() > 0 &&
         (e = hipMemcpyAsync(d_slot, col_slot.data(), sizeof(int32_t) * col_slot.size(),
                             hipMemcpyHostToDevice, st)) != hipSuccess) ||
        (col_row.size() > 0 &&
         (e = hipMemcpyAsync(d_row, col_row.data(), sizeof(int32_t) * col_row.size(),
                             hipMemcpyHostToDevice, st)) != hipSuccess) ||
        (long_cols.size() > 0 &&
         (e = hipMemcpyAsync(d_lcols, long_cols.data(), sizeof(int32_t) * long_cols.size(),
                             hipMemcpyHostToDevice, st)) != hipSuccess) ||
        (e = hipMemcpyAsync(d_loff, long_col_off.data(), sizeof(int64_t) * long_col_off.size(),
                            hipMemcpyHostToDevice, st)) != hipSuccess ||
        (trand &&
         (e = hipMemcpyAsync(d_tptr, trand_ptr.data(), sizeof(int64_t) * trand_ptr.size(),
                             hipMemcpyHostToDevice, st)) != hipSuccess) ||
        (trand_slot.size() > 0 &&
         ((e = hipMemcpyAsync(d_tslot, trand_slot.data(), sizeof(int32_t) * trand_slot.size(),
                              hipMemcpyHostToDevice, st)) != hipSuccess ||
          (e = hipMemcpyAsync(d_trow, trand_row.data(), sizeof(int32_t) * trand_row.size(),
                              hipMemcpyHostToDevice, st)) != hipSuccess)) ||
        (e = hipStreamSynchronize(st)) != hipSuccess) {
        hipFree(d_ptr);
        hipFree(d_off);
        hipFree(d_slot);
        hipFree(d_row);
        hipFree(d_lcols);
        hipFree(d_loff);
        hipFree(d_tptr);
        hipFree(d_tslot);
        hipFree(d_trow);
        return hip_fail(e, "upload of the column index");
    }
    g->d_long_cols = d_lcols;
    g->d_long_col_off = d_loff;
    g->max_long_col = max_long_col;
    g->d_col_ptr = d_ptr;
    g->d_col_off_slots = d_off;
    g->d_col_slot = d_slot;
    g->d_col_row = d_row;
    g->d_trand_ptr = d_tptr;
    g->d_trand_slot = d_tslot;
    g->d_trand_row = d_trow;
    return DIFFUSER_OK;
}

// Lists the graph's long rows (more than kLongRow slots) for the generic
// kernels' long-row companions. Enqueued on `st`; synchronises it.
diffuser_status build_long_rows(diffuser_graph* g, hipStream_t st) {
    const int32_t G = g->num_graphs;
    const int64_t n = g->n;
    g->long_off.assign(G + 1, 0);
    g->max_long = 0;
    const int64_t bound = g->max_row_slots + (g->rand_apart() ? g->rnd_width : 0);
    int32_t* flags = nullptr;
    int64_t *offsets = nullptr, *dmax = nullptr;
    hipError_t e;
    struct tmp_guard {
        void* p[3];
        ~tmp_guard() {
            for (void* q : p) hipFree(q);
        }
    };
    std::vector<int64_t> totals(G, 0);
    if (bound > kLongRow) {
        if ((e = dev_alloc(&flags, (size_t)G * n)) != hipSuccess ||
            (e = dev_alloc(&offsets, (size_t)G * (n + 1))) != hipSuccess ||
            (e = dev_alloc(&dmax, (size_t)G)) != hipSuccess) {
            hipFree(flags);
            hipFree(offsets);
            hipFree(dmax);
            return alloc_status(e, "device allocation for the long-row list");
        }
    }
    tmp_guard tmps{{flags, offsets, dmax}};
    if (bound > kLongRow) {
        if ((e = launch_long_flags(*g, flags, st)) != hipSuccess ||
            (e = launch_scan(n, G, flags, offsets, dmax, st)) != hipSuccess)
            return hip_fail(e, "long-row flag launch");
        for (int32_t gr = 0; gr < G; ++gr)
            if ((e = hipMemcpyAsync(&totals[gr], offsets + (int64_t)gr * (n + 1) + n,
                                    sizeof(int64_t), hipMemcpyDeviceToHost, st)) != hipSuccess)
                return hip_fail(e, "copy of long-row counts");
        if ((e = hipStreamSynchronize(st)) != hipSuccess) return hip_fail(e, "long-row count");
    }
    for (int32_t gr = 0; gr < G; ++gr) {
        g->long_off[gr + 1] = g->long_off[gr] + totals[gr];
        g->max_long = std::max(g->max_long, totals[gr]);
    }
    if ((e = dev_alloc(&g->d_long_rows, (size_t)g->long_off[G])) != hipSuccess ||
        (e = dev_alloc(&g->d_long_off, (size_t)G + 1)) != hipSuccess)
        return alloc_status(e, "device allocation of the long-row list");
    if ((e = hipMemcpyAsync(g->d_long_off, g->long_off.data(), sizeof(int64_t) * (G + 1),
                            hipMemcpyHostToDevice, st)) != hipSuccess)
        return hip_fail(e, "copy of long-row offsets");
    if (g->max_long > 0 && (e = launch_long_fill(*g, flags, offsets, st)) != hipSuccess)
        return hip_fail(e, "long-row fill launch");
    if ((e = hipStreamSynchronize(st)) != hipSuccess) return hip_fail(e, "long-row list");
    return DIFFUSER_OK;
}

// Builds the slot -> CSR position map (once, under bw_mutex) with one
// kernel on `st`, then waits for it.
diffuser_status ensure_slot_csr(diffuser_graph* g, hipStream_t st) {
    std::lock_guard<std::mutex> lock(g->bw_mutex);
    if (g->d_slot_csr != nullptr) return DIFFUSER_OK;
    for (int64_t e : g->nnz)
        if (e >= (1ll << 31))
            return fail(DIFFUSER_ERR_INVALID_ARG, "CSR order needs fewer than 2^31 edges per graph");
    int32_t* map = nullptr;
    hipError_t e = dev_alloc(&map, (size_t)g->slot_off[g->num_graphs]);
    if (e != hipSuccess) return alloc_status(e, "device allocation of the slot -> CSR map");
    if ((e = launch_slot_csr(*g, map, st)) != hipSuccess ||
        (e = hipStreamSynchronize(st)) != hipSuccess) {
        hipFree(map);
        return hip_fail(e, "slot -> CSR map build");
    }
    g->d_slot_csr = map;
    return DIFFUSER_OK;
}

// Edges of all (b, h) blocks in CSR order.
int64_t total_csr_elems(const diffuser_graph* g, int32_t B, int32_t H) {
    if (g->num_graphs == 1) return (int64_t)B * H * g->nnz[0];
    return (int64_t)H * g->col_off[g->num_graphs];
}

// Workspace of diffuser_layer_forward: the [B*n][3 H d] projection (reused
// for the merged heads), Q, K, V, Z, the whole path's own workspace and
// the GEMM library's workspace.
constexpr size_t kBlasWorkspace = (size_t)32 << 20;

struct layer_layout {
    size_t t, h, attn, total;
};

layer_layout make_layer_layout(const diffuser_graph* g, int32_t B, int32_t H, int32_t d,
                               diffuser_dtype dtype) {
    layer_layout w;
    const size_t es = elem_size(dtype);
    w.t = align_up((size_t)B * g->n * 3 * H * d * es);
    w.h = align_up((size_t)B * H * g->n * d * es);
    w.attn = layout(g, B, H, d, dtype).total;
    w.total = w.t + 4 * w.h + w.attn + kBlasWorkspace;
    return w;
}

}  // namespace

diffuser_status fail(diffuser_status s, const std::string& msg) {
    g_last_error = msg;
    return s;
}

}  // namespace diffuser

using namespace diffuser;

extern "C" {

const char* diffuser_status_string(diffuser_status s) {
    switch (s) {
        case DIFFUSER_OK: return "DIFFUSER_OK";
        case DIFFUSER_ERR_INVALID_ARG: return "DIFFUSER_ERR_INVALID_ARG";
        case DIFFUSER_ERR_UNSUPPORTED: return "DIFFUSER_ERR_UNSUPPORTED";
        case DIFFUSER_ERR_OUT_OF_MEMORY: return "DIFFUSER_ERR_OUT_OF_MEMORY";
        case DIFFUSER_ERR_HIP: return "DIFFUSER_ERR_HIP";
        case DIFFUSER_ERR_INTERNAL: return "DIFFUSER_ERR_INTERNAL";
    }
    return "DIFFUSER_ERR_UNKNOWN";
}

const char* diffuser_last_error(void) { return g_last_error.c_str(); }

diffuser_status diffuser_build_graph(const diffuser_graph_desc* desc, void* stream,
                                     diffuser_graph** out) {
    return diffuser_build_graph_layout(desc, DIFFUSER_EXTRAS_RANDOM, stream, out);
}

diffuser_status diffuser_build_graph_layout(const diffuser_graph_desc* desc, int32_t layout,
                                            void* stream, diffuser_graph** out) {
    g_last_error.clear();
    if (!desc || !out) return fail(DIFFUSER_ERR_INVALID_ARG, "desc and out must be non-NULL");
    if (layout != DIFFUSER_EXTRAS_RANDOM && layout != DIFFUSER_EXTRAS_EVEN)
        return fail(DIFFUSER_ERR_INVALID_ARG, "layout must be DIFFUSER_EXTRAS_RANDOM or _EVEN");
    const int64_t n = desc->n;
    if (n < 1 || n > kMaxN) return fail(DIFFUSER_ERR_INVALID_ARG, "n must lie in [1, 2^24]");
    if (desc->window_radius < 0) return fail(DIFFUSER_ERR_INVALID_ARG, "window_radius < 0");
    if (desc->num_global < 0 || desc->num_global > n)
        return fail(DIFFUSER_ERR_INVALID_ARG, "num_global must lie in [0, n]");
    if (desc->num_global > 0 && !desc->global_idx)
        return fail(DIFFUSER_ERR_INVALID_ARG, "global_idx is NULL");
    for (int32_t k = 0; k < desc->num_global; ++k) {
        const int32_t p = desc->global_idx[k];
        if (p < 0 || p >= n) return fail(DIFFUSER_ERR_INVALID_ARG, "global index out of range");
        if (k > 0 && p <= desc->global_idx[k - 1])
            return fail(DIFFUSER_ERR_INVALID_ARG, "global_idx must be strictly increasing");
    }
    if (desc->num_random < 0) return fail(DIFFUSER_ERR_INVALID_ARG, "num_random < 0");
    if (desc->num_graphs < 1 || desc->num_graphs > 65535)
        return fail(DIFFUSER_ERR_INVALID_ARG, "num_graphs must lie in [1, 65535]");
    if (desc->causal != 0 && desc->causal != 1)
        return fail(DIFFUSER_ERR_INVALID_ARG, "causal must be 0 or 1");
    if ((int64_t)desc->num_graphs * n >= (1ll << 44))
        return fail(DIFFUSER_ERR_INVALID_ARG, "num_graphs * n too large for the draw counter");
    if (desc->num_random > kMaxSampledRandom &&
        max_pool(n, desc->window_radius, desc->global_idx, desc->num_global) > desc->num_random)
        return fail(DIFFUSER_ERR_UNSUPPORTED,
                    "num_random above 1024 with a pool larger than the budget");

    hipStream_t st = static_cast<hipStream_t>(stream);
    diffuser_graph* g = new (std::nothrow) diffuser_graph();
    if (!g) return fail(DIFFUSER_ERR_OUT_OF_MEMORY, "host allocation of the graph");
    graph_guard guard{g};
    g->n = n;
    g->num_graphs = desc->num_graphs;
    g->structured = true;
    g->radius = desc->window_radius;
    g->num_global = desc->num_global;
    g->num_random = desc->num_random;
    g->rnd_width = (int32_t)std::min<int64_t>(desc->num_random, n);
    g->causal = desc->causal;
    g->seed = desc->seed;
    g->random_layout = layout;
    g->scheduled = n <= kMaxScheduledN;
    g->rand_layout = !g->scheduled        ? diffuser_graph::RandLayout::kRow
                     : n <= kMaxResidentN ? diffuser_graph::RandLayout::kOctet
                                          : diffuser_graph::RandLayout::kGroup;
    g->key_batches = ((g->rnd_width + 7) / 8 + kOctBatch - 1) / kOctBatch;
    hipGetDevice(&g->device);

    const int64_t rows = (int64_t)g->num_graphs * n;
    const int64_t nrb = (n + kRowBlock - 1) / kRowBlock;
    int32_t* d_deg = nullptr;
    int32_t* d_slots = nullptr;
    int32_t* d_status = nullptr;
    int64_t* d_max = nullptr;
    int32_t* d_gcount = nullptr;
    hipError_t e;
    // Globals below the start of every key chunk (G is ascending).
    const int64_t nchunks = (n + kChunkRows - 1) / kChunkRows;
    std::vector<int32_t> gchunk((size_t)nchunks + 1);
    for (int64_t c = 0; c <= nchunks; ++c)
        gchunk[c] = (int32_t)(std::lower_bound(desc->global_idx, desc->global_idx + g->num_global,
                                               (int64_t)c * kChunkRows) - desc->global_idx);
    if ((e = dev_alloc(&g->d_global, g->num_global)) != hipSuccess ||
        (e = dev_alloc(&g->d_gchunk, (size_t)nchunks + 1)) != hipSuccess ||
        (e = dev_alloc(&g->d_rnd, (size_t)rows * std::max(g->rnd_width, 1))) != hipSuccess ||
        (e = dev_alloc(&g->d_rslot, (size_t)rows * std::max(g->rnd_width, 1))) != hipSuccess ||
        (e = dev_alloc(&g->d_row_info, (size_t)rows * 4)) != hipSuccess ||
        (e = dev_alloc(&g->d_rnd_cnt, rows)) != hipSuccess ||
        (e = dev_alloc(&g->d_row_ptr, (size_t)g->num_graphs * (n + 1))) != hipSuccess ||
        (e = dev_alloc(&g->d_col_off, g->num_graphs + 1)) != hipSuccess ||
        (e = dev_alloc(&g->d_seg_ptr, (size_t)g->num_graphs * (n + 1))) != hipSuccess ||
        (e = dev_alloc(&g->d_slot_off, g->num_graphs + 1)) != hipSuccess ||
        (e = dev_alloc(&g->d_grp_ptr, (size_t)g->num_graphs * (nrb + 1))) != hipSuccess ||
        (e = dev_alloc(&g->d_grp_off, g->num_graphs + 1)) != hipSuccess ||
        (e = dev_alloc(&d_deg, rows)) != hipSuccess ||
        (e = dev_alloc(&d_slots, rows)) != hipSuccess ||
        (e = dev_alloc(&d_status, 1)) != hipSuccess ||
        (e = dev_alloc(&d_max, 4 * (size_t)g->num_graphs)) != hipSuccess ||
        (e = dev_alloc(&d_gcount, (size_t)g->num_graphs * nrb)) != hipSuccess ||
        (g->octet() &&
         ((e = dev_alloc(&g->d_rb_oct, (size_t)g->num_graphs * nrb)) != hipSuccess ||
          (e = dev_alloc(&g->d_rb_roff, (size_t)g->num_graphs * (nrb + 1))) != hipSuccess))) {
        hipFree(d_deg);
        hipFree(d_slots);
        hipFree(d_status);
        hipFree(d_max);
        hipFree(d_gcount);
        return alloc_status(e, "device allocation for the graph build");
    }
    struct tmp_guard {
        void* p[5];
        ~tmp_guard() {
            for (void* q : p) hipFree(q);
        }
    } tmps{{d_deg, d_slots, d_status, d_max, d_gcount}};

    if (g->num_global > 0 &&
        (e = hipMemcpyAsync(g->d_global, desc->global_idx, sizeof(int32_t) * g->num_global,
                            hipMemcpyHostToDevice, st)) != hipSuccess)
        return hip_fail(e, "copy of global_idx");
    if ((e = hipMemcpyAsync(g->d_gchunk, gchunk.data(), sizeof(int32_t) * gchunk.size(),
                            hipMemcpyHostToDevice, st)) != hipSuccess)
        return hip_fail(e, "copy of the global chunk table");
    if ((e = hipMemsetAsync(d_status, 0, sizeof(int32_t), st)) != hipSuccess)
        return hip_fail(e, "status clear");
    if ((e = launch_draw(*g, d_deg, d_slots, d_status, st)) != hipSuccess)
        return hip_fail(e, "draw launch");
    if ((e = launch_scan(n, g->num_graphs, d_deg, g->d_row_ptr, d_max, st)) != hipSuccess ||
        (e = launch_scan(n, g->num_graphs, d_slots, g->d_seg_ptr, d_max + g->num_graphs, st)) !=
            hipSuccess)
        return hip_fail(e, "scan launch");
    if (g->scheduled &&
        ((e = launch_sched_count(*g, d_gcount, st)) != hipSuccess ||
         (e = launch_scan(nrb, g->num_graphs, d_gcount, g->d_grp_ptr, d_max + 2 * g->num_graphs,
                          st)) != hipSuccess))
        return hip_fail(e, "schedule count launch");
    if (g->octet() && (e = launch_rb_octets(*g, d_max + 3 * g->num_graphs, st)) != hipSuccess)
        return hip_fail(e, "random octet count launch");
    int32_t status = 0;
    std::vector<int64_t> maxes(3 * (size_t)g->num_graphs);
    std::vector<int64_t> last_e(g->num_graphs), last_s(g->num_graphs), last_g(g->num_graphs, 0);
    g->octets.assign(g->num_graphs, 0);
    if ((e = hipMemcpyAsync(&status, d_status, sizeof(int32_t), hipMemcpyDeviceToHost, st)) !=
            hipSuccess ||
        (e = hipMemcpyAsync(maxes.data(), d_max, sizeof(int64_t) * 2 * g->num_graphs,
                            hipMemcpyDeviceToHost, st)) != hipSuccess)
        return hip_fail(e, "copy of build status");
    for (int32_t gr = 0; gr < g->num_graphs; ++gr) {
        if ((e = hipMemcpyAsync(&last_e[gr], g->d_row_ptr + (int64_t)gr * (n + 1) + n,
                                sizeof(int64_t), hipMemcpyDeviceToHost, st)) != hipSuccess ||
            (e = hipMemcpyAsync(&last_s[gr], g->d_seg_ptr + (int64_t)gr * (n + 1) + n,
                                sizeof(int64_t), hipMemcpyDeviceToHost, st)) != hipSuccess ||
            (g->scheduled &&
             (e = hipMemcpyAsync(&last_g[gr], g->d_grp_ptr + (int64_t)gr * (nrb + 1) + nrb,
                                 sizeof(int64_t), hipMemcpyDeviceToHost, st)) != hipSuccess) ||
            (g->octet() &&
             (e = hipMemcpyAsync(&g->octets[gr], g->d_rb_roff + (int64_t)gr * (nrb + 1) + nrb,
                                 sizeof(int64_t), hipMemcpyDeviceToHost, st)) != hipSuccess))
            return hip_fail(e, "copy of edge counts");
    }
    if ((e = hipStreamSynchronize(st)) != hipSuccess) return hip_fail(e, "graph draw");
    if (status != 0)
        return fail(DIFFUSER_ERR_INTERNAL, "random draw budget (2^20 draws per row) exhausted");
    g->nnz = last_e;
    g->groups = last_g;
    g->slots.assign(g->num_graphs, 0);
    g->col_off.assign(g->num_graphs + 1, 0);
    g->slot_off.assign(g->num_graphs + 1, 0);
    g->grp_off.assign(g->num_graphs + 1, 0);
    for (int32_t gr = 0; gr < g->num_graphs; ++gr) {
        g->slots[gr] = last_s[gr] + (g->grouped() ? (int64_t)kGroupSlots * last_g[gr]
                                     : g->octet() ? 8 * kRowBlock * g->octets[gr]
                                                  : 0);
        g->col_off[gr + 1] = g->col_off[gr] + last_e[gr];
        g->slot_off[gr + 1] = g->slot_off[gr] + g->slots[gr];
        g->grp_off[gr + 1] = g->grp_off[gr] + last_g[gr];
    }
    g->max_row_len = *std::max_element(maxes.begin(), maxes.begin() + g->num_graphs);
    g->max_row_slots =
        *std::max_element(maxes.begin() + g->num_graphs, maxes.begin() + 2 * g->num_graphs);
    const int64_t ngroups = g->grp_off[g->num_graphs];
    if ((e = dev_alloc(&g->d_col_idx, g->col_off[g->num_graphs])) != hipSuccess ||
        (e = dev_alloc(&g->d_slot_col, g->slot_off[g->num_graphs])) != hipSuccess ||
        (e = dev_alloc(&g->d_slot_row, g->slot_off[g->num_graphs])) != hipSuccess ||
        (e = dev_alloc(&g->d_grp_cptr, g->scheduled ? (size_t)g->num_graphs * nrb *
                                                          ((n + kChunkRows - 1) / kChunkRows + 1)
                                                    : 1)) != hipSuccess ||
        (e = dev_alloc(&g->d_sched_row, (size_t)ngroups * 4)) != hipSuccess ||
        (e = dev_alloc(&g->d_sched_j, (size_t)ngroups * 16)) != hipSuccess ||
        (e = dev_alloc(&g->d_sched_k, (size_t)ngroups * kGroupSlots)) != hipSuccess ||
        (e = dev_alloc(&g->d_sched_off, (size_t)ngroups * 16)) != hipSuccess)
        return alloc_status(e, "device allocation of the columns");
    if ((e = hipMemcpyAsync(g->d_col_off, g->col_off.data(), sizeof(int64_t) * (g->num_graphs + 1),
                            hipMemcpyHostToDevice, st)) != hipSuccess ||
        (e = hipMemcpyAsync(g->d_slot_off, g->slot_off.data(),
                            sizeof(int64_t) * (g->num_graphs + 1), hipMemcpyHostToDevice, st)) !=
            hipSuccess ||
        (e = hipMemcpyAsync(g->d_grp_off, g->grp_off.data(),
                            sizeof(int64_t) * (g->num_graphs + 1), hipMemcpyHostToDevice, st)) !=
            hipSuccess)
        return hip_fail(e, "copy of offsets");
    if ((e = launch_fill(*g, st)) != hipSuccess) return hip_fail(e, "fill launch");
    if (g->scheduled && (e = launch_sched_fill(*g, st)) != hipSuccess)
        return hip_fail(e, "schedule fill launch");
    if (g->octet()) {
        // Tables of the resident-slice diffusion step; d_gcount (graphs x nrb
        // int32) is free again and holds the row-block costs.
        // 64 lanes x 8 uint16 entries per (row block, batch).
        if ((e = dev_alloc(&g->d_rkey, (size_t)g->num_graphs * nrb * g->key_batches * 512)) !=
                hipSuccess ||
            (e = dev_alloc(&g->d_rb_cost, (size_t)g->num_graphs * (nrb + 1))) != hipSuccess ||
            (e = dev_alloc(&g->d_rb_cost_max, (size_t)g->num_graphs)) != hipSuccess)
            return alloc_status(e, "device allocation of the resident tables");
        if ((e = launch_res_tables(*g, d_gcount, st)) != hipSuccess)
            return hip_fail(e, "resident tables launch");
    }
    if ((e = hipStreamSynchronize(st)) != hipSuccess) return hip_fail(e, "graph fill");
    if (auto s = build_long_rows(g, st)) return s;
    guard.g = nullptr;
    *out = g;
    return DIFFUSER_OK;
}

diffuser_status diffuser_graph_from_csr(int64_t n, int32_t num_graphs, const int64_t* row_ptr_host,
                                        const int32_t* col_idx_host, void* stream,
                                        diffuser_graph** out) {
    g_last_error.clear();
    if (!out || !row_ptr_host) return fail(DIFFUSER_ERR_INVALID_ARG, "NULL argument");
    if (n < 1 || n > kMaxN) return fail(DIFFUSER_ERR_INVALID_ARG, "n must lie in [1, 2^24]");
    if (num_graphs < 1 || num_graphs > 65535)
        return fail(DIFFUSER_ERR_INVALID_ARG, "num_graphs must lie in [1, 65535]");
    std::vector<int64_t> nnz(num_graphs), col_off(num_graphs + 1, 0);
    int64_t max_len = 0;
    for (int32_t gr = 0; gr < num_graphs; ++gr) {
        const int64_t* rp = row_ptr_host + (int64_t)gr * (n + 1);
        if (rp[0] != 0) return fail(DIFFUSER_ERR_INVALID_ARG, "row_ptr must start at 0");
        for (int64_t i = 0; i < n; ++i) {
            if (rp[i + 1] < rp[i]) return fail(DIFFUSER_ERR_INVALID_ARG, "row_ptr decreasing");
            max_len = std::max(max_len, rp[i + 1] - rp[i]);
        }
        nnz[gr] = rp[n];
        col_off[gr + 1] = col_off[gr] + rp[n];
    }
    if (col_off[num_graphs] > 0 && !col_idx_host)
        return fail(DIFFUSER_ERR_INVALID_ARG, "col_idx is NULL");
    if (col_off[num_graphs] >= (1ll << 40))
        return fail(DIFFUSER_ERR_INVALID_ARG, "too many edges");
    for (int32_t gr = 0; gr < num_graphs; ++gr) {
        const int64_t* rp = row_ptr_host + (int64_t)gr * (n + 1);
        const int32_t* c = col_idx_host + col_off[gr];
        for (int64_t i = 0; i < n; ++i) {
            bool self = false;
            for (int64_t e = rp[i]; e < rp[i + 1]; ++e) {
                if (c[e] < 0 || c[e] >= n)
                    return fail(DIFFUSER_ERR_INVALID_ARG, "column index out of range");
                if (e > rp[i] && c[e] <= c[e - 1])
                    return fail(DIFFUSER_ERR_INVALID_ARG, "row columns must be strictly ascending");
                self |= c[e] == i;
            }
            if (!self) return fail(DIFFUSER_ERR_INVALID_ARG, "every row needs its self edge");
        }
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    diffuser_graph* g = new (std::nothrow) diffuser_graph();
    if (!g) return fail(DIFFUSER_ERR_OUT_OF_MEMORY, "host allocation of the graph");
    graph_guard guard{g};
    g->n = n;
    g->num_graphs = num_graphs;
    g->structured = false;
    g->nnz = nnz;
    g->col_off = col_off;
    g->max_row_len = max_len;
    // The weight slots of an imported graph are its CSR entries.
    g->slots = nnz;
    g->slot_off = col_off;
    g->max_row_slots = max_len;
    hipGetDevice(&g->device);
    hipError_t e;
    const size_t rp_bytes = sizeof(int64_t) * num_graphs * (n + 1);
    const size_t ci_bytes = sizeof(int32_t) * col_off[num_graphs];
    const size_t off_bytes = sizeof(int64_t) * (num_graphs + 1);
    // Row of every edge (the slot_row of an imported graph).
    std::vector<int32_t> edge_row((size_t)col_off[num_graphs]);
    for (int32_t gr = 0; gr < num_graphs; ++gr) {
        const int64_t* rp = row_ptr_host + (int64_t)gr * (n + 1);
        for (int64_t i = 0; i < n; ++i)
            for (int64_t q = rp[i]; q < rp[i + 1]; ++q) edge_row[col_off[gr] + q] = (int32_t)i;
    }
    if ((e = dev_alloc(&g->d_row_ptr, (size_t)num_graphs * (n + 1))) != hipSuccess ||
        (e = dev_alloc(&g->d_col_idx, col_off[num_graphs])) != hipSuccess ||
        (e = dev_alloc(&g->d_col_off, num_graphs + 1)) != hipSuccess ||
        (e = dev_alloc(&g->d_seg_ptr, (size_t)num_graphs * (n + 1))) != hipSuccess ||
        (e = dev_alloc(&g->d_slot_col, col_off[num_graphs])) != hipSuccess ||
        (e = dev_alloc(&g->d_slot_row, col_off[num_graphs])) != hipSuccess ||
        (e = dev_alloc(&g->d_slot_off, num_graphs + 1)) != hipSuccess)
        return alloc_status(e, "device allocation of the imported graph");
    if ((e = hipMemcpyAsync(g->d_row_ptr, row_ptr_host, rp_bytes, hipMemcpyHostToDevice, st)) !=
            hipSuccess ||
        (e = hipMemcpyAsync(g->d_seg_ptr, row_ptr_host, rp_bytes, hipMemcpyHostToDevice, st)) !=
            hipSuccess ||
        (ci_bytes > 0 &&
         ((e = hipMemcpyAsync(g->d_col_idx, col_idx_host, ci_bytes, hipMemcpyHostToDevice, st)) !=
              hipSuccess ||
          (e = hipMemcpyAsync(g->d_slot_col, col_idx_host, ci_bytes, hipMemcpyHostToDevice, st)) !=
              hipSuccess ||
          (e = hipMemcpyAsync(g->d_slot_row, edge_row.data(), ci_bytes, hipMemcpyHostToDevice,
                              st)) != hipSuccess)) ||
        (e = hipMemcpyAsync(g->d_col_off, col_off.data(), off_bytes, hipMemcpyHostToDevice, st)) !=
            hipSuccess ||
        (e = hipMemcpyAsync(g->d_slot_off, col_off.data(), off_bytes, hipMemcpyHostToDevice,
                            st)) != hipSuccess)
        return hip_fail(e, "copy of the imported graph");
    if ((e = hipStreamSynchronize(st)) != hipSuccess) return hip_fail(e, "graph import");
    if (auto s = build_long_rows(g, st)) return s;
    guard.g = nullptr;
    *out = g;
    return DIFFUSER_OK;
}

diffuser_status diffuser_build_block_graph(const diffuser_block_graph_desc* desc, void* stream,
                                          diffuser_graph** out) {
    g_last_error.clear();
    if (!desc || !out) return fail(DIFFUSER_ERR_INVALID_ARG, "NULL argument");
    const int64_t n = desc->n;
    if (n < 1 || n > kMaxN) return fail(DIFFUSER_ERR_INVALID_ARG, "n must lie in [1, 2^24]");
    if (desc->block < 1 || n % desc->block != 0)
        return fail(DIFFUSER_ERR_INVALID_ARG, "block must be >= 1 and divide n");
    const int64_t N = n / desc->block;
    if (desc->local_blocks < 1 || desc->local_blocks % 2 == 0)
        return fail(DIFFUSER_ERR_INVALID_ARG, "local_blocks must be odd and >= 1");
    if (desc->num_global_blocks < 0 || desc->num_global_blocks > N)
        return fail(DIFFUSER_ERR_INVALID_ARG, "num_global_blocks must lie in [0, n / block]");
    if (desc->num_random_blocks < 0)
        return fail(DIFFUSER_ERR_INVALID_ARG, "num_random_blocks must be >= 0");
    if (desc->num_graphs < 1 || desc->num_graphs > 65535)
        return fail(DIFFUSER_ERR_INVALID_ARG, "num_graphs must lie in [1, 65535]");
    if (N > (1 << 20)) return fail(DIFFUSER_ERR_INVALID_ARG, "too many blocks");
    std::vector<std::vector<int32_t>> keys;
    if (!build_block_lists(N, desc->local_blocks, desc->num_random_blocks,
                           desc->num_global_blocks, desc->num_graphs, desc->seed, keys))
        return fail(DIFFUSER_ERR_INTERNAL, "random block draws exceeded their budget");
    int64_t total = 0;
    for (const auto& ks : keys) total += (int64_t)ks.size() * desc->block * desc->block;
    if (total >= (1ll << 40)) return fail(DIFFUSER_ERR_INVALID_ARG, "too many edges");
    std::vector<int64_t> row_ptr;
    std::vector<int32_t> cols;
    block_lists_to_csr(n, desc->block, desc->num_graphs, keys, row_ptr, cols);
    diffuser_graph* g = nullptr;
    if (auto s = diffuser_graph_from_csr(n, desc->num_graphs, row_ptr.data(), cols.data(), stream,
                                         &g))
        return s;
    graph_guard guard{g};
    // Block lists: d_bptr per graph with absolute indices into d_bcol.
    std::vector<int32_t> bptr((size_t)desc->num_graphs * (N + 1)), bcol;
    int32_t longest = 0;
    for (int64_t gr = 0; gr < desc->num_graphs; ++gr)
        for (int64_t I = 0; I < N; ++I) {
            const auto& ks = keys[(size_t)(gr * N + I)];
            bptr[(size_t)(gr * (N + 1) + I)] = (int32_t)bcol.size();
            bcol.insert(bcol.end(), ks.begin(), ks.end());
            longest = std::max(longest, (int32_t)ks.size());
            if (I + 1 == N) bptr[(size_t)(gr * (N + 1) + N)] = (int32_t)bcol.size();
        }
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e;
    if ((e = dev_alloc(&g->d_bptr, bptr.size())) != hipSuccess ||
        (e = dev_alloc(&g->d_bcol, bcol.size())) != hipSuccess)
        return alloc_status(e, "device allocation of the block lists");
    if ((e = hipMemcpyAsync(g->d_bptr, bptr.data(), sizeof(int32_t) * bptr.size(),
                            hipMemcpyHostToDevice, st)) != hipSuccess ||
        (e = hipMemcpyAsync(g->d_bcol, bcol.data(), sizeof(int32_t) * bcol.size(),
                            hipMemcpyHostToDevice, st)) != hipSuccess)
        return hip_fail(e, "copy of the block lists");
    if ((e = hipStreamSynchronize(st)) != hipSuccess) return hip_fail(e, "block graph build");
    g->blocked = true;
    g->block = desc->block;
    g->nblocks = N;
    g->max_key_blocks = longest;
    g->global_blocks = desc->num_global_blocks;
    guard.g = nullptr;
    *out = g;
    return DIFFUSER_OK;
}

diffuser_status diffuser_build_dilated_graph(int64_t n, int32_t radius, int32_t dilation,
                                            int32_t num_global, const int32_t* global_idx,
                                            void* stream, diffuser_graph** out) {
    g_last_error.clear();
    if (!out) return fail(DIFFUSER_ERR_INVALID_ARG, "NULL argument");
    if (n < 1 || n > kMaxN) return fail(DIFFUSER_ERR_INVALID_ARG, "n must lie in [1, 2^24]");
    if (radius < 0 || dilation < 1)
        return fail(DIFFUSER_ERR_INVALID_ARG, "radius must be >= 0 and dilation >= 1");
    if (num_global < 0 || num_global > n)
        return fail(DIFFUSER_ERR_INVALID_ARG, "num_global must lie in [0, n]");
    if (num_global > 0 && !global_idx) return fail(DIFFUSER_ERR_INVALID_ARG, "global_idx is NULL");
    for (int32_t q = 0; q < num_global; ++q)
        if (global_idx[q] < 0 || global_idx[q] >= n || (q > 0 && global_idx[q] <= global_idx[q - 1]))
            return fail(DIFFUSER_ERR_INVALID_ARG,
                        "global_idx must be strictly increasing in [0, n)");
    if ((int64_t)num_global * n + n * (2 * (int64_t)radius + 1) >= (1ll << 40))
        return fail(DIFFUSER_ERR_INVALID_ARG, "too many edges");
    std::vector<int64_t> row_ptr;
    std::vector<int32_t> cols;
    dilated_csr(n, radius, dilation, global_idx, num_global, row_ptr, cols);
    return diffuser_graph_from_csr(n, 1, row_ptr.data(), cols.data(), stream, out);
}

diffuser_status diffuser_graph_info(const diffuser_graph* g, int64_t* n, int32_t* num_graphs,
                                    int64_t* nnz, int64_t* slots) {
    g_last_error.clear();
    if (auto s = check_graph(g)) return s;
    if (n) *n = g->n;
    if (num_graphs) *num_graphs = g->num_graphs;
    if (nnz) std::copy(g->nnz.begin(), g->nnz.end(), nnz);
    if (slots) std::copy(g->slots.begin(), g->slots.end(), slots);
    return DIFFUSER_OK;
}

diffuser_status diffuser_graph_copy_slots(const diffuser_graph* g, int32_t graph,
                                          int32_t* slot_row_host, int32_t* slot_col_host,
                                          void* stream) {
    g_last_error.clear();
    if (auto s = check_graph(g)) return s;
    if (graph < 0 || graph >= g->num_graphs)
        return fail(DIFFUSER_ERR_INVALID_ARG, "graph index out of range");
    if (g->slots[graph] > 0 && (!slot_row_host || !slot_col_host))
        return fail(DIFFUSER_ERR_INVALID_ARG, "NULL output array");
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e;
    const size_t bytes = sizeof(int32_t) * g->slots[graph];
    if (g->slots[graph] > 0 &&
        ((e = hipMemcpyAsync(slot_row_host, g->d_slot_row + g->slot_off[graph], bytes,
                             hipMemcpyDeviceToHost, st)) != hipSuccess ||
         (e = hipMemcpyAsync(slot_col_host, g->d_slot_col + g->slot_off[graph], bytes,
                             hipMemcpyDeviceToHost, st)) != hipSuccess))
        return hip_fail(e, "copy of the slot layout");
    if ((e = hipStreamSynchronize(st)) != hipSuccess) return hip_fail(e, "slot layout copy");
    return DIFFUSER_OK;
}

diffuser_status diffuser_graph_copy_csr(const diffuser_graph* g, int32_t graph,
                                        int64_t* row_ptr_host, int32_t* col_idx_host,
                                        void* stream) {
    g_last_error.clear();
    if (auto s = check_graph(g)) return s;
    if (graph < 0 || graph >= g->num_graphs)
        return fail(DIFFUSER_ERR_INVALID_ARG, "graph index out of range");
    if (!row_ptr_host || (!col_idx_host && g->nnz[graph] > 0))
        return fail(DIFFUSER_ERR_INVALID_ARG, "NULL output array");
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e;
    if ((e = hipMemcpyAsync(row_ptr_host, g->d_row_ptr + (int64_t)graph * (g->n + 1),
                            sizeof(int64_t) * (g->n + 1), hipMemcpyDeviceToHost, st)) !=
            hipSuccess ||
        (g->nnz[graph] > 0 &&
         (e = hipMemcpyAsync(col_idx_host, g->d_col_idx + g->col_off[graph],
                             sizeof(int32_t) * g->nnz[graph], hipMemcpyDeviceToHost, st)) !=
             hipSuccess))
        return hip_fail(e, "copy of the CSR");
    if ((e = hipStreamSynchronize(st)) != hipSuccess) return hip_fail(e, "CSR copy");
    return DIFFUSER_OK;
}

void diffuser_graph_destroy(diffuser_graph* g) {
    if (!g) return;
    hipDeviceSynchronize();
    free_graph_memory(g);
    delete g;
}

diffuser_status diffuser_attn_workspace_size(const diffuser_graph* g, int32_t B, int32_t H,
                                             int32_t d_h, int32_t d_v, diffuser_dtype dtype,
                                             size_t* bytes) {
    g_last_error.clear();
    if (!bytes) return fail(DIFFUSER_ERR_INVALID_ARG, "bytes is NULL");
    if (auto s = check_shape(g, B, H, d_h, dtype, "d_h")) return s;
    if (auto s = check_shape(g, B, H, d_v, dtype, "d_v")) return s;
    *bytes = layout(g, B, H, d_v, dtype).total;
    return DIFFUSER_OK;
}

namespace {

// The whole path; theta == nullptr: the PPR recurrence with alpha, else
// the general coefficients theta[0..K_steps].
diffuser_status attn_impl(const void* Q, const void* K, const void* V, diffuser_dtype dtype,
                          int32_t B, int32_t H, int32_t d_h, int32_t d_v, const diffuser_graph* g,
                          int32_t K_steps, float alpha, const float* theta, void* Z,
                          void* workspace, size_t ws_bytes, void* stream) {
    g_last_error.clear();
    if (auto s = check_shape(g, B, H, d_h, dtype, "d_h")) return s;
    if (auto s = check_shape(g, B, H, d_v, dtype, "d_v")) return s;
    if (auto s = theta ? check_theta(K_steps, theta) : check_alpha_k(K_steps, alpha)) return s;
    for (auto pr : {std::make_pair(Q, "Q"), std::make_pair(K, "K"), std::make_pair(V, "V"),
                    std::make_pair((const void*)Z, "Z"), std::make_pair((const void*)workspace,
                                                                          "workspace")})
        if (auto s = check_ptr(pr.first, pr.second)) return s;
    const ws_layout w = layout(g, B, H, d_v, dtype);
    if (ws_bytes < w.total) return fail(DIFFUSER_ERR_INVALID_ARG, "workspace too small");
    const size_t es = elem_size(dtype);
    const size_t qk_bytes = (size_t)B * H * g->n * d_h * es;
    const size_t vz_bytes = (size_t)B * H * g->n * d_v * es;
    if (overlaps(Z, vz_bytes, Q, qk_bytes) || overlaps(Z, vz_bytes, K, qk_bytes) ||
        overlaps(Z, vz_bytes, V, vz_bytes) || overlaps(Z, vz_bytes, workspace, ws_bytes))
        return fail(DIFFUSER_ERR_INVALID_ARG, "Z overlaps an input or the workspace");
    hipStream_t st = static_cast<hipStream_t>(stream);
    char* ws = static_cast<char*>(workspace);
    void* A = ws;
    void* tmp = ws + w.a_bytes;
    float* row_scale = reinterpret_cast<float*>(ws + w.a_bytes + w.z_bytes);
    float* part = reinterpret_cast<float*>(ws + w.a_bytes + w.z_bytes + w.s_bytes);
    const float scale_log2 = (float)(1.0 / std::sqrt((double)d_h) * 1.4426950408889634);
    hipError_t e = launch_scores_softmax(*g, attn_shape{B, H, d_h, dtype}, Q, K, A, row_scale,
                                         scale_log2, st, w.p_bytes ? part : nullptr);
    if (e != hipSuccess) return hip_fail(e, "score/softmax launch");
    if (theta)
        return run_diffusion_theta(g, attn_shape{B, H, d_v, dtype}, A, row_scale, V, Z, tmp, part,
                                   K_steps, theta, st);
    return run_diffusion(g, attn_shape{B, H, d_v, dtype}, A, row_scale, V, Z, tmp, part, K_steps,
                         alpha, st);
}

}  // namespace

diffuser_status diffuser_attn(const void* Q, const void* K, const void* V, diffuser_dtype dtype,
                              int32_t B, int32_t H, int32_t d_h, int32_t d_v,
                              const diffuser_graph* g, int32_t K_steps, float alpha, void* Z,
                              void* workspace, size_t ws_bytes, void* stream) {
    return attn_impl(Q, K, V, dtype, B, H, d_h, d_v, g, K_steps, alpha, nullptr, Z, workspace,
                     ws_bytes, stream);
}

diffuser_status diffuser_attn_theta(const void* Q, const void* K, const void* V,
                                    diffuser_dtype dtype, int32_t B, int32_t H, int32_t d_h,
                                    int32_t d_v, const diffuser_graph* g, int32_t K_steps,
                                    const float* theta, void* Z, void* workspace,
                                    size_t ws_bytes, void* stream) {
    return attn_impl(Q, K, V, dtype, B, H, d_h, d_v, g, K_steps, 0.0f, theta, Z, workspace,
                     ws_bytes, stream);
}

diffuser_status diffuser_scores_softmax(const void* Q, const void* K, diffuser_dtype dtype,
                                        int32_t B, int32_t H, int32_t d_h,
                                        const diffuser_graph* g, void* A_out, void* workspace,
                                        size_t ws_bytes, void* stream) {
    g_last_error.clear();
    (void)workspace;
    (void)ws_bytes;
    if (auto s = check_shape(g, B, H, d_h, dtype, "d_h")) return s;
    if (auto s = check_ptr(Q, "Q")) return s;
    if (auto s = check_ptr(K, "K")) return s;
    if (auto s = check_ptr(A_out, "A_out", false)) return s;
    if (reinterpret_cast<uintptr_t>(A_out) % elem_size(dtype))
        return fail(DIFFUSER_ERR_INVALID_ARG, "A_out is not element aligned");
    const size_t es = elem_size(dtype);
    const size_t qk_bytes = (size_t)B * H * g->n * d_h * es;
    const size_t a_bytes = (size_t)total_a_elems(g, B, H) * es;
    if (overlaps(A_out, a_bytes, Q, qk_bytes) || overlaps(A_out, a_bytes, K, qk_bytes))
        return fail(DIFFUSER_ERR_INVALID_ARG, "A_out overlaps Q or K");
    const float scale_log2 = (float)(1.0 / std::sqrt((double)d_h) * 1.4426950408889634);
    hipError_t e = launch_scores_softmax(*g, attn_shape{B, H, d_h, dtype}, Q, K, A_out, nullptr,
                                         scale_log2, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "score/softmax launch");
    return DIFFUSER_OK;
}

namespace {

// Workspace of diffuser_diffuse(_theta): the Z ping-pong buffer when there
// are two or more steps, then the block-tile step's partial sums whenever a
// diffusion step is launched (theta's nested form launches one even at
// K_steps = 0).
size_t diffuse_ws_need(const diffuser_graph* g, int32_t B, int32_t H, int32_t d_v,
                       diffuser_dtype dtype, int32_t K_steps, bool theta) {
    const size_t z_need = align_up((size_t)B * H * g->n * d_v * elem_size(dtype));
    const bool launches = theta || K_steps >= 1;
    return (K_steps >= 2 ? z_need : 0) + (launches ? part_bytes(g, B, H, d_v, dtype) : 0);
}

diffuser_status diffuse_impl(const void* A, const void* V, diffuser_dtype dtype, int32_t B,
                             int32_t H, int32_t d_v, const diffuser_graph* g, int32_t K_steps,
                             float alpha, const float* theta, void* Z, void* workspace,
                             size_t ws_bytes, void* stream) {
    g_last_error.clear();
    if (auto s = check_shape(g, B, H, d_v, dtype, "d_v")) return s;
    if (auto s = theta ? check_theta(K_steps, theta) : check_alpha_k(K_steps, alpha)) return s;
    if (auto s = check_ptr(A, "A", false)) return s;
    if (reinterpret_cast<uintptr_t>(A) % elem_size(dtype))
        return fail(DIFFUSER_ERR_INVALID_ARG, "A is not element aligned");
    if (auto s = check_ptr(V, "V")) return s;
    if (auto s = check_ptr(Z, "Z")) return s;
    const size_t es = elem_size(dtype);
    const size_t vz_bytes = (size_t)B * H * g->n * d_v * es;
    const size_t a_bytes = (size_t)total_a_elems(g, B, H) * es;
    const size_t z_need = align_up(vz_bytes);
    const size_t ws_need = diffuse_ws_need(g, B, H, d_v, dtype, K_steps, theta != nullptr);
    const size_t p_need = ws_need - (K_steps >= 2 ? z_need : 0);
    if (ws_need > 0) {
        if (auto s = check_ptr(workspace, "workspace")) return s;
        if (ws_bytes < ws_need) return fail(DIFFUSER_ERR_INVALID_ARG, "workspace too small");
    }
    if (overlaps(Z, vz_bytes, A, a_bytes) || overlaps(Z, vz_bytes, V, vz_bytes) ||
        (ws_need > 0 && overlaps(Z, vz_bytes, workspace, ws_need)))
        return fail(DIFFUSER_ERR_INVALID_ARG, "Z overlaps an input or the workspace");
    // The caller's workspace holds the Z ping-pong buffer, then the
    // block-tile step's partial sums.
    float* part = p_need ? reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                                    (K_steps >= 2 ? z_need : 0))
                         : nullptr;
    if (theta)
        return run_diffusion_theta(g, attn_shape{B, H, d_v, dtype}, A, nullptr, V, Z, workspace,
                                   part, K_steps, theta, static_cast<hipStream_t>(stream));
    return run_diffusion(g, attn_shape{B, H, d_v, dtype}, A, nullptr, V, Z, workspace, part,
                         K_steps, alpha, static_cast<hipStream_t>(stream));
}

}  // namespace

diffuser_status diffuser_diffuse_workspace_size(const diffuser_graph* g, int32_t B, int32_t H,
                                                int32_t d_v, int32_t K_steps, diffuser_dtype dtype,
                                                size_t* bytes) {
    g_last_error.clear();
    if (!bytes) return fail(DIFFUSER_ERR_INVALID_ARG, "bytes is NULL");
    if (auto s = check_shape(g, B, H, d_v, dtype, "d_v")) return s;
    if (K_steps < 0) return fail(DIFFUSER_ERR_INVALID_ARG, "K_steps must be >= 0");
    *bytes = diffuse_ws_need(g, B, H, d_v, dtype, K_steps, true);
    return DIFFUSER_OK;
}

// Scratch of diffuser_diffuse_noalloc: a file-scope device array, one copy
// per GPU that the library runs on, kept until the process ends. Host code
// uses only the address hipGetSymbolAddress returns for it on each device.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch (looked up once per device).
diffuser_status scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(DIFFUSER_ERR_INTERNAL, "device index out of range");
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "address of the scratch array");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return DIFFUSER_OK;
}

}  // namespace

diffuser_status diffuser_diffuse_noalloc(const void* A, const void* V, diffuser_dtype dtype,
                                         int32_t B, int32_t H, int32_t d_v,
                                         const diffuser_graph* g, int32_t K_steps, float alpha,
                                         void* Z, void* stream) {
    g_last_error.clear();
    if (auto s = check_shape(g, B, H, d_v, dtype, "d_v")) return s;
    if (K_steps < 0) return fail(DIFFUSER_ERR_INVALID_ARG, "K_steps must be >= 0");
    const size_t need = diffuse_ws_need(g, B, H, d_v, dtype, K_steps, false);
    if (need > kNoAllocScratchBytes)
        return fail(DIFFUSER_ERR_INVALID_ARG,
                    "needs " + std::to_string(need) + " bytes of scratch; the allocation-free "
                    "entry point holds " + std::to_string(kNoAllocScratchBytes));
    void* ws = nullptr;
    if (need > 0)
        if (auto s = scratch_address(&ws)) return s;
    return diffuse_impl(A, V, dtype, B, H, d_v, g, K_steps, alpha, nullptr, Z, ws,
                        need > 0 ? kNoAllocScratchBytes : 0, stream);
}

diffuser_status diffuser_diffuse(const void* A, const void* V, diffuser_dtype dtype, int32_t B,
                                 int32_t H, int32_t d_v, const diffuser_graph* g,
                                 int32_t K_steps, float alpha, void* Z, void* workspace,
                                 size_t ws_bytes, void* stream) {
    return diffuse_impl(A, V, dtype, B, H, d_v, g, K_steps, alpha, nullptr, Z, workspace,
                        ws_bytes, stream);
}

diffuser_status diffuser_diffuse_theta(const void* A, const void* V, diffuser_dtype dtype,
                                       int32_t B, int32_t H, int32_t d_v,
                                       const diffuser_graph* g, int32_t K_steps,
                                       const float* theta, void* Z, void* workspace,
                                       size_t ws_bytes, void* stream) {
    return diffuse_impl(A, V, dtype, B, H, d_v, g, K_steps, 0.0f, theta, Z, workspace, ws_bytes,
                        stream);
}

diffuser_status diffuser_csr_workspace_size(const diffuser_graph* g, int32_t B, int32_t H,
                                            int32_t d, int32_t K_steps, diffuser_dtype dtype,
                                            size_t* bytes) {
    g_last_error.clear();
    if (!bytes) return fail(DIFFUSER_ERR_INVALID_ARG, "bytes is NULL");
    if (auto s = check_shape(g, B, H, d, dtype, "d")) return s;
    if (K_steps < 0) return fail(DIFFUSER_ERR_INVALID_ARG, "K_steps must be >= 0");
    *bytes = align_up((size_t)total_a_elems(g, B, H) * elem_size(dtype)) +
             diffuse_ws_need(g, B, H, d, dtype, K_steps, false);
    return DIFFUSER_OK;
}

diffuser_status diffuser_scores_softmax_csr(const void* Q, const void* K, diffuser_dtype dtype,
                                            int32_t B, int32_t H, int32_t d_h,
                                            const diffuser_graph* g, void* A_csr,
                                            void* workspace, size_t ws_bytes, void* stream) {
    g_last_error.clear();
    if (auto s = check_shape(g, B, H, d_h, dtype, "d_h")) return s;
    if (auto s = check_ptr(A_csr, "A_csr", false)) return s;
    if (reinterpret_cast<uintptr_t>(A_csr) % elem_size(dtype))
        return fail(DIFFUSER_ERR_INVALID_ARG, "A_csr is not element aligned");
    if (auto s = check_ptr(workspace, "workspace")) return s;
    const size_t es = elem_size(dtype);
    const size_t a_need = align_up((size_t)total_a_elems(g, B, H) * es);
    if (ws_bytes < a_need) return fail(DIFFUSER_ERR_INVALID_ARG, "workspace too small");
    const size_t csr_bytes = (size_t)total_csr_elems(g, B, H) * es;
    const size_t qk_bytes = (size_t)B * H * g->n * d_h * es;
    if (overlaps(A_csr, csr_bytes, workspace, a_need) || overlaps(A_csr, csr_bytes, Q, qk_bytes) ||
        overlaps(A_csr, csr_bytes, K, qk_bytes))
        return fail(DIFFUSER_ERR_INVALID_ARG, "A_csr overlaps Q, K or the workspace");
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (auto s = ensure_slot_csr(const_cast<diffuser_graph*>(g), st)) return s;
    // The weights in the slot layout (in the workspace), then permuted.
    if (auto s = diffuser_scores_softmax(Q, K, dtype, B, H, d_h, g, workspace, nullptr, 0, stream))
        return s;
    hipError_t e = launch_slots_csr_permute(*g, B, H, es, workspace, A_csr, true, st);
    if (e != hipSuccess) return hip_fail(e, "slot -> CSR permutation launch");
    return DIFFUSER_OK;
}

diffuser_status diffuser_diffuse_csr(const void* A_csr, const void* V, diffuser_dtype dtype,
                                     int32_t B, int32_t H, int32_t d_v, const diffuser_graph* g,
                                     int32_t K_steps, float alpha, void* Z, void* workspace,
                                     size_t ws_bytes, void* stream) {
    g_last_error.clear();
    if (auto s = check_shape(g, B, H, d_v, dtype, "d_v")) return s;
    if (auto s = check_alpha_k(K_steps, alpha)) return s;
    if (auto s = check_ptr(A_csr, "A_csr", false)) return s;
    if (reinterpret_cast<uintptr_t>(A_csr) % elem_size(dtype))
        return fail(DIFFUSER_ERR_INVALID_ARG, "A_csr is not element aligned");
    if (auto s = check_ptr(workspace, "workspace")) return s;
    const size_t es = elem_size(dtype);
    const size_t a_need = align_up((size_t)total_a_elems(g, B, H) * es);
    const size_t need = a_need + diffuse_ws_need(g, B, H, d_v, dtype, K_steps, false);
    if (ws_bytes < need) return fail(DIFFUSER_ERR_INVALID_ARG, "workspace too small");
    const size_t csr_bytes = (size_t)total_csr_elems(g, B, H) * es;
    const size_t v_bytes = (size_t)B * H * g->n * d_v * es;
    if (overlaps(A_csr, csr_bytes, workspace, need) || overlaps(V, v_bytes, workspace, need))
        return fail(DIFFUSER_ERR_INVALID_ARG, "A_csr or V overlaps the workspace");
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (auto s = ensure_slot_csr(const_cast<diffuser_graph*>(g), st)) return s;
    // The weights into the slot layout at the workspace's start; the rest
    // of it serves the diffusion steps.
    hipError_t e = launch_slots_csr_permute(*g, B, H, es, A_csr, workspace, false, st);
    if (e != hipSuccess) return hip_fail(e, "CSR -> slot permutation launch");
    return diffuse_impl(workspace, V, dtype, B, H, d_v, g, K_steps, alpha, nullptr, Z,
                        static_cast<char*>(workspace) + a_need, ws_bytes - a_need, stream);
}


diffuser_status diffuser_attn_backward_workspace_size(const diffuser_graph* g, int32_t B,
                                                     int32_t H, int32_t d, int32_t K_steps,
                                                     diffuser_dtype dtype, size_t* bytes) {
    g_last_error.clear();
    if (!bytes) return fail(DIFFUSER_ERR_INVALID_ARG, "bytes is NULL");
    if (auto s = check_shape(g, B, H, d, dtype, "d")) return s;
    if (K_steps < 0) return fail(DIFFUSER_ERR_INVALID_ARG, "K_steps must be >= 0");
    *bytes = backward_layout(g, B, H, d, K_steps).total;
    return DIFFUSER_OK;
}

diffuser_status diffuser_attn_backward(const void* Q, const void* K, const void* V,
                                       const void* dZ, diffuser_dtype dtype, int32_t B, int32_t H,
                                       int32_t d, const diffuser_graph* g, int32_t K_steps,
                                       float alpha, void* dQ, void* dK, void* dV, void* workspace,
                                       size_t ws_bytes, void* stream) {
    g_last_error.clear();
    if (auto s = check_shape(g, B, H, d, dtype, "d")) return s;
    if (auto s = check_alpha_k(K_steps, alpha)) return s;
    const size_t bytes = (size_t)B * H * g->n * d * elem_size(dtype);
    const void* ins[4] = {Q, K, V, dZ};
    const void* outs[3] = {dQ, dK, dV};
    const char* in_names[4] = {"Q", "K", "V", "dZ"};
    const char* out_names[3] = {"dQ", "dK", "dV"};
    for (int k = 0; k < 4; ++k)
        if (auto s = check_ptr(ins[k], in_names[k])) return s;
    for (int k = 0; k < 3; ++k)
        if (auto s = check_ptr(outs[k], out_names[k])) return s;
    if (auto s = check_ptr(workspace, "workspace")) return s;
    const bw_layout w = backward_layout(g, B, H, d, K_steps);
    if (ws_bytes < w.total) return fail(DIFFUSER_ERR_INVALID_ARG, "workspace too small");
    for (int k = 0; k < 3; ++k) {
        for (int l = 0; l < 4; ++l)
            if (overlaps(outs[k], bytes, ins[l], bytes))
                return fail(DIFFUSER_ERR_INVALID_ARG, "an output overlaps an input");
        for (int l = k + 1; l < 3; ++l)
            if (overlaps(outs[k], bytes, outs[l], bytes))
                return fail(DIFFUSER_ERR_INVALID_ARG, "outputs overlap");
        if (overlaps(outs[k], bytes, workspace, ws_bytes))
            return fail(DIFFUSER_ERR_INVALID_ARG, "an output overlaps the workspace");
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (auto s = ensure_col_index(const_cast<diffuser_graph*>(g), st)) return s;
    char* ws = static_cast<char*>(workspace);
    BackwardArgs p;
    p.B = B;
    p.H = H;
    p.d = d;
    p.dtype = dtype;
    p.K_steps = K_steps;
    p.alpha = alpha;
    p.scale = (float)(1.0 / std::sqrt((double)d));
    p.Q = Q;
    p.K = K;
    p.V = V;
    p.dZ = dZ;
    p.dQ = dQ;
    p.dK = dK;
    p.dVout = dV;
    p.a_count = total_a_elems(g, B, H);
    p.A = reinterpret_cast<float*>(ws);
    p.dA = reinterpret_cast<float*>(ws + w.a);
    p.At = reinterpret_cast<float*>(ws + 2 * w.a);
    p.Zs = reinterpret_cast<float*>(ws + 3 * w.a);
    p.Gs = reinterpret_cast<float*>(ws + 3 * w.a + w.zs);
    p.dV = reinterpret_cast<float*>(ws + 3 * w.a + w.zs + w.gs);
    const float scale_log2 = (float)(1.0 / std::sqrt((double)d) * 1.4426950408889634);
    // p.dV (B H n d floats) is free until the G steps: the row scales.
    hipError_t e = launch_scores_softmax_f32(*g, attn_shape{B, H, d, dtype}, Q, K, p.A,
                                             scale_log2, st, p.dV);
    if (e != hipSuccess) return hip_fail(e, "score/softmax launch");
    e = launch_backward(*g, p, st);
    if (e != hipSuccess) return hip_fail(e, "backward launch");
    return DIFFUSER_OK;
}

diffuser_status diffuser_layer_workspace_size(const diffuser_graph* g, int32_t B, int32_t H,
                                             int32_t d, int32_t d_model, diffuser_dtype dtype,
                                             size_t* bytes) {
    g_last_error.clear();
    if (!bytes) return fail(DIFFUSER_ERR_INVALID_ARG, "bytes is NULL");
    if (auto s = check_shape(g, B, H, d, dtype, "d")) return s;
    if (d_model < 1) return fail(DIFFUSER_ERR_INVALID_ARG, "d_model must be >= 1");
    *bytes = make_layer_layout(g, B, H, d, dtype).total;
    return DIFFUSER_OK;
}

diffuser_status diffuser_layer_forward(const void* X, const void* W_qkv, const void* W_o,
                                       diffuser_dtype dtype, int32_t B, int32_t H, int32_t d,
                                       int32_t d_model, const diffuser_graph* g, int32_t K_steps,
                                       float alpha, void* Y, void* workspace, size_t ws_bytes,
                                       void* stream) {
    g_last_error.clear();
    if (auto s = check_shape(g, B, H, d, dtype, "d")) return s;
    if (d_model < 1) return fail(DIFFUSER_ERR_INVALID_ARG, "d_model must be >= 1");
    if (auto s = check_alpha_k(K_steps, alpha)) return s;
    for (auto pr : {std::make_pair(X, "X"), std::make_pair(W_qkv, "W_qkv"),
                    std::make_pair(W_o, "W_o"), std::make_pair((const void*)Y, "Y"),
                    std::make_pair((const void*)workspace, "workspace")})
        if (auto s = check_ptr(pr.first, pr.second)) return s;
    const layer_layout w = make_layer_layout(g, B, H, d, dtype);
    if (ws_bytes < w.total) return fail(DIFFUSER_ERR_INVALID_ARG, "workspace too small");
    const size_t es = elem_size(dtype);
    const size_t y_bytes = (size_t)B * g->n * d_model * es;
    if (overlaps(Y, y_bytes, X, y_bytes) || overlaps(Y, y_bytes, workspace, ws_bytes) ||
        overlaps(Y, y_bytes, W_qkv, (size_t)d_model * 3 * H * d * es) ||
        overlaps(Y, y_bytes, W_o, (size_t)H * d * d_model * es))
        return fail(DIFFUSER_ERR_INVALID_ARG, "Y overlaps an input or the workspace");
    hipStream_t st = static_cast<hipStream_t>(stream);
    char* ws = static_cast<char*>(workspace);
    void* t = ws;
    void* q = ws + w.t;
    void* k = ws + w.t + w.h;
    void* v = ws + w.t + 2 * w.h;
    void* z = ws + w.t + 3 * w.h;
    void* attn_ws = ws + w.t + 4 * w.h;
    void* blas_ws = ws + w.t + 4 * w.h + w.attn;
    const int64_t rows = (int64_t)B * g->n;
    if (auto s = blas_gemm(g->device, dtype, rows, 3 * (int64_t)H * d, d_model, X, W_qkv, t,
                           blas_ws, kBlasWorkspace, st))
        return s;
    hipError_t e = launch_split_heads(dtype, B, (int32_t)g->n, H, d, t, q, k, v, st);
    if (e != hipSuccess) return hip_fail(e, "head split launch");
    if (auto s = diffuser_attn(q, k, v, dtype, B, H, d, d, g, K_steps, alpha, z, attn_ws, w.attn,
                               stream))
        return s;
    e = launch_merge_heads(dtype, B, (int32_t)g->n, H, d, z, t, st);
    if (e != hipSuccess) return hip_fail(e, "head merge launch");
    return blas_gemm(g->device, dtype, rows, d_model, (int64_t)H * d, t, W_o, Y, blas_ws,
                     kBlasWorkspace, st);
}

}  // extern "C"
