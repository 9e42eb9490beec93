// Edge scores and edge softmax on weight-slot rows ("Diffuser" reading notes,
// section 2.1, eqs. S.1-S.5; "1.2.1 Static sparsity", section 1, eqs. 1-3):
//   s_ij = q_i . k_j / sqrt(d_h) for j in N(i),
//   A_ij = exp(s_ij - m_i) / sum_{u in N(i)} exp(s_iu - m_i),  m_i = max_j s_ij.
// The normalisation runs over exactly the row's neighbour set.
//
// Generic path (any slot layout: the row segment, then any scheduled random
// slots). One wavefront per row; padding slots (column -1) get weight 0. A
// group of L lanes covers one key row with 16-byte loads (L = d * elem_size
// / 16), so a wave scores 64 / L edges per step, and issues the loads of
// kUnroll steps before it uses any of them. The scale folds log2(e) so the
// exponentials are exp2.
// Pass 1 keeps an online (max, sum) per lane group; pass 2 recomputes the
// scores and writes A in the storage type.
// Long rows (more than kLongRow slots) are left to a companion kernel that
// gives each one a workgroup of kLongWaves waves, each scoring a contiguous
// share of the row; the waves' maxima and sums are merged in wave order.
#include <type_traits>

#include "internal.h"
#include "vec.h"

namespace diffuser {
namespace {

constexpr int kWave = 64;
constexpr int kWavesPerBlock = 4;
constexpr int kUnroll = 4;
constexpr int kLongWaves = 16;

// Dot products q . k_j of the slots base + u EPI + grp (u < kUnroll) of the
// row that lie below e1, reduced over the group's L lanes; j[u] = -1 and
// row 0 for padding, slot[u] = -1 past e1.
template <typename T, int D>
__device__ __forceinline__ void slot_dots(const RowSlots& rs, const T* Kb,
                                          const float (&q)[chunk<T>::kElems], int64_t base,
                                          int64_t e1, int grp, int32_t (&j)[kUnroll],
                                          int64_t (&slot)[kUnroll], float (&dot)[kUnroll]) {
    constexpr int E = chunk<T>::kElems;
    constexpr int L = D / E;
    constexpr int EPI = kWave / L;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const int64_t e = base + u * EPI + grp;
        j[u] = -1;
        slot[u] = e < e1 ? rs.slot(e, j[u]) : -1;
    }
    float k[kUnroll][E];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
        chunk<T>::load(Kb + (int64_t)(j[u] >= 0 ? j[u] : 0) * D, k[u]);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        dot[u] = 0.0f;
#pragma unroll
        for (int c = 0; c < E; ++c) dot[u] = fmaf(q[c], k[u][c], dot[u]);
    }
#pragma unroll
    for (int off = 1; off < L; off <<= 1)
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) dot[u] += __shfl_xor(dot[u], off);
}

// (m, l) <- the online-softmax merge of (m, l) and (m2, l2).
__device__ __forceinline__ void merge_ml(float& m, float& l, float m2, float l2);

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// A row whose weights, shifted by less than the row maximum, sum to this or
// more is redone with its exact maximum.
constexpr float kSumLimit = 18446744073709551616.0f;   // 2^64

template <typename T, typename TA, int D>
__global__ __launch_bounds__(kWave * kWavesPerBlock)
void k_scores_softmax(GenericGraph gg, int32_t H, int32_t BH, const T* __restrict__ Q,
                      const T* __restrict__ K, TA* __restrict__ A, float* __restrict__ row_scale,
                      float scale_log2) {
    constexpr int E = chunk<T>::kElems;
    constexpr int L = D / E;          // lanes per edge
    constexpr int EPI = kWave / L;    // edges per iteration
    static_assert(L >= 1 && L <= kWave && (kWave % L) == 0, "unsupported head width");

    const int wave = threadIdx.x / kWave;
    const int lane = __lane_id();
    const int64_t n = gg.n;
    int64_t i;
    int32_t bh;
    if (!xcd_row_item<kWavesPerBlock>(n, BH, wave, i, bh)) return;
    const int32_t b = bh / H, h = bh - b * H;
    const int32_t gr = gg.num_graphs == 1 ? 0 : b;
    const RowSlots rs = gg.row(gr, i);
    const int64_t e1 = rs.count();
    if (e1 > kLongRow) return;   // k_scores_long's
    TA* Ab = A + a_block_offset(gg.slot_off, gg.num_graphs, H, b, h);
    const int sub = lane % L, grp = lane / L;

    float q[E];
    chunk<T>::load(Q + ((int64_t)bh * n + i) * D + sub * E, q);
    const T* Kb = K + (int64_t)bh * n * D + sub * E;

    auto dots = [&](int64_t base, int32_t (&j)[kUnroll], int64_t (&slot)[kUnroll],
                    float (&dot)[kUnroll]) {
        slot_dots<T, D>(rs, Kb, q, base, e1, grp, j, slot, dot);
    };

    if (std::is_same<TA, float>::value && row_scale != nullptr) {
        // fp32 weights for the diffusion step (fused mode): one pass with the
        // row's own score as the shift (the self-loop is an edge of every
        // row, so it is at most the row maximum), unnormalised weights and
        // c_i = 1 / (their sum). A row whose weights sum to 2^64 or more
        // falls through to the exact two passes below.
        float ks[E];
        chunk<T>::load(Kb + i * D, ks);
        float sii = 0.0f;
#pragma unroll
        for (int c = 0; c < E; ++c) sii = fmaf(q[c], ks[c], sii);
#pragma unroll
        for (int off = 1; off < L; off <<= 1) sii += __shfl_xor(sii, off);
        const float ms = sii * scale_log2;
        float total = 0.0f;
        for (int64_t base = 0; base < e1; base += EPI * kUnroll) {
            int32_t j[kUnroll];
            int64_t slot[kUnroll];
            float dot[kUnroll];
            dots(base, j, slot, dot);
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                if (slot[u] >= 0 && sub == 0) {
                    const float a = j[u] >= 0 ? fast_exp2(dot[u] * scale_log2 - ms) : 0.0f;
                    chunk<TA>::store1(Ab + slot[u], a);
                    total += a;
                }
            }
        }
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) total += __shfl_xor(total, off);
        if (total < kSumLimit) {
            if (lane == 0) row_scale[(int64_t)bh * n + i] = 1.0f / total;
            return;
        }
    }

    float m = -INFINITY, l = 0.0f;
    for (int64_t base = 0; base < e1; base += EPI * kUnroll) {
        int32_t j[kUnroll];
        int64_t slot[kUnroll];
        float dot[kUnroll];
        dots(base, j, slot, dot);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if (j[u] >= 0) {
                const float t = dot[u] * scale_log2;
                const float mn = fmaxf(m, t);
                l = l * fast_exp2(m - mn) + fast_exp2(t - mn);
                m = mn;
            }
        }
    }
    // Merge the per-group (max, sum) pairs.
#pragma unroll
    for (int off = L; off < kWave; off <<= 1) {
        const float m2 = __shfl_xor(m, off);
        const float l2 = __shfl_xor(l, off);
        merge_ml(m, l, m2, l2);
    }
    const float inv = 1.0f / l;

    float stored_sum = 0.0f;  // sum of the weights as stored (after rounding)
    for (int64_t base = 0; base < e1; base += EPI * kUnroll) {
        int32_t j[kUnroll];
        int64_t slot[kUnroll];
        float dot[kUnroll];
        dots(base, j, slot, dot);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if (slot[u] >= 0 && sub == 0) {
                const float a = j[u] >= 0 ? fast_exp2(dot[u] * scale_log2 - m) * inv : 0.0f;
                chunk<TA>::store1(Ab + slot[u], a);
                stored_sum += chunk<TA>::round(a);
            }
        }
    }
    if (row_scale != nullptr) {
        // 1 / (row sum of the stored weights): applied by the diffusion step,
        // it keeps the stored operator row-stochastic, so storage rounding
        // of A does not compound over the K steps.
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) stored_sum += __shfl_xor(stored_sum, off);
        if (lane == 0) row_scale[(int64_t)bh * n + i] = 1.0f / stored_sum;
    }
}

__device__ __forceinline__ void merge_ml(float& m, float& l, float m2, float l2) {
    const float mn = fmaxf(m, m2);
    const float a = m == -INFINITY ? 0.0f : l * fast_exp2(m - mn);
    const float c = m2 == -INFINITY ? 0.0f : l2 * fast_exp2(m2 - mn);
    l = a + c;
    m = mn;
}

// One long row per workgroup (long row blockIdx.x of the graph of pair
// blockIdx.y): the same passes as k_scores_softmax, each wave over its
// contiguous share of the row's slots, with the row's shift, maximum and
// sums merged across the waves in wave order through LDS.
template <typename T, typename TA, int D>
__global__ __launch_bounds__(kWave * kLongWaves)
void k_scores_long(GenericGraph gg, int32_t H, const T* __restrict__ Q, const T* __restrict__ K,
                   TA* __restrict__ A, float* __restrict__ row_scale, float scale_log2) {
    constexpr int E = chunk<T>::kElems;
    constexpr int L = D / E;
    constexpr int EPI = kWave / L;
    __shared__ float red[2][kLongWaves];
    const int32_t bh = blockIdx.y;
    const int32_t b = bh / H, h = bh - b * H;
    const int32_t gr = gg.num_graphs == 1 ? 0 : b;
    const int64_t li = gg.long_off[gr] + blockIdx.x;
    if (li >= gg.long_off[gr + 1]) return;   // the whole workgroup
    const int64_t n = gg.n;
    const int64_t i = gg.long_rows[li];
    const RowSlots rs = gg.row(gr, i);
    const int wave = threadIdx.x / kWave;
    const int lane = __lane_id();
    const int64_t cnt = rs.count();
    const int64_t e0 = cnt * wave / kLongWaves, e1 = cnt * (wave + 1) / kLongWaves;
    TA* Ab = A + a_block_offset(gg.slot_off, gg.num_graphs, H, b, h);
    const int sub = lane % L, grp = lane / L;

    float q[E];
    chunk<T>::load(Q + ((int64_t)bh * n + i) * D + sub * E, q);
    const T* Kb = K + (int64_t)bh * n * D + sub * E;
    auto dots = [&](int64_t base, int32_t (&j)[kUnroll], int64_t (&slot)[kUnroll],
                    float (&dot)[kUnroll]) {
        slot_dots<T, D>(rs, Kb, q, base, e1, grp, j, slot, dot);
    };
    // Sum of one value per wave (lane 0's), in wave order, in every thread.
    auto wave_sum = [&](float v) -> float {
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) v += __shfl_xor(v, off);
        if (lane == 0) red[0][wave] = v;
        __syncthreads();
        float t = 0.0f;
        for (int w = 0; w < kLongWaves; ++w) t += red[0][w];
        __syncthreads();
        return t;
    };

    if (std::is_same<TA, float>::value && row_scale != nullptr) {
        // The fused single pass, shifted by the row's own score.
        float ks[E];
        chunk<T>::load(Kb + i * D, ks);
        float sii = 0.0f;
#pragma unroll
        for (int c = 0; c < E; ++c) sii = fmaf(q[c], ks[c], sii);
#pragma unroll
        for (int off = 1; off < L; off <<= 1) sii += __shfl_xor(sii, off);
        const float ms = sii * scale_log2;
        float total = 0.0f;
        for (int64_t base = e0; base < e1; base += EPI * kUnroll) {
            int32_t j[kUnroll];
            int64_t slot[kUnroll];
            float dot[kUnroll];
            dots(base, j, slot, dot);
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                if (slot[u] >= 0 && sub == 0) {
                    const float a = j[u] >= 0 ? fast_exp2(dot[u] * scale_log2 - ms) : 0.0f;
                    chunk<TA>::store1(Ab + slot[u], a);
                    total += a;
                }
            }
        }
        total = wave_sum(total);
        if (total < kSumLimit) {
            if (threadIdx.x == 0) row_scale[(int64_t)bh * n + i] = 1.0f / total;
            return;
        }
    }

    float m = -INFINITY, l = 0.0f;
    for (int64_t base = e0; base < e1; base += EPI * kUnroll) {
        int32_t j[kUnroll];
        int64_t slot[kUnroll];
        float dot[kUnroll];
        dots(base, j, slot, dot);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if (j[u] >= 0) {
                const float t = dot[u] * scale_log2;
                const float mn = fmaxf(m, t);
                l = l * fast_exp2(m - mn) + fast_exp2(t - mn);
                m = mn;
            }
        }
    }
#pragma unroll
    for (int off = L; off < kWave; off <<= 1) {
        const float m2 = __shfl_xor(m, off);
        const float l2 = __shfl_xor(l, off);
        merge_ml(m, l, m2, l2);
    }
    if (lane == 0) {
        red[0][wave] = m;
        red[1][wave] = l;
    }
    __syncthreads();
    m = -INFINITY;
    l = 0.0f;
    for (int w = 0; w < kLongWaves; ++w) merge_ml(m, l, red[0][w], red[1][w]);
    __syncthreads();
    const float inv = 1.0f / l;

    float stored_sum = 0.0f;
    for (int64_t base = e0; base < e1; base += EPI * kUnroll) {
        int32_t j[kUnroll];
        int64_t slot[kUnroll];
        float dot[kUnroll];
        dots(base, j, slot, dot);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if (slot[u] >= 0 && sub == 0) {
                const float a = j[u] >= 0 ? fast_exp2(dot[u] * scale_log2 - m) * inv : 0.0f;
                chunk<TA>::store1(Ab + slot[u], a);
                stored_sum += chunk<TA>::round(a);
            }
        }
    }
    if (row_scale != nullptr) {
        stored_sum = wave_sum(stored_sum);
        if (threadIdx.x == 0) row_scale[(int64_t)bh * n + i] = 1.0f / stored_sum;
    }
}

// Zeroes the dummy slots of the random area (no row owns them) in every
// (b, h) block of A.
template <typename T>
__global__ __launch_bounds__(256)
void k_zero_dummies(int64_t n, int32_t H, int32_t num_graphs, const int64_t* __restrict__ slot_off,
                    const int32_t* __restrict__ slot_col, const int64_t* __restrict__ seg_ptr,
                    T* __restrict__ A) {
    const int32_t bh = blockIdx.y;
    const int32_t b = bh / H, h = bh - b * H;
    const int32_t gr = num_graphs == 1 ? 0 : b;
    const int64_t base = seg_ptr[(int64_t)gr * (n + 1) + n];              // random area start
    const int64_t len = slot_off[gr + 1] - slot_off[gr] - base;           // to the graph's end
    const int32_t* cols = slot_col + slot_off[gr] + base;
    T* Ab = A + a_block_offset(slot_off, num_graphs, H, b, h) + base;
    for (int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; s < len;
         s += (int64_t)gridDim.x * blockDim.x)
        if (cols[s] < 0) chunk<T>::store1(Ab + s, 0.0f);
}

// A[s] *= c[row(s)] over the slots of each (b, h) block of fp32 weights
// (padding, row -1, untouched): stored weights normalised by their rows'
// scale. Four slots per thread (a graph's slots are a multiple of 8, its
// blocks 32-byte aligned).
__global__ __launch_bounds__(256)
void k_scale_rows(int64_t n, int32_t H, int32_t num_graphs, const int64_t* __restrict__ slot_off,
                  const int32_t* __restrict__ slot_row, const float* __restrict__ c,
                  float* __restrict__ A) {
    const int32_t bh = blockIdx.y;
    const int32_t b = bh / H, h = bh - b * H;
    const int32_t gr = num_graphs == 1 ? 0 : b;
    const int64_t quads = (slot_off[gr + 1] - slot_off[gr]) / 4;
    const int4* rows = reinterpret_cast<const int4*>(slot_row + slot_off[gr]);
    const float* cb = c + (int64_t)bh * n;
    float4* Ab = reinterpret_cast<float4*>(A + a_block_offset(slot_off, num_graphs, H, b, h));
    for (int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; s < quads;
         s += (int64_t)gridDim.x * blockDim.x) {
        const int4 r = rows[s];
        float4 w = Ab[s];
        if (r.x >= 0) w.x *= cb[r.x];
        if (r.y >= 0) w.y *= cb[r.y];
        if (r.z >= 0) w.z *= cb[r.z];
        if (r.w >= 0) w.w *= cb[r.w];
        Ab[s] = w;
    }
}

template <typename T, int D>
hipError_t launch_t(const diffuser_graph& g, const attn_shape& s, const void* Q, const void* K,
                    void* A, float* row_scale, float scale_log2, hipStream_t st) {
    const dim3 grid = xcd_row_grid(g.n, s.B * s.H, kWavesPerBlock);
    hipLaunchKernelGGL((k_scores_softmax<T, T, D>), grid, dim3(kWave * kWavesPerBlock), 0, st,
                       generic_graph(g), s.H, s.B * s.H, static_cast<const T*>(Q),
                       static_cast<const T*>(K), static_cast<T*>(A), row_scale, scale_log2);
    if (g.max_long > 0)
        hipLaunchKernelGGL((k_scores_long<T, T, D>), dim3((unsigned)g.max_long, (unsigned)(s.B * s.H)),
                           dim3(kWave * kLongWaves), 0, st, generic_graph(g), s.H,
                           static_cast<const T*>(Q), static_cast<const T*>(K),
                           static_cast<T*>(A), row_scale, scale_log2);
    if (g.rand_apart())
        hipLaunchKernelGGL((k_zero_dummies<T>), dim3(64, (unsigned)(s.B * s.H)), dim3(256), 0, st,
                           g.n, s.H, g.num_graphs, g.d_slot_off, g.d_slot_col, g.d_seg_ptr,
                           static_cast<T*>(A));
    return hipGetLastError();
}

template <typename T>
hipError_t launch_d(const diffuser_graph& g, const attn_shape& s, const void* Q, const void* K,
                    void* A, float* row_scale, float scale_log2, hipStream_t st) {
    switch (s.d) {
        case 16: return launch_t<T, 16>(g, s, Q, K, A, row_scale, scale_log2, st);
        case 32: return launch_t<T, 32>(g, s, Q, K, A, row_scale, scale_log2, st);
        case 64: return launch_t<T, 64>(g, s, Q, K, A, row_scale, scale_log2, st);
        case 128: return launch_t<T, 128>(g, s, Q, K, A, row_scale, scale_log2, st);
        default: return hipErrorInvalidValue;
    }
}

template <typename T, int D>
hipError_t launch_f32_t(const diffuser_graph& g, const attn_shape& s, const void* Q, const void* K,
                        float* A, float scale_log2, hipStream_t st) {
    const dim3 grid = xcd_row_grid(g.n, s.B * s.H, kWavesPerBlock);
    hipLaunchKernelGGL((k_scores_softmax<T, float, D>), grid, dim3(kWave * kWavesPerBlock), 0, st,
                       generic_graph(g), s.H, s.B * s.H, static_cast<const T*>(Q),
                       static_cast<const T*>(K), A, nullptr, scale_log2);
    if (g.max_long > 0)
        hipLaunchKernelGGL((k_scores_long<T, float, D>), dim3((unsigned)g.max_long, (unsigned)(s.B * s.H)),
                           dim3(kWave * kLongWaves), 0, st, generic_graph(g), s.H,
                           static_cast<const T*>(Q), static_cast<const T*>(K), A, nullptr,
                           scale_log2);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_f32_d(const diffuser_graph& g, const attn_shape& s, const void* Q, const void* K,
                        float* A, float scale_log2, hipStream_t st) {
    switch (s.d) {
        case 16: return launch_f32_t<T, 16>(g, s, Q, K, A, scale_log2, st);
        case 32: return launch_f32_t<T, 32>(g, s, Q, K, A, scale_log2, st);
        case 64: return launch_f32_t<T, 64>(g, s, Q, K, A, scale_log2, st);
        case 128: return launch_f32_t<T, 128>(g, s, Q, K, A, scale_log2, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_zero_dummies_f32(const diffuser_graph& g, const attn_shape& s, void* A,
                                  hipStream_t st) {
    if (g.rand_apart())
        hipLaunchKernelGGL((k_zero_dummies<float>), dim3(64, (unsigned)(s.B * s.H)), dim3(256), 0,
                           st, g.n, s.H, g.num_graphs, g.d_slot_off, g.d_slot_col, g.d_seg_ptr,
                           static_cast<float*>(A));
    return hipGetLastError();
}

hipError_t launch_scores_softmax_f32(const diffuser_graph& g, const attn_shape& s, const void* Q,
                                     const void* K, float* A, float scale_log2, hipStream_t st,
                                     float* row_scale) {
    // Built d = 64 graphs: the fused LDS-window pass (weights and row
    // scales), then the weights normalised in place.
    if (row_scale != nullptr && (reinterpret_cast<uintptr_t>(A) & 15u) == 0 &&
        rows_scores_any_supported(g, s)) {
        hipError_t e = launch_scores_rows(g, s, Q, K, A, row_scale, scale_log2, st);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(k_scale_rows, dim3(256, (unsigned)(s.B * s.H)), dim3(256), 0, st, g.n,
                           s.H, g.num_graphs, g.d_slot_off, g.d_slot_row, row_scale, A);
        return hipGetLastError();
    }
    if (s.dtype == DIFFUSER_F32) return launch_f32_d<float>(g, s, Q, K, A, scale_log2, st);
    return launch_f32_d<bf16_t>(g, s, Q, K, A, scale_log2, st);
}

hipError_t launch_scores_softmax(const diffuser_graph& g, const attn_shape& s, const void* Q,
                                 const void* K, void* A, float* row_scale, float scale_log2,
                                 hipStream_t st, float* part) {
    const bool aligned = (reinterpret_cast<uintptr_t>(A) & 15u) == 0;
    if (aligned && fast_block_supported(g, s))
        return launch_block_scores(g, s, Q, K, A, row_scale, scale_log2, row_scale == nullptr, part,
                                   st);
    if (aligned && fast_scores_supported(g, s))
        return launch_scores_fast(g, s, Q, K, A, row_scale, scale_log2, row_scale == nullptr, st);
    if (aligned && row_scale != nullptr && rows_scores_supported(g, s))
        return launch_scores_rows(g, s, Q, K, A, row_scale, scale_log2, st);
    if (s.dtype == DIFFUSER_F32) return launch_d<float>(g, s, Q, K, A, row_scale, scale_log2, st);
    return launch_d<bf16_t>(g, s, Q, K, A, row_scale, scale_log2, st);
}

}  // namespace diffuser
