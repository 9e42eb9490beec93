// Backward of the whole path: the chain rule through the PPR recurrence
// ("Diffuser" reading notes, section 2.4, eq. S.7), the edge softmax
// (section 2.1, eqs. S.1-S.5) and the edge scores. For one (b, h), with
// G_K = dZ and k = K-1 .. 0:
//   dA_ij += (1 - alpha) G_{k+1}[i] . Z_k[j]      (edges of the graph)
//   dV    += alpha G_{k+1}
//   G_k    = (1 - alpha) A^T G_{k+1}
// then dV += G_0 (Z_0 = V), dS_ij = A_ij (dA_ij - sum_u A_iu dA_iu),
// dQ_i = sum_j dS_ij k_j / sqrt(d_h), dK_j = sum_i dS_ij q_i / sqrt(d_h).
//
// Every intermediate (A, dA, the states Z_k, G_k, dV) is fp32; the outputs
// are rounded to the storage type once, and every sum has a fixed order.
//
// On built graphs with d = 64 and enough rows the products run on the fp32
// LDS-window step kernels (the states and dQ; on bidirectional graphs also
// G_k and dK, over A^T laid out in the graph's own slot geometry), dA's
// dense parts on MFMA (dots_mfma.hip) with its random slots here, and the
// softmax gradient reads each segment as quads. Everything else runs on
// generic kernels over the weight slots (any graph, fp32 or bf16 storage,
// d in {16, 32, 64, 128}): rows and columns with more than kLongRow entries
// are split over the waves of one workgroup by companion kernels;
// row-wise products walk a row's slots, the transposed ones the graph's
// column index (the slots of each column by ascending row) with the
// weights first copied into that order, so only the rows of X are
// gathered; dA takes all K terms in one pass over the slots, from the
// stored states G_1 .. G_K; each wave splits its row or column over groups
// of lanes and adds the groups' partial sums in a fixed order. dV is one
// pass over the stored states at the end.
#include <algorithm>
#include <type_traits>

#include "internal.h"
#include "vec.h"

namespace diffuser {
namespace {

constexpr int kWave = 64;
constexpr int kWavesPerBlock = 4;
constexpr int kThreads = kWave * kWavesPerBlock;
// Slot steps whose index and row loads a wave issues before it uses any of
// them: the products are bound by the latency of those dependent loads.
constexpr int kUnroll = 4;


__device__ __forceinline__ float ld(const float* p) { return *p; }
__device__ __forceinline__ float ld(const bf16_t* p) { return bf16_to_f32(p->bits); }
__device__ __forceinline__ void st(float* p, float v) { *p = v; }
__device__ __forceinline__ void st(bf16_t* p, float v) { p->bits = (uint16_t)f32_to_bf16(v); }

// Four channels of row r of X as floats.
template <typename TX>
__device__ __forceinline__ void ld4(const TX* p, float (&x)[4]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = ld(p + e);
}

// Y[i] = a * sum_{slots s of row i} W[s] X[col(s)] + b * U[i], one wave per
// row: groups of L = D / 4 lanes take one slot each (lane = 4 channels),
// so 64 / L slots are in flight per step; the groups' partial sums are
// added in a fixed order at the end.
template <typename TX, typename TU, typename TY, int D>
__global__ __launch_bounds__(kThreads)
void k_rows(GenericGraph gg, int32_t H, int32_t BH, const float* __restrict__ W,
            const TX* __restrict__ X, const TU* __restrict__ U, TY* __restrict__ Y, float a,
            float b) {
    constexpr int L = D / 4, EPI = kWave / L;
    const int wave = threadIdx.x / kWave, lane = __lane_id();
    const int64_t n = gg.n;
    int64_t i;
    int32_t bh;
    if (!xcd_row_item<kWavesPerBlock>(n, BH, wave, i, bh)) return;
    const int32_t bb = bh / H, hh = bh - bb * H;
    const int32_t gr = gg.num_graphs == 1 ? 0 : bb;
    const RowSlots rs = gg.row(gr, i);
    const float* Wb = W + a_block_offset(gg.slot_off, gg.num_graphs, H, bb, hh);
    const int sub = lane % L, grp = lane / L;
    const TX* Xb = X + (int64_t)bh * n * D + 4 * sub;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    const int64_t cnt = rs.count();
    if (cnt > kLongRow) return;   // k_rows_long's
    for (int64_t base = 0; base < cnt; base += EPI * kUnroll) {
        // Slots base + u EPI + grp; padding and slots past the row read
        // column 0 with weight 0.
        int32_t j[kUnroll];
        int64_t s[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t e = base + u * EPI + grp;
            j[u] = -1;
            s[u] = 0;
            if (e < cnt) s[u] = rs.slot(e, j[u]);
        }
        float w[kUnroll], x[kUnroll][4];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            w[u] = j[u] >= 0 ? Wb[s[u]] : 0.0f;
            ld4(Xb + (int64_t)(j[u] >= 0 ? j[u] : 0) * D, x[u]);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[c] = fmaf(w[u], x[u][c], acc[c]);
    }
#pragma unroll
    for (int off = L; off < kWave; off <<= 1)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[c] += __shfl_xor(acc[c], off);
    if (grp == 0) {
        const int64_t o = ((int64_t)bh * n + i) * D + 4 * sub;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            float y = a * acc[c];
            if (U != nullptr) y += b * ld(U + o + c);
            st(Y + o + c, y);
        }
    }
}

// Column index of one graph family: col_ptr [graphs][n + 1], col_slot (slot
// numbers within the graph, ascending row within a column), slot_row.
struct ColIndex {
    int64_t n;
    int32_t num_graphs;
    const int64_t* col_ptr;
    const int64_t* col_off;    // [graphs + 1] start of each graph's col_slot run
    const int32_t* col_slot;
    const int32_t* col_row;    // row of each col_slot entry
    const int64_t* slot_off;   // [graphs + 1]
};

// Wt[e] = W[col_slot[e]] for every column-index entry e of each (b, h)
// (both at the (b, h) block's slot offset): the weights in column order.
// Workgroup items are (b, h, block of kThreads entries) on an XCD-aware grid
// over `blocks` entry blocks per (b, h).
__global__ __launch_bounds__(kThreads)
void k_to_columns(ColIndex ci, int32_t H, int32_t BH, int64_t blocks, const float* __restrict__ W,
                  float* __restrict__ Wt) {
    int64_t eb;
    int32_t bh;
    if (!xcd_row_item<1>(blocks, BH, 0, eb, bh)) return;
    const int32_t bb = bh / H, hh = bh - bb * H;
    const int32_t gr = ci.num_graphs == 1 ? 0 : bb;
    const int64_t count = ci.col_off[gr + 1] - ci.col_off[gr];
    const int64_t e = eb * kThreads + threadIdx.x;
    if (e >= count) return;
    const int64_t off = a_block_offset(ci.slot_off, ci.num_graphs, H, bb, hh);
    Wt[off + e] = W[off + ci.col_slot[ci.col_off[gr] + e]];
}

// Y[j] = a * sum_{entries e of column j} Wt[e] X[col_row[e]], one wave per
// column, lanes grouped as in k_rows; Wt holds the weights in column order
// (k_to_columns).
template <typename TX, typename TY, int D>
__global__ __launch_bounds__(kThreads)
void k_cols(ColIndex ci, int32_t H, int32_t BH, const float* __restrict__ Wt,
            const TX* __restrict__ X, TY* __restrict__ Y, float a) {
    constexpr int L = D / 4, EPI = kWave / L;
    const int wave = threadIdx.x / kWave, lane = __lane_id();
    const int64_t n = ci.n;
    int64_t j;
    int32_t bh;
    if (!xcd_row_item<kWavesPerBlock>(n, BH, wave, j, bh)) return;
    const int32_t bb = bh / H, hh = bh - bb * H;
    const int32_t gr = ci.num_graphs == 1 ? 0 : bb;
    const int64_t* cp = ci.col_ptr + (int64_t)gr * (n + 1);
    const int32_t* crow = ci.col_row + ci.col_off[gr];
    const float* Wb = Wt + a_block_offset(ci.slot_off, ci.num_graphs, H, bb, hh);
    const int sub = lane % L, grp = lane / L;
    const TX* Xb = X + (int64_t)bh * n * D + 4 * sub;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    const int64_t e0 = cp[j], e1 = cp[j + 1];
    if (e1 - e0 > kLongRow) return;   // k_cols_long's
    for (int64_t base = e0; base < e1; base += EPI * kUnroll) {
        // Entries base + u EPI + grp; those past the column read entry e0
        // with weight 0.
        int64_t i[kUnroll];
        float w[kUnroll], x[kUnroll][4];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t e = base + u * EPI + grp;
            const bool ok = e < e1;
            i[u] = crow[ok ? e : e0];
            w[u] = ok ? Wb[e] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) ld4(Xb + i[u] * D, x[u]);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[c] = fmaf(w[u], x[u][c], acc[c]);
    }
#pragma unroll
    for (int off = L; off < kWave; off <<= 1)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[c] += __shfl_xor(acc[c], off);
    if (grp == 0) {
        const int64_t o = ((int64_t)bh * n + j) * D + 4 * sub;
#pragma unroll
        for (int c = 0; c < 4; ++c) st(Y + o + c, a * acc[c]);
    }
}

// The slots [e0, e1) of one row for k_edge_dots (lane group grp, channel
// quad sub).
template <int D>
__device__ __forceinline__ void edge_dots_range(const RowSlots& rs, const float* Gi,
                                                const float* Zb, int64_t stride, int32_t K,
                                                float* dAb, float a, int64_t e0, int64_t e1,
                                                int grp, int sub) {
    constexpr int L = D / 4, EPI = kWave / L;
    const int64_t cnt = e1;
    for (int64_t base = e0; base < cnt; base += EPI * kUnroll) {
        int32_t j[kUnroll];
        int64_t s[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t e = base + u * EPI + grp;
            j[u] = -1;
            s[u] = -1;
            if (e < cnt) s[u] = rs.slot(e, j[u]);
        }
        float dot[kUnroll] = {};
        for (int32_t k = 0; k < K; ++k) {
            const float4 g = *reinterpret_cast<const float4*>(Gi + k * stride);
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const float4 z = *reinterpret_cast<const float4*>(
                    Zb + k * stride + (int64_t)(j[u] >= 0 ? j[u] : 0) * D);
                dot[u] += g.x * z.x + g.y * z.y + g.z * z.z + g.w * z.w;
            }
        }
#pragma unroll
        for (int off = 1; off < L; off <<= 1)
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) dot[u] += __shfl_xor(dot[u], off);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            if (s[u] >= 0 && sub == 0) dAb[s[u]] = j[u] >= 0 ? a * dot[u] : 0.0f;
    }
}

// v plus the value of the lane of its DPP row that `ctrl` names.
template <int ctrl>
__device__ __forceinline__ float dpp_add(float v) {
    return v + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), ctrl, 0xf, 0xf, true));
}
// Sum over a row of 16 lanes (every lane gets it): lane pairs, quads, the
// halves of 8 and of 16.
__device__ __forceinline__ float row16_sum(float v) {
    v = dpp_add<0xB1>(v);    // quad_perm [1, 0, 3, 2]
    v = dpp_add<0x4E>(v);    // quad_perm [2, 3, 0, 1]
    v = dpp_add<0x141>(v);   // row_half_mirror
    v = dpp_add<0x140>(v);   // row_mirror
    return v;
}
// Lane u of the caller's row of 16 lanes (DPP row_newbcast).
template <int u>
__device__ __forceinline__ int32_t row16_lane(int32_t v) {
    return __builtin_amdgcn_mov_dpp(v, 0x150 + u, 0xf, 0xf, false);
}

// The random slots of row i for D = 64 (a lane group is one DPP row of 16
// lanes): per step of 16 edges, lane u < 4 of group q loads the slot and
// lane 4 + u the column of edge base + 4 u + q, handed round the group; each group
// sums its four edges' K dot products over its 16 lanes, and lane u stores
// edge u's value: one index load and one store per step.
__device__ __forceinline__ void rand_dots64(const RowSlots& rs, const float* Gi, const float* Zb,
                                            int64_t stride, int32_t K, float* dAb, float a,
                                            int grp, int sub) {
    const int32_t nr = rs.rcnt;
    // The row's first kHeld states of G stay in registers for all its edges.
    constexpr int kHeld = 6;
    float4 gh[kHeld];
#pragma unroll
    for (int k = 0; k < kHeld; ++k)
        gh[k] = k < K && nr > 0 ? *reinterpret_cast<const float4*>(Gi + k * stride)
                                : make_float4(0.f, 0.f, 0.f, 0.f);
    // Lanes 0-3 of a group load slots, lanes 4-7 columns: one load per step.
    const int32_t* ixp = (sub & 4) ? rs.rcol : rs.rslot;
    for (int32_t base = 0; base < nr; base += 4 * kUnroll) {
        const int32_t el = base + 4 * (sub & 3) + grp;
        const int32_t ix = el < nr ? ixp[el] : -1;
        const int32_t sl = ix;   // this lane's slot (lanes 0-3 store)
        const int32_t s[kUnroll] = {row16_lane<0>(ix), row16_lane<1>(ix), row16_lane<2>(ix),
                                    row16_lane<3>(ix)};
        int32_t j[kUnroll] = {row16_lane<4>(ix), row16_lane<5>(ix), row16_lane<6>(ix),
                              row16_lane<7>(ix)};
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) j[u] = s[u] >= 0 ? j[u] : 0;
        float dot[kUnroll] = {};
#pragma unroll
        for (int32_t k = 0; k < kHeld; ++k) {
            if (k >= K) break;
            const float4 g = gh[k];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const float4 z = *reinterpret_cast<const float4*>(Zb + k * stride + (int64_t)j[u] * 64);
                dot[u] += g.x * z.x + g.y * z.y + g.z * z.z + g.w * z.w;
            }
        }
        for (int32_t k = kHeld; k < K; ++k) {
            const float4 g = *reinterpret_cast<const float4*>(Gi + k * stride);
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const float4 z = *reinterpret_cast<const float4*>(Zb + k * stride + (int64_t)j[u] * 64);
                dot[u] += g.x * z.x + g.y * z.y + g.z * z.z + g.w * z.w;
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) dot[u] = row16_sum(dot[u]);
        const int u = sub & 3;
        const float dv = u == 0 ? dot[0] : u == 1 ? dot[1] : u == 2 ? dot[2] : dot[3];
        if (sub < 4 && sl >= 0) dAb[sl] = a * dv;
    }
}

// dA[s] = a * sum_{k < K} G_{k+1}[i] . Z_k[col(s)] for the slots of row i
// (padding slots get 0): groups of L lanes take one slot each (L = D / 4
// lanes of 4 channels); state k of G or Z starts at k * stride. kRandOnly:
// only the row's random slots (kept apart from its segment), whatever the
// row's length.
template <int D, bool kRandOnly>
__global__ __launch_bounds__(kThreads)
void k_edge_dots(GenericGraph gg, int32_t H, int32_t BH, const float* __restrict__ Gs,
                 const float* __restrict__ Zs, int64_t stride, int32_t K, float* __restrict__ dA,
                 float a) {
    constexpr int L = D / 4;
    const int wave = threadIdx.x / kWave, lane = __lane_id();
    const int64_t n = gg.n;
    int64_t i;
    int32_t bh;
    if (!xcd_row_item<kWavesPerBlock>(n, BH, wave, i, bh)) return;
    const int32_t bb = bh / H, hh = bh - bb * H;
    const int32_t gr = gg.num_graphs == 1 ? 0 : bb;
    const RowSlots rs = gg.row(gr, i);
    float* dAb = dA + a_block_offset(gg.slot_off, gg.num_graphs, H, bb, hh);
    const int sub = lane % L, grp = lane / L;
    const float* Gi = Gs + stride + ((int64_t)bh * n + i) * D + 4 * sub;
    const float* Zb = Zs + (int64_t)bh * n * D + 4 * sub;
    const int64_t cnt = rs.count();
    if (kRandOnly) {
        if constexpr (D == 64) rand_dots64(rs, Gi, Zb, stride, K, dAb, a, grp, sub);
        else if (rs.rcnt > 0) edge_dots_range<D>(rs, Gi, Zb, stride, K, dAb, a, rs.seg_len, cnt, grp, sub);
        return;
    }
    if (cnt > kLongRow) return;   // k_edge_dots_long's
    edge_dots_range<D>(rs, Gi, Zb, stride, K, dAb, a, 0, cnt, grp, sub);
}

// Long rows and columns (more than kLongRow entries, a global row's or
// column's n, say): one workgroup of kLongWaves waves per (pair, long row or
// column), long row (column) blockIdx.x of the pair's graph, each wave a
// contiguous share of the entries gathered as k_rows / k_cols / k_edge_dots
// do. The row and column products add the waves' partial sums in wave order
// through LDS; dA needs no sum across entries.
constexpr int kLongWaves = 16;
constexpr int kLongThreads = kWave * kLongWaves;

template <typename TX, typename TU, typename TY, int D>
__global__ __launch_bounds__(kLongThreads)
void k_rows_long(GenericGraph gg, int32_t H, const float* __restrict__ W,
                 const TX* __restrict__ X, const TU* __restrict__ U, TY* __restrict__ Y,
                 float a, float b) {
    constexpr int L = D / 4, EPI = kWave / L;
    __shared__ float part[kLongWaves][D];
    const int32_t bh = blockIdx.y;
    const int32_t bb = bh / H, hh = bh - bb * H;
    const int32_t gr = gg.num_graphs == 1 ? 0 : bb;
    const int64_t li = gg.long_off[gr] + blockIdx.x;
    if (li >= gg.long_off[gr + 1]) return;   // the whole workgroup
    const int64_t n = gg.n;
    const int64_t i = gg.long_rows[li];
    const RowSlots rs = gg.row(gr, i);
    const float* Wb = W + a_block_offset(gg.slot_off, gg.num_graphs, H, bb, hh);
    const int wave = threadIdx.x / kWave, lane = __lane_id();
    const int sub = lane % L, grp = lane / L;
    const TX* Xb = X + (int64_t)bh * n * D + 4 * sub;
    const int64_t cnt = rs.count();
    const int64_t e0 = cnt * wave / kLongWaves, e1 = cnt * (wave + 1) / kLongWaves;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int64_t base = e0; base < e1; base += EPI * kUnroll) {
        int32_t j[kUnroll];
        int64_t s[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t e = base + u * EPI + grp;
            j[u] = -1;
            s[u] = 0;
            if (e < e1) s[u] = rs.slot(e, j[u]);
        }
        float w[kUnroll], x[kUnroll][4];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            w[u] = j[u] >= 0 ? Wb[s[u]] : 0.0f;
            ld4(Xb + (int64_t)(j[u] >= 0 ? j[u] : 0) * D, x[u]);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[c] = fmaf(w[u], x[u][c], acc[c]);
    }
#pragma unroll
    for (int off = L; off < kWave; off <<= 1)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[c] += __shfl_xor(acc[c], off);
    if (grp == 0) {
#pragma unroll
        for (int c = 0; c < 4; ++c) part[wave][4 * sub + c] = acc[c];
    }
    __syncthreads();
    if (threadIdx.x < D) {
        const int c = threadIdx.x;
        float t = 0.0f;
        for (int w = 0; w < kLongWaves; ++w) t += part[w][c];
        const int64_t o = ((int64_t)bh * n + i) * D + c;
        float y = a * t;
        if (U != nullptr) y += b * ld(U + o);
        st(Y + o, y);
    }
}

template <typename TX, typename TY, int D>
__global__ __launch_bounds__(kLongThreads)
void k_cols_long(ColIndex ci, int32_t H, const int32_t* __restrict__ long_cols,
                 const int64_t* __restrict__ long_col_off, const float* __restrict__ Wt,
                 const TX* __restrict__ X, TY* __restrict__ Y, float a) {
    constexpr int L = D / 4, EPI = kWave / L;
    __shared__ float part[kLongWaves][D];
    const int32_t bh = blockIdx.y;
    const int32_t bb = bh / H, hh = bh - bb * H;
    const int32_t gr = ci.num_graphs == 1 ? 0 : bb;
    const int64_t li = long_col_off[gr] + blockIdx.x;
    if (li >= long_col_off[gr + 1]) return;   // the whole workgroup
    const int64_t n = ci.n;
    const int64_t j = long_cols[li];
    const int64_t* cp = ci.col_ptr + (int64_t)gr * (n + 1);
    const int32_t* crow = ci.col_row + ci.col_off[gr];
    const float* Wb = Wt + a_block_offset(ci.slot_off, ci.num_graphs, H, bb, hh);
    const int wave = threadIdx.x / kWave, lane = __lane_id();
    const int sub = lane % L, grp = lane / L;
    const TX* Xb = X + (int64_t)bh * n * D + 4 * sub;
    const int64_t c_lo = cp[j], cnt = cp[j + 1] - cp[j];
    const int64_t e0 = c_lo + cnt * wave / kLongWaves, e1 = c_lo + cnt * (wave + 1) / kLongWaves;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int64_t base = e0; base < e1; base += EPI * kUnroll) {
        int64_t r[kUnroll];
        float w[kUnroll], x[kUnroll][4];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t e = base + u * EPI + grp;
            const bool ok = e < e1;
            r[u] = crow[ok ? e : c_lo];
            w[u] = ok ? Wb[e] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) ld4(Xb + r[u] * D, x[u]);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[c] = fmaf(w[u], x[u][c], acc[c]);
    }
#pragma unroll
    for (int off = L; off < kWave; off <<= 1)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[c] += __shfl_xor(acc[c], off);
    if (grp == 0) {
#pragma unroll
        for (int c = 0; c < 4; ++c) part[wave][4 * sub + c] = acc[c];
    }
    __syncthreads();
    if (threadIdx.x < D) {
        const int c = threadIdx.x;
        float t = 0.0f;
        for (int w = 0; w < kLongWaves; ++w) t += part[w][c];
        st(Y + ((int64_t)bh * n + j) * D + c, a * t);
    }
}

template <int D>
__global__ __launch_bounds__(kLongThreads)
void k_edge_dots_long(GenericGraph gg, int32_t H, const float* __restrict__ Gs,
                      const float* __restrict__ Zs, int64_t stride, int32_t K,
                      float* __restrict__ dA, float a) {
    constexpr int L = D / 4;
    const int32_t bh = blockIdx.y;
    const int32_t bb = bh / H, hh = bh - bb * H;
    const int32_t gr = gg.num_graphs == 1 ? 0 : bb;
    const int64_t li = gg.long_off[gr] + blockIdx.x;
    if (li >= gg.long_off[gr + 1]) return;   // the whole workgroup
    const int64_t n = gg.n;
    const int64_t i = gg.long_rows[li];
    const RowSlots rs = gg.row(gr, i);
    float* dAb = dA + a_block_offset(gg.slot_off, gg.num_graphs, H, bb, hh);
    const int wave = threadIdx.x / kWave, lane = __lane_id();
    const int sub = lane % L, grp = lane / L;
    const float* Gi = Gs + stride + ((int64_t)bh * n + i) * D + 4 * sub;
    const float* Zb = Zs + (int64_t)bh * n * D + 4 * sub;
    const int64_t cnt = rs.count();
    edge_dots_range<D>(rs, Gi, Zb, stride, K, dAb, a, cnt * wave / kLongWaves,
                       cnt * (wave + 1) / kLongWaves, grp, sub);
}

// dS = A (dA - sum_row A dA) * scale, in place of dA; one wave per row.
__global__ __launch_bounds__(kThreads)
void k_softmax_grad(GenericGraph gg, int32_t H, int32_t BH, const float* __restrict__ A,
                    float* __restrict__ dA, float scale) {
    const int wave = threadIdx.x / kWave, lane = __lane_id();
    const int64_t n = gg.n;
    int64_t i;
    int32_t bh;
    if (!xcd_row_item<kWavesPerBlock>(n, BH, wave, i, bh)) return;
    const int32_t bb = bh / H, hh = bh - bb * H;
    const int32_t gr = gg.num_graphs == 1 ? 0 : bb;
    const RowSlots rs = gg.row(gr, i);
    const int64_t off = a_block_offset(gg.slot_off, gg.num_graphs, H, bb, hh);
    const float* Ab = A + off;
    float* dAb = dA + off;
    const int64_t cnt = rs.count();
    float sum = 0.0f;
    for (int64_t e = lane; e < cnt; e += kWave) {
        int32_t j;
        const int64_t s = rs.slot(e, j);
        if (j >= 0) sum += Ab[s] * dAb[s];
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
    for (int64_t e = lane; e < cnt; e += kWave) {
        int32_t j;
        const int64_t s = rs.slot(e, j);
        if (j >= 0) dAb[s] = Ab[s] * (dAb[s] - sum) * scale;
    }
}

// The same on built graphs, whose padding slots hold A = 0 and dA = 0: a
// row's segment is read as whole 16-byte quads (a segment starts on and
// spans a multiple of 8 slots) with no column lookups, its random slots
// through the row's slot list; a lane keeps the values it read for the
// write when the row fits one pass.
__global__ __launch_bounds__(kThreads)
void k_softmax_grad_built(GenericGraph gg, int32_t H, int32_t BH, const float* __restrict__ A,
                          float* __restrict__ dA, float scale) {
    const int wave = threadIdx.x / kWave, lane = __lane_id();
    const int64_t n = gg.n;
    int64_t i;
    int32_t bh;
    if (!xcd_row_item<kWavesPerBlock>(n, BH, wave, i, bh)) return;
    const int32_t bb = bh / H, hh = bh - bb * H;
    const int32_t gr = gg.num_graphs == 1 ? 0 : bb;
    const RowSlots rs = gg.row(gr, i);
    const int64_t off = a_block_offset(gg.slot_off, gg.num_graphs, H, bb, hh);
    const float4* A4 = reinterpret_cast<const float4*>(A + off + rs.seg_begin);
    float4* dA4 = reinterpret_cast<float4*>(dA + off + rs.seg_begin);
    const float* Ab = A + off;
    float* dAb = dA + off;
    const int64_t quads = rs.seg_len / 4;
    float sum = 0.0f;
    float4 a0 = make_float4(0.f, 0.f, 0.f, 0.f), d0 = a0;
    float ar = 0.0f, dr = 0.0f;
    if (lane < quads) {
        a0 = A4[lane];
        d0 = dA4[lane];
        sum = a0.x * d0.x + a0.y * d0.y + a0.z * d0.z + a0.w * d0.w;
    }
    for (int64_t qd = lane + kWave; qd < quads; qd += kWave) {
        const float4 x = A4[qd], y = dA4[qd];
        sum += x.x * y.x + x.y * y.y + x.z * y.z + x.w * y.w;
    }
    if (lane < rs.rcnt) {
        ar = Ab[rs.rslot[lane]];
        dr = dAb[rs.rslot[lane]];
        sum += ar * dr;
    }
    for (int32_t e = lane + kWave; e < rs.rcnt; e += kWave) sum += Ab[rs.rslot[e]] * dAb[rs.rslot[e]];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
    if (lane < quads)
        dA4[lane] = make_float4(a0.x * (d0.x - sum) * scale, a0.y * (d0.y - sum) * scale,
                                a0.z * (d0.z - sum) * scale, a0.w * (d0.w - sum) * scale);
    for (int64_t qd = lane + kWave; qd < quads; qd += kWave) {
        const float4 x = A4[qd], y = dA4[qd];
        dA4[qd] = make_float4(x.x * (y.x - sum) * scale, x.y * (y.y - sum) * scale,
                              x.z * (y.z - sum) * scale, x.w * (y.w - sum) * scale);
    }
    if (lane < rs.rcnt) dAb[rs.rslot[lane]] = ar * (dr - sum) * scale;
    for (int32_t e = lane + kWave; e < rs.rcnt; e += kWave) {
        const int32_t s = rs.rslot[e];
        dAb[s] = Ab[s] * (dAb[s] - sum) * scale;
    }
}

// y = a * x + b * y elementwise over count values (x of type TX).
template <typename TX>
__global__ __launch_bounds__(kThreads)
void k_axpby(int64_t count, const TX* __restrict__ x, float* __restrict__ y, float a, float b) {
    for (int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x; e < count;
         e += (int64_t)gridDim.x * kThreads)
        y[e] = a * ld(x + e) + (b == 0.0f ? 0.0f : b * y[e]);
}

// dV = alpha (G_K + .. + G_1) + G_0, rounded to TY once, summed from G_K
// down as a running alpha G_k + acc; four values per thread (count is a
// multiple of 4).
template <typename TY>
__global__ __launch_bounds__(kThreads)
void k_dv_sum(int64_t count, const float* __restrict__ Gs, int64_t stride, int32_t K, float alpha,
              TY* __restrict__ out) {
    for (int64_t e = 4 * ((int64_t)blockIdx.x * kThreads + threadIdx.x); e < count;
         e += 4 * (int64_t)gridDim.x * kThreads) {
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int32_t k = K; k >= 1; --k) {
            const float4 g = *reinterpret_cast<const float4*>(Gs + k * stride + e);
            acc = k == K ? make_float4(alpha * g.x, alpha * g.y, alpha * g.z, alpha * g.w)
                         : make_float4(alpha * g.x + acc.x, alpha * g.y + acc.y,
                                       alpha * g.z + acc.z, alpha * g.w + acc.w);
        }
        const float4 g0 = *reinterpret_cast<const float4*>(Gs + e);
        st(out + e, acc.x + g0.x);
        st(out + e + 1, acc.y + g0.y);
        st(out + e + 2, acc.z + g0.z);
        st(out + e + 3, acc.w + g0.w);
    }
}

dim3 grid_elems(int64_t count) {
    int64_t blocks = (count + kThreads - 1) / kThreads;
    if (blocks > 65536) blocks = 65536;
    return dim3((unsigned)(blocks < 1 ? 1 : blocks));
}

template <typename T, int D>
hipError_t backward_t(const diffuser_graph& g, const BackwardArgs& p, hipStream_t stream) {
    const GenericGraph gg = generic_graph(g);
    ColIndex ci;
    ci.n = g.n;
    ci.num_graphs = g.num_graphs;
    ci.col_ptr = g.d_col_ptr;
    ci.col_off = g.d_col_off_slots;
    ci.col_slot = g.d_col_slot;
    ci.col_row = g.d_col_row;
    ci.slot_off = g.d_slot_off;
    const int32_t BH = p.B * p.H;
    const dim3 rows = xcd_row_grid(g.n, BH, kWavesPerBlock);
    const dim3 blk(kThreads);
    const int64_t cnt = (int64_t)BH * g.n * D;
    int64_t max_entries = 0;
    for (int32_t gr = 0; gr < g.num_graphs; ++gr)
        max_entries = std::max(max_entries, g.slots[gr]);
    const int64_t entry_blocks = (max_entries + kThreads - 1) / kThreads;
    const dim3 entries = xcd_row_grid(entry_blocks, BH, 1);
    const T* V = static_cast<const T*>(p.V);
    const float keep = 1.0f - p.alpha;
    const int32_t K = p.K_steps;

    // Forward states Z_0 = V, Z_{k+1} = (1 - alpha) A Z_k + alpha V (fp32).
    if (K > 0)
        hipLaunchKernelGGL((k_axpby<T>), grid_elems(cnt), blk, 0, stream, cnt, V, p.Zs, 1.0f,
                           0.0f);
    const dim3 longs((unsigned)std::max<int64_t>(g.max_long, 1), (unsigned)BH);
    const dim3 long_cols((unsigned)std::max<int64_t>(g.max_long_col, 1), (unsigned)BH);
    const dim3 lblk(kLongThreads);
    // On built graphs (d = 64) the states come from the LDS-window step kernels.
    const bool rows_states = D == 64 && rows_states_supported(g, p.B, p.H, D);
    for (int32_t k = 1; k < K && rows_states; ++k) {
        const hipError_t e = launch_states_rows(
            g, p.B, p.H, p.A, p.Zs + (size_t)(k - 1) * cnt, V,
            std::is_same<T, float>::value ? DIFFUSER_F32 : DIFFUSER_BF16, p.Zs + (size_t)k * cnt,
            step_coefs{keep, p.alpha}, stream);
        if (e != hipSuccess) return e;
    }
    for (int32_t k = 1; k < K && !rows_states; ++k) {
        hipLaunchKernelGGL((k_rows<float, T, float, D>), rows, blk, 0, stream, gg, p.H, BH, p.A,
                           p.Zs + (size_t)(k - 1) * cnt, V, p.Zs + (size_t)k * cnt, keep,
                           p.alpha);
        if (g.max_long > 0)
            hipLaunchKernelGGL((k_rows_long<float, T, float, D>), longs, lblk, 0, stream, gg, p.H,
                               p.A, p.Zs + (size_t)(k - 1) * cnt, V, p.Zs + (size_t)k * cnt,
                               keep, p.alpha);
    }
    // G_K = dZ, G_k = (1 - alpha) A^T G_{k+1}; dV = alpha (G_K + .. + G_1).
    hipLaunchKernelGGL((k_axpby<T>), grid_elems(cnt), blk, 0, stream, cnt,
                       static_cast<const T*>(p.dZ), p.Gs + (size_t)K * cnt, 1.0f, 0.0f);
    // On bidirectional built graphs (d = 64) A^T is laid out in the graph's
    // own slot geometry and the products run on the LDS-window step kernels.
    const bool rows_cols = D == 64 && K > 0 && rows_transposed_supported(g, p.B, p.H, D);
    if (rows_cols) {
        const hipError_t e = launch_transpose_struct(g, p.B, p.H, p.A, p.At, stream);
        if (e != hipSuccess) return e;
    } else if (K > 0) {
        hipLaunchKernelGGL(k_to_columns, entries, blk, 0, stream, ci, p.H, BH, entry_blocks, p.A,
                           p.At);
    }
    for (int32_t k = K - 1; k >= 0; --k) {
        const float* Gk1 = p.Gs + (size_t)(k + 1) * cnt;
        if (rows_cols) {
            const hipError_t e = launch_transposed_rows(g, p.B, p.H, p.At, p.A, Gk1,
                                                        p.Gs + (size_t)k * cnt, keep, stream);
            if (e != hipSuccess) return e;
            continue;
        }
        hipLaunchKernelGGL((k_cols<float, float, D>), rows, blk, 0, stream, ci, p.H, BH, p.At, Gk1,
                           p.Gs + (size_t)k * cnt, keep);
        if (g.max_long_col > 0)
            hipLaunchKernelGGL((k_cols_long<float, float, D>), long_cols, lblk, 0, stream, ci, p.H,
                               g.d_long_cols, g.d_long_col_off, p.At, Gk1,
                               p.Gs + (size_t)k * cnt, keep);
    }
    // dA = (1 - alpha) sum_k G_{k+1} Z_k^T on the edges (on built d = 64
    // graphs the window bands, global columns and global rows on MFMA, the
    // random edges gathered).
    if (D == 64 && K > 0 && mfma_dots_supported(g, D)) {
        const hipError_t e = launch_dots_dense(g, p.B, p.H, p.Gs, p.Zs, cnt, K, keep, p.dA, stream);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((k_edge_dots<D, true>), rows, blk, 0, stream, gg, p.H, BH, p.Gs, p.Zs,
                           cnt, K, p.dA, keep);
    } else {
        hipLaunchKernelGGL((k_edge_dots<D, false>), rows, blk, 0, stream, gg, p.H, BH, p.Gs, p.Zs, cnt, K,
                           p.dA, keep);
        if (g.max_long > 0)
            hipLaunchKernelGGL((k_edge_dots_long<D>), longs, lblk, 0, stream, gg, p.H, p.Gs, p.Zs,
                               cnt, K, p.dA, keep);
    }
    // dV = (sum of alpha G_{k+1}) + G_0, in one pass over the states.
    hipLaunchKernelGGL((k_dv_sum<T>), grid_elems(cnt / 4), blk, 0, stream, cnt, p.Gs, cnt, K,
                       p.alpha, static_cast<T*>(p.dVout));
    // dS, then dQ = dS K and dK = dS^T Q (the 1 / sqrt(d_h) inside dS).
    if (rows_states)
        hipLaunchKernelGGL(k_softmax_grad_built, rows, blk, 0, stream, gg, p.H, BH, p.A, p.dA,
                           p.scale);
    else
        hipLaunchKernelGGL(k_softmax_grad, rows, blk, 0, stream, gg, p.H, BH, p.A, p.dA, p.scale);
    // On built d = 64 graphs both products run on the LDS-window step kernels
    // (dK on bidirectional graphs, with dS^T in the graph's slot geometry).
    if (rows_states) {
        const hipError_t e = launch_grad_rows(g, p.B, p.H, p.dA, p.dA, false, p.K, p.dQ, p.dtype,
                                              1.0f, stream);
        if (e != hipSuccess) return e;
    } else {
        hipLaunchKernelGGL((k_rows<T, T, T, D>), rows, blk, 0, stream, gg, p.H, BH, p.dA,
                           static_cast<const T*>(p.K), static_cast<const T*>(nullptr),
                           static_cast<T*>(p.dQ), 1.0f, 0.0f);
        if (g.max_long > 0)
            hipLaunchKernelGGL((k_rows_long<T, T, T, D>), longs, lblk, 0, stream, gg, p.H, p.dA,
                               static_cast<const T*>(p.K), static_cast<const T*>(nullptr),
                               static_cast<T*>(p.dQ), 1.0f, 0.0f);
    }
    if (rows_states && rows_transposed_supported(g, p.B, p.H, D)) {
        hipError_t e = launch_transpose_struct(g, p.B, p.H, p.dA, p.At, stream);
        if (e == hipSuccess)
            e = launch_grad_rows(g, p.B, p.H, p.At, p.dA, true, p.Q, p.dK, p.dtype, 1.0f, stream);
        return e;
    }
    hipLaunchKernelGGL(k_to_columns, entries, blk, 0, stream, ci, p.H, BH, entry_blocks, p.dA,
                       p.At);
    hipLaunchKernelGGL((k_cols<T, T, D>), rows, blk, 0, stream, ci, p.H, BH, p.At,
                       static_cast<const T*>(p.Q), static_cast<T*>(p.dK), 1.0f);
    if (g.max_long_col > 0)
        hipLaunchKernelGGL((k_cols_long<T, T, D>), long_cols, lblk, 0, stream, ci, p.H,
                           g.d_long_cols, g.d_long_col_off, p.At, static_cast<const T*>(p.Q),
                           static_cast<T*>(p.dK), 1.0f);
    return hipGetLastError();
}

template <typename T>
hipError_t backward_d(const diffuser_graph& g, const BackwardArgs& p, hipStream_t st) {
    switch (p.d) {
        case 16: return backward_t<T, 16>(g, p, st);
        case 32: return backward_t<T, 32>(g, p, st);
        case 64: return backward_t<T, 64>(g, p, st);
        case 128: return backward_t<T, 128>(g, p, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_backward(const diffuser_graph& g, const BackwardArgs& p, hipStream_t st) {
    if (p.dtype == DIFFUSER_F32) return backward_d<float>(g, p, st);
    return backward_d<bf16_t>(g, p, st);
}

}  // namespace diffuser
