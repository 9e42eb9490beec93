// One diffusion step ("Diffuser" reading notes, section 2.4, eq. S.7):
//   Z_{k+1}[i] = (1 - alpha) * sum_{j in N(i)} A_ij Z_k[j] + alpha * V[i],
// written as keep * c_i * sum_j A_ij Z_k[j] + restart * V[i] so that the
// same step also evaluates general coefficients (section 2.3, eq. S.6) in
// nested form. The edge weights A are the same in every step; only Z changes.
//
// Generic path (any slot layout: the row segment, then any scheduled random
// slots; padding slots are skipped). One wavefront
// per row. A group of L lanes gathers one neighbour row of Z_k
// with 16-byte loads (L = d * elem_size / 16), so a wave consumes 64 / L
// edges per step, and issues the loads of kUnroll steps before it uses any
// of them (the step is bound by these dependent index and row loads); the
// groups' partial sums are reduced at the end and the restart term is fused
// into the store.
// Long rows (more than kLongRow slots, a global row's n, say) are left to
// a companion kernel that gives each one a workgroup of kLongWaves waves:
// every wave sums a contiguous share of the row's slots as above, and the
// waves' partial sums are added in wave order, so no wave walks a whole
// long row and every sum keeps a fixed order.
#include "internal.h"
#include "vec.h"

namespace diffuser {
namespace {

constexpr int kWave = 64;
constexpr int kWavesPerBlock = 4;
constexpr int kUnroll = 4;
constexpr int kLongWaves = 16;

// acc (lane group grp's share) += sum over slots [e0, e1) of the row,
// group grp taking slots e0 + u EPI + grp of each step.
template <typename T, int D>
__device__ __forceinline__ void gather_slots(const RowSlots& rs, const T* Ab, const T* Zb,
                                             int64_t e0, int64_t e1, int grp,
                                             float (&acc)[chunk<T>::kElems]) {
    constexpr int E = chunk<T>::kElems;
    constexpr int EPI = kWave / (D / E);
    for (int64_t base = e0; base < e1; base += EPI * kUnroll) {
        // Padding and slots past the range read row 0 with weight 0.
        int32_t j[kUnroll];
        int64_t slot[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t e = base + u * EPI + grp;
            j[u] = -1;
            slot[u] = e < e1 ? rs.slot(e, j[u]) : 0;
        }
        float a[kUnroll], z[kUnroll][E];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            a[u] = j[u] >= 0 ? chunk<T>::load1(Ab + slot[u]) : 0.0f;
            chunk<T>::load(Zb + (int64_t)(j[u] >= 0 ? j[u] : 0) * D, z[u]);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
#pragma unroll
            for (int c = 0; c < E; ++c) acc[c] = fmaf(a[u], z[u][c], acc[c]);
    }
}

template <typename T, int D>
__global__ __launch_bounds__(kWave * kWavesPerBlock)
void k_diffuse_step(GenericGraph gg, int32_t H, int32_t BH, const T* __restrict__ A,
                    const T* __restrict__ Zk,
                    const T* __restrict__ V, T* __restrict__ Zn,
                    const float* __restrict__ row_scale, step_coefs kc) {
    constexpr int E = chunk<T>::kElems;
    constexpr int L = D / E;
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
    if (e1 > kLongRow) return;   // k_diffuse_long's
    const T* Ab = A + a_block_offset(gg.slot_off, gg.num_graphs, H, b, h);
    const int sub = lane % L, grp = lane / L;
    const T* Zb = Zk + (int64_t)bh * n * D + sub * E;

    float acc[E];
#pragma unroll
    for (int c = 0; c < E; ++c) acc[c] = 0.0f;
    gather_slots<T, D>(rs, Ab, Zb, 0, e1, grp, acc);
#pragma unroll
    for (int off = L; off < kWave; off <<= 1) {
#pragma unroll
        for (int c = 0; c < E; ++c) acc[c] += __shfl_xor(acc[c], off);
    }
    if (grp == 0) {
        const int64_t o = ((int64_t)bh * n + i) * D + sub * E;
        float v[E];
        chunk<T>::load(V + o, v);
        const float keep =
            row_scale == nullptr ? kc.keep : kc.keep * row_scale[(int64_t)bh * n + i];
#pragma unroll
        for (int c = 0; c < E; ++c) v[c] = keep * acc[c] + kc.restart * v[c];
        chunk<T>::store(Zn + o, v);
    }
}

// One long row per workgroup: long row blockIdx.x of the graph of pair
// blockIdx.y.
template <typename T, int D>
__global__ __launch_bounds__(kWave * kLongWaves)
void k_diffuse_long(GenericGraph gg, int32_t H, const T* __restrict__ A,
                    const T* __restrict__ Zk, const T* __restrict__ V, T* __restrict__ Zn,
                    const float* __restrict__ row_scale, step_coefs kc) {
    constexpr int E = chunk<T>::kElems;
    constexpr int L = D / E;
    __shared__ float part[kLongWaves][D];
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
    const T* Ab = A + a_block_offset(gg.slot_off, gg.num_graphs, H, b, h);
    const int sub = lane % L, grp = lane / L;
    const T* Zb = Zk + (int64_t)bh * n * D + sub * E;

    float acc[E];
#pragma unroll
    for (int c = 0; c < E; ++c) acc[c] = 0.0f;
    gather_slots<T, D>(rs, Ab, Zb, e0, e1, grp, acc);
#pragma unroll
    for (int off = L; off < kWave; off <<= 1) {
#pragma unroll
        for (int c = 0; c < E; ++c) acc[c] += __shfl_xor(acc[c], off);
    }
    if (grp == 0) {
#pragma unroll
        for (int c = 0; c < E; ++c) part[wave][sub * E + c] = acc[c];
    }
    __syncthreads();
    if (threadIdx.x < L) {
        const int s = threadIdx.x;
        float v[E];
#pragma unroll
        for (int c = 0; c < E; ++c) {
            float t = 0.0f;
            for (int w = 0; w < kLongWaves; ++w) t += part[w][s * E + c];
            acc[c] = t;
        }
        const int64_t o = ((int64_t)bh * n + i) * D + s * E;
        chunk<T>::load(V + o, v);
        const float keep =
            row_scale == nullptr ? kc.keep : kc.keep * row_scale[(int64_t)bh * n + i];
#pragma unroll
        for (int c = 0; c < E; ++c) v[c] = keep * acc[c] + kc.restart * v[c];
        chunk<T>::store(Zn + o, v);
    }
}

template <typename T, int D>
hipError_t launch_t(const diffuser_graph& g, const attn_shape& s, const void* A, const void* Zk,
                    const void* V, void* Zn, const float* row_scale, step_coefs kc,
                    hipStream_t st) {
    const dim3 grid = xcd_row_grid(g.n, s.B * s.H, kWavesPerBlock);
    hipLaunchKernelGGL((k_diffuse_step<T, D>), grid, dim3(kWave * kWavesPerBlock), 0, st,
                       generic_graph(g), s.H, s.B * s.H, static_cast<const T*>(A),
                       static_cast<const T*>(Zk), static_cast<const T*>(V),
                       static_cast<T*>(Zn), row_scale, kc);
    if (g.max_long > 0)
        hipLaunchKernelGGL((k_diffuse_long<T, D>), dim3((unsigned)g.max_long, (unsigned)(s.B * s.H)),
                           dim3(kWave * kLongWaves), 0, st, generic_graph(g), s.H,
                           static_cast<const T*>(A), static_cast<const T*>(Zk),
                           static_cast<const T*>(V), static_cast<T*>(Zn), row_scale, kc);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_d(const diffuser_graph& g, const attn_shape& s, const void* A, const void* Zk,
                    const void* V, void* Zn, const float* row_scale, step_coefs kc,
                    hipStream_t st) {
    switch (s.d) {
        case 16: return launch_t<T, 16>(g, s, A, Zk, V, Zn, row_scale, kc, st);
        case 32: return launch_t<T, 32>(g, s, A, Zk, V, Zn, row_scale, kc, st);
        case 64: return launch_t<T, 64>(g, s, A, Zk, V, Zn, row_scale, kc, st);
        case 128: return launch_t<T, 128>(g, s, A, Zk, V, Zn, row_scale, kc, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

GenericGraph generic_graph(const diffuser_graph& g) {
    GenericGraph gg;
    gg.n = g.n;
    gg.num_graphs = g.num_graphs;
    gg.rnd_width = g.rnd_width;
    gg.seg_ptr = g.d_seg_ptr;
    gg.slot_col = g.d_slot_col;
    gg.slot_off = g.d_slot_off;
    gg.rnd = g.rand_apart() ? g.d_rnd : nullptr;
    gg.rnd_cnt = g.rand_apart() ? g.d_rnd_cnt : nullptr;
    gg.rslot = g.rand_apart() ? g.d_rslot : nullptr;
    gg.long_rows = g.d_long_rows;
    gg.long_off = g.d_long_off;
    return gg;
}

hipError_t launch_diffuse_step(const diffuser_graph& g, const attn_shape& s, const void* A,
                               const void* Zk, const void* V, void* Zn, const float* row_scale,
                               step_coefs kc, hipStream_t st) {
    if (s.dtype == DIFFUSER_F32)
        return launch_d<float>(g, s, A, Zk, V, Zn, row_scale, kc, st);
    return launch_d<bf16_t>(g, s, A, Zk, V, Zn, row_scale, kc, st);
}

}  // namespace diffuser
