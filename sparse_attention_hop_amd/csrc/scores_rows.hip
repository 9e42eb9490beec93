// Fused edge scores and edge softmax on built graphs with fp32 storage
// ("Diffuser" reading notes, section 2.1, eqs. S.1-S.5; "1.2.1 Static
// sparsity", section 1, eqs. 1-3):
//   s_ij = q_i . k_j / sqrt(d_h) on the edges of row i,
//   w_ij = exp(s_ij - m_i) stored, c_i = 1 / sum_j w_ij,
// so that c_i w_ij is the row's softmax. As in the generic kernel the shift
// m_i is the row's own score (the self-loop is an edge of every row, so it
// is at most the maximum and the largest weight is at least 1); a row whose
// weights sum to 2^64 or more is redone with its exact maximum, and its
// stored weights are then normalised, with c_i over them as stored.
//
// One wavefront per row, as in the generic kernel, with the key rows of the
// window band and of the global columns served from LDS: a workgroup of 16
// waves owns 64 consecutive rows of one (batch, head) pair and first copies
// into LDS every key row a window slot of its rows can name and the g
// global key rows, by direct global-to-LDS loads. A lane holds 4 channels
// of q_i and of a key row (lane group q, lanes 16 q .. + 15); each group
// scores 4 slots at a time, its dot products reduced over the group's 16
// lanes:
//  * window slots: 16 consecutive columns per step, lane group q taking
//    columns 4 q .. 4 q + 3, key rows from LDS, the four weights stored in
//    one 16-byte store; block padding stores 0;
//  * global-column slots: the same over the row's global slots (G[t] from
//    LDS in global order), padding (a global in the window or, when causal,
//    above the row) stores 0;
//  * random edges: key rows gathered from K in global memory, four
//    consecutive edges per lane group, their slots and columns in one
//    16-byte load each.
// Global rows with more than kLongRow slots (a global row's segment is every
// column, or when causal every column up to the row) go to a second kernel
// that scores each key row, read once, for four of them; the shorter
// global rows of a causal graph's first rows are scored here from K in
// global memory. The random area's dummy slots are zeroed as the generic
// pass does.
#include "internal.h"
#include "mfma_util.h"
#include "vec.h"

namespace diffuser {
namespace {

constexpr int kWave = 64;
constexpr int kWaves = 16;
constexpr int kThreads = kWave * kWaves;
constexpr int kRowsPerWave = 4;
constexpr int kRowsPerGroup = kWaves * kRowsPerWave;
constexpr int kLdsLimit = 160 * 1024;
constexpr int kGlobPad = 16;   // zero key rows past the globals (a global tile reads up to 15 past g)
constexpr int64_t kMinGroups = 1024;
constexpr float kSumLimit = 18446744073709551616.0f;   // 2^64

struct SRowsArgs {
    int64_t n;
    int32_t H, num_graphs, radius, causal, g;
    int32_t win_rows;
    int32_t items, per_xcd, blocks;
    GenericGraph gg;
    const int4* row_info;          // [graphs][n]
    const int32_t* G;              // [g]
    const void* Q;                 // fp32 or bf16 (the kernels' T)
    const void* K;
    float* A;
    float* row_scale;              // [B*H][n]
    float scale_log2;              // log2(e) / sqrt(d_h)
};

// Four channels of a query or key row as floats, from global memory or LDS.
__device__ __forceinline__ f32x4 bf4(u32x2 u) {
    return f32x4{bf16_to_f32(u[0] & 0xffffu), bf16_to_f32(u[0] >> 16), bf16_to_f32(u[1] & 0xffffu),
                 bf16_to_f32(u[1] >> 16)};
}
__device__ __forceinline__ f32x4 ld4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ f32x4 ld4(const bf16_t* p) { return bf4(*reinterpret_cast<const u32x2*>(p)); }

__device__ __forceinline__ float dot4(const f32x4& q, const f32x4& k) {
    return fmaf(q[3], k[3], fmaf(q[2], k[2], fmaf(q[1], k[1], q[0] * k[0])));
}

// v plus the value of the lane that DPP control `ctrl` names.
template <int ctrl>
__device__ __forceinline__ float dpp_add(float v) {
    return v + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), ctrl, 0xf, 0xf, true));
}

// Lane u of the caller's row of 16 lanes (DPP row_newbcast).
template <int u>
__device__ __forceinline__ int32_t row16_lane(int32_t v) {
    return __builtin_amdgcn_mov_dpp(v, 0x150 + u, 0xf, 0xf, false);
}

// Sum over the 16 lanes of a lane group (every lane gets it), by DPP within
// each row of 16 lanes: lane pairs, then quads (quad permutations), then
// the two halves of 8 (half-row mirror) and of 16 (row mirror); each step
// pairs lanes that hold sums of disjoint sets.
__device__ __forceinline__ float group_sum(float v) {
    v = dpp_add<0xB1>(v);    // quad_perm [1, 0, 3, 2]
    v = dpp_add<0x4E>(v);    // quad_perm [2, 3, 0, 1]
    v = dpp_add<0x141>(v);   // row_half_mirror
    v = dpp_add<0x140>(v);   // row_mirror
    return v;
}

// LDS layout of the key rows: a row's 16-byte pieces are permuted so that
// the 16 consecutive rows one MFMA operand read touches (lane m reading row
// base + m at one channel offset) fall on distinct banks: piece position
// u ^ (row mod 16) for fp32 rows (16 pieces), u ^ ((row / 2) mod 8) for
// bf16 rows (8 pieces, two rows per bank cycle).
template <typename T>
__device__ __forceinline__ int32_t kpiece(int32_t row, int32_t u) {
    if constexpr (sizeof(T) == 4) return u ^ (row & 15);
    else return u ^ ((row >> 1) & 7);
}
// Channels ch .. ch + 3 (ch a multiple of 4) of LDS key row `row`.
__device__ __forceinline__ f32x4 klds4(const float LDS_AS* lds, int32_t row, int32_t ch) {
    return *reinterpret_cast<const f32x4 LDS_AS*>(lds + row * 64 + 4 * kpiece<float>(row, ch >> 2));
}
__device__ __forceinline__ f32x4 klds4(const bf16_t LDS_AS* lds, int32_t row, int32_t ch) {
    return bf4(*reinterpret_cast<const u32x2 LDS_AS*>(lds + row * 64 + 8 * kpiece<bf16_t>(row, ch >> 3) +
                                                     (ch & 7)));
}
__device__ __forceinline__ i16x4 klds4_bf16(const bf16_t LDS_AS* lds, int32_t row, int32_t ch) {
    return *reinterpret_cast<const i16x4 LDS_AS*>(lds + row * 64 + 8 * kpiece<bf16_t>(row, ch >> 3) +
                                                  (ch & 7));
}

// The band products of one 16 x 16 tile over the 64 channels: D[row m][key
// n] = Q[m] . K[n], lane (m, kq) supplying channels 16 s + 4 kq .. + 3 of
// query row m (from qrow, which points at channel 4 kq of it) and of key
// row `krow` (from LDS) for chunk s.
__device__ __forceinline__ f32x4 tile_dots(const float* qrow, const float LDS_AS* lds,
                                           int32_t krow, int kq) {
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const f32x4 q = ld4(qrow + 16 * s);
        const f32x4 z = klds4(lds, krow, 16 * s + 4 * kq);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(q[e], z[e], acc, 0, 0, 0);
    }
    return acc;
}
__device__ __forceinline__ f32x4 tile_dots(const bf16_t* qrow, const bf16_t LDS_AS* lds,
                                           int32_t krow, int kq) {
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s)
        acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
            *reinterpret_cast<const i16x4*>(qrow + 16 * s), klds4_bf16(lds, krow, 16 * s + 4 * kq),
            acc, 0, 0, 0);
    return acc;
}
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

template <int D, typename T>
__global__ __launch_bounds__(kThreads, 8)
void k_scores_rows_f32(SRowsArgs a) {
    static_assert(D == 64, "one 16-lane group per key row");
    constexpr int U = D * (int)sizeof(T) / 16;   // 16-byte pieces of a key row
    extern __shared__ __align__(16) char lds_raw[];
    T LDS_AS* lds = (T LDS_AS*)lds_raw;
    const int lane = __lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int sub = lane & 15, grp = lane >> 4;

    const int32_t item = (int32_t)(blockIdx.x & 7u) * a.per_xcd + (int32_t)(blockIdx.x >> 3);
    if (item >= a.items) return;
    const int32_t bh = item / a.blocks;
    const int64_t r0 = (int64_t)(item - bh * a.blocks) * kRowsPerGroup;
    const int32_t b = bh / a.H, h = bh - b * a.H;
    const int32_t gr = a.num_graphs == 1 ? 0 : b;
    const int64_t n = a.n;
    float* Abh = a.A + a_block_offset(a.gg.slot_off, a.num_graphs, a.H, b, h);
    const int4* info = a.row_info + (int64_t)gr * n;
    const __amdgpu_buffer_rsrc_t rG = buffer_rsrc(a.G, (uint32_t)(4 * a.g));
    const int64_t w0 = (r0 - a.radius < 0 ? 0 : r0 - a.radius) & ~7ll;
    const T* Qg = static_cast<const T*>(a.Q);
    const T* Kbh = static_cast<const T*>(a.K) + (int64_t)bh * n * D;

    // ---- key rows into LDS (as the fp32 diffusion step's) -----------------
    {
        const int32_t rows = a.win_rows + a.g + kGlobPad;
        const int32_t units = rows * U;
        char LDS_AS* ldsb = (char LDS_AS*)lds_raw;
        for (int32_t p0 = 64 * wave; p0 < units; p0 += 64 * kWaves) {
            const int32_t p = p0 + lane;
            const int32_t r = p / U, u = p - r * U;
            int64_t k = -1;
            if (r < a.win_rows) k = w0 + r;
            else if (r < a.win_rows + a.g) k = a.G[r - a.win_rows];
            const bool live = p < units && k >= 0 && k < n;
            if (live)
                dma16(reinterpret_cast<const char*>(Kbh + k * D) + 16 * kpiece<T>(r, u),
                      (void LDS_AS*)(ldsb + 16 * p0));
            else if (p < units)
                *reinterpret_cast<f32x4 LDS_AS*>(ldsb + 16 * p) = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
    // Shifts: each row's own score (the self-loop is an edge of every row).
    float LDS_AS* msh = reinterpret_cast<float LDS_AS*>(lds + (int64_t)(a.win_rows + a.g + kGlobPad) * D);
    float LDS_AS* psum = msh + kRowsPerGroup;   // [4][kRowsPerGroup] band sums per tile quarter
    i32x4 LDS_AS* rinfo = reinterpret_cast<i32x4 LDS_AS*>(psum + 4 * kRowsPerGroup);   // [kRowsPerGroup]
    full_barrier();
#pragma unroll 1
    for (int u = 0; u < kRowsPerWave; ++u) {
        const int64_t i = r0 + kWaves * u + wave;
        float ms = 0.0f;
        if (i < n) {
            const f32x4 q = ld4(Qg + ((int64_t)bh * n + i) * D + 4 * sub);
            ms = a.scale_log2 * group_sum(dot4(q, klds4(lds, (int32_t)(i - w0), 4 * sub)));
        }
        if (lane == 0) {
            msh[kWaves * u + wave] = ms;
            const int4 ri = i < n ? info[i] : make_int4(0, 0, -1, 0);
            rinfo[kWaves * u + wave] = i32x4{ri.x, ri.y, ri.z, ri.w};
        }
    }
    __syncthreads();

    // ---- window bands and global columns on MFMA ---------------------------
    // Wave w: block w / 4 (16 rows), tiles w mod 4, + 4, ... of its keys:
    // the window keys (16 consecutive per tile, from the first row's block
    // start through the last row's last window slot), then the globals.
    // Each weight exp(s - m_row) goes to its row's slot (0 for padding and
    // keys not the row's); the tiles' row sums meet in psum. Row and key
    // numbers fit 32 bits here (n < 2^31).
    {
        const int m = lane & 15, kq = lane >> 4;
        const int bb = wave >> 2, tq = wave & 3;
        const int32_t n32 = (int32_t)n, r = a.radius;
        const int32_t i0 = (int32_t)r0 + 16 * bb;
        float rsum[4] = {0.f, 0.f, 0.f, 0.f};
        if (i0 < n32) {
            const int32_t il = i0 + 15 < n32 ? i0 + 15 : n32 - 1;
            const int32_t J0 = (i0 - r < 0 ? 0 : i0 - r) & ~7;
            const int32_t wend_l = a.causal ? il : (il + r > n32 - 1 ? n32 - 1 : il + r);
            const int32_t twin = ((wend_l | 7) - J0) / 16 + 1;
            const int32_t ntile = twin + (a.g + 15) / 16;
            const int32_t qi = i0 + m;
            const T* qrow = Qg + ((int64_t)bh * n + (qi < n32 ? qi : i0)) * D + 4 * kq;
#pragma unroll 1
            for (int32_t t = tq; t < ntile; t += 4) {
                int32_t krow;
                if (t < twin) krow = min(J0 + 16 * t + m - (int32_t)w0, a.win_rows - 1);
                else krow = a.win_rows + 16 * (t - twin) + m;
                const f32x4 d = tile_dots(qrow, lds, krow, kq);
                const int32_t gt = 16 * (t - twin) + m;   // a global tile's slot
                const int32_t gc = t >= twin && gt < a.g ? a.G[gt] : -1;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    // the lane's output row i0 + 4 kq + v
                    const int32_t i = i0 + 4 * kq + v;
                    const i32x4 ri = rinfo[16 * bb + 4 * kq + v];
                    if (i >= n32 || ri[2] < 0) continue;   // past n, or a global row
                    const int32_t lo = i - r < 0 ? 0 : i - r;
                    const int32_t hi = i + r > n32 - 1 ? n32 - 1 : i + r;
                    int32_t slot;
                    bool ok;
                    if (t < twin) {
                        const int32_t j = J0 + 16 * t + m;
                        const int32_t s2 = j - ri[1];
                        if (s2 < 0 || s2 >= ri[2]) continue;
                        slot = ri[0] + s2;
                        ok = j >= lo && j <= (a.causal ? i : hi);
                    } else {
                        if (gt >= ri[3]) continue;
                        slot = ri[0] + ri[2] + gt;
                        ok = gc >= 0 && (gc < lo || gc > hi) && (!a.causal || gc <= i);
                    }
                    const float w = ok ? __builtin_amdgcn_exp2f(a.scale_log2 * d[v] -
                                                                msh[16 * bb + 4 * kq + v])
                                       : 0.0f;
                    Abh[slot] = w;
                    rsum[v] += w;
                }
            }
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const float t = group_sum(rsum[v]);
            if (m == 0) psum[tq * kRowsPerGroup + 16 * bb + 4 * kq + v] = t;
        }
    }
    __syncthreads();

#pragma unroll 1
    for (int u = 0; u < kRowsPerWave; ++u) {
        const int64_t i = r0 + kWaves * u + wave;
        if (i >= n) break;
        const int4 ri = info[i];
        const RowSlots rs = a.gg.row(gr, i);
        if (rs.count() > kLongRow) continue;   // a long global row: k_scores_grows_f32's
        // A global row here is one of a causal graph's first rows: its
        // segment holds its columns 0 .. i in order.
        const bool grow = ri.z < 0;
        const f32x4 q = ld4(Qg + ((int64_t)bh * n + i) * D + 4 * sub);
        const int64_t lo = i - a.radius < 0 ? 0 : i - a.radius;
        const int64_t hi = i + a.radius > n - 1 ? n - 1 : i + a.radius;
        const int64_t wend = a.causal ? i : hi;
        const int64_t last = a.causal ? i : n - 1;
        const int64_t wb0 = ri.y;
        const int32_t wseg = ri.z, gseg = ri.w;
        const int32_t nr = rs.rcnt;

        // Every slot of the row, four per lane group per step: f(kind, t0 or
        // the slots, valid[4], scaled scores[4]); kind 0 window (slots
        // seg + t0 .. + 3), 1 global (seg + wseg + t0 ..), 2 random, 3 a
        // short global row (seg + t0 ..).
        auto sweep = [&](bool band, auto&& f) {
            if (grow) {
                const int32_t len = (int32_t)rs.seg_len;
                for (int32_t tb = 0; tb < len; tb += 16) {
                    const int32_t t0 = tb + 4 * grp;
                    bool ok[4];
                    f32x4 kz[4];
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        ok[v] = t0 + v < len && t0 + v <= last;
                        kz[v] = ld4(Kbh + (int64_t)(ok[v] ? t0 + v : 0) * D + 4 * sub);
                    }
                    float s[4];
#pragma unroll
                    for (int v = 0; v < 4; ++v) s[v] = a.scale_log2 * group_sum(dot4(q, kz[v]));
                    f(3, t0, u32x4{0u, 0u, 0u, 0u}, ok, s);
                }
                return;
            }
            for (int32_t tb = 0; band && tb < wseg; tb += 16) {
                const int32_t t0 = tb + 4 * grp;
                bool ok[4];
                float s[4];
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int64_t c = wb0 + t0 + v;
                    ok[v] = t0 < wseg && c >= lo && c <= wend;
                    s[v] = a.scale_log2 * group_sum(dot4(q, klds4(lds, (int32_t)(ok[v] ? c - w0 : 0), 4 * sub)));
                }
                f(0, t0, u32x4{0u, 0u, 0u, 0u}, ok, s);
            }
            for (int32_t tb = 0; band && tb < gseg; tb += 16) {
                const int32_t t0 = tb + 4 * grp;
                const u32x4 gk = bload16(rG, t0 < min(gseg, a.g) ? 4u * (uint32_t)t0 : kOutside, 0u);
                bool ok[4];
                float s[4];
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int64_t k = (int32_t)gk[v];
                    ok[v] = t0 + v < min(gseg, a.g) && (k < lo || k > hi) && k <= last;
                    s[v] = a.scale_log2 * group_sum(dot4(q, klds4(lds, a.win_rows + (ok[v] ? t0 + v : 0), 4 * sub)));
                }
                f(1, t0, u32x4{0u, 0u, 0u, 0u}, ok, s);
            }
            for (int32_t eb = 0; eb < nr; eb += 16) {
                const int32_t e0 = eb + 4 * grp;
                // one index load per lane: slots from lanes 0-3, columns
                // from lanes 4-7 of the group (DPP row_newbcast)
                const int32_t el = e0 + (sub & 3);
                const int32_t ix = el < nr ? ((sub & 4) ? rs.rcol : rs.rslot)[el] : 0;
                const u32x4 sl = u32x4{(uint32_t)row16_lane<0>(ix), (uint32_t)row16_lane<1>(ix),
                                       (uint32_t)row16_lane<2>(ix), (uint32_t)row16_lane<3>(ix)};
                const u32x4 cl = u32x4{(uint32_t)row16_lane<4>(ix), (uint32_t)row16_lane<5>(ix),
                                       (uint32_t)row16_lane<6>(ix), (uint32_t)row16_lane<7>(ix)};
                bool ok[4];
                f32x4 kz[4];
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    ok[v] = e0 + v < nr;
                    kz[v] = ld4(Kbh + (int64_t)(ok[v] ? (int32_t)cl[v] : 0) * D + 4 * sub);
                }
                float s[4];
#pragma unroll
                for (int v = 0; v < 4; ++v) s[v] = a.scale_log2 * group_sum(dot4(q, kz[v]));
                f(2, e0, sl, ok, s);
            }
        };
        // The weights w[4] of one step into A (lane sub == 0 of the group).
        auto store = [&](int kind, int32_t t0, const u32x4& sl, const bool (&ok)[4],
                         const float (&w)[4]) {
            if (sub != 0) return;
            if (kind == 3) {
                if (t0 < rs.seg_len)
                    *reinterpret_cast<f32x4*>(Abh + ri.x + t0) = f32x4{w[0], w[1], w[2], w[3]};
            } else if (kind == 0) {
                if (t0 < wseg)
                    *reinterpret_cast<f32x4*>(Abh + ri.x + t0) = f32x4{w[0], w[1], w[2], w[3]};
            } else if (kind == 1) {
                if (t0 < gseg)
                    *reinterpret_cast<f32x4*>(Abh + ri.x + wseg + t0) = f32x4{w[0], w[1], w[2], w[3]};
            } else {
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    if (ok[v]) Abh[sl[v]] = w[v];
            }
        };

        // The fused single pass, shifted by the row's own score: the random
        // edges here (a short global row: every slot), the band's weights and
        // sums from the MFMA tiles.
        const float ms = msh[i - r0];
        float total = 0.0f;
        if (!grow)
            for (int t = 0; t < 4; ++t) total += psum[t * kRowsPerGroup + (i - r0)];
        float rtot = 0.0f;
        sweep(false, [&](int kind, int32_t t0, const u32x4& sl, const bool (&ok)[4], const float (&s)[4]) {
            float w[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) w[v] = ok[v] ? __builtin_amdgcn_exp2f(s[v] - ms) : 0.0f;
            store(kind, t0, sl, ok, w);
            if (sub == 0) rtot += (w[0] + w[1]) + (w[2] + w[3]);
        });
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) rtot += __shfl_xor(rtot, off);
        total += rtot;
        if (total < kSumLimit) {
            if (lane == 0) a.row_scale[(int64_t)bh * n + i] = 1.0f / total;
            continue;
        }
        // Redone with the exact maximum: its (max, sum), then the normalised
        // weights and c_i over them as stored.
        float m = -INFINITY;
        sweep(true, [&](int, int32_t, const u32x4&, const bool (&ok)[4], const float (&s)[4]) {
#pragma unroll
            for (int v = 0; v < 4; ++v) m = ok[v] ? fmaxf(m, s[v]) : m;
        });
#pragma unroll
        for (int off = 16; off < kWave; off <<= 1) m = fmaxf(m, __shfl_xor(m, off));
        float l = 0.0f;
        sweep(true, [&](int, int32_t, const u32x4&, const bool (&ok)[4], const float (&s)[4]) {
#pragma unroll
            for (int v = 0; v < 4; ++v) l += ok[v] ? __builtin_amdgcn_exp2f(s[v] - m) : 0.0f;
        });
#pragma unroll
        for (int off = 16; off < kWave; off <<= 1) l += __shfl_xor(l, off);
        const float inv = 1.0f / l;
        float stored = 0.0f;
        sweep(true, [&](int kind, int32_t t0, const u32x4& sl, const bool (&ok)[4], const float (&s)[4]) {
            float w[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) w[v] = ok[v] ? __builtin_amdgcn_exp2f(s[v] - m) * inv : 0.0f;
            store(kind, t0, sl, ok, w);
            if (sub == 0) stored += (w[0] + w[1]) + (w[2] + w[3]);
        });
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) stored += __shfl_xor(stored, off);
        if (lane == 0) a.row_scale[(int64_t)bh * n + i] = 1.0f / stored;
    }
}

// Long global rows, kGRows per workgroup: the 16 waves split the keys into
// contiguous ranges and score every key row, read once per workgroup, for
// all kGRows rows (lane group q taking 4 consecutive keys, their weights
// stored with one 16-byte store per row); a row's sums meet in LDS in wave
// order. A row whose weights reach 2^64 is redone by the whole workgroup
// with its exact maximum: the maximum, the sum, then the normalised weights
// and c_i over them as stored. Short global rows (a causal graph's first
// rows) are the row kernel's.
constexpr int kGRows = 4;

template <int D, typename T>
__global__ __launch_bounds__(kThreads)
void k_scores_grows_f32(SRowsArgs a, int32_t gblocks) {
    __shared__ float red[kWaves][kGRows];
    const int lane = __lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int sub = lane & 15, grp = lane >> 4;
    const int32_t bh = blockIdx.x / gblocks;
    const int32_t q0 = (blockIdx.x - bh * gblocks) * kGRows;
    const int32_t b = bh / a.H, h = bh - b * a.H;
    const int32_t gr = a.num_graphs == 1 ? 0 : b;
    const int64_t n = a.n;
    float* Abh = a.A + a_block_offset(a.gg.slot_off, a.num_graphs, a.H, b, h);
    const T* Qg = static_cast<const T*>(a.Q);
    const T* Kbh = static_cast<const T*>(a.K) + (int64_t)bh * n * D;
    const int4* info = a.row_info + (int64_t)gr * n;
    const int64_t* sp = a.gg.seg_ptr + (int64_t)gr * (n + 1);
    // The rows: segment start, last column (-1: not this kernel's), q, shift.
    uint32_t seg[kGRows];
    int64_t seglen[kGRows];   // slots of the row's segment (when causal, columns 0 .. i, padded)
    int64_t last[kGRows];
    f32x4 q[kGRows];
    float ms[kGRows];
#pragma unroll
    for (int r = 0; r < kGRows; ++r) {
        const int32_t qi = q0 + r;
        const int64_t i = qi < a.g ? a.G[qi] : -1;
        seglen[r] = i >= 0 ? sp[i + 1] - sp[i] : 0;
        const bool mine = seglen[r] > kLongRow;
        seg[r] = mine ? (uint32_t)info[i].x : 0u;
        last[r] = !mine ? -1 : a.causal ? i : n - 1;
        q[r] = mine ? ld4(Qg + ((int64_t)bh * n + i) * D + 4 * sub) : f32x4{0.f, 0.f, 0.f, 0.f};
        ms[r] = mine ? a.scale_log2 * group_sum(dot4(q[r], ld4(Kbh + i * D + 4 * sub))) : 0.0f;
    }
    const int64_t k0 = n * wave / kWaves, k1 = n * (wave + 1) / kWaves;
    // f(r, j0, ok[4], scaled scores[4]) for every row and every 4 keys of the wave.
    auto sweep = [&](auto&& f) {
        for (int64_t kb = k0 & ~3ll; kb < k1; kb += 16) {
            const int64_t j0 = kb + 4 * grp;
            f32x4 kz[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int64_t j = j0 + v;
                kz[v] = ld4(Kbh + (j >= k0 && j < k1 ? j : 0) * D + 4 * sub);
            }
#pragma unroll
            for (int r = 0; r < kGRows; ++r) {
                if (last[r] < 0) continue;
                bool ok[4];
                float sc[4];
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int64_t j = j0 + v;
                    ok[v] = j >= k0 && j < k1 && j <= last[r];
                    sc[v] = a.scale_log2 * group_sum(dot4(q[r], kz[v]));
                }
                f(r, j0, ok, sc);
            }
        }
    };
    // One value per (wave, row) summed (or maxed) over the waves in wave
    // order, into every thread.
    auto merge = [&](float (&v)[kGRows], bool is_max) {
#pragma unroll
        for (int r = 0; r < kGRows; ++r) {
#pragma unroll
            for (int off = 16; off < kWave; off <<= 1) {
                const float o = __shfl_xor(v[r], off);
                v[r] = is_max ? fmaxf(v[r], o) : v[r] + o;
            }
            if (lane == 0) red[wave][r] = v[r];
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < kGRows; ++r) {
            float t = is_max ? -INFINITY : 0.0f;
            for (int w = 0; w < kWaves; ++w) t = is_max ? fmaxf(t, red[w][r]) : t + red[w][r];
            v[r] = t;
        }
        __syncthreads();
    };
    // Weights w[4] of row r at keys j0 .. j0 + 3 (all four in the segment).
    auto store = [&](int r, int64_t j0, const float (&w)[4]) {
        if (sub == 0 && j0 >= 0)
            *reinterpret_cast<f32x4*>(Abh + seg[r] + j0) = f32x4{w[0], w[1], w[2], w[3]};
    };

    // The fused single pass, shifted by each row's own score. Keys of the
    // 4-key block outside the wave's range are another wave's to store.
    float total[kGRows];
#pragma unroll
    for (int r = 0; r < kGRows; ++r) total[r] = 0.0f;
    sweep([&](int r, int64_t j0, const bool (&ok)[4], const float (&sc)[4]) {
        float w[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) w[v] = ok[v] ? __builtin_amdgcn_exp2f(sc[v] - ms[r]) : 0.0f;
        // (a segment is a multiple of 8 slots: the 4 keys lie in it or past it)
        if (j0 < seglen[r]) {
            if (j0 >= k0 && j0 + 3 < k1) store(r, j0, w);
            else if (sub == 0)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    if (j0 + v >= k0 && j0 + v < k1) Abh[seg[r] + j0 + v] = w[v];
        }
        if (sub == 0) total[r] += (w[0] + w[1]) + (w[2] + w[3]);
    });
    // Slots past column n - 1 (a segment is a multiple of 8 slots) weigh 0.
    if (k1 == n && sub == 0) {
#pragma unroll
        for (int r = 0; r < kGRows; ++r) {
            if (last[r] < 0) continue;
            for (int64_t j = n + grp; j < seglen[r]; j += 4) Abh[seg[r] + j] = 0.0f;
        }
    }
    merge(total, false);
    bool redo = false;
#pragma unroll
    for (int r = 0; r < kGRows; ++r) {
        if (last[r] < 0) continue;
        if (total[r] < kSumLimit) {
            if (threadIdx.x == 0) a.row_scale[(int64_t)bh * n + a.G[q0 + r]] = 1.0f / total[r];
        } else {
            redo = true;
        }
    }
    if (!redo) return;   // the same in every thread
    // Rows whose weights reached 2^64, redone with the exact maximum.
    float m[kGRows], l[kGRows], st[kGRows];
#pragma unroll
    for (int r = 0; r < kGRows; ++r) {
        m[r] = -INFINITY;
        l[r] = 0.0f;
        st[r] = 0.0f;
        if (total[r] < kSumLimit) last[r] = -1;   // done
    }
    sweep([&](int r, int64_t, const bool (&ok)[4], const float (&sc)[4]) {
#pragma unroll
        for (int v = 0; v < 4; ++v) m[r] = ok[v] ? fmaxf(m[r], sc[v]) : m[r];
    });
    merge(m, true);
    sweep([&](int r, int64_t, const bool (&ok)[4], const float (&sc)[4]) {
        if (sub == 0)
#pragma unroll
            for (int v = 0; v < 4; ++v) l[r] += ok[v] ? __builtin_amdgcn_exp2f(sc[v] - m[r]) : 0.0f;
    });
    merge(l, false);
    sweep([&](int r, int64_t j0, const bool (&ok)[4], const float (&sc)[4]) {
        const float inv = 1.0f / l[r];
        float w[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) w[v] = ok[v] ? __builtin_amdgcn_exp2f(sc[v] - m[r]) * inv : 0.0f;
        if (sub == 0 && j0 < seglen[r])
#pragma unroll
            for (int v = 0; v < 4; ++v)
                if (j0 + v >= k0 && j0 + v < k1) Abh[seg[r] + j0 + v] = w[v];
        if (sub == 0) st[r] += (w[0] + w[1]) + (w[2] + w[3]);
    });
    merge(st, false);
#pragma unroll
    for (int r = 0; r < kGRows; ++r)
        if (last[r] >= 0 && threadIdx.x == 0)
            a.row_scale[(int64_t)bh * n + a.G[q0 + r]] = 1.0f / st[r];
}

// Key rows of the window run: the group's rows, the radius on either side
// (on the left only when causal) and the 8-column alignment of its start.
// A per-row slot outside its row's window or global set reads LDS row 0
// with a zero weight, and a band tile's keys past the run read its last
// row, so no rows are needed past the run.
int32_t win_rows(const diffuser_graph& g) {
    return kRowsPerGroup + (g.causal ? 1 : 2) * g.radius + 8;
}

// The key rows (window run, globals and kGlobPad zero rows), then the rows'
// shifts, the band sums of the four tile quarters and the rows' geometry.
int32_t lds_bytes(const diffuser_graph& g, diffuser_dtype dt) {
    return (win_rows(g) + g.num_global + kGlobPad) * 64 * (dt == DIFFUSER_F32 ? 4 : 2) +
           9 * kRowsPerGroup * 4;
}

template <typename T>
hipError_t launch_args(const diffuser_graph& g, const attn_shape& s, const SRowsArgs& a,
                       hipStream_t st) {
    static int attr_device = -1;
    if (attr_device != g.device) {
        hipError_t e =
            hipFuncSetAttribute(reinterpret_cast<const void*>(&k_scores_rows_f32<64, T>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, kLdsLimit);
        if (e != hipSuccess) return e;
        attr_device = g.device;
    }
    hipLaunchKernelGGL((k_scores_rows_f32<64, T>), dim3((unsigned)(8 * a.per_xcd)),
                       dim3(kThreads), (size_t)lds_bytes(g, s.dtype), st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (g.num_global > 0) {
        const int32_t gblocks = (g.num_global + kGRows - 1) / kGRows;
        hipLaunchKernelGGL((k_scores_grows_f32<64, T>), dim3((unsigned)(s.B * s.H * gblocks)),
                           dim3(kThreads), 0, st, a, gblocks);
        e = hipGetLastError();
    }
    return e;
}

SRowsArgs make_sargs(const diffuser_graph& g, const attn_shape& s, const void* Q, const void* K,
                     void* A, float* row_scale, float scale_log2) {
    SRowsArgs a;
    a.n = g.n;
    a.H = s.H;
    a.num_graphs = g.num_graphs;
    a.radius = g.radius;
    a.causal = g.causal;
    a.g = g.num_global;
    a.win_rows = win_rows(g);
    a.blocks = (int32_t)((g.n + kRowsPerGroup - 1) / kRowsPerGroup);
    a.items = s.B * s.H * a.blocks;
    a.per_xcd = (a.items + 7) / 8;
    a.gg = generic_graph(g);
    a.row_info = reinterpret_cast<const int4*>(g.d_row_info);
    a.G = g.d_global;
    a.Q = Q;
    a.K = K;
    a.A = static_cast<float*>(A);
    a.row_scale = row_scale;
    a.scale_log2 = scale_log2;
    return a;
}

}  // namespace

bool rows_scores_supported(const diffuser_graph& g, const attn_shape& s) {
    return s.dtype == DIFFUSER_F32 && rows_scores_any_supported(g, s);
}

bool rows_scores_any_supported(const diffuser_graph& g, const attn_shape& s) {
    if (!g.structured || !g.rand_apart() || g.d_row_info == nullptr || s.d != 64 ||
        g.n <= kLongRow)
        return false;
    for (int64_t x : g.slots)
        if (4 * x >= (1ll << 31)) return false;
    const int64_t groups = (int64_t)s.B * s.H * ((g.n + kRowsPerGroup - 1) / kRowsPerGroup);
    // Every long row must be a global row: a row's window blocks, global
    // slots and random edges stay within kLongRow.
    const int64_t row_max = 2 * (int64_t)g.radius + 16 + ((g.num_global + 7) & ~7) + g.rnd_width;
    return groups >= kMinGroups && 2 * lds_bytes(g, s.dtype) <= kLdsLimit && row_max <= kLongRow;
}

hipError_t launch_scores_rows(const diffuser_graph& g, const attn_shape& s, const void* Q,
                              const void* K, void* A, float* row_scale, float scale_log2,
                              hipStream_t st) {
    const SRowsArgs a = make_sargs(g, s, Q, K, A, row_scale, scale_log2);
    const hipError_t e = s.dtype == DIFFUSER_F32 ? launch_args<float>(g, s, a, st)
                                                 : launch_args<bf16_t>(g, s, a, st);
    if (e != hipSuccess) return e;
    return launch_zero_dummies_f32(g, s, A, st);
}

}  // namespace diffuser
