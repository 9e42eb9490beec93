// Diffusion step on built graphs with fp32 states (keys fp32 or bf16), the
// key rows of the window band and of the global columns served from LDS:
//   Z_{k+1}[i] = keep * c_i * sum_j A_ij Z_k[j] + restart * V[i]
// ("Diffuser" reading notes, section 2.4, eq. S.7, with keep = 1 - alpha and
// restart = alpha; other coefficients evaluate section 2.3's eq. S.6 in
// nested form; c_i rescales the stored weights of row i to sum to one, or
// is 1). The same kernels serve the backward's products with fp32 weights:
// the recomputed states, the transposed products (A^T laid out in the
// graph's slot geometry, the random edges listed by column) and dQ, dK.
//
// A workgroup of 16 waves owns kRowsPerGroup consecutive rows of one
// (batch, head) pair. It first copies into LDS, by direct global-to-LDS
// loads, every key row that a window slot of its rows can name (one
// contiguous run of Z_k around its rows) and the key rows of the g global
// columns. The window and global slots, most of a row's edges, are then a
// dense product per block of 16 rows on MFMA (k_diffuse_rows_mma), which
// reads each key row from LDS once per block instead of once per row; the
// random edges are gathered from Z_k in global memory a row at a time, and
// the restart term is fused into the store. Global rows (whose segment is
// every column) go to a second kernel, 16 of them against each key row on
// MFMA.
#include <algorithm>
#include <type_traits>

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
constexpr int kGlobPad = 16;       // zero rows past the globals (a global step reads up to 15 past gs)
constexpr int kLdsLimit = 160 * 1024;
constexpr int64_t kMinGroups = 1024;   // workgroups below which the generic step is used

struct RowsArgs {
    int64_t n;
    int32_t H, num_graphs, radius, causal, g;
    int32_t win_rows;              // key rows of the window run in LDS (padding included)
    int32_t items, per_xcd, blocks;   // work items, per XCD, row groups per pair
    GenericGraph gg;
    const int4* row_info;          // [graphs][n]
    const int32_t* G;              // [g]
    const float* A;
    const float* AR;               // weights of the random edges' slots (A unless transposed)
    // Random edges by column (transposed products), or null: the graph's rows.
    const int64_t* t_ptr;          // [graphs][n + 1]
    const int32_t* t_slot;
    const int32_t* t_row;
    const void* Z;                 // key rows (the kernels' TX)
    const void* V;                 // restart rows (TV), or null when restart = 0
    void* Zn;                      // output rows (TY)
    const float* row_scale;        // [B*H][n] or null
    float keep, restart;
};

// Four channels of a row (fp32 or bf16) as floats, from global memory or a
// buffer load, and four floats stored as a row's channels.
__device__ __forceinline__ f32x4 bf4(u32x2 u) {
    return f32x4{bf16_to_f32(u[0] & 0xffffu), bf16_to_f32(u[0] >> 16), bf16_to_f32(u[1] & 0xffffu),
                 bf16_to_f32(u[1] >> 16)};
}
__device__ __forceinline__ f32x4 ld4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ f32x4 ld4(const bf16_t* p) { return bf4(*reinterpret_cast<const u32x2*>(p)); }
template <typename TX>
__device__ __forceinline__ f32x4 bload4(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    if constexpr (sizeof(TX) == 4) return __builtin_bit_cast(f32x4, bload16(r, voff, 0u));
    else return bf4(bload8(r, voff, 0u));
}
__device__ __forceinline__ void st4(float* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }
__device__ __forceinline__ void st4(bf16_t* p, f32x4 v) {
    *reinterpret_cast<u32x2*>(p) = u32x2{f32_to_bf16(v[0]) | (f32_to_bf16(v[1]) << 16),
                                         f32_to_bf16(v[2]) | (f32_to_bf16(v[3]) << 16)};
}

// keep * acc + restart * V[o .. o + 3], with no read of V when restart = 0.
template <typename TV>
__device__ __forceinline__ f32x4 restart4(const RowsArgs& a, int64_t o, float keep, f32x4 acc) {
    if (a.restart == 0.0f) return keep * acc;
    return keep * acc + a.restart * ld4(static_cast<const TV*>(a.V) + o);
}

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// Lane u of the caller's row of 16 lanes (DPP row_newbcast).
template <int u>
__device__ __forceinline__ int32_t row16_lane(int32_t v) {
    return __builtin_amdgcn_mov_dpp(v, 0x150 + u, 0xf, 0xf, false);
}

__device__ __forceinline__ void fma4(float (&acc)[4], float w, const f32x4& z) {
    acc[0] = fmaf(w, z[0], acc[0]);
    acc[1] = fmaf(w, z[1], acc[1]);
    acc[2] = fmaf(w, z[2], acc[2]);
    acc[3] = fmaf(w, z[3], acc[3]);
}

// LDS element position of channel c of run row k: a row's 16-byte pieces
// are permuted by ((k >> 2) & 3), so that the four rows one MFMA operand
// read touches (rows 4 apart) fall on distinct banks.
template <typename TX>
__device__ __forceinline__ int32_t zpos(int32_t k, int32_t c) {
    if constexpr (sizeof(TX) == 4)
        return k * 64 + ((c >> 2) ^ (((k >> 2) & 3) << 2)) * 4 + (c & 3);
    else
        return k * 64 + ((c >> 3) ^ (((k >> 2) & 3) << 1)) * 8 + (c & 7);
}
// The 16-byte piece a staging lane fetches for position `pos` of run row r.
template <typename TX>
__device__ __forceinline__ int32_t zpiece(int32_t r, int32_t pos) {
    if constexpr (sizeof(TX) == 4) return pos ^ (((r >> 2) & 3) << 2);
    else return pos ^ (((r >> 2) & 3) << 1);
}
__device__ __forceinline__ float zld(const float LDS_AS* base, int32_t p) { return base[p]; }
__device__ __forceinline__ float zld(const bf16_t LDS_AS* base, int32_t p) {
    return bf16_to_f32(*reinterpret_cast<const uint16_t LDS_AS*>(base + p));
}

// The same step with the window band and the global columns of each block
// of 16 rows on v_mfma_f32_16x16x4_f32: wave w takes the rows of block
// w / 4 against channels 16 (w mod 4) .. + 15,
//   D[row][channel] += W[row][key] Z[key][channel]
// over the block's window keys and the g globals, four keys per product:
// lane (m, kq) = (lane mod 16, lane / 16) supplies the weights of row m for
// keys base + 4 kq .. + 3 (one 16-byte load) and channel m of those keys'
// rows from LDS, product e pairing key base + 4 kq + e in both operands.
// A weight whose key lies outside its row's window (or, for a global slot,
// inside it or above a causal row) is 0. The block's sums go to LDS; then
// each row's random edges are gathered (a wave per row, lane group q
// taking edges 4 q .. 4 q + 3 of each step of 16, their slots and columns
// in one 16-byte load each) and added to them. Eight waves per SIMD (two workgroups per CU): at most 64
// registers per lane.
template <int D, typename TX, typename TV, typename TY>
__global__ __launch_bounds__(kThreads, 8)
void k_diffuse_rows_mma(RowsArgs a) {
    static_assert(D == 64, "four 16-channel tiles per block");
    constexpr int L = D / 4;
    constexpr int NG = kWave / L;
    constexpr int U = D * (int)sizeof(TX) / 16;
    extern __shared__ __align__(16) char lds_raw[];
    TX LDS_AS* lds = (TX LDS_AS*)lds_raw;
    float LDS_AS* csum = (float LDS_AS*)lds_raw;   // [4][64][64], after the products
    const int lane = __lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int sub = lane % L, grp = lane / L;

    const int32_t item = (int32_t)(blockIdx.x & 7u) * a.per_xcd + (int32_t)(blockIdx.x >> 3);
    if (item >= a.items) return;
    const int32_t bh = item / a.blocks;
    const int64_t r0 = (int64_t)(item - bh * a.blocks) * kRowsPerGroup;
    const int32_t b = bh / a.H, h = bh - b * a.H;
    const int32_t gr = a.num_graphs == 1 ? 0 : b;
    const int64_t n = a.n, r = a.radius;
    const float* Abh = a.A + a_block_offset(a.gg.slot_off, a.num_graphs, a.H, b, h);
    const TX* Zbh = static_cast<const TX*>(a.Z) + (int64_t)bh * n * D;
    const int4* info = a.row_info + (int64_t)gr * n;
    const int64_t pair_slots = a.num_graphs == 1 ? a.gg.slot_off[1]
                                                 : a.gg.slot_off[gr + 1] - a.gg.slot_off[gr];
    const __amdgpu_buffer_rsrc_t rA = buffer_rsrc(Abh, (uint32_t)(4 * pair_slots));
    const __amdgpu_buffer_rsrc_t rAR = buffer_rsrc(
        a.AR + a_block_offset(a.gg.slot_off, a.num_graphs, a.H, b, h), (uint32_t)(4 * pair_slots));
    const __amdgpu_buffer_rsrc_t rG = buffer_rsrc(a.G, (uint32_t)(4 * a.g));

    // ---- key rows into LDS (pieces permuted by zpiece) ---------------------
    const int64_t w0 = (r0 - r < 0 ? 0 : r0 - r) & ~7ll;
    {
        const int32_t rows = a.win_rows + a.g + kGlobPad;
        const int32_t units = rows * U;
        char LDS_AS* ldsb = (char LDS_AS*)lds_raw;
        for (int32_t p0 = 64 * wave; p0 < units; p0 += 64 * kWaves) {
            const int32_t p = p0 + lane;
            const int32_t rr = p / U, pos = p - rr * U;
            int64_t k = -1;
            if (rr < a.win_rows) k = w0 + rr;
            else if (rr < a.win_rows + a.g) k = a.G[rr - a.win_rows];
            const bool live = p < units && k >= 0 && k < n;
            if (live)
                dma16(reinterpret_cast<const char*>(Zbh + k * D) + 16 * zpiece<TX>(rr, pos),
                      (void LDS_AS*)(ldsb + 16 * p0));
            else if (p < units)
                *reinterpret_cast<f32x4 LDS_AS*>(ldsb + 16 * p) = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
    // The group's row geometry and random-edge counts (or list starts) in
    // LDS past the key rows and the partial sums, loaded once by the last
    // wave.
    const int32_t aux = max((a.win_rows + a.g + kGlobPad) * D * (int)sizeof(TX),
                            4 * kRowsPerGroup * 64 * 4);
    i32x4 LDS_AS* rinfo = reinterpret_cast<i32x4 LDS_AS*>((char LDS_AS*)lds_raw + aux);   // [64]
    int64_t LDS_AS* rlist = reinterpret_cast<int64_t LDS_AS*>(rinfo + kRowsPerGroup);   // [65]
    if (wave == kWaves - 1) {
        const int64_t ir = r0 + lane;
        const int4 t = ir < n ? info[ir] : make_int4(0, 0, -1, 0);
        rinfo[lane] = i32x4{t.x, t.y, t.z, t.w};
        if (a.t_ptr != nullptr) {
            rlist[lane] = a.t_ptr[(int64_t)gr * (n + 1) + (ir < n ? ir : n)];
            if (lane == 0)
                rlist[kRowsPerGroup] =
                    a.t_ptr[(int64_t)gr * (n + 1) + (r0 + kRowsPerGroup < n ? r0 + kRowsPerGroup : n)];
        } else {
            rlist[lane] = ir < n && a.gg.rslot != nullptr ? a.gg.rnd_cnt[(int64_t)gr * n + ir] : 0;
        }
    }
    full_barrier();

    // ---- window band and global columns, a quarter of the keys per wave ------
    // Wave w takes the rows of block w / 4 and every fourth 16-key chunk
    // (from chunk w mod 4) of its window keys and globals, against all 64
    // channels (four tiles), so each weight is loaded once; the four
    // quarters' partial sums meet in LDS.
    const int m = lane & 15, kq = lane >> 4;
    const int64_t ib0 = r0 + 16 * (wave >> 2);
    const int kqt = wave & 3;
    f32x4 acc16[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) acc16[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (ib0 < n) {
        const int64_t i = ib0 + m;   // this lane's weight row
        const i32x4 rv = rinfo[i - r0];
        const int4 ri = make_int4(rv[0], rv[1], rv[2], rv[3]);
        const bool live = i < n && ri.z >= 0;
        const int64_t lo = i - r < 0 ? 0 : i - r;
        const int64_t hi = i + r > n - 1 ? n - 1 : i + r;
        const int64_t wend = a.causal ? i : hi;
        const int64_t last = a.causal ? i : n - 1;
        // The block's window keys: from its first row's block start through
        // the last slot of its last row's window.
        const int64_t ibl = ib0 + 15 < n ? ib0 + 15 : n - 1;
        const int64_t J0 = (ib0 - r < 0 ? 0 : ib0 - r) & ~7ll;
        const int64_t wend_l = a.causal ? ibl : (ibl + r > n - 1 ? n - 1 : ibl + r);
        const int32_t nch = (int32_t)(((wend_l | 7) - J0) / 16 + 1);
        const int32_t gch = (a.g + 15) / 16;
        for (int32_t c = kqt; c < nch + gch; c += 4) {
            u32x4 wv;
            int32_t kl[4];
            bool ok[4];
            if (c < nch) {
                const int64_t key0 = J0 + 16 * c + 4 * kq;
                const int64_t s0 = key0 - ri.y;
                const bool in = live && s0 >= 0 && s0 < ri.z;
                wv = bload16(rA, in ? 4u * (uint32_t)(ri.x + s0) : kOutside, 0u);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int64_t key = key0 + e;
                    ok[e] = live && key >= lo && key <= wend;
                    kl[e] = (int32_t)min(key - w0, (int64_t)a.win_rows - 1);
                }
            } else {
                const int32_t t0 = 16 * (c - nch) + 4 * kq;
                const bool in = live && t0 < ri.w;
                wv = bload16(rA, in ? 4u * (uint32_t)(ri.x + ri.z + t0) : kOutside, 0u);
                const u32x4 gk = bload16(rG, t0 < a.g ? 4u * (uint32_t)t0 : kOutside, 0u);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int64_t kc = (int32_t)gk[e];
                    ok[e] = in && t0 + e < a.g && (kc < lo || kc > hi) && kc <= last;
                    kl[e] = a.win_rows + t0 + e;
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float we = ok[e] ? __uint_as_float(wv[e]) : 0.0f;
#pragma unroll
                for (int ct = 0; ct < 4; ++ct)
                    acc16[ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                        we, zld(lds, zpos<TX>(kl[e], 16 * ct + m)), acc16[ct], 0, 0, 0);
            }
        }
    }
    __syncthreads();   // every wave is done with the key rows
    // Lane (m, kq) holds rows 4 kq + v of its block at channels 16 ct + m;
    // quarter kqt's partial sums go to csum[kqt].
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int v = 0; v < 4; ++v)
            csum[(kqt * kRowsPerGroup + 16 * (wave >> 2) + 4 * kq + v) * 64 + 16 * ct + m] =
                acc16[ct][v];
    __syncthreads();

    // ---- random edges per row, gathered, plus the block sums ----------------
#pragma unroll 1
    for (int u = 0; u < kRowsPerWave; ++u) {
        const int64_t i = r0 + kWaves * u + wave;
        if (i >= n) break;
        const int32_t li = kWaves * u + wave;
        if (rinfo[li][2] < 0) continue;   // a global row: k_diffuse_grows_f32's
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
        int32_t nr;
        const int32_t *rslot, *rcol;
        if (a.t_ptr == nullptr) {
            const int64_t row = (int64_t)gr * n + i;
            nr = (int32_t)rlist[li];
            rslot = a.gg.rslot + row * a.gg.rnd_width;
            rcol = a.gg.rnd + row * a.gg.rnd_width;
        } else {
            const int64_t t0 = rlist[li];
            nr = (int32_t)(rlist[li + 1] - t0);
            rslot = a.t_slot + t0;
            rcol = a.t_row + t0;
        }
        // Indices, one load per lane per two steps of 16 edges: lane sub of
        // group grp fetches the slot (sub mod 8 < 4) or the column (sub mod
        // 8 >= 4) of edge base + 16 (sub / 8) + 4 grp + (sub mod 4); each
        // step's four slots and columns are then broadcast from the group's
        // lanes (DPP row_newbcast), as are the four weights from the lanes
        // that load them.
        const int vv = sub & 3;
        const int32_t* ixp = (sub & 4) ? rcol : rslot;
        auto idx = [&](int32_t base) -> int32_t {
            const int32_t e = base + 16 * (sub >> 3) + 4 * grp + vv;
            return e < nr ? ixp[e] : 0;
        };
        // One step of 16 edges from index lanes 8 h .. 8 h + 7.
        auto step = [&](auto hc, int32_t base, int32_t ix) {
            constexpr int h = decltype(hc)::value;
            const int32_t sl[4] = {row16_lane<8 * h + 0>(ix), row16_lane<8 * h + 1>(ix),
                                   row16_lane<8 * h + 2>(ix), row16_lane<8 * h + 3>(ix)};
            const int32_t cl[4] = {row16_lane<8 * h + 4>(ix), row16_lane<8 * h + 5>(ix),
                                   row16_lane<8 * h + 6>(ix), row16_lane<8 * h + 7>(ix)};
            const int32_t slv = vv == 0 ? sl[0] : vv == 1 ? sl[1] : vv == 2 ? sl[2] : sl[3];
            const bool okw = base + 4 * grp + vv < nr;
            const int wl = __builtin_amdgcn_raw_buffer_load_b32(
                rAR, okw ? (int)(4u * (uint32_t)slv) : (int)kOutside, 0, 0);
            f32x4 z[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const bool ok = base + 4 * grp + v < nr;
                z[v] = ld4(Zbh + (int64_t)(ok ? cl[v] : 0) * D + 4 * sub);
            }
            float w[4];
            w[0] = __int_as_float(row16_lane<0>(wl));
            w[1] = __int_as_float(row16_lane<1>(wl));
            w[2] = __int_as_float(row16_lane<2>(wl));
            w[3] = __int_as_float(row16_lane<3>(wl));
#pragma unroll
            for (int v = 0; v < 4; ++v) fma4(acc, w[v], z[v]);
        };
        int32_t ix = idx(0);
        for (int32_t base = 0; base < nr; base += 8 * NG) {
            const int32_t ixn = idx(base + 8 * NG);
            step(std::integral_constant<int, 0>{}, base, ix);
            if (base + 4 * NG < nr) step(std::integral_constant<int, 1>{}, base + 4 * NG, ix);
            ix = ixn;
        }
#pragma unroll
        for (int off = L; off < kWave; off <<= 1) {
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[c] += __shfl_xor(acc[c], off);
        }
        if (grp == 0) {
            f32x4 bs = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int q = 0; q < 4; ++q)
                bs = bs + *reinterpret_cast<const f32x4 LDS_AS*>(
                              csum + (q * kRowsPerGroup + (i - r0)) * 64 + 4 * sub);
            const int64_t o = ((int64_t)bh * n + i) * D + 4 * sub;
            const float keep =
                a.row_scale == nullptr ? a.keep : a.keep * a.row_scale[(int64_t)bh * n + i];
            st4(static_cast<TY*>(a.Zn) + o,
                restart4<TV>(a, o, keep, f32x4{acc[0], acc[1], acc[2], acc[3]} + bs));
        }
    }
}

// Global rows, 16 per workgroup, on v_mfma_f32_16x16x4_f32: the 16 waves
// split the keys into contiguous ranges and each computes, over its range,
//   D_ct[row][n] += W[row][key] Z[key][4 n + ct]      (ct = 0..3)
// for the workgroup's 16 rows (a global row's segment holds its columns in
// order), so lane (n, kq) reads channels 4 n .. 4 n + 3 of a key row with
// one 16-byte load and ends with four consecutive channels of each of its
// rows. Keys outside the wave's range, past n or (causal) above the row
// weigh 0. The waves' partial sums meet in LDS and are added in wave order.

// kGTiles tiles of 16 global rows per workgroup share each key row's load.
template <int D, typename TX, typename TV, typename TY, int kGTiles>
__global__ __launch_bounds__(kThreads)
void k_diffuse_grows_f32(RowsArgs a, int32_t gblocks) {
    constexpr int kGTile = 16 * kGTiles;
    static_assert(D == 64, "four channel tiles of 16");
    __shared__ f32x4 part[kWaves][16][16];   // [wave][row of a tile][channels 4 n ..]
    const int lane = __lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int m = lane & 15, kq = lane >> 4;
    const int32_t bh = blockIdx.x / gblocks;
    const int32_t q0 = (blockIdx.x - bh * gblocks) * kGTile;
    const int32_t b = bh / a.H, h = bh - b * a.H;
    const int32_t gr = a.num_graphs == 1 ? 0 : b;
    const int64_t n = a.n;
    const float* Abh = a.A + a_block_offset(a.gg.slot_off, a.num_graphs, a.H, b, h);
    const TX* Zbh = static_cast<const TX*>(a.Z) + (int64_t)bh * n * D;
    const int4* info = a.row_info + (int64_t)gr * n;
    const int64_t pair_slots = a.num_graphs == 1 ? a.gg.slot_off[1]
                                                 : a.gg.slot_off[gr + 1] - a.gg.slot_off[gr];
    const __amdgpu_buffer_rsrc_t rA = buffer_rsrc(Abh, (uint32_t)(4 * pair_slots));
    const __amdgpu_buffer_rsrc_t rZ = buffer_rsrc(Zbh, (uint32_t)(sizeof(TX) * n * D));
    // This lane's weight rows (row m of each tile) and their last columns.
    uint32_t seg[kGTiles];
    int64_t last[kGTiles];
#pragma unroll
    for (int tl = 0; tl < kGTiles; ++tl) {
        const int32_t q = q0 + 16 * tl + m;
        const int64_t gi = q < a.g ? a.G[q] : -1;
        seg[tl] = gi >= 0 ? (uint32_t)info[gi].x : 0u;
        last[tl] = gi < 0 ? -1 : a.causal ? gi : n - 1;
    }
    f32x4 acc[kGTiles][4];
#pragma unroll
    for (int tl = 0; tl < kGTiles; ++tl)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) acc[tl][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int64_t k0 = n * wave / kWaves, k1 = n * (wave + 1) / kWaves;
    for (int64_t kb = k0 & ~15ll; kb < k1; kb += 16) {
        const int64_t key0 = kb + 4 * kq;   // this lane's keys key0 .. key0 + 3
        u32x4 w[kGTiles];
#pragma unroll
        for (int tl = 0; tl < kGTiles; ++tl) {
            const bool any = key0 <= last[tl] && key0 + 3 >= k0 && key0 < k1;
            w[tl] = bload16(rA, any ? 4u * (seg[tl] + (uint32_t)key0) : kOutside, 0u);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int64_t key = key0 + e;
            const bool zk = key >= k0 && key < k1;
            const f32x4 z = bload4<TX>(rZ, zk ? (uint32_t)((key * D + 4 * m) * sizeof(TX)) : kOutside);
#pragma unroll
            for (int tl = 0; tl < kGTiles; ++tl) {
                const float we = zk && key <= last[tl] ? __uint_as_float(w[tl][e]) : 0.0f;
#pragma unroll
                for (int ct = 0; ct < 4; ++ct)
                    acc[tl][ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(we, z[ct], acc[tl][ct], 0, 0, 0);
            }
        }
    }
    // Lane (n, kq) holds rows 4 kq + v of each tile at channels 4 n + ct;
    // the tiles' partial sums meet in LDS one tile at a time.
#pragma unroll
    for (int tl = 0; tl < kGTiles; ++tl) {
        if (tl > 0) __syncthreads();   // the previous tile's sums are read
#pragma unroll
        for (int v = 0; v < 4; ++v)
            part[wave][4 * kq + v][m] =
                f32x4{acc[tl][0][v], acc[tl][1][v], acc[tl][2][v], acc[tl][3][v]};
        __syncthreads();
        for (int t = threadIdx.x; t < 16 * 16; t += kThreads) {
            const int rr = t / 16, c4 = t - rr * 16;
            const int32_t q = q0 + 16 * tl + rr;
            if (q >= a.g) continue;
            f32x4 sum = f32x4{0.f, 0.f, 0.f, 0.f};
            for (int ww = 0; ww < kWaves; ++ww) sum = sum + part[ww][rr][c4];
            const int64_t i = a.G[q];
            const int64_t o = ((int64_t)bh * n + i) * D + 4 * c4;
            const float keep =
                a.row_scale == nullptr ? a.keep : a.keep * a.row_scale[(int64_t)bh * n + i];
            st4(static_cast<TY*>(a.Zn) + o, restart4<TV>(a, o, keep, sum));
        }
    }
}

// Transposed weights of a bidirectional built graph in the graph's own
// slot geometry, for the transposed product A^T X: the columns of A^T's
// row j are the rows i with an edge (i, j), which on these graphs are the
// window rows |i - j| <= r, the global rows and, for a global j, every
// row; so row j's window slot for column i and its global slot t (for
// G[t]) hold A_ij and A_{G[t] j}, and a global row j's slot i holds A_ij.
// The random edges are listed by column apart. Padding slots are 0. For a
// source row i, A_ij lies in its full segment when i is global, in its
// window when |i - j| <= r, and otherwise (j is then a global column) in
// its global slot for j.
//
// k_transpose_band: the rows j of a tile of kTRows that are not global. A
// workgroup reads, one wave per source row with a lane per column, the
// tile's columns of every source row that can be a window row of the tile
// (rows j0 - r .. j0 + kTRows - 1 + r) and of every global row into LDS,
// then writes each destination row's slots with a lane per slot.
constexpr int kTRows = 64;
constexpr int kTStride = kTRows + 1;   // LDS row stride (column reads fall on distinct banks)

__global__ __launch_bounds__(kThreads)
void k_transpose_band(RowsArgs a, float* __restrict__ At, int32_t tiles) {
    extern __shared__ float tl[];
    const int lane = __lane_id();
    const int wave = threadIdx.x / kWave;
    constexpr int kW = kWaves;
    const int64_t n = a.n;
    const int32_t bh = blockIdx.x / tiles;
    const int64_t j0 = (int64_t)(blockIdx.x - bh * tiles) * kTRows;
    const int32_t b = bh / a.H, h = bh - b * a.H;
    const int32_t gr = a.num_graphs == 1 ? 0 : b;
    const int64_t off = a_block_offset(a.gg.slot_off, a.num_graphs, a.H, b, h);
    const float* Ab = a.A + off;
    float* Atb = At + off;
    const int4* info = a.row_info + (int64_t)gr * n;
    const int64_t r = a.radius;
    const int64_t ib = j0 - r < 0 ? 0 : j0 - r;
    const int64_t ie = j0 + kTRows - 1 + r > n - 1 ? n - 1 : j0 + kTRows - 1 + r;
    const int32_t nsrc = (int32_t)(ie - ib + 1);
    const int32_t rows = nsrc + a.g;
    float* win = tl;                                  // [nsrc][kTStride], then [g][kTStride]
    int4* sinfo = reinterpret_cast<int4*>(tl + (((int64_t)rows * kTStride + 3) & ~3ll));   // [rows]
    int4* dinfo = sinfo + rows;                                              // [kTRows]
    // The geometry of the source rows (window rows, then the global rows)
    // and of the destination rows.
    for (int32_t u = threadIdx.x; u < rows + kTRows; u += kThreads) {
        if (u < rows) {
            sinfo[u] = info[u < nsrc ? ib + u : a.G[u - nsrc]];
        } else {
            const int64_t jd = j0 + (u - rows);
            dinfo[u - rows] = jd < n ? info[jd] : make_int4(0, 0, -1, 0);
        }
    }
    __syncthreads();
    const int64_t j = j0 + lane;   // this lane's column
#pragma unroll 4
    for (int32_t u = wave; u < rows; u += kW) {
        const int4 ri = sinfo[u];
        float w = 0.0f;
        if (u < nsrc) {
            const int64_t i = ib + u;
            if (j < n && j >= i - r && j <= i + r) w = Ab[(int64_t)ri.x + (ri.z < 0 ? j : j - ri.y)];
        } else if (j < n) {
            w = Ab[(int64_t)ri.x + j];   // a global row's column j
        }
        win[(int64_t)u * kTStride + lane] = w;
    }
    __syncthreads();
    const float* glob = win + (int64_t)nsrc * kTStride;
    for (int32_t jj = wave; jj < kTRows; jj += kW) {
        const int64_t jd = j0 + jj;
        const int4 rj = dinfo[jj];
        if (jd >= n || rj.z < 0) continue;   // past n, or a global row: k_transpose_grows's
        const int64_t nslot = (int64_t)rj.z + rj.w;
        for (int64_t s = lane; s < nslot; s += kWave) {
            float w = 0.0f;
            if (s < rj.z) {
                const int64_t i = rj.y + s;
                if (i < n && i >= jd - r && i <= jd + r) w = win[(i - ib) * kTStride + jj];
            } else {
                const int64_t t = s - rj.z;
                if (t < a.g) {
                    const int64_t i = a.G[t];
                    if (i < jd - r || i > jd + r) w = glob[t * kTStride + jj];
                }
            }
            Atb[(int64_t)rj.x + s] = w;
        }
    }
}

// Global destination rows j = G[q] (a global column of A: every row has an
// edge to it): one wave per row, a lane per slot.
__global__ __launch_bounds__(kThreads)
void k_transpose_grows(RowsArgs a, float* __restrict__ At) {
    const int lane = __lane_id();
    const int wave = threadIdx.x / kWave;
    const int64_t n = a.n;
    const int32_t per = (a.g + kWaves - 1) / kWaves;
    const int32_t bh = blockIdx.x / per;
    const int32_t q = (blockIdx.x - bh * per) * kWaves + wave;
    if (q >= a.g) return;
    const int32_t b = bh / a.H, h = bh - b * a.H;
    const int32_t gr = a.num_graphs == 1 ? 0 : b;
    const int64_t off = a_block_offset(a.gg.slot_off, a.num_graphs, a.H, b, h);
    const float* Ab = a.A + off;
    float* Atb = At + off;
    const int4* info = a.row_info + (int64_t)gr * n;
    const int64_t j = a.G[q];
    const int4 rj = info[j];
    const int64_t r = a.radius;
    const int64_t nslot = a.gg.row(gr, j).seg_len;
    for (int64_t i = lane; i < nslot; i += kWave) {
        float w = 0.0f;
        if (i < n) {
            const int4 ri = info[i];
            if (ri.z < 0) w = Ab[(int64_t)ri.x + j];
            else if (j >= i - r && j <= i + r) w = Ab[(int64_t)ri.x + (j - ri.y)];
            else w = Ab[(int64_t)ri.x + ri.z + q];
        }
        Atb[(int64_t)rj.x + i] = w;
    }
}

// Key rows of the window run: the group's rows, the radius on either side
// (on the left only when causal) and the 8-column alignment of its start.
// A window slot outside its row's window reads run row 0 with weight 0, so
// the run needs no rows past the last window column.
int32_t win_rows(const diffuser_graph& g) {
    return kRowsPerGroup + (g.causal ? 1 : 2) * g.radius + 8;
}

int32_t lds_bytes(const diffuser_graph& g, int elem_bytes) {
    return (win_rows(g) + g.num_global + kGlobPad) * 64 * elem_bytes;
}

// LDS of k_transpose_band: the source rows of a tile and the global rows,
// kTStride floats and an int4 of geometry each, and the destination rows'
// geometry.
int64_t transpose_lds_bytes(const diffuser_graph& g) {
    const int64_t src = std::min<int64_t>(kTRows + 2 * (int64_t)g.radius, g.n);
    return (src + g.num_global) * (kTStride * 4 + 16) + kTRows * 16 + 16;
}

RowsArgs make_args(const diffuser_graph& g, int32_t B, int32_t H, const float* A, const void* Zk,
                   const void* V, void* Zn, const float* row_scale, step_coefs kc) {
    RowsArgs a;
    a.n = g.n;
    a.H = H;
    a.num_graphs = g.num_graphs;
    a.radius = g.radius;
    a.causal = g.causal;
    a.g = g.num_global;
    a.win_rows = win_rows(g);
    a.blocks = (int32_t)((g.n + kRowsPerGroup - 1) / kRowsPerGroup);
    a.items = B * H * a.blocks;
    a.per_xcd = (a.items + 7) / 8;
    a.gg = generic_graph(g);
    a.row_info = reinterpret_cast<const int4*>(g.d_row_info);
    a.G = g.d_global;
    a.A = A;
    a.AR = A;
    a.t_ptr = nullptr;
    a.t_slot = nullptr;
    a.t_row = nullptr;
    a.Z = Zk;
    a.V = V;
    a.Zn = Zn;
    a.row_scale = row_scale;
    a.keep = kc.keep;
    a.restart = kc.restart;
    return a;
}

// The transposed product's weights: A^T in the graph's slot geometry for
// the window and global slots, A's own slots for the random edges by column.
void set_transposed(RowsArgs& a, const diffuser_graph& g, const float* A) {
    a.AR = A;
    a.t_ptr = g.d_trand_ptr;
    a.t_slot = g.d_trand_slot;
    a.t_row = g.d_trand_row;
}

template <typename TX, typename TV, typename TY>
hipError_t launch_args(const diffuser_graph& g, int32_t B, int32_t H, const RowsArgs& a,
                       hipStream_t st) {
    const int lds = std::max(lds_bytes(g, (int)sizeof(TX)), 4 * kRowsPerGroup * 64 * 4) +
                    kRowsPerGroup * 16 + (kRowsPerGroup + 1) * 8;
    auto kern = &k_diffuse_rows_mma<64, TX, TV, TY>;
    static int attr_device = -1;
    if (attr_device != g.device) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, kLdsLimit);
        if (e != hipSuccess) return e;
        attr_device = g.device;
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)(8 * a.per_xcd)), dim3(kThreads), (size_t)lds, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || g.num_global == 0) return e;
    // Two tiles of 16 global rows per workgroup when that leaves at least
    // half as many workgroups as CUs (measured: 192 workgroups gain, 32
    // lose), else one.
    const int32_t g2 = (g.num_global + 31) / 32;
    if ((int64_t)B * H * g2 >= 128)
        hipLaunchKernelGGL((k_diffuse_grows_f32<64, TX, TV, TY, 2>), dim3((unsigned)(B * H * g2)),
                           dim3(kThreads), 0, st, a, g2);
    else
        hipLaunchKernelGGL((k_diffuse_grows_f32<64, TX, TV, TY, 1>),
                           dim3((unsigned)(B * H * ((g.num_global + 15) / 16))), dim3(kThreads), 0,
                           st, a, (g.num_global + 15) / 16);
    return hipGetLastError();
}

}  // namespace

bool rows_diffuse_supported(const diffuser_graph& g, const attn_shape& s) {
    return s.dtype == DIFFUSER_F32 && rows_states_supported(g, s.B, s.H, s.d);
}

bool rows_states_supported(const diffuser_graph& g, int32_t B, int32_t H, int32_t d) {
    if (!g.structured || !g.rand_apart() || g.d_row_info == nullptr || d != 64) return false;
    for (int64_t x : g.slots)
        if (4 * x >= (1ll << 31)) return false;   // byte offsets of a pair's weights fit 31 bits
    // Enough row groups to give every CU two workgroups twice over; fewer
    // rows run faster one wave per row on the generic step.
    const int64_t groups = (int64_t)B * H * ((g.n + kRowsPerGroup - 1) / kRowsPerGroup);
    return groups >= kMinGroups && 2 * lds_bytes(g, 4) <= kLdsLimit;
}

hipError_t launch_diffuse_rows(const diffuser_graph& g, const attn_shape& s, const void* A,
                               const void* Zk, const void* V, void* Zn, const float* row_scale,
                               step_coefs kc, hipStream_t st) {
    const RowsArgs a = make_args(g, s.B, s.H, static_cast<const float*>(A), Zk, V, Zn, row_scale, kc);
    return launch_args<float, float, float>(g, s.B, s.H, a, st);
}

bool rows_transposed_supported(const diffuser_graph& g, int32_t B, int32_t H, int32_t d) {
    return !g.causal && g.d_trand_ptr != nullptr && transpose_lds_bytes(g) <= kLdsLimit &&
           rows_states_supported(g, B, H, d);
}

hipError_t launch_transpose_struct(const diffuser_graph& g, int32_t B, int32_t H, const float* A,
                                   float* At, hipStream_t st) {
    const RowsArgs a =
        make_args(g, B, H, A, nullptr, nullptr, nullptr, nullptr, step_coefs{0.f, 0.f});
    static int attr_device = -1;
    if (attr_device != g.device) {
        const hipError_t e =
            hipFuncSetAttribute(reinterpret_cast<const void*>(&k_transpose_band),
                                hipFuncAttributeMaxDynamicSharedMemorySize, kLdsLimit);
        if (e != hipSuccess) return e;
        attr_device = g.device;
    }
    const int32_t tiles = (int32_t)((g.n + kTRows - 1) / kTRows);
    hipLaunchKernelGGL(k_transpose_band, dim3((unsigned)(B * H * tiles)), dim3(kThreads),
                       (size_t)transpose_lds_bytes(g), st, a, At, tiles);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || g.num_global == 0) return e;
    const int32_t per = (g.num_global + kWaves - 1) / kWaves;
    hipLaunchKernelGGL(k_transpose_grows, dim3((unsigned)(B * H * per)), dim3(kThreads), 0, st, a,
                       At);
    return hipGetLastError();
}

hipError_t launch_transposed_rows(const diffuser_graph& g, int32_t B, int32_t H, const float* At,
                                  const float* A, const float* X, float* Y, float scale,
                                  hipStream_t st) {
    RowsArgs a = make_args(g, B, H, At, X, nullptr, Y, nullptr, step_coefs{scale, 0.f});
    set_transposed(a, g, A);
    return launch_args<float, float, float>(g, B, H, a, st);
}

hipError_t launch_states_rows(const diffuser_graph& g, int32_t B, int32_t H, const float* A,
                              const float* Zk, const void* V, diffuser_dtype v_dtype, float* Zn,
                              step_coefs kc, hipStream_t st) {
    const RowsArgs a = make_args(g, B, H, A, Zk, V, Zn, nullptr, kc);
    if (v_dtype == DIFFUSER_F32) return launch_args<float, float, float>(g, B, H, a, st);
    return launch_args<float, bf16_t, float>(g, B, H, a, st);
}

hipError_t launch_grad_rows(const diffuser_graph& g, int32_t B, int32_t H, const float* W,
                            const float* WR, bool transposed, const void* X, void* Y,
                            diffuser_dtype dtype, float scale, hipStream_t st) {
    RowsArgs a = make_args(g, B, H, W, X, nullptr, Y, nullptr, step_coefs{scale, 0.f});
    if (transposed) set_transposed(a, g, WR);
    if (dtype == DIFFUSER_F32) return launch_args<float, float, float>(g, B, H, a, st);
    return launch_args<bf16_t, float, bf16_t>(g, B, H, a, st);
}

}  // namespace diffuser
