// The backward's edge values on built graphs,
//   dA_ij = f sum_{k < K} G_{k+1}[i] . Z_k[j]      (f = 1 - alpha)
// (the chain rule through "Diffuser" reading notes, section 2.4, eq. S.7),
// with the dense parts of the graph on v_mfma_f32_16x16x4_f32:
//  * k_dots_band: one wave per block of 16 rows: the block's window band
//    (every key a window slot of one of its rows names, in tiles of 16
//    consecutive keys) and its global columns (tiles of 16 globals), each
//    tile a 16 x 16 product
//      D[row][key] += G_{k+1}[row] . Z_k[key]
//    accumulated over the 64 channels and all K states in registers, then
//    written once into the rows' window and global slots (0 where a slot is
//    padding or the key is not the row's);
//  * k_dots_glob: one wave per tile of 16 keys: the global rows (whose
//    segment holds their columns in order), 16 at a time, against the tile;
//  * the random edges stay per-edge gathers (the generic kernel limited to
//    the random slots).
// Operands: lane l = 16 kq + m supplies row m of a 16-row tile; for chunk s
// of 16 channels it holds channels 16 s + 4 kq .. + 3 of that row (one
// 16-byte load), and product e of the chunk pairs element e of both
// operands, so the k index kq names the same channel in both. The result
// lane l holds D[4 kq + v][m], v = 0..3.
#include "internal.h"
#include "mfma_util.h"

namespace diffuser {
namespace {

constexpr int kWave = 64;
constexpr int kWavesPerBlock = 4;
constexpr int kThreads = kWave * kWavesPerBlock;
constexpr int kTiles = 6;   // key tiles accumulated per pass of k_dots_band
constexpr int kQTiles = 4;  // global-row tiles per pass of k_dots_glob

struct DotsArgs {
    int64_t n;
    int32_t H, num_graphs, radius, causal, g, K;
    int32_t nrb;                // row blocks of 16 per pair
    int32_t nkt;                // key tiles of 16 per pair (global rows)
    int32_t BH;
    int64_t stride;             // elements between consecutive states
    const int64_t* slot_off;
    const int64_t* seg_ptr;     // [graphs][n + 1]
    const int4* row_info;       // [graphs][n]
    const int32_t* G;           // [g]
    const float* Gs;            // G_0 .. G_K
    const float* Zs;            // Z_0 .. Z_{K-1}
    float* dA;
    float f;
};

__device__ __forceinline__ f32x4 ld4z(const float* p, bool ok) {
    return ok ? *reinterpret_cast<const f32x4*>(p) : f32x4{0.f, 0.f, 0.f, 0.f};
}

// acc += the 16 x 16 x 16-channel product of one chunk (four k steps).
__device__ __forceinline__ f32x4 mfma_chunk(f32x4 acc, const f32x4& x, const f32x4& y) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x[0], y[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x[1], y[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x[2], y[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x[3], y[3], acc, 0, 0, 0);
    return acc;
}

// Window block start and last window slot's key of row i (the graph
// builder's segment geometry: window blocks of 8 from (lo & ~7) through
// the last window column).
__device__ __forceinline__ void window_span(int64_t i, int64_t n, int64_t r, bool causal,
                                            int64_t& wb0, int64_t& wlast) {
    const int64_t lo = i - r < 0 ? 0 : i - r;
    const int64_t hi = i + r > n - 1 ? n - 1 : i + r;
    const int64_t wend = causal ? i : hi;
    wb0 = lo & ~7ll;
    wlast = wb0 + (wend - wb0) / 8 * 8 + 7;
}

__global__ __launch_bounds__(kThreads)
void k_dots_band(DotsArgs a) {
    const int lane = __lane_id();
    const int wave = threadIdx.x / kWave;
    const int m = lane & 15, kq = lane >> 4;
    const int64_t item = (int64_t)blockIdx.x * kWavesPerBlock + wave;
    if (item >= (int64_t)a.BH * a.nrb) return;
    const int32_t bh = (int32_t)(item / a.nrb);
    const int64_t i0 = (item - (int64_t)bh * a.nrb) * 16;
    const int32_t b = bh / a.H, h = bh - b * a.H;
    const int32_t gr = a.num_graphs == 1 ? 0 : b;
    const int64_t n = a.n, r = a.radius;
    const int4* info = a.row_info + (int64_t)gr * n;
    float* dAb = a.dA + a_block_offset(a.slot_off, a.num_graphs, a.H, b, h);
    // Keys of the block's window slots: from the first row's block start
    // through the last row's last window slot.
    int64_t J0, wl_first, wb_last, Jend;
    window_span(i0, n, r, a.causal, J0, wl_first);
    window_span(i0 + 15 < n ? i0 + 15 : n - 1, n, r, a.causal, wb_last, Jend);
    const int32_t twin = (int32_t)((Jend - J0) / 16 + 1);
    const int32_t T = twin + (a.g + 15) / 16;
    const int64_t qi = i0 + m;   // this lane's query row
    const float* Gq = a.Gs + a.stride + ((int64_t)bh * n + (qi < n ? qi : 0)) * 64 + 4 * kq;
    const float* Zb = a.Zs + (int64_t)bh * n * 64 + 4 * kq;

    for (int32_t tp = 0; tp < T; tp += kTiles) {
        f32x4 acc[kTiles];
#pragma unroll
        for (int tt = 0; tt < kTiles; ++tt) acc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int32_t k = 0; k < a.K; ++k) {
            f32x4 q[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) q[s] = ld4z(Gq + k * a.stride + 16 * s, qi < n);
#pragma unroll
            for (int tt = 0; tt < kTiles; ++tt) {
                const int32_t t = tp + tt;
                if (t >= T) continue;   // the same in every lane
                int64_t key;
                bool kok;
                if (t < twin) {
                    key = J0 + 16 * t + m;
                    kok = key < n;
                } else {
                    const int32_t gt = 16 * (t - twin) + m;
                    kok = gt < a.g;
                    key = kok ? a.G[gt] : 0;
                }
                const float* Zk = Zb + k * a.stride + (kok ? key : 0) * 64;
#pragma unroll
                for (int s = 0; s < 4; ++s) acc[tt] = mfma_chunk(acc[tt], q[s], ld4z(Zk + 16 * s, kok));
            }
        }
        // Lane holds rows i0 + 4 kq + v against key m of each tile.
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int64_t i = i0 + 4 * kq + v;
            if (i >= n) continue;
            const int4 ri = info[i];
            if (ri.z < 0) continue;   // a global row: k_dots_glob's
            const int64_t lo = i - r < 0 ? 0 : i - r;
            const int64_t hi = i + r > n - 1 ? n - 1 : i + r;
            const int64_t wend = a.causal ? i : hi;
            const int64_t last = a.causal ? i : n - 1;
#pragma unroll
            for (int tt = 0; tt < kTiles; ++tt) {
                const int32_t t = tp + tt;
                if (t >= T) continue;
                if (t < twin) {
                    const int64_t j = J0 + 16 * t + m;
                    const int64_t s = j - ri.y;
                    if (s >= 0 && s < ri.z)
                        dAb[(int64_t)ri.x + s] = j >= lo && j <= wend ? a.f * acc[tt][v] : 0.0f;
                } else {
                    const int32_t gt = 16 * (t - twin) + m;
                    if (gt < ri.w) {
                        const int64_t c = gt < a.g ? a.G[gt] : -1;
                        const bool ok = c >= 0 && (c < lo || c > hi) && c <= last;
                        dAb[(int64_t)ri.x + ri.z + gt] = ok ? a.f * acc[tt][v] : 0.0f;
                    }
                }
            }
        }
    }
}

// k_dots_band with the key rows in LDS: a workgroup of 16 waves owns 64
// consecutive rows (four blocks); for each state k it copies the key rows
// of Z_k that a window slot of its rows can name (one contiguous run) and
// the g global rows into LDS by direct global-to-LDS loads, a row's 16-byte
// pieces permuted by (row mod 16) so that the 16 rows one operand read
// touches fall on distinct banks; wave w takes the tiles w mod 4,
// w mod 4 + 4, ... of block w / 4. Every key row is then read from L2 once
// per 64 rows and state instead of once per block of 16.
constexpr int kLdsWaves = 16;
constexpr int kLdsThreads = kWave * kLdsWaves;
constexpr int kWaveTiles = 4;     // tiles per wave: at most 16 per block
constexpr int kLdsPad = 16;       // zero rows past the globals (a global tile reads up to 15 past g)

__global__ __launch_bounds__(kLdsThreads, 8)
void k_dots_band_lds(DotsArgs a, int32_t groups, int32_t per_xcd, int32_t win_rows) {
    extern __shared__ __align__(16) char lds_raw[];
    float LDS_AS* lds = (float LDS_AS*)lds_raw;
    const int lane = __lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int m = lane & 15, kq = lane >> 4;
    const int32_t item = (int32_t)(blockIdx.x & 7u) * per_xcd + (int32_t)(blockIdx.x >> 3);
    if (item >= a.BH * groups) return;
    const int32_t bh = item / groups;
    const int64_t r0 = (int64_t)(item - bh * groups) * 64;
    const int32_t b = bh / a.H, h = bh - b * a.H;
    const int32_t gr = a.num_graphs == 1 ? 0 : b;
    const int64_t n = a.n, r = a.radius;
    const int4* info = a.row_info + (int64_t)gr * n;
    float* dAb = a.dA + a_block_offset(a.slot_off, a.num_graphs, a.H, b, h);
    const int64_t w0 = (r0 - r < 0 ? 0 : r0 - r) & ~7ll;
    // This wave's block and tiles.
    const int64_t i0 = r0 + 16 * (wave >> 2);
    const int tq = wave & 3;
    int64_t J0, wl_first, wb_last, Jend;
    window_span(i0 < n ? i0 : n - 1, n, r, a.causal, J0, wl_first);
    window_span(i0 + 15 < n ? i0 + 15 : n - 1, n, r, a.causal, wb_last, Jend);
    const int32_t twin = (int32_t)((Jend - J0) / 16 + 1);
    const int32_t T = i0 < n ? twin + (a.g + 15) / 16 : 0;
    const int64_t qi = i0 + m;
    const float* Gq = a.Gs + a.stride + ((int64_t)bh * n + (qi < n ? qi : 0)) * 64 + 4 * kq;
    const int32_t rows = win_rows + a.g + kLdsPad;
    f32x4 acc[kWaveTiles];
#pragma unroll
    for (int tt = 0; tt < kWaveTiles; ++tt) acc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int32_t k = 0; k < a.K; ++k) {
        if (k > 0) __syncthreads();   // every wave is done with state k - 1's rows
        const float* Zk = a.Zs + (int64_t)k * a.stride + (int64_t)bh * n * 64;
        for (int32_t p0 = 64 * wave; p0 < rows * 16; p0 += 64 * kLdsWaves) {
            const int32_t p = p0 + lane;
            const int32_t rr = p >> 4, pos = p & 15;
            int64_t key = -1;
            if (rr < win_rows) key = w0 + rr;
            else if (rr < win_rows + a.g) key = a.G[rr - win_rows];
            if (p < rows * 16 && key >= 0 && key < n)
                dma16(Zk + key * 64 + 4 * (pos ^ (rr & 15)), (void LDS_AS*)(lds + 4 * p0));
            else if (p < rows * 16)
                *reinterpret_cast<f32x4 LDS_AS*>(lds + 4 * p) = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        f32x4 q[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) q[s] = ld4z(Gq + k * a.stride + 16 * s, qi < n);
        full_barrier();
#pragma unroll
        for (int tt = 0; tt < kWaveTiles; ++tt) {
            const int32_t t = tq + 4 * tt;
            if (t >= T) continue;   // the same in every lane
            int32_t kl;
            if (t < twin) {
                const int64_t key = J0 + 16 * t + m;
                kl = (int32_t)min(key - w0, (int64_t)win_rows - 1);
            } else {
                kl = win_rows + 16 * (t - twin) + m;
            }
            const float LDS_AS* row = lds + (int64_t)kl * 64;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const f32x4 z =
                    *reinterpret_cast<const f32x4 LDS_AS*>(row + 4 * ((4 * s + kq) ^ (kl & 15)));
                acc[tt] = mfma_chunk(acc[tt], q[s], z);
            }
        }
    }
    // Lane holds rows i0 + 4 kq + v against key m of each of its tiles.
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int64_t i = i0 + 4 * kq + v;
        if (i >= n) continue;
        const int4 ri = info[i];
        if (ri.z < 0) continue;   // a global row: k_dots_glob's
        const int64_t lo = i - r < 0 ? 0 : i - r;
        const int64_t hi = i + r > n - 1 ? n - 1 : i + r;
        const int64_t wend = a.causal ? i : hi;
        const int64_t last = a.causal ? i : n - 1;
#pragma unroll
        for (int tt = 0; tt < kWaveTiles; ++tt) {
            const int32_t t = tq + 4 * tt;
            if (t >= T) continue;
            if (t < twin) {
                const int64_t j = J0 + 16 * t + m;
                const int64_t s = j - ri.y;
                if (s >= 0 && s < ri.z)
                    dAb[(int64_t)ri.x + s] = j >= lo && j <= wend ? a.f * acc[tt][v] : 0.0f;
            } else {
                const int32_t gt = 16 * (t - twin) + m;
                if (gt < ri.w) {
                    const int64_t c = gt < a.g ? a.G[gt] : -1;
                    const bool ok = c >= 0 && (c < lo || c > hi) && c <= last;
                    dAb[(int64_t)ri.x + ri.z + gt] = ok ? a.f * acc[tt][v] : 0.0f;
                }
            }
        }
    }
}

// Each wave takes kKTiles tiles of 16 keys, so every global row's operand
// load serves them all.
constexpr int kKTiles = 2;

__global__ __launch_bounds__(kThreads)
void k_dots_glob(DotsArgs a) {
    const int lane = __lane_id();
    const int wave = threadIdx.x / kWave;
    const int m = lane & 15, kq = lane >> 4;
    const int64_t nkp = (a.nkt + kKTiles - 1) / kKTiles;
    const int64_t item = (int64_t)blockIdx.x * kWavesPerBlock + wave;
    if (item >= (int64_t)a.BH * nkp) return;
    const int32_t bh = (int32_t)(item / nkp);
    const int64_t j0 = (item - (int64_t)bh * nkp) * 16 * kKTiles;
    const int32_t b = bh / a.H, h = bh - b * a.H;
    const int32_t gr = a.num_graphs == 1 ? 0 : b;
    const int64_t n = a.n;
    const int4* info = a.row_info + (int64_t)gr * n;
    const int64_t* sp = a.seg_ptr + (int64_t)gr * (n + 1);
    float* dAb = a.dA + a_block_offset(a.slot_off, a.num_graphs, a.H, b, h);
    int64_t key[kKTiles];   // this lane's key row of each tile
    const float* Zk[kKTiles];
#pragma unroll
    for (int kt = 0; kt < kKTiles; ++kt) {
        key[kt] = j0 + 16 * kt + m;
        Zk[kt] = a.Zs + ((int64_t)bh * n + (key[kt] < n ? key[kt] : 0)) * 64 + 4 * kq;
    }
    const float* Gb = a.Gs + a.stride + (int64_t)bh * n * 64 + 4 * kq;

    for (int32_t qp = 0; qp < a.g; qp += 16 * kQTiles) {
        f32x4 acc[kQTiles][kKTiles];
#pragma unroll
        for (int qt = 0; qt < kQTiles; ++qt)
#pragma unroll
            for (int kt = 0; kt < kKTiles; ++kt) acc[qt][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int32_t k = 0; k < a.K; ++k) {
            f32x4 z[kKTiles][4];
#pragma unroll
            for (int kt = 0; kt < kKTiles; ++kt)
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    z[kt][s] = ld4z(Zk[kt] + k * a.stride + 16 * s, key[kt] < n);
#pragma unroll
            for (int qt = 0; qt < kQTiles; ++qt) {
                const int32_t q0 = qp + 16 * qt;
                if (q0 >= a.g) continue;   // the same in every lane
                const bool qok = q0 + m < a.g;
                const int64_t gi = qok ? a.G[q0 + m] : 0;
                const float* Gq = Gb + k * a.stride + gi * 64;
                // rows of the product = global rows, columns = keys
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const f32x4 gq = ld4z(Gq + 16 * s, qok);
#pragma unroll
                    for (int kt = 0; kt < kKTiles; ++kt)
                        acc[qt][kt] = mfma_chunk(acc[qt][kt], gq, z[kt][s]);
                }
            }
        }
        // Lane holds global rows q0 + 4 kq + v against key j0 + 16 kt + m.
#pragma unroll
        for (int qt = 0; qt < kQTiles; ++qt) {
            const int32_t q0 = qp + 16 * qt;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int32_t q = q0 + 4 * kq + v;
                if (q >= a.g) continue;
                const int64_t i = a.G[q];
                const int64_t seglen = sp[i + 1] - sp[i];
                const int64_t last = a.causal ? i : n - 1;
#pragma unroll
                for (int kt = 0; kt < kKTiles; ++kt)
                    if (key[kt] < seglen)
                        dAb[(int64_t)info[i].x + key[kt]] =
                            key[kt] <= last ? a.f * acc[qt][kt][v] : 0.0f;
            }
        }
    }
}

DotsArgs make_args(const diffuser_graph& g, int32_t B, int32_t H, const float* Gs, const float* Zs,
                   int64_t stride, int32_t K, float f, float* dA) {
    DotsArgs a;
    a.n = g.n;
    a.H = H;
    a.num_graphs = g.num_graphs;
    a.radius = g.radius;
    a.causal = g.causal;
    a.g = g.num_global;
    a.K = K;
    a.BH = B * H;
    a.nrb = (int32_t)((g.n + 15) / 16);
    a.nkt = (int32_t)(((g.n + 7) / 8 * 8 + 15) / 16);
    a.stride = stride;
    a.slot_off = g.d_slot_off;
    a.seg_ptr = g.d_seg_ptr;
    a.row_info = reinterpret_cast<const int4*>(g.d_row_info);
    a.G = g.d_global;
    a.Gs = Gs;
    a.Zs = Zs;
    a.dA = dA;
    a.f = f;
    return a;
}

// Key rows of a 64-row group's window run (its rows, the radius on either
// side, or on the left when causal, and the 8-column alignment).
int32_t lds_win_rows(const diffuser_graph& g) {
    return 64 + (g.causal ? 1 : 2) * g.radius + 8;
}

// k_dots_band_lds serves a graph whose blocks have at most 16 tiles and
// whose window run and globals fit two workgroups per CU.
bool lds_band_fits(const diffuser_graph& g) {
    const int64_t twin = (15 + (g.causal ? 1 : 2) * (int64_t)g.radius + 14) / 16 + 1;
    const int64_t tiles = twin + (g.num_global + 15) / 16;
    const int64_t bytes = (int64_t)(lds_win_rows(g) + g.num_global + kLdsPad) * 256;
    return tiles <= 4 * kWaveTiles && 2 * bytes <= 160 * 1024;
}

}  // namespace

bool mfma_dots_supported(const diffuser_graph& g, int32_t d) {
    if (!g.structured || !g.rand_apart() || g.d_row_info == nullptr || d != 64) return false;
    for (int64_t x : g.slots)
        if (x >= (1ll << 31)) return false;   // slot numbers in int4 row geometry
    return true;
}

hipError_t launch_dots_dense(const diffuser_graph& g, int32_t B, int32_t H, const float* Gs,
                             const float* Zs, int64_t stride, int32_t K, float f, float* dA,
                             hipStream_t st) {
    const DotsArgs a = make_args(g, B, H, Gs, Zs, stride, K, f, dA);
    hipError_t e;
    const int32_t wrows = lds_win_rows(g);
    if (lds_band_fits(g)) {
        static int attr_device = -1;
        if (attr_device != g.device) {
            e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_dots_band_lds),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
            if (e != hipSuccess) return e;
            attr_device = g.device;
        }
        const int32_t groups = (int32_t)((g.n + 63) / 64);
        const int32_t per_xcd = (a.BH * groups + 7) / 8;
        hipLaunchKernelGGL(k_dots_band_lds, dim3((unsigned)(8 * per_xcd)), dim3(kLdsThreads),
                           (size_t)(wrows + g.num_global + kLdsPad) * 256, st, a, groups, per_xcd,
                           wrows);
    } else {
        const int64_t band = ((int64_t)a.BH * a.nrb + kWavesPerBlock - 1) / kWavesPerBlock;
        hipLaunchKernelGGL(k_dots_band, dim3((unsigned)band), dim3(kThreads), 0, st, a);
    }
    e = hipGetLastError();
    if (e != hipSuccess || g.num_global == 0) return e;
    const int64_t glob =
        ((int64_t)a.BH * ((a.nkt + kKTiles - 1) / kKTiles) + kWavesPerBlock - 1) / kWavesPerBlock;
    hipLaunchKernelGGL(k_dots_glob, dim3((unsigned)glob), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace diffuser
