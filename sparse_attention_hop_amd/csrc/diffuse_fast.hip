// Diffusion step on built graphs, bf16 storage, head width 64:
//   Z_{k+1}[i] = (1 - alpha) * c_i * sum_j A_ij Z_k[j] + alpha * V[i]
// ("Diffuser" reading notes, section 2.4, eq. S.7; c_i rescales the stored
// weights of row i to sum to one, or is 1).
//
// Each workgroup streams Z_k of one (batch, head) through LDS in chunks of
// 256 rows, and every edge reads its neighbour row from LDS, never from L2:
//  * window edges: the band of a 16-row block is a dense 16 x 32 weight
//    block per 32 key columns; v_mfma_f32_16x16x32_bf16 multiplies it with
//    the chunk's key rows (the weight slots of a window are 8-aligned column
//    blocks, so each lane's 8 weights are one aligned 16-byte load);
//  * global columns: the g global rows of Z_k are staged once per
//    workgroup and multiplied as a dense 16 x g block by MFMA;
//  * random edges: dot2 (two edges of one row per instruction, lane =
//    channel) from the chunk holding their key rows; each 16-lane group's
//    result is moved into the MFMA accumulator layout with permlane swaps.
// Global rows (full rows of length n) get workgroups of their own: 32 rows,
// the 8 waves split each chunk's columns and add their partial sums in a
// fixed order at the end.
// Workgroups are numbered so that each XCD (workgroup id mod 8) works
// through a contiguous range of (batch, head) pairs, keeping Z_k of the
// pairs in flight resident in that XCD's L2.
#include "internal.h"
#include "vec.h"

namespace diffuser {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kWaves = 16;
constexpr int kThreads = kWave * kWaves;
constexpr int kD = 64;            // head width
constexpr int kNB = kD / 16;      // 16-channel MFMA blocks
constexpr int kZS = 72;           // LDS row stride in bf16 (144 B: 16-B aligned, bank-spread)
constexpr int kGrowRows = 32;     // global rows per global-row workgroup
constexpr int kStage = 16;        // random edges per row staged per pass
constexpr int kChunk = 512;       // key rows per LDS chunk

struct FastArgs {
    int64_t n;
    int32_t H, num_graphs, radius, g, causal, rnd_width, nchunks, chunk;
    const int64_t* slot_ptr;   // [graphs][n + 1]
    const int64_t* slot_off;   // [graphs + 1]
    const int32_t* G;          // [g]
    const int32_t* rnd;        // [graphs][n][rnd_width]
    const int32_t* rnd_cnt;    // [graphs][n]
    const int32_t* bnd;        // [graphs][n][nchunks + 1]
    const uint16_t* A;
    const uint16_t* Z;
    const uint16_t* V;
    uint16_t* Zn;
    const float* row_scale;    // [B*H][n] or null
    float alpha;
    int32_t BH, tiles_per_bh, grow_per_bh, per_xcd, total_items;
};

__device__ __forceinline__ int32_t count_less(const int32_t* a, int32_t len, int64_t x) {
    int32_t lo = 0, hi = len;
    while (lo < hi) {
        int32_t mid = (lo + hi) >> 1;
        if ((int64_t)a[mid] < x) lo = mid + 1; else hi = mid;
    }
    return lo;
}

__device__ __forceinline__ bool is_global_pos(const int32_t* G, int32_t g, int64_t j) {
    int32_t k = count_less(G, g, j);
    return k < g && G[k] == j;
}

__device__ __forceinline__ int64_t round8(int64_t x) { return (x + 7) & ~7ll; }

__device__ __forceinline__ f32x4 mfma(const u32x4& a, const u32x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// B operand of a 16x16x32 MFMA: 8 consecutive LDS rows (k) of one channel.
__device__ __forceinline__ u32x4 load_b(const uint16_t* rows, int ch) {
    u32x4 b;
#pragma unroll
    for (int t = 0; t < 4; ++t)
        b[t] = (uint32_t)rows[(2 * t) * kZS + ch] | ((uint32_t)rows[(2 * t + 1) * kZS + ch] << 16);
    return b;
}

// Copies rows [r0, r0 + count) of the (b, h) slab of Z into LDS (zero for
// rows at or beyond n).
__device__ __forceinline__ void load_rows(uint16_t* dst, const uint16_t* Zbh, int64_t n,
                                          int64_t r0, int count) {
    for (int idx = threadIdx.x; idx < count * 8; idx += kThreads) {
        const int row = idx >> 3, part = idx & 7;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (r0 + row < n) v = *reinterpret_cast<const u32x4*>(Zbh + (r0 + row) * kD + part * 8);
        *reinterpret_cast<u32x4*>(dst + row * kZS + part * 8) = v;
    }
}

__device__ __forceinline__ uint16_t to_bf16(float x) { return (uint16_t)f32_to_bf16(x); }

// v_permlane32_swap / v_permlane16_swap with both registers declared
// read-write. (Through the compiler builtins, the second result of a swap
// was dropped when both results stayed live, so the swaps are written out.)
// a <-> b: lanes 32-63 of a trade places with lanes 0-31 of b.
__device__ __forceinline__ void swap32(float& a, float& b) {
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
// a <-> b: the odd 16-lane rows of a trade places with the even rows of b.
__device__ __forceinline__ void swap16(float& a, float& b) {
    asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}

// Restart and store of one 16x16 accumulator block (rows row0 + 4*(l/16) + e,
// channel ch) unless the row is outside [0, n) or flagged in skip_mask.
__device__ __forceinline__ void store_block(const FastArgs& a, int32_t bh, int64_t row0, int ch,
                                            const f32x4& acc, uint32_t skip_mask, int mask_base) {
    const int lane = __lane_id();
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int rl = 4 * (lane >> 4) + e;   // row within the 16-row block
        const int64_t i = row0 + rl;
        if (i >= a.n || ((skip_mask >> (mask_base + rl)) & 1u)) continue;
        const int64_t o = ((int64_t)bh * a.n + i) * kD + ch;
        const float keep = a.row_scale ? (1.0f - a.alpha) * a.row_scale[(int64_t)bh * a.n + i]
                                       : 1.0f - a.alpha;
        const float v = bf16_to_f32(a.V[o]);
        a.Zn[o] = to_bf16(keep * acc[e] + a.alpha * v);
    }
}

template <int RPW>  // rows per wave (multiple of 16, at most 32)
__global__ __launch_bounds__(kThreads)
void k_diffuse_fast(FastArgs a) {
    extern __shared__ __align__(16) uint16_t lds[];
    constexpr int MB = RPW / 16;
    const int lane = __lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);

    // XCD-aware numbering: workgroup id mod 8 is the XCD; each XCD walks a
    // contiguous range of items (grow workgroups of a pair come first).
    const int32_t item = (blockIdx.x & 7) * a.per_xcd + (blockIdx.x >> 3);
    if (item >= a.total_items) return;
    const int32_t per_bh = a.grow_per_bh + a.tiles_per_bh;
    const int32_t bh = item / per_bh;
    const int32_t sub = item - bh * per_bh;
    const int32_t b = bh / a.H, h = bh - b * a.H;
    const int32_t gr = a.num_graphs == 1 ? 0 : b;
    const int64_t n = a.n;
    const int64_t* sp = a.slot_ptr + (int64_t)gr * (n + 1);
    const uint16_t* Abh = a.A + a_block_offset(a.slot_off, a.num_graphs, a.H, b, h);
    const uint16_t* Zbh = a.Z + (int64_t)bh * n * kD;
    uint16_t* zc = lds;                               // chunk: a.chunk rows
    uint16_t* zg = lds + a.chunk * kZS;               // globals: round32(g) rows
    const int gpad = (a.g + 31) & ~31;
    // Random-edge staging, per wave: byte offsets of the key rows within the
    // chunk [RPW][kStage] and their weights [RPW][kStage].
    uint32_t* st_off = reinterpret_cast<uint32_t*>(zg + gpad * kZS) + wave * (RPW * kStage * 3 / 2);
    uint16_t* st_a = reinterpret_cast<uint16_t*>(st_off + RPW * kStage);
    const int nl = lane & 15, kg = lane >> 4;

    if (sub < a.grow_per_bh) {
        // ---------------- global rows -------------------------------------
        const int q0 = sub * kGrowRows;
        f32x4 acc[2][kNB];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int nb = 0; nb < kNB; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
        // A-operand rows of this lane: global rows q0 + 16 mb + (lane % 16).
        int64_t rbase[2], rslots[2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            const int q = q0 + 16 * mb + nl;
            rbase[mb] = 0;
            rslots[mb] = 0;
            if (q < a.g) {
                const int64_t i = a.G[q];
                rbase[mb] = sp[i];
                rslots[mb] = sp[i + 1] - sp[i];
            }
        }
        for (int c = 0; c < a.nchunks; ++c) {
            const int64_t c0 = (int64_t)c * a.chunk;
            __syncthreads();
            load_rows(zc, Zbh, n, c0, a.chunk);
            __syncthreads();
            const int64_t cend = min((int64_t)a.chunk, n - c0);
            for (int kc = 32 * wave; kc < cend; kc += 32 * kWaves) {
                u32x4 bop[kNB];
#pragma unroll
                for (int nb = 0; nb < kNB; ++nb) bop[nb] = load_b(zc + (kc + 8 * kg) * kZS, 16 * nb + nl);
#pragma unroll
                for (int mb = 0; mb < 2; ++mb) {
                    const int64_t col = c0 + kc + 8 * kg;
                    u32x4 aop = {0u, 0u, 0u, 0u};
                    if (col < rslots[mb])
                        aop = *reinterpret_cast<const u32x4*>(Abh + rbase[mb] + col);
#pragma unroll
                    for (int nb = 0; nb < kNB; ++nb) acc[mb][nb] = mfma(aop, bop[nb], acc[mb][nb]);
                }
            }
        }
        // Fixed-order tree reduction of the 8 waves' partial sums in LDS.
        __syncthreads();
        float* red = reinterpret_cast<float*>(lds);   // kWaves/2 waves x 2 x kNB x 4 x 64 floats
        for (int half = kWaves / 2; half >= 1; half >>= 1) {
            if (wave >= half && wave < 2 * half) {
                float* dst = red + (wave - half) * (2 * kNB * 4 * kWave);
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                    for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            dst[((mb * kNB + nb) * 4 + e) * kWave + lane] = acc[mb][nb][e];
            }
            __syncthreads();
            if (wave < half) {
                const float* src = red + wave * (2 * kNB * 4 * kWave);
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                    for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            acc[mb][nb][e] += src[((mb * kNB + nb) * 4 + e) * kWave + lane];
            }
            __syncthreads();
        }
        if (wave == 0) {
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int q = q0 + 16 * mb + 4 * kg + e;
                    if (q >= a.g) continue;
                    const int64_t i = a.G[q];
#pragma unroll
                    for (int nb = 0; nb < kNB; ++nb) {
                        const int64_t o = ((int64_t)bh * n + i) * kD + 16 * nb + nl;
                        const float keep = a.row_scale
                            ? (1.0f - a.alpha) * a.row_scale[(int64_t)bh * n + i]
                            : 1.0f - a.alpha;
                        a.Zn[o] = to_bf16(keep * acc[mb][nb][e] + a.alpha * bf16_to_f32(a.V[o]));
                    }
                }
            }
        }
        return;
    }

    // ---------------- row tile --------------------------------------------
    const int64_t r0w = (int64_t)(sub - a.grow_per_bh) * (RPW * kWaves) + (int64_t)RPW * wave;
    f32x4 acc[MB][kNB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Per-lane row data for the A operand (row r0w + 16 mb + lane % 16).
    int32_t sbase[MB], wb0[MB], wseg[MB], gseg[MB];
    bool rok[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int64_t i = r0w + 16 * mb + nl;
        rok[mb] = i < n && !is_global_pos(a.G, a.g, i);
        sbase[mb] = 0; wb0[mb] = 0; wseg[mb] = 0; gseg[mb] = 0;
        if (rok[mb]) {
            const int64_t lo = i - a.radius < 0 ? 0 : i - a.radius;
            const int64_t hi = i + a.radius > n - 1 ? n - 1 : i + a.radius;
            const int64_t wend = a.causal ? i : hi;
            sbase[mb] = (int32_t)sp[i];
            wb0[mb] = (int32_t)(lo & ~7ll);
            wseg[mb] = (int32_t)((wend - wb0[mb]) / 8 * 8 + 8);
            gseg[mb] = (int32_t)round8(a.causal ? count_less(a.G, a.g, lo) : a.g);
        }
    }
    // Rows of this wave that are global or beyond n (not written here).
    uint32_t skip = 0;
    {
        const int64_t i = r0w + (lane & 31);
        const bool s = (lane < RPW) && (i >= n || is_global_pos(a.G, a.g, i));
        skip = (uint32_t)__ballot(s);
    }
    // Random-edge bookkeeping: lane w < RPW owns row r0w + w.
    const int64_t my_row = r0w + (lane < RPW ? lane : 0);
    const bool my_ok = lane < RPW && my_row < n;
    const int32_t* my_bnd = a.bnd + ((int64_t)gr * n + (my_ok ? my_row : 0)) * (a.nchunks + 1);
    int32_t my_rseg = 0;   // offset of my row's random segment within A's (b, h) block
    if (my_ok) {
        const int64_t i = my_row;
        if (!is_global_pos(a.G, a.g, i)) {
            const int64_t lo = i - a.radius < 0 ? 0 : i - a.radius;
            const int64_t hi = i + a.radius > n - 1 ? n - 1 : i + a.radius;
            const int64_t wend = a.causal ? i : hi;
            const int64_t w0 = lo & ~7ll;
            const int64_t ws = (wend - w0) / 8 * 8 + 8;
            const int64_t gs = round8(a.causal ? count_less(a.G, a.g, lo) : a.g);
            my_rseg = (int32_t)(sp[i] + ws + gs);
        }
    }
    const int32_t* rnd_gr = a.rnd + (int64_t)gr * n * a.rnd_width;

    // Band of this wave: key columns [band_lo, band_hi].
    const int64_t wr_last = min(r0w + RPW - 1, n - 1);
    const int64_t band_lo = (r0w - a.radius < 0 ? 0 : r0w - a.radius) & ~31ll;
    const int64_t band_hi = a.causal ? wr_last : min(n - 1, wr_last + a.radius);

    // Global columns, staged once.
    for (int idx = threadIdx.x; idx < gpad * 8; idx += kThreads) {
        const int q = idx >> 3, part = idx & 7;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (q < a.g) v = *reinterpret_cast<const u32x4*>(Zbh + (int64_t)a.G[q] * kD + part * 8);
        *reinterpret_cast<u32x4*>(zg + q * kZS + part * 8) = v;
    }
    __syncthreads();
    if (r0w < n) {
        for (int q = 0; q < gpad; q += 32) {
            u32x4 bop[kNB];
#pragma unroll
            for (int nb = 0; nb < kNB; ++nb) bop[nb] = load_b(zg + (q + 8 * kg) * kZS, 16 * nb + nl);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                u32x4 aop = {0u, 0u, 0u, 0u};
                if (rok[mb] && q + 8 * kg < gseg[mb])
                    aop = *reinterpret_cast<const u32x4*>(Abh + sbase[mb] + wseg[mb] + q + 8 * kg);
#pragma unroll
                for (int nb = 0; nb < kNB; ++nb) acc[mb][nb] = mfma(aop, bop[nb], acc[mb][nb]);
            }
        }
    }

    // ---- software pipeline over key-row chunks ----------------------------
    // While chunk c is multiplied, chunk c + 1's rows of Z_k and the first
    // kStage random edges of each row in it are fetched into registers.
    constexpr int kZPer = kChunk * 8 / kThreads;     // 16-byte pieces per thread
    constexpr int kSPer = RPW / 4;                   // staged entries per lane
    u32x4 zr[kZPer];
    int32_t sj[kSPer];
    uint32_t sw[kSPer];
    uint32_t sv = 0;                                 // valid bits of the staged entries
    int32_t b0 = my_ok ? my_bnd[0] : 0;
    int32_t b1 = my_ok ? my_bnd[1] : 0;
    int32_t b2 = (my_ok && a.nchunks >= 2) ? my_bnd[2] : 0;

    auto fetch_chunk = [&](int c) {
        const int64_t c0 = (int64_t)c * kChunk;
#pragma unroll
        for (int t = 0; t < kZPer; ++t) {
            const int idx = threadIdx.x + t * kThreads;
            const int row = idx >> 3, part = idx & 7;
            zr[t] = u32x4{0u, 0u, 0u, 0u};
            if (c0 + row < n) zr[t] = *reinterpret_cast<const u32x4*>(Zbh + (c0 + row) * kD + part * 8);
        }
    };
    auto store_chunk = [&]() {
#pragma unroll
        for (int t = 0; t < kZPer; ++t) {
            const int idx = threadIdx.x + t * kThreads;
            const int row = idx >> 3, part = idx & 7;
            *reinterpret_cast<u32x4*>(zc + row * kZS + part * 8) = zr[t];
        }
    };
    // Lane l stages entry (l % 16) of rows 4 it + l / 16; every address is
    // clamped into the row's arrays, invalid entries are masked at store time.
    auto fetch_stage = [&](int32_t start, int32_t end, int32_t pass) {
        sv = 0;
#pragma unroll
        for (int it = 0; it < kSPer; ++it) {
            const int w = 4 * it + (lane >> 4);
            const int32_t s = __shfl(start, w) + pass;
            const int32_t e = __shfl(end, w);
            const int32_t rs = __shfl(my_rseg, w);
            const int32_t k = s + (lane & 15);
            const int32_t kc = k < a.rnd_width - 1 ? k : a.rnd_width - 1;
            const int64_t rw = r0w + w < n ? r0w + w : n - 1;
            sj[it] = rnd_gr[rw * a.rnd_width + kc];
            sw[it] = Abh[rs + kc];
            sv |= (k < e ? 1u : 0u) << it;
        }
    };
    auto store_stage = [&](int64_t c0) {
#pragma unroll
        for (int it = 0; it < kSPer; ++it) {
            const int w = 4 * it + (lane >> 4);
            const bool v = (sv >> it) & 1u;
            st_off[w * kStage + (lane & 15)] = v ? (uint32_t)(sj[it] - c0) * (kZS * 2) : 0u;
            st_a[w * kStage + (lane & 15)] = v ? (uint16_t)sw[it] : (uint16_t)0;
        }
    };
    const uint32_t lane_byte = 2u * (uint32_t)lane;
    const char* zb = reinterpret_cast<const char*>(zc);
    // Random edges of rows staged in LDS: lane = channel, two edges of one
    // row per dot2, then the 4 x 4 transpose of 16-lane groups into the MFMA
    // layout (x[g4] holds row 4 g4 + r with lane = channel; afterwards x[nb]
    // holds channel block nb with lane 16 g4 + n = row 4 g4 + r).
    auto random_pass = [&](int32_t start, int32_t end, int32_t pass) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float x[4];
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int w = 16 * mb + 4 * g4 + r;
                    int32_t cnt = __builtin_amdgcn_readlane(end, w) -
                                  __builtin_amdgcn_readlane(start, w) - pass;
                    cnt = cnt < kStage ? cnt : kStage;
                    const u32x4* so = reinterpret_cast<const u32x4*>(st_off + w * kStage);
                    const uint2* sa = reinterpret_cast<const uint2*>(st_a + w * kStage);
                    float xs = 0.0f;
                    for (int32_t p = 0; p < cnt; p += 4) {
                        const u32x4 o = so[p >> 2];
                        const uint2 ap = sa[p >> 2];
                        const uint32_t z0 = *reinterpret_cast<const uint16_t*>(zb + o[0] + lane_byte);
                        const uint32_t z1 = *reinterpret_cast<const uint16_t*>(zb + o[1] + lane_byte);
                        const uint32_t z2 = *reinterpret_cast<const uint16_t*>(zb + o[2] + lane_byte);
                        const uint32_t z3 = *reinterpret_cast<const uint16_t*>(zb + o[3] + lane_byte);
                        xs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, ap.x),
                                                             __builtin_bit_cast(bf16x2, z0 | (z1 << 16)),
                                                             xs, false);
                        xs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, ap.y),
                                                             __builtin_bit_cast(bf16x2, z2 | (z3 << 16)),
                                                             xs, false);
                    }
                    x[g4] = xs;
                }
                swap32(x[0], x[2]);
                swap32(x[1], x[3]);
                swap16(x[0], x[1]);
                swap16(x[2], x[3]);
                acc[mb][0][r] += x[0];
                acc[mb][1][r] += x[1];
                acc[mb][2][r] += x[2];
                acc[mb][3][r] += x[3];
            }
        }
    };

    fetch_chunk(0);
    fetch_stage(b0, b1, 0);
    for (int c = 0; c < a.nchunks; ++c) {
        const int64_t c0 = (int64_t)c * kChunk;
        const int32_t cs = b0, ce = b1;
        __syncthreads();
        store_chunk();
        store_stage(c0);
        __syncthreads();
        if (c + 1 < a.nchunks) {
            b0 = b1;
            b1 = b2;
            b2 = (my_ok && c + 3 <= a.nchunks) ? my_bnd[c + 3] : 0;
            fetch_chunk(c + 1);
            fetch_stage(b0, b1, 0);
        }
        if (r0w >= n) continue;

        // Window band.
        const int64_t k_lo = max(band_lo, c0);
        const int64_t k_hi = min(band_hi, c0 + kChunk - 1);
        for (int64_t kc = k_lo; kc <= k_hi; kc += 32) {
            u32x4 bop[kNB];
#pragma unroll
            for (int nb = 0; nb < kNB; ++nb)
                bop[nb] = load_b(zc + (kc - c0 + 8 * kg) * kZS, 16 * nb + nl);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const int32_t off = (int32_t)(kc + 8 * kg) - wb0[mb];
                u32x4 aop = {0u, 0u, 0u, 0u};
                if (rok[mb] && off >= 0 && off < wseg[mb])
                    aop = *reinterpret_cast<const u32x4*>(Abh + sbase[mb] + off);
#pragma unroll
                for (int nb = 0; nb < kNB; ++nb) acc[mb][nb] = mfma(aop, bop[nb], acc[mb][nb]);
            }
        }

        // Random edges in this chunk: the first kStage per row were staged
        // above; any further ones (rare) are staged and used pass by pass.
        random_pass(cs, ce, 0);
        const bool more = __ballot(lane < RPW && ce - cs > kStage) != 0;
        if (more) {
            const uint32_t keep_sv = sv;
            int32_t keep_j[kSPer];
            uint32_t keep_w[kSPer];
#pragma unroll
            for (int t = 0; t < kSPer; ++t) { keep_j[t] = sj[t]; keep_w[t] = sw[t]; }
            int32_t most = 0;
            for (int w = 0; w < RPW; ++w) {
                const int32_t cnt = __builtin_amdgcn_readlane(ce, w) - __builtin_amdgcn_readlane(cs, w);
                most = cnt > most ? cnt : most;
            }
            for (int32_t pass = kStage; pass < most; pass += kStage) {
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                fetch_stage(cs, ce, pass);
                store_stage(c0);
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                random_pass(cs, ce, pass);
            }
            sv = keep_sv;
#pragma unroll
            for (int t = 0; t < kSPer; ++t) { sj[t] = keep_j[t]; sw[t] = keep_w[t]; }
        }
    }

    if (r0w >= n) return;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb)
            store_block(a, bh, r0w + 16 * mb, 16 * nb + nl, acc[mb][nb], skip, 16 * mb);
}

}  // namespace

bool fast_diffuse_supported(const diffuser_graph& g, const attn_shape& s) {
    return g.structured && s.dtype == DIFFUSER_BF16 && s.d == kD && g.d_bnd != nullptr &&
           g.chunk == kChunk;
}

constexpr int kRPW = 16;   // rows per wave

size_t fast_diffuse_lds_bytes(const diffuser_graph& g) {
    const int gpad = (g.num_global + 31) & ~31;
    const size_t chunk = (size_t)g.chunk * kZS * 2 + (size_t)gpad * kZS * 2 +
                         (size_t)kWaves * kRPW * kStage * 6;
    const size_t red = (size_t)(kWaves / 2) * 2 * kNB * 4 * kWave * 4;   // global-row reduction
    return chunk > red ? chunk : red;
}

hipError_t launch_diffuse_fast(const diffuser_graph& g, const attn_shape& s, const void* A,
                               const void* Zk, const void* V, void* Zn, const float* row_scale,
                               float alpha, hipStream_t st) {
    constexpr int RPW = kRPW;
    FastArgs a;
    a.n = g.n;
    a.H = s.H;
    a.num_graphs = g.num_graphs;
    a.radius = g.radius;
    a.g = g.num_global;
    a.causal = g.causal;
    a.rnd_width = g.rnd_width;
    a.chunk = g.chunk;
    a.nchunks = (int32_t)((g.n + g.chunk - 1) / g.chunk);
    a.slot_ptr = g.d_slot_ptr;
    a.slot_off = g.d_slot_off;
    a.G = g.d_global;
    a.rnd = g.d_rnd;
    a.rnd_cnt = g.d_rnd_cnt;
    a.bnd = g.d_bnd;
    a.A = static_cast<const uint16_t*>(A);
    a.Z = static_cast<const uint16_t*>(Zk);
    a.V = static_cast<const uint16_t*>(V);
    a.Zn = static_cast<uint16_t*>(Zn);
    a.row_scale = row_scale;
    a.alpha = alpha;
    a.BH = s.B * s.H;
    a.tiles_per_bh = (int32_t)((g.n + RPW * kWaves - 1) / (RPW * kWaves));
    a.grow_per_bh = (g.num_global + kGrowRows - 1) / kGrowRows;
    a.total_items = a.BH * (a.tiles_per_bh + a.grow_per_bh);
    a.per_xcd = (a.total_items + 7) / 8;
    const size_t lds = fast_diffuse_lds_bytes(g);
    static bool attr_set = false;   // dynamic LDS above 64 KB must be enabled once
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_diffuse_fast<RPW>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           160 * 1024);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    hipLaunchKernelGGL(k_diffuse_fast<RPW>, dim3((unsigned)(8 * a.per_xcd)), dim3(kThreads), lds,
                       st, a);
    return hipGetLastError();
}

}  // namespace diffuser
