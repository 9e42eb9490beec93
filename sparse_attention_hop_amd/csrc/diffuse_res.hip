// Diffusion step on built graphs whose random edges sit in the row segments
// (n up to kMaxResidentN), bf16 storage, head width 32 or 64, with a whole
// channel slice of Z_k resident in LDS:
//   Z_{k+1}[i] = keep * c_i * sum_j A_ij Z_k[j] + restart * V[i]
// ("Diffuser" reading notes, section 2.4, eq. S.7, with keep = 1 - alpha and
// restart = alpha; other coefficients evaluate section 2.3's eq. S.6 in
// nested form; c_i rescales the stored weights of row i to sum to one, or
// is 1).
//
// A workgroup owns one (batch, head) pair, one channel slice of CB
// 16-channel blocks and one piece of the pair's rows. It loads the slice of
// every key row of Z_k into LDS once (one plane of 32-byte rows per channel
// block, a zero row after the last), so the random edges, which may point
// anywhere, read LDS like the window and the global columns, and no key row
// is streamed twice. After that one barrier every wave works alone: it walks
// its own run of 16-row blocks and, for each, sums 32-key products with
// v_mfma_f32_16x16x32_bf16
//   D[channel][row] += Z^T[channel][key] * W^T[key][row]
// where lane (row m, k-group kg) supplies 8 consecutive weight slots:
//  * window band: 32 consecutive keys, 8 slots of the lane's own row;
//  * global columns: 32 global slots at a time;
//  * random edges, in octets: product (octet o, t) takes k-group kg from row
//    4 t + ((kg + o) mod 4), its random edges 8 o .. 8 o + 7, so 4 products
//    cover 8 random edges of each of the block's 16 rows. The block's
//    random weights sit in an octet area (octet o of row m at 16 o + m, 8
//    slots each), so one 16-byte load per lane fetches a batch of 4 octets
//    of all 16 rows with no lane idle: lane (m, kg) takes octet
//    (m - kg) mod 4 of row m, which is exactly its operand in the one
//    product of the batch it serves; in the other 15 it gives zeros. The
//    keys of a batch (16-bit key-row slots) come from the graph's key
//    table, one contiguous kilobyte, 16 bytes per lane, each quad of lanes
//    holding 4 octets that a DPP broadcast hands round.
// Every weight load is a buffer load: a lane whose slots lie outside its
// row's part is given an offset past the buffer and reads zeros, with no
// branch; the step's own offset rides in the scalar offset. The next row
// block's row geometry is loaded while the current one is summed.
// Z^T comes from LDS with ds_read_b64_tr_b16 (each lane reads 4 channels of
// one key row; the read hands every lane one channel of 4 key rows).
// Global rows (full rows of length n) come in blocks of 16 dealt round the
// row pieces; each block is split by key range over waves of its piece,
// whose fp32 partial sums meet in LDS and are added in a fixed order at the
// end.
// Pieces are cut so that their cost (band steps, global-column steps and
// random products per row block, plus the global rows) is even, and so are
// the waves' runs inside a piece. Workgroup ids are numbered so that each
// XCD (id mod 8) takes a contiguous run of pairs, the channel slices of one
// (pair, piece) back to back: their shared weights are then read from HBM
// once and from that XCD's L2 for the other slices.
#include <cmath>
#include <type_traits>

#include "internal.h"
#include "mfma_util.h"

namespace diffuser {
namespace {

constexpr int kWave = 64;
constexpr int kWaves = 16;
constexpr int kThreads = kWave * kWaves;
constexpr int kLdsLimit = 160 * 1024;
constexpr int kGlobItems = 16;     // most partial-sum slots of the global rows (key-part items)
constexpr int kMaxGcolRegs = 2;    // global-column steps whose key rows stay in registers

struct ResArgs {
    int64_t n;
    int32_t n_pad;                 // zero row slot (n rounded up to 32)
    int32_t H, num_graphs, radius, g, causal, nrb;
    int32_t nsl, S;                // channel slices per pair, row pieces per slice
    int32_t items, per_xcd;
    int32_t ngb, ks;               // global row blocks, key parts of each
    int32_t gweight;               // cost of a global-row step in row-block cost units
    int32_t gsteps;                // 32-key steps of a full row
    int32_t plane;                 // LDS bytes of one channel block's plane
    int32_t red_off;               // LDS byte offset of the global rows' partial sums
    int32_t batches;               // key-table batches per row block
    const int64_t* slot_off;       // [graphs + 1]
    const int64_t* seg_ptr;        // [graphs][n + 1]
    const int4* row_info;          // [graphs][n]
    const int32_t* G;              // [g]
    const uint16_t* rkey;          // [graphs][nrb][batches][64][8]
    const int32_t* rb_oct;         // [graphs][nrb]
    const int64_t* rb_roff;        // [graphs][nrb + 1]
    const int64_t* cost;           // [graphs][nrb + 1]
    const uint16_t* A;
    const uint16_t* Z;
    const uint16_t* V;
    uint16_t* Zn;
    const float* row_scale;        // [B*H][n] or null
    float keep, restart;
};

__device__ __forceinline__ uint32_t lds_addr(const char LDS_AS* p) {
    return (uint32_t)(uintptr_t)p;
}

__device__ __forceinline__ i16x4 tr_read(uint32_t addr) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LDS_AS*)(uintptr_t)addr);
}

// Slot of key row k within a plane (res_unit of the graph builder): bit 2
// flipped when bit 3 is set.
__device__ __forceinline__ uint32_t unit_of(uint32_t k) { return k ^ ((k >> 1) & 4u); }

// Z^T operand from the two transposed reads at r1 (keys 8 kg + 0..3) and r2
// (keys 8 kg + 4..7).
__device__ __forceinline__ u32x4 z_op(uint32_t r1, uint32_t r2) {
    const u32x2 l = __builtin_bit_cast(u32x2, tr_read(r1));
    const u32x2 h = __builtin_bit_cast(u32x2, tr_read(r2));
    return u32x4{l[0], l[1], h[0], h[1]};
}

// Every lane of a quad takes the value of quad lane J.
template <int J>
__device__ __forceinline__ uint32_t quad_bcast(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, J * 0x55, 0xf, 0xf, true);
}

__device__ __forceinline__ int32_t uniform_load32i(const int32_t* p) {
    const uint64_t u = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
    return *reinterpret_cast<const __attribute__((address_space(4))) int32_t*>(
        ((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ int64_t uniform_load64i(const int64_t* p) {
    const uint64_t u = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
    return *reinterpret_cast<const __attribute__((address_space(4))) int64_t*>(
        ((uint64_t)hi << 32) | lo);
}

// Smallest row block rb in [0, nrb] with cost[rb] >= c (cost ascending).
__device__ __forceinline__ int32_t first_rb(const int64_t* cost, int32_t nrb, int64_t c) {
    int32_t lo = 0, hi = nrb;
    while (lo < hi) {
        const int32_t mid = (lo + hi) >> 1;
        if (uniform_load64i(cost + mid) < c) lo = mid + 1; else hi = mid;
    }
    return lo;
}

template <int KD, int CB>
__global__ __launch_bounds__(kThreads)
void k_diffuse_res(ResArgs a) {
    extern __shared__ __align__(128) char lds_raw[];
    char LDS_AS* lds = (char LDS_AS*)lds_raw;
    const int lane = __lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int kg = lane >> 4;                 // k-group of the MFMA operands
    const int m = lane & 15;                  // row (W^T) / channel (Z^T) of the lane
    const uint32_t a8 = 8u * (lane & 3), q4 = (lane >> 2) & 3;

    const int32_t item = (int32_t)(blockIdx.x & 7u) * a.per_xcd + (int32_t)(blockIdx.x >> 3);
    if (item >= a.items) return;
    const int32_t slice = item % a.nsl;
    const int32_t piece = (item / a.nsl) % a.S;
    const int32_t bh = item / (a.nsl * a.S);
    const int32_t b = bh / a.H, h = bh - b * a.H;
    const int32_t gr = a.num_graphs == 1 ? 0 : b;
    const int64_t n = a.n;
    const uint16_t* Abh = a.A + a_block_offset(a.slot_off, a.num_graphs, a.H, b, h);
    const uint16_t* Zbh = a.Z + (int64_t)bh * n * KD;
    const int4* info = a.row_info + (int64_t)gr * n;
    const int ch0 = slice * 16 * CB;          // first channel of the slice

    // ---- the slice of every key row into LDS ---------------------------
    // Plane nb (channel block nb of the slice), slot u holds key row
    // unit_of(u), 32 bytes; slots of keys >= n and the zero row n_pad are 0.
    {
        const int32_t per_plane = (a.n_pad + 1) * 2;   // 16-byte pieces of a plane
        const int32_t units = per_plane * CB;
        for (int32_t p0 = 64 * wave; p0 < units; p0 += 64 * kWaves) {
            const int32_t p = p0 + lane;
            const int32_t nb = p / per_plane;
            const int32_t q = p - nb * per_plane;
            const uint32_t k = unit_of((uint32_t)(q >> 1));
            const bool live = p < units && (int64_t)k < n;
            if (live)
                dma16(Zbh + (int64_t)k * KD + ch0 + 16 * nb + 8 * (q & 1), lds + 16 * p0);
            else if (p < units)
                *reinterpret_cast<u32x4 LDS_AS*>(lds + 16 * p) = u32x4{0u, 0u, 0u, 0u};
        }
    }

    // Lane address of piece a8 of plane nb's slot 0.
    uint32_t base[CB];
#pragma unroll
    for (int nb = 0; nb < CB; ++nb) base[nb] = lds_addr(lds) + (uint32_t)(nb * a.plane) + a8;
    // Slots of this lane's key rows within a 32-key step (keys 8 kg + q4 and
    // 8 kg + 4 + q4) as byte offsets.
    const uint32_t U1 = unit_of(8u * kg + q4) << 5, U2 = unit_of(8u * kg + 4u + q4) << 5;
    // Global-column steps: key-row byte offsets held in registers.
    const int ngs = (a.g + 31) >> 5;
    uint32_t gu1[kMaxGcolRegs], gu2[kMaxGcolRegs];
#pragma unroll
    for (int s = 0; s < kMaxGcolRegs; ++s) {
        const int qa = 32 * s + 8 * kg + (int)q4;
        gu1[s] = (qa < a.g ? unit_of((uint32_t)a.G[qa]) : (uint32_t)a.n_pad) << 5;
        gu2[s] = (qa + 4 < a.g ? unit_of((uint32_t)a.G[qa + 4]) : (uint32_t)a.n_pad) << 5;
    }

    // ---- this wave's work ----------------------------------------------
    // Global row block gb belongs to piece gb mod S (npg of them here, each
    // split into ks key parts, one wave per part). Pieces then take runs of
    // regular row blocks so that global plus regular cost is even: piece q
    // starts at the cost boundary B_q = clamp(ctot q / S - gunit G_q) with
    // G_q the global blocks of the pieces before it (kept ascending).
    const int64_t* cost = a.cost + (int64_t)gr * (a.nrb + 1);
    const int64_t creg = uniform_load64i(cost + a.nrb);
    const int32_t npg = a.g > 0 && a.ngb > piece ? (a.ngb - piece + a.S - 1) / a.S : 0;
    const int64_t gunit = (int64_t)a.gsteps * a.gweight;
    const int64_t ctot = (a.g > 0 ? (int64_t)a.ngb * gunit : 0) + creg;
    int64_t ra = 0, rz = creg, bnd = 0, gq = 0;
    for (int32_t q = 0; q <= a.S; ++q) {
        const int64_t bq = q == a.S ? creg : min(max(ctot * q / a.S - gunit * gq, bnd), creg);
        if (q == piece) ra = bq;
        if (q == piece + 1) rz = bq;
        bnd = bq;
        if (a.g > 0 && a.ngb > q) gq += (a.ngb - q + a.S - 1) / a.S;
    }
    // The piece's range of regular cost, split evenly over the waves.
    const int64_t wa = ra + (rz - ra) * wave / kWaves, wz = ra + (rz - ra) * (wave + 1) / kWaves;
    const int32_t rb_begin = first_rb(cost, a.nrb, wa);
    const int32_t rb_end = (piece == a.S - 1 && wave == kWaves - 1) ? a.nrb : first_rb(cost, a.nrb, wz);

    const int64_t pair_slots = a.num_graphs == 1 ? a.slot_off[1] : a.slot_off[gr + 1] - a.slot_off[gr];
    const __amdgpu_buffer_rsrc_t rA = buffer_rsrc(Abh, (uint32_t)(2 * pair_slots));
    const uint16_t* rk = a.rkey + (int64_t)gr * a.nrb * a.batches * 512;
    const __amdgpu_buffer_rsrc_t rK = buffer_rsrc(rk, (uint32_t)(a.nrb * a.batches * 1024));
    const int32_t* oct = a.rb_oct + (int64_t)gr * a.nrb;
    const int64_t* roffs = a.rb_roff + (int64_t)gr * (a.nrb + 1);
    const int64_t rand_base = a.seg_ptr[(int64_t)gr * (n + 1) + n];   // random area's first slot

    full_barrier();   // the slice is in LDS

    // Global rows: item `wave` = (this piece's global row block wave / ks,
    // key part wave % ks).
    const bool grows = npg > 0;
    if (grows && wave < npg * a.ks) {
        const int gb = piece + (wave / a.ks) * a.S, part = wave % a.ks;
        const int q = 16 * gb + m;
        uint32_t wv = kOutside;   // lane offset of its row's slots 8 kg ..
        int32_t wlen = 0;
        if (q < a.g) {
            const int64_t i = a.G[q];
            const int64_t* sp = a.seg_ptr + (int64_t)gr * (n + 1);
            wv = (uint32_t)(2 * (info[i].x + 8 * kg));
            wlen = (int32_t)(sp[i + 1] - sp[i]);
        }
        f32x4 acc[CB];
#pragma unroll
        for (int nb = 0; nb < CB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int s0 = a.gsteps * part / a.ks, s1 = a.gsteps * (part + 1) / a.ks;
        // Steps in batches of kGB, the next batch's weights loaded before the
        // current batch's products.
        constexpr int kGB = 8;
        u32x4 wa[kGB], wb[kGB];
        auto fetch = [&](u32x4 (&w)[kGB], int sb) {
#pragma unroll
            for (int t = 0; t < kGB; ++t) {
                const bool ok = 32 * (sb + t) + 8 * kg < wlen && sb + t < s1;
                w[t] = bload16(rA, ok ? wv : kOutside, (uint32_t)(64 * (sb + t)));
            }
        };
        auto mult = [&](const u32x4 (&w)[kGB], int sb) {
#pragma unroll
            for (int t = 0; t < kGB; ++t) {
                if (sb + t < s1) {
                    const uint32_t kb = (uint32_t)(32 * (sb + t)) << 5;
#pragma unroll
                    for (int nb = 0; nb < CB; ++nb)
                        acc[nb] = mfma_bf16(z_op(base[nb] + kb + U1, base[nb] + kb + U2), w[t],
                                            acc[nb]);
                }
            }
        };
        fetch(wa, s0);
        for (int sb = s0; sb < s1; sb += 2 * kGB) {
            fetch(wb, sb + kGB);
            mult(wa, sb);
            if (sb + kGB >= s1) break;
            fetch(wa, sb + 2 * kGB);
            mult(wb, sb + kGB);
        }
        float LDS_AS* red = (float LDS_AS*)(lds + a.red_off);
#pragma unroll
        for (int nb = 0; nb < CB; ++nb)
#pragma unroll
            for (int e = 0; e < 4; ++e) red[((wave * CB + nb) * 4 + e) * kWave + lane] = acc[nb][e];
    }

    // Random batches: this lane serves product (octet 4 b + jstar, tstar) of
    // every batch b, with octet jstar of its own row m.
    const uint32_t jstar = (uint32_t)(m - kg) & 3u, pstar = 4u * jstar + (uint32_t)(m >> 2);
    const uint32_t wv_lane = (jstar * 16u + (uint32_t)m) * 16u;   // bytes into a batch
    const uint32_t kv_lane = 16u * (uint32_t)lane;

    // Regular row blocks, software-pipelined: the loads of block rb + 1
    // are issued as soon as the registers they land in are free (its band
    // and global-column weights after rb's band products, its random
    // batches after rb's random products, its restart inputs after rb's
    // store), so each group of loads has a phase of other work to arrive
    // in. The row geometry runs two blocks ahead. Every load is issued
    // unconditionally, past the end of its buffer where there is nothing to
    // fetch, so the loads retire in a fixed order.
    constexpr int kMaxBand = 5;   // band steps whose weights are fetched up front
    const __amdgpu_buffer_rsrc_t rI = buffer_rsrc(info, (uint32_t)(16 * n));
    auto info_at = [&](int32_t rb) -> int4 {
        const int64_t i = (int64_t)rb * kRowBlock + m;
        const u32x4 v = bload16(rI, i < n ? (uint32_t)(16 * i) : kOutside, 0u);
        return make_int4((int32_t)v[0], (int32_t)v[1], (int32_t)v[2], (int32_t)v[3]);
    };
    // Geometry of row block rb (rb >= rb_end: an empty block).
    struct Geo {
        int64_t r0, band_lo;
        int32_t nbs, noct, nbat;
        uint32_t wsoff, ksoff;
        int32_t riz, riw, dlane;
        uint32_t vband, vglob;
        bool rok;
    };
    auto geo = [&](int32_t rb, const int4& ri) -> Geo {
        Geo G;
        const bool live = rb < rb_end;
        G.r0 = (int64_t)rb * kRowBlock;
        const int64_t i = G.r0 + m;
        G.rok = live && i < n && ri.z >= 0;
        G.riz = G.rok ? ri.z : 0;
        G.riw = G.rok ? ri.w : 0;
        const int64_t last = min(G.r0 + kRowBlock - 1, n - 1);
        G.band_lo = (G.r0 - a.radius < 0 ? 0 : G.r0 - a.radius) & ~31ll;
        const int64_t band_hi = a.causal ? last : min(n - 1, last + a.radius);
        G.nbs = G.band_lo <= band_hi ? (int)((band_hi - G.band_lo) >> 5) + 1 : 0;
        G.dlane = (int32_t)G.band_lo + 8 * kg - ri.y;
        G.vband = (uint32_t)(2 * (ri.x + 8 * kg - ri.y));
        G.vglob = (uint32_t)(2 * (ri.x + ri.z + 8 * kg));
        const int32_t rbc = rb < a.nrb ? rb : a.nrb - 1;
        G.noct = live ? uniform_load32i(oct + rbc) : 0;
        G.nbat = (G.noct + kOctBatch - 1) / kOctBatch;
        G.wsoff = (uint32_t)(2 * (rand_base + 8 * kRowBlock * uniform_load64i(roffs + rbc)));
        G.ksoff = (uint32_t)rbc * (uint32_t)a.batches * 1024u;
        return G;
    };
    u32x4 bw[kMaxBand], gw[kMaxGcolRegs];
    auto issue_band = [&](const Geo& G) {
#pragma unroll
        for (int t = 0; t < kMaxBand; ++t) {
            const bool ok = (uint32_t)(G.dlane + 32 * t) < (uint32_t)G.riz && t < G.nbs;
            bw[t] = bload16(rA, ok ? G.vband : kOutside, (uint32_t)(2 * (G.band_lo + 32 * t)));
        }
#pragma unroll
        for (int s = 0; s < kMaxGcolRegs; ++s) {
            const bool ok = 32 * s + 8 * kg < G.riw && s < ngs;
            gw[s] = bload16(rA, ok ? G.vglob : kOutside, (uint32_t)(64 * s));
        }
    };
    u32x4 w0, w1, k0, k1;
    auto rload = [&](const Geo& G, u32x4& w, u32x4& kk, int b) {
        w = bload16(rA, (int32_t)(4 * b + (int32_t)jstar) < G.noct ? wv_lane : kOutside,
                    G.wsoff + 1024u * (uint32_t)b);
        kk = bload16(rK, b < G.nbat ? kv_lane : kOutside, G.ksoff + 1024u * (uint32_t)b);
    };
    auto issue_rand = [&](const Geo& G) {
        rload(G, w0, k0, 0);
        rload(G, w1, k1, 1);
    };
    u32x2 vin[CB];
    float cs = 1.0f;
    auto issue_v = [&](const Geo& G) {
        const int64_t i = G.r0 + m;
        const int64_t ic = i < n ? i : n - 1;
#pragma unroll
        for (int nb = 0; nb < CB; ++nb)
            vin[nb] = *reinterpret_cast<const u32x2*>(a.V + ((int64_t)bh * n + ic) * KD + ch0 +
                                                      16 * nb + 4 * kg);
        cs = a.row_scale != nullptr ? a.row_scale[(int64_t)bh * n + ic] : 1.0f;
    };

    int4 ri_next = info_at(rb_begin + 1);
    Geo G = geo(rb_begin, info_at(rb_begin));
    issue_band(G);
    issue_rand(G);
    issue_v(G);
    for (int32_t rb = rb_begin; rb < rb_end; ++rb) {
        const Geo Gn = geo(rb + 1, ri_next);
        ri_next = info_at(rb + 2);

        f32x4 acc[CB];
#pragma unroll
        for (int nb = 0; nb < CB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
        // Window band (32-key steps from band_lo) and global columns.
#pragma unroll
        for (int t = 0; t < kMaxBand; ++t) {
            if (t < G.nbs) {
                const uint32_t kb = (uint32_t)(G.band_lo + 32 * t) << 5;
#pragma unroll
                for (int nb = 0; nb < CB; ++nb)
                    acc[nb] = mfma_bf16(z_op(base[nb] + kb + U1, base[nb] + kb + U2), bw[t], acc[nb]);
            }
        }
        for (int t = kMaxBand; t < G.nbs; ++t) {
            const bool ok = (uint32_t)(G.dlane + 32 * t) < (uint32_t)G.riz;
            const u32x4 w = bload16(rA, ok ? G.vband : kOutside, (uint32_t)(2 * (G.band_lo + 32 * t)));
            const uint32_t kb = (uint32_t)(G.band_lo + 32 * t) << 5;
#pragma unroll
            for (int nb = 0; nb < CB; ++nb)
                acc[nb] = mfma_bf16(z_op(base[nb] + kb + U1, base[nb] + kb + U2), w, acc[nb]);
        }
#pragma unroll
        for (int s = 0; s < kMaxGcolRegs; ++s) {
            if (s < ngs) {
#pragma unroll
                for (int nb = 0; nb < CB; ++nb)
                    acc[nb] = mfma_bf16(z_op(base[nb] + gu1[s], base[nb] + gu2[s]), gw[s], acc[nb]);
            }
        }
        for (int s = kMaxGcolRegs; s < ngs; ++s) {
            const bool ok = 32 * s + 8 * kg < G.riw;
            const u32x4 w = bload16(rA, ok ? G.vglob : kOutside, (uint32_t)(64 * s));
            const int qa = 32 * s + 8 * kg + (int)q4;
            const uint32_t u1 = (qa < a.g ? unit_of((uint32_t)a.G[qa]) : (uint32_t)a.n_pad) << 5;
            const uint32_t u2 =
                (qa + 4 < a.g ? unit_of((uint32_t)a.G[qa + 4]) : (uint32_t)a.n_pad) << 5;
#pragma unroll
            for (int nb = 0; nb < CB; ++nb)
                acc[nb] = mfma_bf16(z_op(base[nb] + u1, base[nb] + u2), w, acc[nb]);
        }
        issue_band(Gn);

        // Random batches. Octet ob + J of a batch: quad lane J's keys for
        // every lane of the quad, then its 4 products.
        // ko: the lane's 8 key-row slots of the batch as byte offsets in a
        // plane (entry 2t + h of word t's half h); the products of octet J
        // take quad lane J's, each added to the plane base in one
        // broadcast add.
        auto octet = [&](const u32x4& w, const uint32_t (&ko)[8], auto jc, int ob) {
            constexpr int J = decltype(jc)::value;
            if (ob + J >= G.noct) return;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const uint32_t o1 = quad_bcast<J>(ko[2 * t]), o2 = quad_bcast<J>(ko[2 * t + 1]);
                const bool mine = pstar == (uint32_t)(4 * J + t);
                const u32x4 wt = u32x4{mine ? w[0] : 0u, mine ? w[1] : 0u, mine ? w[2] : 0u,
                                       mine ? w[3] : 0u};
#pragma unroll
                for (int nb = 0; nb < CB; ++nb)
                    acc[nb] = mfma_bf16(z_op(base[nb] + o1, base[nb] + o2), wt, acc[nb]);
            }
        };
        auto rbatch = [&](const u32x4& w, const u32x4& kk, int b) {
            const int ob = kOctBatch * b;
            uint32_t ko[8];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                ko[2 * t] = (kk[t] & 0xffffu) << 5;
                ko[2 * t + 1] = (kk[t] >> 16) << 5;
            }
            octet(w, ko, std::integral_constant<int, 0>{}, ob);
            octet(w, ko, std::integral_constant<int, 1>{}, ob);
            octet(w, ko, std::integral_constant<int, 2>{}, ob);
            octet(w, ko, std::integral_constant<int, 3>{}, ob);
        };
        rbatch(w0, k0, 0);
        rbatch(w1, k1, 1);
        // Blocks with more than 2 batches: the rest, each loaded on the spot.
        for (int b = 2; b < G.nbat; ++b) {
            u32x4 w, kk;
            rload(G, w, kk, b);
            rbatch(w, kk, b);
        }
        issue_rand(Gn);

        // Restart and store: lane (m, kg) holds channels 4 kg .. + 3 of each
        // channel block for row r0 + m.
        if (G.rok) {
            const float keep = a.keep * cs;
            uint16_t* out = a.Zn + ((int64_t)bh * n + G.r0 + m) * KD + ch0 + 4 * kg;
#pragma unroll
            for (int nb = 0; nb < CB; ++nb) {
                u32x2 o;
                o[0] = to_bf16_pair(keep * acc[nb][0] + a.restart * bf16_lo(vin[nb][0]),
                                    keep * acc[nb][1] + a.restart * bf16_hi(vin[nb][0]));
                o[1] = to_bf16_pair(keep * acc[nb][2] + a.restart * bf16_lo(vin[nb][1]),
                                    keep * acc[nb][3] + a.restart * bf16_hi(vin[nb][1]));
                *reinterpret_cast<u32x2*>(out + 16 * nb) = o;
            }
        }
        issue_v(Gn);
        G = Gn;
    }

    // Global rows: fixed-order sum of each block's key parts, restart, store.
    if (grows) {
        __syncthreads();
        const float LDS_AS* red = (const float LDS_AS*)(lds + a.red_off);
        const int per = CB * 4 * kWave;   // partial sums of one item
        for (int idx = threadIdx.x; idx < npg * per; idx += kThreads) {
            const int lg = idx / per, r = idx - lg * per;
            const int l = r & 63, e = (r >> 6) & 3, nb = r >> 8;
            const int q = 16 * (piece + lg * a.S) + (l & 15);
            if (q >= a.g) continue;
            float sum = 0.0f;
            for (int part = 0; part < a.ks; ++part) sum += red[(lg * a.ks + part) * per + r];
            const int64_t i = a.G[q];
            const int ch = ch0 + 16 * nb + 4 * (l >> 4) + e;
            const int64_t o = ((int64_t)bh * n + i) * KD + ch;
            const float keep = a.row_scale ? a.keep * a.row_scale[(int64_t)bh * n + i] : a.keep;
            a.Zn[o] = (uint16_t)f32_to_bf16(keep * sum + a.restart * bf16_to_f32(a.V[o]));
        }
    }
}

// Channel blocks held per workgroup for head width d and n keys: the most
// (at most two: more would leave too few registers for the loads in
// flight) whose planes fit beside the global rows' partial sums, or 0 when
// none does.
struct ResPlan {
    int cb, ngb, gslots, lds, plane, red_off;
};

ResPlan res_plan(const diffuser_graph& g, int d) {
    ResPlan p{0, 0, 0, 0, 0, 0};
    const int64_t npad = res_npad(g.n);
    const int ngb = (g.num_global + 15) / 16;
    if (ngb > kGlobItems) return p;
    const int64_t plane = (npad + 1) * 32;   // the loader packs the planes back to back
    for (int cb = d / 16 > 2 ? 2 : d / 16; cb >= 1; cb >>= 1) {
        // Partial-sum slots for the global rows' key parts: kGlobItems, or
        // half as many (down to one per global row block) when that lets
        // the planes fit.
        for (int slots = kGlobItems; slots >= ngb && slots >= 1; slots >>= 1) {
            const int64_t red = g.num_global > 0 ? (int64_t)slots * cb * 4 * kWave * 4 : 0;
            if (plane * cb + red <= kLdsLimit) {
                p.cb = cb;
                p.ngb = ngb;
                p.gslots = g.num_global > 0 ? slots : 0;
                p.plane = (int)plane;
                p.red_off = (int)(plane * cb);
                p.lds = (int)(plane * cb + red);
                return p;
            }
            if (g.num_global == 0) break;
        }
    }
    return p;
}

int device_cus(int device) {
    static int cached_dev = -1, cached_cus = 0;
    if (cached_dev != device) {
        hipDeviceProp_t prop;
        cached_cus = hipGetDeviceProperties(&prop, device) == hipSuccess ? prop.multiProcessorCount
                                                                          : 256;
        cached_dev = device;
    }
    return cached_cus > 0 ? cached_cus : 256;
}

template <int KD, int CB>
hipError_t launch_kernel(const ResArgs& a, int lds, int device, hipStream_t st) {
    static int attr_device = -1;
    const void* kern = reinterpret_cast<const void*>(&k_diffuse_res<KD, CB>);
    if (attr_device != device) {
        hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           kLdsLimit);
        if (e != hipSuccess) return e;
        attr_device = device;
    }
    hipLaunchKernelGGL((k_diffuse_res<KD, CB>), dim3((unsigned)(8 * a.per_xcd)), dim3(kThreads),
                       (size_t)lds, st, a);
    return hipGetLastError();
}

}  // namespace

bool res_diffuse_supported(const diffuser_graph& g, const attn_shape& s) {
    if (!g.structured || !g.octet() || g.d_rkey == nullptr || g.d_rb_cost == nullptr ||
        s.dtype != DIFFUSER_BF16 || (s.d != 64 && s.d != 32))
        return false;
    for (int64_t x : g.slots)
        if (2 * x >= (1ll << 31)) return false;
    const int64_t nrb = (g.n + kRowBlock - 1) / kRowBlock;
    if (nrb * g.key_batches * 1024 >= (1ll << 31)) return false;
    return res_plan(g, s.d).cb > 0;
}

hipError_t launch_diffuse_res(const diffuser_graph& g, const attn_shape& s, const void* A,
                              const void* Zk, const void* V, void* Zn, const float* row_scale,
                              step_coefs kc, hipStream_t st) {
    const ResPlan p = res_plan(g, s.d);
    ResArgs a;
    a.n = g.n;
    a.n_pad = (int32_t)res_npad(g.n);
    a.H = s.H;
    a.num_graphs = g.num_graphs;
    a.radius = g.radius;
    a.g = g.num_global;
    a.causal = g.causal;
    a.nrb = (int32_t)((g.n + kRowBlock - 1) / kRowBlock);
    a.nsl = s.d / 16 / p.cb;
    a.ngb = p.ngb;
    a.gweight = 2;
    a.gsteps = (int32_t)(res_npad(g.n) / 32);
    a.plane = p.plane;
    a.red_off = p.red_off;
    a.batches = g.key_batches;
    // Row pieces per (pair, slice): the S in 1..8 that minimises the
    // estimated time, rounds of workgroups (one per CU) times each
    // workgroup's time, a fixed part (the slice load and its barrier, worth
    // about kFixedBlocks row blocks of one wave) plus the row blocks of its
    // busiest wave.
    constexpr int64_t kFixedBlocks = 4;
    const int64_t units = (int64_t)s.B * s.H * a.nsl;
    const int64_t cus = device_cus(g.device);
    int best = 1;
    int64_t best_cost = -1;
    for (int S = 1; S <= 8; ++S) {
        if (S > 1 && (int64_t)a.nrb < 16ll * S) break;
        const int64_t rounds = (units * S + cus - 1) / cus;
        const int64_t per_wave = ((a.nrb + S - 1) / S + kWaves - 1) / kWaves;
        const int64_t cost = rounds * (kFixedBlocks + per_wave);
        if (best_cost < 0 || cost < best_cost) {
            best_cost = cost;
            best = S;
        }
    }
    a.S = best;
    // Key parts per global row block: a piece holds at most ceil(ngb / S)
    // blocks, all of whose parts fit in the plan's partial-sum slots.
    a.ks = p.ngb > 0 ? p.gslots / ((p.ngb + a.S - 1) / a.S) : 0;
    a.items = (int32_t)(units * a.S);
    a.per_xcd = (a.items + 7) / 8;
    a.slot_off = g.d_slot_off;
    a.seg_ptr = g.d_seg_ptr;
    a.row_info = reinterpret_cast<const int4*>(g.d_row_info);
    a.G = g.d_global;
    a.rkey = g.d_rkey;
    a.rb_oct = g.d_rb_oct;
    a.rb_roff = g.d_rb_roff;
    a.cost = g.d_rb_cost;
    a.A = static_cast<const uint16_t*>(A);
    a.Z = static_cast<const uint16_t*>(Zk);
    a.V = static_cast<const uint16_t*>(V);
    a.Zn = static_cast<uint16_t*>(Zn);
    a.row_scale = row_scale;
    a.keep = kc.keep;
    a.restart = kc.restart;
    if (s.d == 64) {
        if (p.cb == 2) return launch_kernel<64, 2>(a, p.lds, g.device, st);
        return launch_kernel<64, 1>(a, p.lds, g.device, st);
    }
    if (p.cb == 2) return launch_kernel<32, 2>(a, p.lds, g.device, st);
    return launch_kernel<32, 1>(a, p.lds, g.device, st);
}

}  // namespace diffuser
