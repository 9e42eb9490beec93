// Diffusion step on scheduled graphs, bf16 storage, head width 64:
//   Z_{k+1}[i] = keep * c_i * sum_j A_ij Z_k[j] + restart * V[i]
// ("Diffuser" reading notes, section 2.4, eq. S.7, with keep = 1 - alpha and
// restart = alpha; other coefficients evaluate section 2.3's eq. S.6 in
// nested form; c_i rescales the stored weights of row i to sum to one, or
// is 1).
//
// Every part of the sum is a v_mfma_f32_16x16x32_bf16 product
//   D[channel][row] += Z^T[channel][key] * W^T[key][row]
// over 16 rows, 16 channels and 32 keys. The Z^T operand comes from LDS
// with ds_read_b64_tr_b16 (each lane reads 4 channels of one key row; the
// read hands every lane one channel of 4 key rows); the W^T operand is 8
// consecutive weight slots of one row, one 16-byte load.
//  * window edges: the 32 keys are consecutive columns of the band;
//  * global columns: 32 global slots at a time, in the chunk that holds the
//    globals' key rows (a slot whose global lies in another chunk reads the
//    zero row instead);
//  * random edges: the 32 keys are the slots of one schedule group, whose
//    key rows lie in the current chunk; the weight operand keeps a pair's
//    two weights in the lanes of the pair's row and zeroes them elsewhere.
// A workgroup (16 waves, 16 rows each) streams Z_k of its (batch, head)
// through LDS in chunks of kChunkRows rows, double-buffered with direct
// global-to-LDS loads of the next chunk while the current one is used; each
// wave's schedule groups of the next chunk travel the same way into a
// double-buffered staging area of its own. The weights of the wave's dense
// steps (band and global columns) are loaded once, with the first chunk, and
// used in the chunk that holds their key rows; during the last chunk the
// tile's rows of V (and c_i) travel into the idle buffer for the restart
// term. Rows
// of Z_k sit in LDS at 128 bytes, quarters permuted by key_row_code, which
// spreads the 16 rows of one transposed read over the banks.
// Global rows get workgroups of their own (32 rows; the 16 waves split each
// chunk's keys and add their partial sums in a fixed order at the end).
// Workgroups are numbered so that each XCD (workgroup id mod 8) works
// through a contiguous range of (batch, head) pairs.
#include "internal.h"
#include "mfma_util.h"

namespace diffuser {
namespace {

constexpr int kWave = 64;
constexpr int kWaves = 16;
constexpr int kThreads = kWave * kWaves;
// Head width KD (a template parameter) is 64 or 32: KD / 16 channel blocks;
// a Z row sits in a 128-byte LDS slot either way.
constexpr int kRowBytes = 128;                        // LDS slot of one Z row
constexpr int kBufBytes = (kChunkRows + 1) * kRowBytes;  // chunk + zero row
constexpr int kTileRows = kWaves * kRowBlock;         // rows per row-tile workgroup
constexpr int kGrowRows = 32;                         // global rows per workgroup
// Per-wave staging of one chunk's first kStageGroups schedule groups:
// weights [group][64 B], key-row codes [group][64 B], pair rows [group][16 B].
constexpr int kStageGroups = 6;
constexpr int kStageJ = kStageGroups * 64;
constexpr int kStageR = 2 * kStageGroups * 64;
constexpr int kStageBytes = kStageR + kStageGroups * 16;
constexpr int kMaxBand = 5;                           // band steps per chunk held in registers
constexpr int kMaxGlob = 2;                           // global steps per chunk held in registers
constexpr int kLdsBytes = 2 * kBufBytes + kWaves * 2 * kStageBytes;
static_assert(kLdsBytes <= 160 * 1024, "LDS budget");

static_assert(kWaves * 2 * 4 * 4 * kWave * 4 <= 2 * kBufBytes, "grow partial sums fit");

struct FastArgs {
    int64_t n;
    int32_t H, num_graphs, radius, g, causal, nchunks, nrb;
    const int64_t* slot_off;    // [graphs + 1]
    const int64_t* seg_ptr;     // [graphs][n + 1]
    const int4* row_info;       // [graphs][n]
    const int32_t* G;           // [g]
    const int32_t* gchunk;      // [nchunks + 1] globals below each chunk start
    const int64_t* grp_ptr;     // [graphs][nrb + 1]
    const int64_t* grp_off;     // [graphs + 1]
    const int32_t* grp_cptr;    // [graphs][nrb][nchunks + 1]
    const uint32_t* sched_row;  // [groups][4]
    const uint32_t* sched_j;    // [groups][16]
    const uint16_t* A;
    const uint16_t* Z;
    const uint16_t* V;
    uint16_t* Zn;
    const float* row_scale;     // [B*H][n] or null
    float keep, restart;
    int32_t tiles_per_bh, grow_per_bh, per_xcd, total_items, bh_per_xcd;
};

__device__ __forceinline__ uint32_t lds_addr(const char LDS_AS* p) {
    return (uint32_t)(uintptr_t)p;
}

__device__ __forceinline__ i16x4 tr_read(uint32_t addr) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LDS_AS*)(uintptr_t)addr);
}

// LDS address of the 8 bytes lane `a4` reads from the key row with
// key_row_code `code` of the buffer at `base` (128-byte aligned), for
// channel block 0; XOR with nb << 5 selects channel block nb (the XOR only
// touches address bits 5 and 6, which neither the base nor 8 a4 sets).
__device__ __forceinline__ uint32_t code_addr(uint32_t base_a4, uint32_t code) {
    return base_a4 + (code << 5);
}

// Z^T operand of channel block nb: key rows at addresses r1 (k = 8 kg +
// 0..3) and r2 (k = 8 kg + 4..7).
__device__ __forceinline__ bf16x8 z_operand(uint32_t r1, uint32_t r2, int nb) {
    const i16x4 lo = tr_read(r1 ^ ((uint32_t)nb << 5));
    const i16x4 hi = tr_read(r2 ^ ((uint32_t)nb << 5));
    const u32x2 l = __builtin_bit_cast(u32x2, lo), h = __builtin_bit_cast(u32x2, hi);
    return __builtin_bit_cast(bf16x8, u32x4{l[0], l[1], h[0], h[1]});
}

__device__ __forceinline__ f32x4 mfma(const bf16x8& a, const u32x4& b, const f32x4& c) {
    return mfma_bf16(__builtin_bit_cast(u32x4, a), b, c);
}

// acc[nb] += Z^T(r1, r2) W^T for the four channel blocks.
template <int NB>
__device__ __forceinline__ void mfma4(f32x4 (&acc)[NB], uint32_t r1, uint32_t r2,
                                      const u32x4& w) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[nb] = mfma(z_operand(r1, r2, nb), w, acc[nb]);
}

// Per-lane byte offsets, within a chunk of Z_k rows (2 KD bytes each), of
// the 16 bytes each of this lane's four direct loads fetches: in LDS block
// 4 w + j (8 row slots, 1 KB) lane l writes 16-byte unit l % 8 of slot l / 8,
// which holds the row's logical unit (l % 8) ^ (2 sw), sw the row's quarter
// swizzle; units past the row (KD = 32: logical units 4..7) are not loaded
// (bit j of `live` clear).
struct ChunkLanes {
    uint32_t off[4];
    uint32_t live;
};

template <int KD>
__device__ __forceinline__ ChunkLanes chunk_lanes(int wave, int lane) {
    ChunkLanes cl;
    cl.live = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t pr = (uint32_t)((4 * wave + j) * 8 + (lane >> 3));
        const uint32_t lu = (uint32_t)(lane & 7) ^ ((key_row_code(pr) & 3u) << 1);
        const bool live = lu < (uint32_t)(KD / 8);
        cl.off[j] = live ? pr * (2 * KD) + lu * 16 : 0u;
        cl.live |= (live ? 1u : 0u) << j;
    }
    return cl;
}

// Direct loads of chunk rows [c0, c0 + kChunkRows) of Z_k into `buf`. Rows
// at or beyond n repeat row n - 1 (their weights are zero).
template <int KD>
__device__ __forceinline__ void dma_chunk(char LDS_AS* buf, const uint16_t* Zbh, int64_t n,
                                          int64_t c0, const ChunkLanes& cl, int wave) {
    constexpr uint32_t kRB = 2 * KD;   // bytes of a Z row in memory
    const char* src = reinterpret_cast<const char*>(Zbh + c0 * KD);
    if (c0 + kChunkRows <= n) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (KD == 64 || ((cl.live >> j) & 1u)) dma16(src + cl.off[j], buf + (4 * wave + j) * 1024);
    } else {
        const uint32_t last = (uint32_t)(n - 1 - c0) * kRB;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t o = cl.off[j] < last + kRB ? cl.off[j] : last | (cl.off[j] & (kRB - 1));
            if (KD == 64 || ((cl.live >> j) & 1u)) dma16(src + o, buf + (4 * wave + j) * 1024);
        }
    }
}

// Direct loads of the rows r0 .. r0 + 15 of V (a wave's restart inputs)
// into `vbuf`, row j at vbuf + 2 KD j in order; rows at or beyond n repeat
// row n - 1.
template <int KD>
__device__ __forceinline__ void dma_restart(const FastArgs& a, int32_t bh, int64_t r0,
                                            char LDS_AS* vbuf, int lane) {
    constexpr int kUnits = KD / 8;             // 16-byte units of a row
    constexpr int kRowsPer = kWave / kUnits;   // rows per load instruction
#pragma unroll
    for (int u = 0; u < 16 / kRowsPer; ++u) {
        const int64_t row = min(r0 + kRowsPer * u + lane / kUnits, a.n - 1);
        dma16(a.V + ((int64_t)bh * a.n + row) * KD + 8 * (lane % kUnits), vbuf + 1024 * u);
    }
}

// Restart and store of one lane's accumulators: row `i` (row j of the
// wave's staged restart inputs), channels 16 nb + 4 kg .. + 3 for
// nb < KD / 16.
template <int KD>
__device__ __forceinline__ void store_row(const FastArgs& a, int32_t bh, int64_t i, int j, int kg,
                                          const f32x4 (&acc)[KD / 16], const char LDS_AS* vbuf,
                                          float scale) {
    const float keep = a.keep * scale;
    const int64_t base = ((int64_t)bh * a.n + i) * KD + 4 * kg;
#pragma unroll
    for (int nb = 0; nb < KD / 16; ++nb) {
        const u32x2 v = *reinterpret_cast<const u32x2 LDS_AS*>(vbuf + 2 * KD * j +
                                                             2 * (16 * nb + 4 * kg));
        u32x2 o;
        o[0] = to_bf16_pair(keep * acc[nb][0] + a.restart * bf16_lo(v[0]),
                            keep * acc[nb][1] + a.restart * bf16_hi(v[0]));
        o[1] = to_bf16_pair(keep * acc[nb][2] + a.restart * bf16_lo(v[1]),
                            keep * acc[nb][3] + a.restart * bf16_hi(v[1]));
        *reinterpret_cast<u32x2*>(a.Zn + base + 16 * nb) = o;
    }
}

// Per-lane state of a row-tile wave.
struct TileLane {
    int kg, s16;
    uint32_t a8, q4;         // 8 (lane % 4) and the transposed-read source row
    int4 ri;                 // row info of row r0w + s16
    bool rok;
    int64_t r0w, band_lo, band_hi;
    const int32_t* cptr;     // chunk -> first group of this row block
    int64_t goff, rbase;
    int nbs;                 // band steps (32 columns each from band_lo)
    u32x4 bw[kMaxBand];      // weights of the first kMaxBand band steps
    int ngs;                 // global steps (32 global slots each)
    u32x4 gw[kMaxGlob];      // weights of the first kMaxGlob global steps
    int32_t gv1[kMaxGlob], gv2[kMaxGlob];   // their globals read by this lane (-1: none)
};

// Weights of the band step at key column kc (8 slots of this lane's row).
__device__ __forceinline__ u32x4 band_weights(const TileLane& t, const uint16_t* Abh, int64_t kc) {
    const int32_t off = (int32_t)(kc + 8 * t.kg) - t.ri.y;
    u32x4 w = {0u, 0u, 0u, 0u};
    if (t.rok && off >= 0 && off < t.ri.z) w = load16(Abh + t.ri.x + off);
    return w;
}

// Weights of global step s (global slots 32 s + 8 kg .. + 7 of this lane's row).
__device__ __forceinline__ u32x4 glob_weights(const TileLane& t, const uint16_t* Abh, int s) {
    const int32_t off = 32 * s + 8 * t.kg;
    u32x4 w = {0u, 0u, 0u, 0u};
    if (t.rok && off < t.ri.w) w = load16(Abh + t.ri.x + t.ri.z + off);
    return w;
}

// Key row, within chunk c0, of global slot q when that global lies in
// [q0, q1) (the chunk's globals), else the zero row.
__device__ __forceinline__ uint32_t glob_row(const FastArgs& a, int q, int q0, int q1,
                                             int64_t c0) {
    return (q >= q0 && q < q1) ? (uint32_t)(a.G[q] - c0) : kZeroRow;
}

// Direct loads of chunk c's first kStageGroups schedule groups (weights,
// key-row codes, pair rows) into the staging area `stg`.
__device__ __forceinline__ void dma_groups(const TileLane& t, const FastArgs& a,
                                           const uint16_t* Abh, char LDS_AS* stg, int c, int lane) {
    const int32_t g0 = uniform_load(t.cptr + c);
    const int32_t cnt = min(uniform_load(t.cptr + c + 1) - g0, kStageGroups);
    const uint32_t l16 = 16u * (uint32_t)lane;
    if (lane < 4 * cnt) {
        dma16(reinterpret_cast<const char*>(Abh + t.rbase + (int64_t)kGroupSlots * g0) + l16, stg);
        dma16(reinterpret_cast<const char*>(a.sched_j + (t.goff + g0) * 16) + l16, stg + kStageJ);
    }
    if (lane < cnt)
        dma16(reinterpret_cast<const char*>(a.sched_row + (t.goff + g0) * 4) + l16, stg + kStageR);
}

// One schedule group as this lane uses it: the 8 weights of its k-group,
// the key-row codes of its two transposed reads, the rows of its 4 pairs.
struct GroupLane {
    u32x4 w;
    uint32_t j, r;
};

__device__ __forceinline__ GroupLane group_lane(const TileLane& t, const FastArgs& a,
                                                const uint16_t* Abh, const char LDS_AS* stg,
                                                int32_t g0, int k) {
    GroupLane gl;
    if (k < kStageGroups) {
        gl.w = *reinterpret_cast<const u32x4 LDS_AS*>(stg + 64 * k + 16 * t.kg);
        gl.j = *reinterpret_cast<const uint32_t LDS_AS*>(stg + kStageJ + 64 * k +
                                                         4 * (4 * t.kg + t.q4));
        gl.r = *reinterpret_cast<const uint32_t LDS_AS*>(stg + kStageR + 16 * k + 4 * t.kg);
    } else {
        const int64_t gi = g0 + k;
        gl.w = load16(Abh + t.rbase + (int64_t)kGroupSlots * gi + 8 * t.kg);
        gl.j = a.sched_j[(t.goff + gi) * 16 + 4 * t.kg + t.q4];
        gl.r = a.sched_row[(t.goff + gi) * 4 + t.kg];
    }
    return gl;
}

// One key chunk of a row-tile wave, with chunk c's Z_k rows in `cur` and its
// staged groups in `stg`: loads the weights of the chunk's dense steps,
// starts the direct loads of chunk c + 1 (rows into `nxt`, groups into
// `nstg`), multiplies the random groups, then the dense steps. The LDS
// regions are disjoint, which lets the reads of `cur` and `stg` run while
// the loads into `nxt` and `nstg` are in flight.
template <int KD>
__device__ __forceinline__ void tile_chunk(const TileLane& t, f32x4 (&acc)[KD / 16], const FastArgs& a,
                                           const uint16_t* Abh, const uint16_t* Zbh,
                                           const ChunkLanes& cl, char LDS_AS* __restrict__ nxt,
                                           const char LDS_AS* __restrict__ cur,
                                           char LDS_AS* __restrict__ nstg,
                                           const char LDS_AS* __restrict__ stg, int c, int wave,
                                           int lane) {
    const int64_t c0 = (int64_t)c * kChunkRows;
    const bool more = c + 1 < a.nchunks;
    const uint32_t base = lds_addr(cur) + t.a8;

    // Dense steps of this chunk: global steps [gs0, gs1), band steps
    // [ib0, ib1] (32-column steps from band_lo inside the chunk).
    const int q0 = uniform_load(a.gchunk + c), q1 = uniform_load(a.gchunk + c + 1);
    const int gs0 = q0 >> 5, gs1 = q1 > q0 ? ((q1 - 1) >> 5) + 1 : gs0;
    const int64_t kb0 = max(t.band_lo, c0);
    const int64_t kb1 = min(t.band_hi, c0 + kChunkRows - 1);
    const int ib0 = (int)((kb0 - t.band_lo) >> 5);
    const int ib1 = kb0 <= kb1 ? (int)((kb1 - t.band_lo) >> 5) : ib0 - 1;

    if (more) {
        dma_chunk<KD>(nxt, Zbh, a.n, c0 + kChunkRows, cl, wave);
        dma_groups(t, a, Abh, nstg, c + 1, lane);
    }

    // Random groups.
    const int32_t g0 = uniform_load(t.cptr + c);
    const int32_t gcnt = uniform_load(t.cptr + c + 1) - g0;
    for (int32_t k = 0; k < gcnt; ++k) {
        const GroupLane gl = group_lane(t, a, Abh, stg, g0, k);
        // Pair p of the lane's k-group keeps its two weights when its row
        // (the low 7 bits of byte p) is the lane's row.
        const uint32_t rm = gl.r & 0x7f7f7f7fu;
        u32x4 w;
#pragma unroll
        for (int p = 0; p < 4; ++p) w[p] = ((rm >> (8 * p)) & 0xffu) == (uint32_t)t.s16 ? gl.w[p] : 0u;
        mfma4(acc, code_addr(base, gl.j & 0xffffu), code_addr(base, gl.j >> 16), w);
    }

    // Global steps.
#pragma unroll
    for (int i = 0; i < kMaxGlob; ++i) {
        if (i >= gs0 && i < gs1) {
            const uint32_t r1 = t.gv1[i] >= c0 && t.gv1[i] < c0 + kChunkRows ? (uint32_t)(t.gv1[i] - c0) : kZeroRow;
            const uint32_t r2 = t.gv2[i] >= c0 && t.gv2[i] < c0 + kChunkRows ? (uint32_t)(t.gv2[i] - c0) : kZeroRow;
            mfma4(acc, code_addr(base, key_row_code(r1)), code_addr(base, key_row_code(r2)),
                  t.gw[i]);
        }
    }
    for (int s = max(gs0, kMaxGlob); s < gs1; ++s) {
        const int qa = 32 * s + 8 * t.kg + t.q4;
        mfma4(acc, code_addr(base, key_row_code(glob_row(a, qa, q0, q1, c0))),
              code_addr(base, key_row_code(glob_row(a, qa + 4, q0, q1, c0))),
              glob_weights(t, Abh, s));
    }

    // Window band.
    const uint32_t bb1 = code_addr(base, key_row_code(8u * t.kg + t.q4));
    const uint32_t bb2 = code_addr(base, key_row_code(8u * t.kg + 4u + t.q4));
#pragma unroll
    for (int i = 0; i < kMaxBand; ++i) {
        if (i >= ib0 && i <= ib1) {
            const uint32_t off = (uint32_t)(t.band_lo + 32 * i - c0) * kRowBytes;  // 32-row multiple
            mfma4(acc, bb1 + off, bb2 + off, t.bw[i]);
        }
    }
    for (int i = max(ib0, kMaxBand); i <= ib1; ++i) {
        const int64_t kc = t.band_lo + 32 * i;
        const uint32_t off = (uint32_t)(kc - c0) * kRowBytes;
        mfma4(acc, bb1 + off, bb2 + off, band_weights(t, Abh, kc));
    }
}

// One key chunk of a global-row wave: starts the direct loads of chunk
// c + 1 into `nxt` and multiplies keys c0 + 32 w .. + 31 of `cur`.
template <int KD>
__device__ __forceinline__ void grow_chunk(f32x4 (&acc)[2][KD / 16], const u32x4 (&w)[2],
                                           const uint16_t* Zbh, int64_t n, int nchunks,
                                           const ChunkLanes& cl, char LDS_AS* __restrict__ nxt,
                                           const char LDS_AS* __restrict__ cur, int c, int wave,
                                           uint32_t b1, uint32_t b2) {
    const int64_t c0 = (int64_t)c * kChunkRows;
    if (c + 1 < nchunks) dma_chunk<KD>(nxt, Zbh, n, c0 + kChunkRows, cl, wave);
    if (c0 + 32 * wave < n) {
        const uint32_t base = lds_addr(cur);
#pragma unroll
        for (int nb = 0; nb < KD / 16; ++nb) {
            const bf16x8 zop = z_operand(base + b1, base + b2, nb);
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) acc[mb][nb] = mfma(zop, w[mb], acc[mb][nb]);
        }
    }
}

template <int KD>
__global__ __launch_bounds__(kThreads)
void k_diffuse_sched(FastArgs a) {
    constexpr int NB = KD / 16;   // 16-channel blocks
    extern __shared__ __align__(128) char lds_raw[];
    char LDS_AS* lds = (char LDS_AS*)lds_raw;
    const int lane = __lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int kg = lane >> 4;          // k-group of the MFMA operands
    const int s16 = lane & 15;         // row (W^T) / channel (Z^T) index
    const uint32_t a8 = 8u * (lane & 3), q4 = (lane >> 2) & 3;   // transposed-read source

    const WorkItem wi = work_item(blockIdx.x, a.per_xcd, a.total_items, a.grow_per_bh,
                                  a.tiles_per_bh, a.bh_per_xcd);
    if (!wi.valid) return;
    const int32_t bh = wi.bh;
    const int32_t sub = wi.sub;
    const int32_t b = bh / a.H, h = bh - b * a.H;
    const int32_t gr = a.num_graphs == 1 ? 0 : b;
    const int64_t n = a.n;
    const uint16_t* Abh = a.A + a_block_offset(a.slot_off, a.num_graphs, a.H, b, h);
    const uint16_t* Zbh = a.Z + (int64_t)bh * n * KD;
    const int4* info = a.row_info + (int64_t)gr * n;
    char LDS_AS* buf[2] = {lds, lds + kBufBytes};
    const ChunkLanes cl = chunk_lanes<KD>(wave, lane);

    // Zero row kChunkRows of both buffers (the key row of dummy slots).
    if (threadIdx.x < 16) {
        *reinterpret_cast<u32x4 LDS_AS*>(buf[threadIdx.x >> 3] + kChunkRows * kRowBytes +
                                        (threadIdx.x & 7) * 16) = u32x4{0u, 0u, 0u, 0u};
    }

    if (sub < a.grow_per_bh) {
        // ---------------- global rows -------------------------------------
        const int q0 = sub * kGrowRows;
        int64_t wbase[2];
        int64_t wlen[2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            const int q = q0 + 16 * mb + s16;
            wbase[mb] = 0;
            wlen[mb] = 0;
            if (q < a.g) {
                const int64_t i = a.G[q];
                const int64_t* sp = a.seg_ptr + (int64_t)gr * (n + 1);
                wbase[mb] = info[i].x;
                wlen[mb] = sp[i + 1] - sp[i];
            }
        }
        auto fetch_w = [&](u32x4 (&w)[2], int64_t kc) {
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) {
                w[mb] = u32x4{0u, 0u, 0u, 0u};
                if (kc + 8 * kg < wlen[mb]) w[mb] = load16(Abh + wbase[mb] + kc + 8 * kg);
            }
        };
        f32x4 acc[2][NB];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
        u32x4 w[2], wn[2];
        fetch_w(w, 32 * wave);
        dma_chunk<KD>(buf[0], Zbh, n, 0, cl, wave);
        const uint32_t b1 = code_addr(a8, key_row_code(32u * wave + 8u * kg + q4));
        const uint32_t b2 = code_addr(a8, key_row_code(32u * wave + 8u * kg + 4u + q4));
        for (int c = 0; c < a.nchunks; ++c) {
            const int64_t c0 = (int64_t)c * kChunkRows;
            full_barrier();   // chunk c in LDS
            if (c + 1 < a.nchunks) fetch_w(wn, c0 + kChunkRows + 32 * wave);
            grow_chunk<KD>(acc, w, Zbh, n, a.nchunks, cl, buf[(c + 1) & 1], buf[c & 1], c, wave, b1,
                           b2);
            w[0] = wn[0];
            w[1] = wn[1];
        }
        // Fixed-order sum of the 16 waves' partial sums.
        full_barrier();
        float LDS_AS* part = (float LDS_AS*)lds;   // [wave][mb][nb][e][lane]
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    part[(((wave * 2 + mb) * NB + nb) * 4 + e) * kWave + lane] = acc[mb][nb][e];
        lds_barrier();
        constexpr int kPer = 2 * NB * 4 * kWave;   // partial sums per wave
        for (int idx = threadIdx.x; idx < kPer; idx += kThreads) {
            float sum = 0.0f;
            for (int w2 = 0; w2 < kWaves; ++w2) sum += part[w2 * kPer + idx];
            const int l = idx & 63, e = (idx >> 6) & 3, nb = (idx >> 8) % NB, mb = (idx >> 8) / NB;
            const int q = q0 + 16 * mb + (l & 15);
            if (q >= a.g) continue;
            const int64_t i = a.G[q];
            const int ch = 16 * nb + 4 * (l >> 4) + e;
            const int64_t o = ((int64_t)bh * n + i) * KD + ch;
            const float keep = a.row_scale ? a.keep * a.row_scale[(int64_t)bh * n + i] : a.keep;
            a.Zn[o] = (uint16_t)f32_to_bf16(keep * sum + a.restart * bf16_to_f32(a.V[o]));
        }
        return;
    }

    // ---------------- row tile --------------------------------------------
    TileLane t;
    t.kg = kg;
    t.s16 = s16;
    t.a8 = a8;
    t.q4 = q4;
    t.r0w = (int64_t)(sub - a.grow_per_bh) * kTileRows + (int64_t)kRowBlock * wave;
    const bool active = t.r0w < n;
    const int64_t my_row = t.r0w + s16;          // W^T column / output row of this lane
    t.ri = make_int4(0, 0, -1, 0);
    if (my_row < n) t.ri = info[my_row];
    t.rok = my_row < n && t.ri.z >= 0;           // a non-global row

    // Band of this wave: key columns [band_lo, band_hi], 32-aligned steps.
    const int64_t wr_last = min(t.r0w + kRowBlock - 1, n - 1);
    t.band_lo = (t.r0w - a.radius < 0 ? 0 : t.r0w - a.radius) & ~31ll;
    t.band_hi = a.causal ? wr_last : min(n - 1, wr_last + a.radius);

    // Schedule groups of this row block, staged chunk by chunk.
    char LDS_AS* stg[2] = {lds + 2 * kBufBytes + (2 * wave) * kStageBytes,
                           lds + 2 * kBufBytes + (2 * wave + 1) * kStageBytes};
    const int64_t rb = active ? t.r0w / kRowBlock : 0;
    t.cptr = a.grp_cptr + ((int64_t)gr * a.nrb + rb) * (a.nchunks + 1);
    t.goff = a.grp_off[gr];
    t.rbase = a.seg_ptr[(int64_t)gr * (n + 1) + n];   // random area of the graph

    dma_chunk<KD>(buf[0], Zbh, n, 0, cl, wave);
    t.nbs = active ? (int)((t.band_hi - t.band_lo) >> 5) + 1 : 0;
    t.ngs = (a.g + 31) >> 5;
#pragma unroll
    for (int i = 0; i < kMaxBand; ++i)
        t.bw[i] = i < t.nbs ? band_weights(t, Abh, t.band_lo + 32 * i) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < kMaxGlob; ++i) {
        t.gw[i] = u32x4{0u, 0u, 0u, 0u};
        t.gv1[i] = t.gv2[i] = -1;
        if (i < t.ngs) {
            const int qa = 32 * i + 8 * kg + (int)q4;
            t.gw[i] = glob_weights(t, Abh, i);
            if (qa < a.g) t.gv1[i] = a.G[qa];
            if (qa + 4 < a.g) t.gv2[i] = a.G[qa + 4];
        }
    }
    if (active) dma_groups(t, a, Abh, stg[0], 0, lane);
    f32x4 acc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

    float scale = 1.0f;   // c_i of this lane's row
    for (int c = 0; c < a.nchunks; ++c) {
        full_barrier();   // chunk c in LDS, chunk c - 1 done by every wave
        if (c + 1 == a.nchunks && active) {
            // The idle buffer takes the restart inputs of the wave's rows.
            dma_restart<KD>(a, bh, t.r0w, buf[(c + 1) & 1] + wave * 2048, lane);
            if (a.row_scale != nullptr && t.rok) scale = a.row_scale[(int64_t)bh * n + my_row];
        }
        if (active) {
            tile_chunk<KD>(t, acc, a, Abh, Zbh, cl, buf[(c + 1) & 1], buf[c & 1],
                           stg[(c + 1) & 1], stg[c & 1], c, wave, lane);
        } else if (c + 1 < a.nchunks) {
            dma_chunk<KD>(buf[(c + 1) & 1], Zbh, n, (int64_t)(c + 1) * kChunkRows, cl, wave);
        }
    }

    if (active) {
        __builtin_amdgcn_s_waitcnt(0x0070);   // this wave's restart inputs have landed
        if (t.rok)
            store_row<KD>(a, bh, my_row, s16, kg, acc, buf[a.nchunks & 1] + wave * 2048, scale);
    }
}

}  // namespace

bool fast_diffuse_supported(const diffuser_graph& g, const attn_shape& s) {
    if (!g.structured || !g.grouped() || s.dtype != DIFFUSER_BF16 || (s.d != 64 && s.d != 32))
        return false;
    for (int64_t x : g.slots)
        if (x >= (1ll << 31)) return false;
    return true;
}

hipError_t launch_diffuse_fast(const diffuser_graph& g, const attn_shape& s, const void* A,
                               const void* Zk, const void* V, void* Zn, const float* row_scale,
                               step_coefs kc, hipStream_t st) {
    FastArgs a;
    a.n = g.n;
    a.H = s.H;
    a.num_graphs = g.num_graphs;
    a.radius = g.radius;
    a.g = g.num_global;
    a.causal = g.causal;
    a.nchunks = (int32_t)((g.n + kChunkRows - 1) / kChunkRows);
    a.nrb = (int32_t)((g.n + kRowBlock - 1) / kRowBlock);
    a.slot_off = g.d_slot_off;
    a.seg_ptr = g.d_seg_ptr;
    a.row_info = reinterpret_cast<const int4*>(g.d_row_info);
    a.G = g.d_global;
    a.gchunk = g.d_gchunk;
    a.grp_ptr = g.d_grp_ptr;
    a.grp_off = g.d_grp_off;
    a.grp_cptr = g.d_grp_cptr;
    a.sched_row = g.d_sched_row;
    a.sched_j = g.d_sched_j;
    a.A = static_cast<const uint16_t*>(A);
    a.Z = static_cast<const uint16_t*>(Zk);
    a.V = static_cast<const uint16_t*>(V);
    a.Zn = static_cast<uint16_t*>(Zn);
    a.row_scale = row_scale;
    a.keep = kc.keep;
    a.restart = kc.restart;
    const int32_t BH = s.B * s.H;
    a.tiles_per_bh = (int32_t)((g.n + kTileRows - 1) / kTileRows);
    a.grow_per_bh = (g.num_global + kGrowRows - 1) / kGrowRows;
    a.total_items = BH * (a.tiles_per_bh + a.grow_per_bh);
    a.bh_per_xcd = 0;   // (b, h)-ordered runs (measured slightly faster here than tiles-first)
    a.per_xcd = a.bh_per_xcd > 0 ? a.bh_per_xcd * (a.tiles_per_bh + a.grow_per_bh)
                                 : (a.total_items + 7) / 8;
    // Dynamic LDS above 64 KB is enabled once per device and instantiation.
    static int attr_device[2] = {-1, -1};
    const int which = s.d == 64 ? 0 : 1;
    const void* kern = s.d == 64 ? reinterpret_cast<const void*>(&k_diffuse_sched<64>)
                                 : reinterpret_cast<const void*>(&k_diffuse_sched<32>);
    if (attr_device[which] != g.device) {
        hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           kLdsBytes);
        if (e != hipSuccess) return e;
        attr_device[which] = g.device;
    }
    const size_t lds = kLdsBytes;
    if (s.d == 64)
        hipLaunchKernelGGL(k_diffuse_sched<64>, dim3((unsigned)(8 * a.per_xcd)), dim3(kThreads),
                           lds, st, a);
    else
        hipLaunchKernelGGL(k_diffuse_sched<32>, dim3((unsigned)(8 * a.per_xcd)), dim3(kThreads),
                           lds, st, a);
    return hipGetLastError();
}

}  // namespace diffuser
