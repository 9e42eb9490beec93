// Edge scores and edge softmax on scheduled graphs, bf16 storage, d_h = 64
// ("Diffuser" reading notes, section 2.1, eqs. S.1-S.5; "1.2.1 Static
// sparsity", section 1, eqs. 1-3):
//   s_ij = q_i . k_j / sqrt(d_h) on the edges of row i,
//   A_ij = exp(s_ij - m_i) / sum_u exp(s_iu - m_i),  m_i = max_j s_ij.
//
// Scores come from v_mfma_f32_16x16x32_bf16 products
//   D[key][row] = sum_c K[key][c] Q[row][c]   (two products for c < 64)
// over 16 keys and 16 rows: the K operand is 8 consecutive channels of one
// key row, read from LDS with ds_read_b128; the Q^T operand 8 channels of
// one query row, held in registers. Lane l of D holds keys 4 (l / 16) .. + 3
// of row l % 16, so each lane owns one row and writes 4 consecutive slots.
//  * window edges: keys are consecutive columns of the band (tiles that lie
//    inside every row's window skip the masking);
//  * global columns: the g global rows of K, staged once per workgroup;
//  * random edges: per schedule group two products with the query rows as
//    the first operand (D[row][key]) against the first and the second
//    slots of the group's 16 pairs; the lane of a pair's row keeps both.
// A workgroup (16 waves, 16 rows each) streams K of its (batch, head)
// through LDS in chunks of kChunkRows rows with direct global-to-LDS loads,
// double-buffered, once per pass. The shift m_i of the exponentials can be
// any value: exp(s - m) / sum exp(s - m) does not depend on it, and any m_i
// at most the row maximum keeps every weight at least as large as with the
// maximum itself (no extra underflow). The kernel takes m_i = the row's own
// score s_ii (the self-loop is an edge of every row); scores above it only
// make weights exceed one. A row whose stored weights sum to 2^64 or more
// (a score far above s_ii) is redone with the exact maximum from a full
// pass, so the weights never overflow.
//   fused mode: one pass writes w_ij = exp(s_ij - m_i) unnormalised and c_i
//     = 1 / (sum of the stored w_ij), which the diffusion step applies;
//   normalised mode: one pass sums w_ij, a second writes w_ij / sum.
// exp(s - m) is evaluated as exp2(x * log2(e) / sqrt(d_h) - m'), x the dot
// product and m' the scaled maximum. Global rows (full rows of length n)
// get workgroups of their own: 32 rows, the 16 waves split each chunk's
// keys and merge their partial sums (and, when redone, maxima) in a fixed
// order; their shift is also the row's own score. K rows sit
// in LDS at 128 bytes, 16-byte units permuted by score_row_code, which
// spreads the 16 rows of one operand read over the banks.
#include "internal.h"
#include "mfma_util.h"

namespace diffuser {
namespace {

constexpr int kWave = 64;
constexpr int kWaves = 16;
constexpr int kThreads = kWave * kWaves;
// A key row sits in a 128-byte LDS slot (64 channels of bf16); a head width
// of 32 fills half of it and leaves channels 32..63 zero, so the second
// product of each tile adds nothing.
constexpr int kRowBytes = 128;
constexpr int kBufBytes = (kChunkRows + 1) * kRowBytes;   // chunk + zero row
constexpr int kTileRows = kWaves * kRowBlock;
constexpr int kGrowRows = 32;
constexpr int kMaxGlobal = 128;
constexpr int kSGroupBytes = 112;   // staged group: codes, pair rows, pair slot offsets
constexpr int kStageGroups = 8;
constexpr int kStageBytes = kStageGroups * kSGroupBytes;
constexpr int kLdsBytes = 2 * kBufBytes + kMaxGlobal * (kRowBytes + 4) + kWaves * kStageBytes;
static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
static_assert(2 * kWaves * kGrowRows * 4 <= 2 * kBufBytes, "grow merge fits");

enum Pass { kPassMax = 0, kPassWriteFused = 1, kPassSum = 2, kPassWriteNorm = 3 };
// A row whose weights (shifted by less than its maximum) sum to this or
// more is redone with its exact maximum: every weight then stays far from
// the float and bf16 overflow threshold (2^128), and so does the sum.
constexpr float kSumLimit = 18446744073709551616.0f;   // 2^64

struct ScoreArgs {
    int32_t n, H, num_graphs, radius, g, causal, nchunks, nrb;
    int32_t kd;                 // head width: 64 or 32
    const int64_t* slot_off;    // [graphs + 1]
    const int64_t* seg_ptr;     // [graphs][n + 1]
    const int4* row_info;       // [graphs][n]
    const int32_t* G;           // [g]
    const int64_t* grp_off;     // [graphs + 1]
    const int32_t* grp_cptr;    // [graphs][nrb][nchunks + 1]
    const uint32_t* sched_row;  // [groups][4]
    const uint16_t* sched_k;    // [groups][32]
    const uint16_t* sched_off;  // [groups][16] pair's first slot in its block's octet area
    const int32_t* rnd_cnt;     // [graphs][n] random edges of each row
    const int32_t* rb_oct;      // [graphs][nrb] random octets of each row block (octet layout)
    const int64_t* rb_roff;     // [graphs][nrb + 1] their prefix sums (octet layout)
    int32_t octet;              // random weights in per-row-block octet areas (else groups)
    const uint16_t* Q;
    const uint16_t* K;
    uint16_t* A;
    float* row_scale;           // [B*H][n] (fused mode)
    float scale_log2;           // log2(e) / sqrt(d_h)
    int32_t normalized;
    int32_t tiles_per_bh, grow_per_bh, per_xcd, total_items, bh_per_xcd;
};

// The K operands (channels 8 kg .. + 7 and 32 + 8 kg .. + 7) of the key row
// with score_row_code `code`.
__device__ __forceinline__ void k_operands(const char LDS_AS* buf, uint32_t code, uint32_t kg,
                                           u32x4& k0, u32x4& k1) {
    const uint32_t o = (code ^ kg) << 4;
    k0 = *reinterpret_cast<const u32x4 LDS_AS*>(buf + o);
    k1 = *reinterpret_cast<const u32x4 LDS_AS*>(buf + (o ^ 64u));   // unit kg + 4
}

// Unscaled dot products of one 16 x 16 tile, D[i][j] = a_i . b_j over the
// 64 channels, where lane (kg, s16) supplies channels 8 kg .. + 7 and
// 32 + 8 kg .. + 7 of a_{s16} (a0, a1) and of b_{s16} (b0, b1) and receives
// D[4 kg + e][s16] in element e. Band and global tiles take keys as a
// (D[key][row]), random groups take query rows as a (D[row][key]).
__device__ __forceinline__ f32x4 dots(const u32x4& a0, const u32x4& a1, const u32x4& b0,
                                      const u32x4& b1) {
    return mfma_bf16(a1, b1, mfma_bf16(a0, b0, f32x4{0.f, 0.f, 0.f, 0.f}));
}

// Direct loads of chunk rows [c0, c0 + kChunkRows) of K into `buf` (wave w
// fills 1 KB blocks 4w .. 4w+3); rows at or beyond n repeat row n - 1. A
// row's logical units past its a.kd channels are not loaded.
__device__ __forceinline__ void dma_chunk(char LDS_AS* buf, const uint16_t* Kbh,
                                          const ScoreArgs& a, int32_t c0, int wave, int lane) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int blk = 4 * wave + t;
        const uint32_t pr = (uint32_t)(blk * 8 + (lane >> 3));
        const uint32_t lu = (uint32_t)(lane & 7) ^ (score_row_code(pr) & 7u);
        const int32_t src = min(c0 + (int32_t)pr, a.n - 1);
        if (lu * 8 < (uint32_t)a.kd)
            __builtin_amdgcn_global_load_lds(Kbh + (int64_t)src * a.kd + lu * 8,
                                             (void LDS_AS*)(buf + blk * 1024), 16, 0, 0);
    }
}

__device__ __forceinline__ float exp2f_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Sum of the two bf16 halves of `w` added to acc (one v_dot2_f32_bf16).
__device__ __forceinline__ float add_pair(uint32_t w, float acc) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w),
                                           __builtin_bit_cast(bf16x2, 0x3f803f80u), acc, false);
}

// acc + a.lo b.lo + a.hi b.hi for two packed bf16 pairs (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), acc, false);
}

// Per-lane state of a row-tile wave (the lane's row is r0w + l % 16).
struct SLane {
    int32_t kg, s16, i, r0w;
    int4 ri;                   // {segment start, window block start, window slots, global slots}
    bool rok;                  // a non-global row below n
    bool block_ok;             // every row of the wave's block is such a row
    int32_t lo;                // window columns [lo, lo + span]
    uint32_t span;
    u32x4 q0, q1;              // Q^T operands
    float m;                   // row maximum of the dot products
    float ms;                  // m * scale_log2
    float sum, inv;            // sum of the weights, its inverse (normalised mode)
    int32_t band_lo, band_hi;
    int32_t gr;                // graph of the (b, h) pair
    uint32_t abase;            // first slot of the row block's octet area (octet layout)
    uint32_t rbase;            // first slot of the random area
    const int32_t* cptr;
    int64_t goff;
    u32x2 po;                  // next chunk's pair slot offsets (octet layout)
    u32x4 pk;                  // next chunk's score codes, compact
    uint32_t pr;               // next chunk's pair rows, compact
    // Random groups put row 4 kg + e in element e of a lane's products:
    float ms4[4];              // shift of rows 4 kg + e
    float inv4[4];             // inverse sums of rows 4 kg + e (normalised write)
    float racc[4];             // their random weights' max (max pass) or sum
};

// Pass-specific treatment of 4 dot products of consecutive slots of the
// lane's row. kMask: valid[] applies (otherwise all four are edges).
template <int P, bool kMask>
__device__ __forceinline__ void consume4(SLane& t, const f32x4& x, const bool (&valid)[4],
                                         float scale_log2, uint16_t* dst) {
    if (P == kPassMax) {
        if (kMask) {
#pragma unroll
            for (int e = 0; e < 4; ++e) t.m = valid[e] ? fmaxf(t.m, x[e]) : t.m;
        } else {
            t.m = fmaxf(fmaxf(t.m, x[0]), fmaxf(x[1], fmaxf(x[2], x[3])));
        }
        return;
    }
    float w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        w[e] = exp2f_fast(__builtin_fmaf(x[e], scale_log2, -t.ms));
        if (kMask) w[e] = valid[e] ? w[e] : 0.0f;
    }
    if (P == kPassSum) {
        t.sum += (w[0] + w[1]) + (w[2] + w[3]);
        return;
    }
    if (P == kPassWriteNorm) {
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] *= t.inv;
    }
    const uint32_t lo = to_bf16_pair(w[0], w[1]), hi = to_bf16_pair(w[2], w[3]);
    if (dst != nullptr) {
        *reinterpret_cast<u32x2*>(dst) = u32x2{lo, hi};
        if (P == kPassWriteFused) t.sum = add_pair(hi, add_pair(lo, t.sum));
    }
}

// One band tile: keys kb .. kb + 15 (rows of `cur` from kb - c0).
template <int P>
__device__ __forceinline__ void band_tile(SLane& t, const ScoreArgs& a, uint16_t* Abh,
                                          const char LDS_AS* cur, int32_t kb, int32_t c0) {
    u32x4 k0, k1;
    k_operands(cur, score_row_code((uint32_t)(kb - c0 + t.s16)), (uint32_t)t.kg, k0, k1);
    const f32x4 x = dots(k0, k1, t.q0, t.q1);
    const int32_t key0 = kb + 4 * t.kg;
    // The whole tile lies in every row's window (a wave-uniform test).
    const bool interior = t.block_ok && kb >= t.r0w + 15 - a.radius &&
                          kb + 15 <= (a.causal ? t.r0w : t.r0w + a.radius) &&
                          kb + 15 <= a.n - 1;
    const bool write = P == kPassWriteFused || P == kPassWriteNorm;
    if (interior) {
        const bool valid[4] = {true, true, true, true};
        consume4<P, false>(t, x, valid, a.scale_log2,
                           write ? Abh + t.ri.x + (key0 - t.ri.y) : nullptr);
        return;
    }
    const uint32_t d = (uint32_t)(key0 - t.lo);
    bool valid[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) valid[e] = t.rok && d + (uint32_t)e <= t.span;
    const int32_t off = key0 - t.ri.y;
    uint16_t* dst = (write && t.rok && off >= 0 && off < t.ri.z) ? Abh + t.ri.x + off : nullptr;
    consume4<P, true>(t, x, valid, a.scale_log2, dst);
}

// Element e = 2 b1 + b0 of x, for a lane-dependent e.
__device__ __forceinline__ float pick4(float x0, float x1, float x2, float x3, bool b0, bool b1) {
    const float lo = b0 ? x1 : x0, hi = b0 ? x3 : x2;
    return b1 ? hi : lo;
}

// One random group. The products are taken with the query rows as the
// first operand: lane (kg, s16) holds, in element e of x0 (x1), the product
// of row 4 kg + e with the key of slot 0 (1) of pair s16, whose row byte
// (row, + 0x40 / 0x80 when the first / second slot is a dummy, 0xFF for a
// dummy pair) is rb. The lane of kg = row / 4 owns the pair: two
// exponentials, the store of its weights at slot `dst` of the (b, h) block
// of A, and the pair's share of row 4 kg + e in racc[e]. In the group layout
// both slots are the group's own (a dummy slot, or a dummy pair, written
// 0 by the lane of kg = 0): one 4-byte store. In the octet layout a dummy
// slot is another edge's or padding, so only the real slots are stored.
template <int P>
__device__ __forceinline__ void random_group(SLane& t, const f32x4& x0, const f32x4& x1,
                                             uint32_t rb, float scale_log2, uint16_t* Abh,
                                             uint32_t dst, bool octet) {
    const uint32_t r = rb & 0x3fu;
    const bool mine = (r >> 2) == (uint32_t)t.kg;
    const bool v0 = mine && (rb & 0x40u) == 0;
    const bool v1 = mine && (rb & 0x80u) == 0;
    const bool b0 = (r & 1u) != 0, b1 = (r & 2u) != 0;
    const float y0 = pick4(x0[0], x0[1], x0[2], x0[3], b0, b1);
    const float y1 = pick4(x1[0], x1[1], x1[2], x1[3], b0, b1);
    float v;
    if (P == kPassMax) {
        v = fmaxf(v0 ? y0 : -INFINITY, v1 ? y1 : -INFINITY);
    } else {
        const float ms = pick4(t.ms4[0], t.ms4[1], t.ms4[2], t.ms4[3], b0, b1);
        float w0 = exp2f_fast(__builtin_fmaf(y0, scale_log2, -ms));
        float w1 = exp2f_fast(__builtin_fmaf(y1, scale_log2, -ms));
        w0 = v0 ? w0 : 0.0f;
        w1 = v1 ? w1 : 0.0f;
        if (P == kPassSum) {
            v = w0 + w1;
        } else {
            if (P == kPassWriteNorm) {
                const float inv = pick4(t.inv4[0], t.inv4[1], t.inv4[2], t.inv4[3], b0, b1);
                w0 *= inv;
                w1 *= inv;
            }
            const uint32_t pw = to_bf16_pair(w0, w1);
            if (!octet) {
                if (mine || (rb == 0xffu && t.kg == 0))
                    *reinterpret_cast<uint32_t*>(Abh + dst) = pw;
            } else if (v0 && v1) {
                *reinterpret_cast<uint32_t*>(Abh + dst) = pw;
            } else if (v0 || v1) {
                Abh[dst + (v0 ? 0u : 1u)] = (uint16_t)(v0 ? pw : pw >> 16);
            }
            if (P == kPassWriteNorm) return;
            v = add_pair(pw, 0.0f);   // fused mode: c_i is over the weights as stored
        }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const bool here = b0 == ((e & 1) != 0) && b1 == ((e & 2) != 0);
        if (P == kPassMax) t.racc[e] = here ? fmaxf(t.racc[e], v) : t.racc[e];
        else t.racc[e] = here ? t.racc[e] + v : t.racc[e];
    }
}

// Start of a pass: random accumulators cleared, the shift (and inverse sum)
// of rows 4 kg + e fetched from the lanes of those rows.
template <int P>
__device__ __forceinline__ void random_begin(SLane& t) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        t.racc[e] = P == kPassMax ? -INFINITY : 0.0f;
        if (P != kPassMax) t.ms4[e] = __shfl(t.ms, 4 * t.kg + e);
        if (P == kPassWriteNorm) t.inv4[e] = __shfl(t.inv, 4 * t.kg + e);
    }
}

// End of a pass: racc[e] over the 16 lanes of kg (row 4 kg + e), then
// into the row's lanes: into m (max pass) or, once per row, into sum.
template <int P>
__device__ __forceinline__ void random_end(SLane& t) {
    if (P == kPassWriteNorm) return;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) {
            const float o = __shfl_xor(t.racc[e], off);
            t.racc[e] = P == kPassMax ? fmaxf(t.racc[e], o) : t.racc[e] + o;
        }
    }
    float row = P == kPassMax ? -INFINITY : 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float o = __shfl(t.racc[e], 16 * (t.s16 >> 2));
        if ((t.s16 & 3) == e) row = o;
    }
    if (P == kPassMax) t.m = fmaxf(t.m, row);
    else if (t.kg == 0) t.sum += row;
}

// One key chunk of a row-tile wave in pass P: band tiles of chunk c, then
// (with the direct loads of chunk c + 1 into `nxt` in flight) the random
// groups of chunk c, whose codes are staged in `stg`.
template <int P>
__device__ __forceinline__ void tile_chunk(SLane& t, const ScoreArgs& a, const uint16_t* Kbh,
                                           uint16_t* Abh, char LDS_AS* __restrict__ nxt,
                                           const char LDS_AS* __restrict__ cur,
                                           char LDS_AS* __restrict__ stg, int c, int wave,
                                           int lane) {
    const int32_t c0 = c * kChunkRows;
    const bool more = c + 1 < a.nchunks;
    const int32_t g0 = uniform_load(t.cptr + c);
    const int32_t gcnt = uniform_load(t.cptr + c + 1) - g0;
    int32_t ncnt = 0;
    if (more) {
        const int32_t n0 = g0 + gcnt;
        ncnt = min(uniform_load(t.cptr + c + 2) - n0, kStageGroups);
        if (lane < 4 * ncnt) {
            t.pk = *reinterpret_cast<const u32x4*>(a.sched_k + (t.goff + n0) * kGroupSlots +
                                                   8 * lane);
            t.pr = a.sched_row[(t.goff + n0) * 4 + lane];
            if (a.octet)
                t.po = *reinterpret_cast<const u32x2*>(a.sched_off + (t.goff + n0) * 16 + 4 * lane);
        }
    }

    // Window band, 16 keys per tile.
    const int32_t k_lo = max(t.band_lo, c0);
    const int32_t k_hi = min(t.band_hi, c0 + kChunkRows - 1);
    for (int32_t kb = k_lo; kb <= k_hi; kb += 16) band_tile<P>(t, a, Abh, cur, kb, c0);

    if (more) dma_chunk(nxt, Kbh, a, c0 + kChunkRows, wave, lane);

    // Random groups: two tiles of 16 slots each. The staged ones read their
    // codes from LDS, any others straight from memory; the two loops are
    // kept apart so that no register is loaded from both places, which would
    // make every LDS read wait for all outstanding memory operations (the
    // next chunk's loads and the weight stores among them).
    // A group's codes and row byte are read one group ahead.
    const int32_t nstaged = min(gcnt, kStageGroups);
    // A pair's first slot: in the octet layout its row block's area base
    // plus the staged offset, in the group layout slot 2 s16 of the group.
    const bool octet = a.octet != 0;
    uint32_t codes_n = *reinterpret_cast<const uint32_t LDS_AS*>(stg + 4 * t.s16);
    uint32_t rb_n = *reinterpret_cast<const uint8_t LDS_AS*>(stg + 64 + t.s16);
    uint32_t off_n = *reinterpret_cast<const uint16_t LDS_AS*>(stg + 80 + 2 * t.s16);
    for (int32_t k = 0; k < nstaged; ++k) {
        const uint32_t codes = codes_n, rb = rb_n, off = off_n;
        if (k + 1 < nstaged) {
            const char LDS_AS* o = stg + (k + 1) * kSGroupBytes;
            codes_n = *reinterpret_cast<const uint32_t LDS_AS*>(o + 4 * t.s16);
            rb_n = *reinterpret_cast<const uint8_t LDS_AS*>(o + 64 + t.s16);
            off_n = *reinterpret_cast<const uint16_t LDS_AS*>(o + 80 + 2 * t.s16);
        }
        f32x4 x[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t code = (codes >> (16 * h)) & 0xffffu;
            u32x4 k0, k1;
            k_operands(cur, code, (uint32_t)t.kg, k0, k1);
            x[h] = dots(t.q0, t.q1, k0, k1);
        }
        const uint32_t dst = octet ? t.abase + off
                                   : t.rbase + (uint32_t)(kGroupSlots * (g0 + k) + 2 * t.s16);
        random_group<P>(t, x[0], x[1], rb, a.scale_log2, Abh, dst, octet);
    }
    for (int32_t k = nstaged; k < gcnt; ++k) {
        const int64_t gi = t.goff + g0 + k;
        const uint32_t codes = reinterpret_cast<const uint32_t*>(a.sched_k + gi * kGroupSlots)[t.s16];
        f32x4 x[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t code = (codes >> (16 * h)) & 0xffffu;
            u32x4 k0, k1;
            k_operands(cur, code, (uint32_t)t.kg, k0, k1);
            x[h] = dots(t.q0, t.q1, k0, k1);
        }
        const uint32_t rb = reinterpret_cast<const uint8_t*>(a.sched_row + gi * 4)[t.s16];
        const uint32_t dst = octet ? t.abase + a.sched_off[gi * 16 + t.s16]
                                   : t.rbase + (uint32_t)(kGroupSlots * (g0 + k) + 2 * t.s16);
        random_group<P>(t, x[0], x[1], rb, a.scale_log2, Abh, dst, octet);
    }
    if (more && lane < 4 * ncnt) {
        char LDS_AS* d = stg + (lane >> 2) * kSGroupBytes;
        *reinterpret_cast<u32x4 LDS_AS*>(d + (lane & 3) * 16) = t.pk;
        *reinterpret_cast<uint32_t LDS_AS*>(d + 64 + (lane & 3) * 4) = t.pr;
        if (octet) *reinterpret_cast<u32x2 LDS_AS*>(d + 80 + (lane & 3) * 8) = t.po;
    }
}

// Global columns of a row-tile wave in pass P (keys = staged global rows).
template <int P>
__device__ __forceinline__ void tile_globals(SLane& t, const ScoreArgs& a, uint16_t* Abh,
                                             const char LDS_AS* zg, const int32_t LDS_AS* gidx,
                                             int gpad) {
    const bool write = P == kPassWriteFused || P == kPassWriteNorm;
    const int32_t hi = (int32_t)t.span + t.lo;   // window end
    for (int qb = 0; qb < gpad; qb += 16) {
        u32x4 k0, k1;
        k_operands(zg, score_row_code((uint32_t)(qb + t.s16)), (uint32_t)t.kg, k0, k1);
        const f32x4 x = dots(k0, k1, t.q0, t.q1);
        const int q0 = qb + 4 * t.kg;
        bool valid[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int q = q0 + e;
            const int32_t p = gidx[q];
            valid[e] = t.rok && q < a.g && (p < t.lo || (!a.causal && p > hi));
        }
        uint16_t* dst = (write && t.rok && q0 < t.ri.w) ? Abh + t.ri.x + t.ri.z + q0 : nullptr;
        consume4<P, true>(t, x, valid, a.scale_log2, dst);
    }
}

// Direct loads of chunk 0 into buffer 0 and of the wave's first staged
// groups.
__device__ __forceinline__ void stage_first(const SLane& t, const ScoreArgs& a,
                                            const uint16_t* Kbh, char LDS_AS* lds,
                                            char LDS_AS* stg, bool active, int wave, int lane) {
    dma_chunk(lds, Kbh, a, 0, wave, lane);
    if (active) {
        const int32_t g0 = uniform_load(t.cptr);
        const int32_t cnt = min(uniform_load(t.cptr + 1) - g0, kStageGroups);
        if (lane < 4 * cnt) {
            char LDS_AS* d = stg + (lane >> 2) * kSGroupBytes;
            *reinterpret_cast<u32x4 LDS_AS*>(d + (lane & 3) * 16) =
                *reinterpret_cast<const u32x4*>(a.sched_k + (t.goff + g0) * kGroupSlots +
                                                8 * lane);
            *reinterpret_cast<uint32_t LDS_AS*>(d + 64 + (lane & 3) * 4) =
                a.sched_row[(t.goff + g0) * 4 + lane];
            if (a.octet)
                *reinterpret_cast<u32x2 LDS_AS*>(d + 80 + (lane & 3) * 8) =
                    *reinterpret_cast<const u32x2*>(a.sched_off + (t.goff + g0) * 16 + 4 * lane);
        }
    }
}

// One pass of a row-tile wave.
template <int P>
__device__ void tile_pass(SLane& t, const ScoreArgs& a, const uint16_t* Kbh, uint16_t* Abh,
                          char LDS_AS* lds, int gpad, bool active, int wave, int lane) {
    char LDS_AS* buf0 = lds;
    char LDS_AS* buf1 = lds + kBufBytes;
    char LDS_AS* zg = lds + 2 * kBufBytes;
    const int32_t LDS_AS* gidx = (const int32_t LDS_AS*)(zg + gpad * kRowBytes);
    char LDS_AS* stg = zg + gpad * (kRowBytes + 4) + wave * kStageBytes;

    random_begin<P>(t);
    if ((P == kPassWriteFused || P == kPassWriteNorm) && a.octet && active && t.kg == 0) {
        // Octet layout: the positions of the block's octet area past a row's
        // random edges (every position of a global row or a row past n)
        // belong to no pair of the schedule; they hold 0.
        const int32_t noct = uniform_load(a.rb_oct + (int64_t)t.gr * a.nrb + t.r0w / kRowBlock);
        const int32_t cnt = t.rok ? a.rnd_cnt[(int64_t)t.gr * a.n + t.i] : 0;
        const uint32_t base = t.abase + 8u * (uint32_t)t.s16;
        for (int32_t e = cnt; e < 8 * noct; ++e) Abh[base + (uint32_t)((e >> 3) * 128 + (e & 7))] = 0;
    }
    stage_first(t, a, Kbh, lds, stg, active, wave, lane);
    full_barrier();
    if (active) tile_globals<P>(t, a, Abh, zg, gidx, gpad);
    for (int c = 0; c < a.nchunks; ++c) {
        if (c > 0) full_barrier();
        if (active) {
            tile_chunk<P>(t, a, Kbh, Abh, (c & 1) ? buf0 : buf1, (c & 1) ? buf1 : buf0, stg, c,
                          wave, lane);
        } else if (c + 1 < a.nchunks) {
            dma_chunk((c & 1) ? buf0 : buf1, Kbh, a, (c + 1) * kChunkRows, wave, lane);
        }
    }
    random_end<P>(t);
    full_barrier();   // every wave is done with the buffers
}

// Max over the 4 lanes of one row (lanes l, l ^ 16, l ^ 32, l ^ 48).
__device__ __forceinline__ float row_max(float x) {
    x = fmaxf(x, __shfl_xor(x, 16));
    return fmaxf(x, __shfl_xor(x, 32));
}
// Sum over the 4 lanes of one row, in a fixed order.
__device__ __forceinline__ float row_sum(float x) {
    x += __shfl_xor(x, 16);
    return x + __shfl_xor(x, 32);
}

// ---------------------------------------------------------------------------
// Global rows: 32 per workgroup (two 16-row blocks); wave w scores keys
// c0 + 32 w .. + 31 of every chunk.
struct GLane {
    int32_t kg, s16;
    int32_t i[2];              // the lane's global rows (or -1)
    int32_t last[2];           // their last key (n - 1, or the row when causal)
    int64_t sbase[2];
    int32_t slen[2];
    u32x4 q0[2], q1[2];
    float m[2], ms[2], sum[2], inv[2];
};

template <int P>
__device__ __forceinline__ void grow_chunk(GLane& t, const ScoreArgs& a, const uint16_t* Kbh,
                                           uint16_t* Abh, char LDS_AS* __restrict__ nxt,
                                           const char LDS_AS* __restrict__ cur, int c, int wave,
                                           int lane, bool prefetch = true) {
    const int32_t c0 = c * kChunkRows;
    if (prefetch && c + 1 < a.nchunks) dma_chunk(nxt, Kbh, a, c0 + kChunkRows, wave, lane);
    if (c0 + 32 * wave >= a.n) return;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        u32x4 k0, k1;
        k_operands(cur, score_row_code((uint32_t)(32 * wave + 16 * h + t.s16)), (uint32_t)t.kg,
                   k0, k1);
        const int32_t key0 = c0 + 32 * wave + 16 * h + 4 * t.kg;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            const f32x4 x = dots(k0, k1, t.q0[mb], t.q1[mb]);
            bool valid[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) valid[e] = key0 + e <= t.last[mb];
            if (P == kPassMax) {
#pragma unroll
                for (int e = 0; e < 4; ++e) t.m[mb] = valid[e] ? fmaxf(t.m[mb], x[e]) : t.m[mb];
                continue;
            }
            float w[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                w[e] = exp2f_fast(__builtin_fmaf(x[e], a.scale_log2, -t.ms[mb]));
                w[e] = valid[e] ? w[e] : 0.0f;
            }
            if (P == kPassSum) {
                t.sum[mb] += (w[0] + w[1]) + (w[2] + w[3]);
                continue;
            }
            if (P == kPassWriteNorm) {
#pragma unroll
                for (int e = 0; e < 4; ++e) w[e] *= t.inv[mb];
            }
            const uint32_t lo = to_bf16_pair(w[0], w[1]), hi = to_bf16_pair(w[2], w[3]);
            if (key0 < t.slen[mb]) {
                *reinterpret_cast<u32x2*>(Abh + t.sbase[mb] + key0) = u32x2{lo, hi};
                if (P == kPassWriteFused) t.sum[mb] = add_pair(hi, add_pair(lo, t.sum[mb]));
            }
        }
    }
}

template <int P>
__device__ void grow_pass(GLane& t, const ScoreArgs& a, const uint16_t* Kbh, uint16_t* Abh,
                          char LDS_AS* lds, int wave, int lane) {
    char LDS_AS* buf0 = lds;
    char LDS_AS* buf1 = lds + kBufBytes;
    dma_chunk(buf0, Kbh, a, 0, wave, lane);
    for (int c = 0; c < a.nchunks; ++c) {
        full_barrier();
        grow_chunk<P>(t, a, Kbh, Abh, (c & 1) ? buf0 : buf1, (c & 1) ? buf1 : buf0, c, wave, lane);
    }
    full_barrier();
}

// Merges the waves' per-row values (max or sum, fixed order) through LDS;
// every lane gets the workgroup value of its rows.
template <bool kMax>
__device__ __forceinline__ void grow_merge(float (&v)[2], char LDS_AS* lds, int wave, int lane) {
    // [wave][32 rows], past the chunk buffers (whose units beyond a head
    // width of 32 must stay zero)
    float LDS_AS* part = (float LDS_AS*)(lds + 2 * kBufBytes);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
        const float x = kMax ? row_max(v[mb]) : row_sum(v[mb]);
        if (lane < 16) part[wave * kGrowRows + 16 * mb + lane] = x;
    }
    lds_barrier();
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
        const int r = 16 * mb + (lane & 15);
        float x = part[r];
        for (int w = 1; w < kWaves; ++w) {
            const float y = part[w * kGrowRows + r];
            x = kMax ? fmaxf(x, y) : x + y;
        }
        v[mb] = x;
    }
    lds_barrier();
}

// One instantiation per head width and random layout: the local copy's kd
// and octet are constants that every (inlined) helper folds.
template <int KD, bool kOctet>
__global__ __launch_bounds__(kThreads)
void k_scores_sched(ScoreArgs args) {
    ScoreArgs a = args;
    a.kd = KD;
    a.octet = kOctet ? 1 : 0;
    extern __shared__ __align__(16) char lds_raw[];
    char LDS_AS* lds = (char LDS_AS*)lds_raw;
    const int lane = __lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int kg = lane >> 4, s16 = lane & 15;

    const WorkItem wi = work_item(blockIdx.x, a.per_xcd, a.total_items, a.grow_per_bh,
                                  a.tiles_per_bh, a.bh_per_xcd);
    if (!wi.valid) return;
    const int32_t bh = wi.bh;
    const int32_t sub = wi.sub;
    const int32_t b = bh / a.H, h = bh - b * a.H;
    const int32_t gr = a.num_graphs == 1 ? 0 : b;
    const int32_t n = a.n;
    uint16_t* Abh = a.A + a_block_offset(a.slot_off, a.num_graphs, a.H, b, h);
    const uint16_t* Kbh = a.K + (int64_t)bh * n * a.kd;
    const uint16_t* Qbh = a.Q + (int64_t)bh * n * a.kd;
    const int4* info = a.row_info + (int64_t)gr * n;

    // Zero row kChunkRows of both buffers (the key row of dummy slots); at
    // head width 32 both buffers whole, whose unloaded units stay zero.
    if (a.kd == 64) {
        if (threadIdx.x < 16)
            *reinterpret_cast<u32x4 LDS_AS*>(lds + (threadIdx.x >> 3) * kBufBytes +
                                            kChunkRows * kRowBytes + (threadIdx.x & 7) * 16) =
                u32x4{0u, 0u, 0u, 0u};
    } else {
        for (int u = threadIdx.x; u < 2 * kBufBytes / 16; u += kThreads)
            *reinterpret_cast<u32x4 LDS_AS*>(lds + 16 * u) = u32x4{0u, 0u, 0u, 0u};
        __syncthreads();
    }

    if (sub < a.grow_per_bh) {
        GLane t;
        t.kg = kg;
        t.s16 = s16;
        const int64_t* sp = a.seg_ptr + (int64_t)gr * (n + 1);
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            const int q = sub * kGrowRows + 16 * mb + s16;
            t.i[mb] = q < a.g ? a.G[q] : -1;
            t.last[mb] = t.i[mb] < 0 ? -1 : (a.causal ? t.i[mb] : n - 1);
            t.sbase[mb] = t.i[mb] >= 0 ? sp[t.i[mb]] : 0;
            t.slen[mb] = t.i[mb] >= 0 ? (int32_t)(sp[t.i[mb] + 1] - sp[t.i[mb]]) : 0;
            const int32_t qi = t.i[mb] >= 0 ? t.i[mb] : 0;
            t.q0[mb] = load16(Qbh + (int64_t)qi * a.kd + 8 * kg);
            t.q1[mb] = a.kd == 64 ? load16(Qbh + (int64_t)qi * a.kd + 32 + 8 * kg)
                                  : u32x4{0u, 0u, 0u, 0u};
            t.m[mb] = -INFINITY;
            t.sum[mb] = 0.0f;
            t.inv[mb] = 0.0f;
        }
        // Shift: the row's own score (a global row reads its own column).
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            const int32_t qi = t.i[mb] >= 0 ? t.i[mb] : 0;
            const u32x4 k0 = load16(Kbh + (int64_t)qi * a.kd + 8 * kg);
            const u32x4 k1 = a.kd == 64 ? load16(Kbh + (int64_t)qi * a.kd + 32 + 8 * kg)
                                        : u32x4{0u, 0u, 0u, 0u};
            float d = 0.0f;
#pragma unroll
            for (int u = 0; u < 4; ++u)
                d = dot2_bf16(t.q1[mb][u], k1[u], dot2_bf16(t.q0[mb][u], k0[u], d));
            t.m[mb] = row_sum(d);
            t.ms[mb] = t.m[mb] * a.scale_log2;
        }
        for (int attempt = 0; attempt < 2; ++attempt) {
            if (attempt == 1) {
                // Some row's weights reached 2^64: the exact maxima instead.
#pragma unroll
                for (int mb = 0; mb < 2; ++mb) {
                    t.m[mb] = -INFINITY;
                    t.sum[mb] = 0.0f;
                }
                grow_pass<kPassMax>(t, a, Kbh, Abh, lds, wave, lane);
                grow_merge<true>(t.m, lds, wave, lane);
#pragma unroll
                for (int mb = 0; mb < 2; ++mb) t.ms[mb] = t.m[mb] * a.scale_log2;
            }
            if (a.normalized) {
                grow_pass<kPassSum>(t, a, Kbh, Abh, lds, wave, lane);
            } else {
                grow_pass<kPassWriteFused>(t, a, Kbh, Abh, lds, wave, lane);
            }
            grow_merge<false>(t.sum, lds, wave, lane);
            const bool big = (t.i[0] >= 0 && !(t.sum[0] < kSumLimit)) ||
                             (t.i[1] >= 0 && !(t.sum[1] < kSumLimit));
            if (attempt == 1 || !__syncthreads_or(big)) break;
        }
        if (a.normalized) {
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) t.inv[mb] = t.i[mb] >= 0 ? 1.0f / t.sum[mb] : 0.0f;
            grow_pass<kPassWriteNorm>(t, a, Kbh, Abh, lds, wave, lane);
        } else if (a.row_scale != nullptr && wave == 0 && kg == 0) {
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
                if (t.i[mb] >= 0) a.row_scale[(int64_t)bh * n + t.i[mb]] = 1.0f / t.sum[mb];
        }
        return;
    }

    // ---------------- row tile --------------------------------------------
    SLane t;
    t.kg = kg;
    t.s16 = s16;
    t.r0w = (sub - a.grow_per_bh) * kTileRows + kRowBlock * wave;
    const bool active = t.r0w < n;
    t.i = t.r0w + s16;
    t.ri = make_int4(0, 0, -1, 0);
    if (t.i < n) t.ri = info[t.i];
    t.rok = t.i < n && t.ri.z >= 0;
    t.block_ok = __all(t.rok);   // wave-uniform
    t.lo = max(t.i - a.radius, 0);
    const int32_t whi = a.causal ? t.i : min(t.i + a.radius, n - 1);
    t.span = (uint32_t)(whi - t.lo);
    const int32_t qi = min(t.i, n - 1);
    t.q0 = load16(Qbh + (int64_t)qi * a.kd + 8 * kg);
    t.q1 = a.kd == 64 ? load16(Qbh + (int64_t)qi * a.kd + 32 + 8 * kg) : u32x4{0u, 0u, 0u, 0u};
    t.m = -INFINITY;
    t.ms = 0.0f;
    t.sum = 0.0f;
    t.inv = 0.0f;
    const int32_t wr_last = min(t.r0w + kRowBlock - 1, n - 1);
    t.band_lo = max(t.r0w - a.radius, 0) & ~15;
    t.band_hi = a.causal ? wr_last : min(n - 1, wr_last + a.radius);
    const int64_t rb = active ? t.r0w / kRowBlock : 0;
    t.cptr = a.grp_cptr + ((int64_t)gr * a.nrb + rb) * (a.nchunks + 1);
    t.goff = a.grp_off[gr];
    t.rbase = (uint32_t)a.seg_ptr[(int64_t)gr * (n + 1) + n];
    t.gr = gr;
    t.abase = a.octet ? t.rbase + (uint32_t)(128 * a.rb_roff[(int64_t)gr * (a.nrb + 1) + rb]) : 0u;
    t.po = u32x2{0u, 0u};
    t.pk = u32x4{0u, 0u, 0u, 0u};
    t.pr = 0u;

    // Staged global rows of K and their positions.
    const int gpad = (a.g + 31) & ~31;
    char LDS_AS* zg = lds + 2 * kBufBytes;
    const int32_t LDS_AS* gidx = (const int32_t LDS_AS*)(zg + gpad * kRowBytes);
    for (int idx = threadIdx.x; idx < gpad * 8; idx += kThreads) {
        const int q = idx >> 3, lu = idx & 7;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (q < a.g && lu * 8 < a.kd) v = load16(Kbh + (int64_t)a.G[q] * a.kd + lu * 8);
        *reinterpret_cast<u32x4 LDS_AS*>(zg + ((score_row_code((uint32_t)q) ^ (uint32_t)lu) << 4)) =
            v;
    }
    for (int q = threadIdx.x; q < gpad; q += kThreads)
        ((int32_t LDS_AS*)gidx)[q] = q < a.g ? a.G[q] : 0;

    // Shift: the row's own score q_i . k_i. The self-loop is an edge of
    // every row, so this is at most the row maximum (the 4 lanes of a row
    // hold 16 channels each).
    {
        const u32x4 k0 = load16(Kbh + (int64_t)qi * a.kd + 8 * kg);
        const u32x4 k1 = a.kd == 64 ? load16(Kbh + (int64_t)qi * a.kd + 32 + 8 * kg)
                                    : u32x4{0u, 0u, 0u, 0u};
        float d = 0.0f;
#pragma unroll
        for (int u = 0; u < 4; ++u) d = dot2_bf16(t.q1[u], k1[u], dot2_bf16(t.q0[u], k0[u], d));
        t.m = row_sum(d);
    }
    t.ms = t.m * a.scale_log2;
    for (int attempt = 0; attempt < 2; ++attempt) {
        if (attempt == 1) {
            // Some row's weights reached 2^64: the exact maxima instead.
            t.m = -INFINITY;
            tile_pass<kPassMax>(t, a, Kbh, Abh, lds, gpad, active, wave, lane);
            t.m = row_max(t.m);
            t.ms = t.m * a.scale_log2;
            t.sum = 0.0f;
        }
        if (a.normalized) {
            tile_pass<kPassSum>(t, a, Kbh, Abh, lds, gpad, active, wave, lane);
        } else {
            tile_pass<kPassWriteFused>(t, a, Kbh, Abh, lds, gpad, active, wave, lane);
        }
        t.sum = row_sum(t.sum);
        if (attempt == 1 || !__syncthreads_or(t.rok && !(t.sum < kSumLimit))) break;
    }
    if (a.normalized) {
        t.inv = t.rok ? 1.0f / t.sum : 0.0f;   // rows without edges here write zeros only
        tile_pass<kPassWriteNorm>(t, a, Kbh, Abh, lds, gpad, active, wave, lane);
    } else if (a.row_scale != nullptr && t.rok && kg == 0) {
        a.row_scale[(int64_t)bh * n + t.i] = 1.0f / t.sum;
    }
}

}  // namespace

bool fast_scores_supported(const diffuser_graph& g, const attn_shape& s) {
    if (!g.structured || !g.scheduled || s.dtype != DIFFUSER_BF16 || (s.d != 64 && s.d != 32))
        return false;
    if (g.num_global > kMaxGlobal) return false;
    for (int64_t x : g.slots)
        if (x >= (1ll << 31)) return false;
    return true;
}

hipError_t launch_scores_fast(const diffuser_graph& g, const attn_shape& s, const void* Q,
                              const void* K, void* A, float* row_scale, float scale_log2,
                              bool normalized, hipStream_t st) {
    ScoreArgs a;
    a.n = (int32_t)g.n;
    a.H = s.H;
    a.num_graphs = g.num_graphs;
    a.radius = (int32_t)std::min<int64_t>(g.radius, g.n);
    a.g = g.num_global;
    a.causal = g.causal;
    a.nchunks = (int32_t)((g.n + kChunkRows - 1) / kChunkRows);
    a.nrb = (int32_t)((g.n + kRowBlock - 1) / kRowBlock);
    a.slot_off = g.d_slot_off;
    a.seg_ptr = g.d_seg_ptr;
    a.row_info = reinterpret_cast<const int4*>(g.d_row_info);
    a.G = g.d_global;
    a.grp_off = g.d_grp_off;
    a.grp_cptr = g.d_grp_cptr;
    a.sched_row = g.d_sched_row;
    a.sched_off = g.d_sched_off;
    a.rnd_cnt = g.d_rnd_cnt;
    a.rb_oct = g.d_rb_oct;
    a.rb_roff = g.d_rb_roff;
    a.octet = g.octet() ? 1 : 0;
    a.sched_k = g.d_sched_k;
    a.Q = static_cast<const uint16_t*>(Q);
    a.K = static_cast<const uint16_t*>(K);
    a.A = static_cast<uint16_t*>(A);
    a.row_scale = row_scale;
    a.scale_log2 = scale_log2;
    a.normalized = normalized ? 1 : 0;
    a.kd = s.d;
    const int32_t BH = s.B * s.H;
    a.tiles_per_bh = (int32_t)((g.n + kTileRows - 1) / kTileRows);
    a.grow_per_bh = (g.num_global + kGrowRows - 1) / kGrowRows;
    a.total_items = BH * (a.tiles_per_bh + a.grow_per_bh);
    a.bh_per_xcd = BH % 8 == 0 ? BH / 8 : 0;
    a.per_xcd = a.bh_per_xcd > 0 ? a.bh_per_xcd * (a.tiles_per_bh + a.grow_per_bh)
                                 : (a.total_items + 7) / 8;
    // Dynamic LDS above 64 KB is enabled once per device and instantiation.
    static int attr_device[4] = {-1, -1, -1, -1};
    const int which = (s.d == 64 ? 0 : 1) + (g.octet() ? 2 : 0);
    const void* kerns[4] = {reinterpret_cast<const void*>(&k_scores_sched<64, false>),
                            reinterpret_cast<const void*>(&k_scores_sched<32, false>),
                            reinterpret_cast<const void*>(&k_scores_sched<64, true>),
                            reinterpret_cast<const void*>(&k_scores_sched<32, true>)};
    if (attr_device[which] != g.device) {
        hipError_t e = hipFuncSetAttribute(kerns[which], hipFuncAttributeMaxDynamicSharedMemorySize,
                                           kLdsBytes);
        if (e != hipSuccess) return e;
        attr_device[which] = g.device;
    }
    const int gpad = (g.num_global + 31) & ~31;
    const size_t lds = (size_t)2 * kBufBytes + (size_t)gpad * (kRowBytes + 4) +
                       (size_t)kWaves * kStageBytes;
    const dim3 grid((unsigned)(8 * a.per_xcd));
    switch (which) {
        case 0: hipLaunchKernelGGL((k_scores_sched<64, false>), grid, dim3(kThreads), lds, st, a); break;
        case 1: hipLaunchKernelGGL((k_scores_sched<32, false>), grid, dim3(kThreads), lds, st, a); break;
        case 2: hipLaunchKernelGGL((k_scores_sched<64, true>), grid, dim3(kThreads), lds, st, a); break;
        default: hipLaunchKernelGGL((k_scores_sched<32, true>), grid, dim3(kThreads), lds, st, a); break;
    }
    return hipGetLastError();
}

}  // namespace diffuser
