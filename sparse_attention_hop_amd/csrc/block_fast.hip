// Block-tile kernels for block graphs ("1.2.1 Static sparsity", section 2,
// eq. 13: every row of query block I reads whole key blocks), block = 64,
// bf16 storage, head width 64. Every (query block, key block) pair is a
// dense 64 x 64 tile, so all of its work is MFMA work:
//  * scores ("Diffuser" reading notes, section 2.1, eqs. S.1-S.5):
//      D[key][row] = sum_c K[key][c] Q[row][c] per 16 x 16 tile
//    (v_mfma_f32_16x16x32_bf16, two per tile for the 64 channels); the K
//    operand is 8 channels of one key row, read from LDS with
//    ds_read_b128, the Q^T operand 8 channels of the lane's row, held in
//    registers. The shift m_i is the row's own score (the diagonal block is
//    among its key blocks, so m_i is at most the row maximum; a row whose
//    weights reach 2^64 is redone with the exact maximum). One pass writes
//    exp(s - m_i) (fused: unnormalised, with c_i = 1 / (sum of the stored
//    weights); normalised: a sum pass, then a pass that writes the weights
//    over their sum). The parts of a split global query block take the
//    exact maximum from a pass of their own.
//  * one diffusion step (section 2.4, eq. S.7, as the scheduled kernel):
//      D[channel][row] += Z^T[channel][key] W^T[key][row]
//    over 32-key steps: the Z^T operand from LDS with ds_read_b64_tr_b16,
//    the W^T operand 8 consecutive weights of the lane's row.
// A workgroup is one (batch, head, query block): 4 waves of 16 rows. It
// streams the key blocks of its query block through two LDS buffers with
// direct global-to-LDS loads, the next block's load in flight while the
// current one is used. Workgroups are numbered so that each XCD works
// through a contiguous range of (batch, head) pairs, whose K or Z_k then
// stays in that XCD's L2.
#include "internal.h"
#include "mfma_util.h"

namespace diffuser {
namespace {

constexpr int kWave = 64;
constexpr int kWaves = 4;
constexpr int kThreads = kWave * kWaves;
constexpr int kBlk = 64;                      // tokens per block
constexpr int kD = 64;                        // head width
constexpr int kNB = 4;                        // 16-channel blocks
constexpr int kRowBytes = kD * 2;
constexpr int kBufBytes = kBlk * kRowBytes;   // one key block of K or Z_k
static_assert(kWaves * 16 == kBlk, "a wave per 16 rows of the query block");
constexpr int kSplit = 8;                     // key blocks per part of a global query block
// A row whose weights (shifted by less than its maximum) sum to this or
// more is redone with its exact maximum, far from the overflow threshold.
constexpr float kSumLimit = 18446744073709551616.0f;   // 2^64

struct BlockArgs {
    int64_t n;
    int32_t H, num_graphs, nblocks;
    const int64_t* slot_off;   // [graphs + 1]
    const int32_t* bptr;       // [graphs][nblocks + 1], absolute
    const int32_t* bcol;
    const uint16_t* X;         // Q (scores) or A (diffusion)
    const uint16_t* Y;         // K (scores) or Z_k (diffusion)
    const uint16_t* V;
    uint16_t* out;             // A (scores) or Z_{k+1} (diffusion)
    float* row_scale;
    float scale_log2, keep, restart;
    int32_t normalized, per_xcd, total;
    int32_t gblocks, gparts;   // global query blocks and the parts each is split into (0: none)
    int32_t total_parts;       // B*H*gblocks*gparts
    float* part;               // diffusion: [B*H][gblocks][gparts][64][64] fp32 partial sums;
                               // scores: pmax then psum, each [B*H][gblocks][gparts][64]
};

// The query block's key-block list and where its rows' weight slots start.
struct BlockRows {
    int32_t k0, nk;      // key blocks bcol[k0 .. k0 + nk)
    int64_t row0;        // slot of row I*64 + 0 within the (b, h) block of A
};

__device__ __forceinline__ BlockRows block_rows(const BlockArgs& a, int32_t gr, int32_t I) {
    const int32_t* bp = a.bptr + (int64_t)gr * (a.nblocks + 1);
    BlockRows r;
    r.k0 = bp[I];
    r.nk = bp[I + 1] - r.k0;
    r.row0 = (int64_t)(r.k0 - bp[0]) * kBlk * kBlk;
    return r;
}

__device__ __forceinline__ uint32_t lds_addr(const char LDS_AS* p) {
    return (uint32_t)(uintptr_t)p;
}

// Work item of workgroup blk (score and diffusion kernels): within a
// (batch, head) pair the parts of its global query blocks come first (gq = I, keys of part p are
// list entries kSplit p ..), then the other query blocks whole (p = -1).
struct DiffItem {
    int32_t bh, I, p;
    bool valid;
};

__device__ __forceinline__ DiffItem diff_item(uint32_t blk, const BlockArgs& a) {
    const int32_t per_bh = a.gblocks * a.gparts + (a.nblocks - a.gblocks);
    const int32_t item = (int32_t)(blk & 7u) * a.per_xcd + (int32_t)(blk >> 3);
    DiffItem it{0, 0, -1, false};
    if (item >= a.total) return it;
    it.bh = item / per_bh;
    const int32_t r = item - it.bh * per_bh;
    if (r < a.gblocks * a.gparts) {
        it.I = r / a.gparts;
        it.p = r - it.I * a.gparts;
    } else {
        it.I = a.gblocks + (r - a.gblocks * a.gparts);
    }
    it.valid = true;
    return it;
}

// ---------------------------------------------------------------------------
// Scores.

// Direct loads of key block J of K into `buf` in the score layout: in LDS
// block 2 w + j (8 rows) lane l writes 16-byte unit l % 8 of row
// 8 (2 w + j) + l / 8, which holds the row's logical unit
// (l % 8) ^ (score_row_code(row) & 7).
__device__ __forceinline__ void dma_k(char LDS_AS* buf, const uint16_t* Kbh, int32_t J, int wave,
                                      int lane) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int blk = 2 * wave + j;
        const uint32_t pr = (uint32_t)(blk * 8 + (lane >> 3));
        const uint32_t lu = (uint32_t)(lane & 7) ^ (score_row_code(pr) & 7u);
        dma16(Kbh + ((int64_t)J * kBlk + pr) * kD + lu * 8, buf + blk * 1024);
    }
}

// Dot products of 16 keys (rows 16 t .. + 15 of the block in `buf`) with
// the lane's row: D[key 16 t + 4 kg + e][row].
__device__ __forceinline__ f32x4 key_tile(const char LDS_AS* buf, int t, uint32_t kg, int s16,
                                          const u32x4& q0, const u32x4& q1) {
    const uint32_t o = (score_row_code((uint32_t)(16 * t + s16)) ^ kg) << 4;
    const u32x4 k0 = *reinterpret_cast<const u32x4 LDS_AS*>(buf + o);
    const u32x4 k1 = *reinterpret_cast<const u32x4 LDS_AS*>(buf + (o ^ 64u));
    return mfma_bf16(k1, q1, mfma_bf16(k0, q0, f32x4{0.f, 0.f, 0.f, 0.f}));
}

enum BlockPass { kBMax = 0, kBSum = 1, kBWrite = 2, kBWriteNorm = 3 };

// One pass over the query block's key blocks. kBMax: m = the row maximum
// of the dot products; kBSum: sum of the weights exp(s - m); kBWrite:
// writes them (bf16) and sums them as stored; kBWriteNorm: writes them
// times inv.
// Key blocks are list entries [kb0, kb1) of the query block; Arow points at
// the slots of entry kb0.
template <int P>
__device__ __forceinline__ void score_pass(const BlockArgs& a, const BlockRows& br, int32_t kb0,
                                           int32_t kb1, const uint16_t* Kbh, uint16_t* Arow,
                                           char LDS_AS* lds, int wave, int lane, const u32x4& q0,
                                           const u32x4& q1, float& m, float ms, float& sum,
                                           float inv) {
    const uint32_t kg = (uint32_t)(lane >> 4);
    const int s16 = lane & 15;
    const int32_t nk = kb1 - kb0;
    dma_k(lds, Kbh, a.bcol[br.k0 + kb0], wave, lane);
    for (int32_t kb = 0; kb < nk; ++kb) {
        full_barrier();   // key block kb in LDS, kb - 1 done by every wave
        const char LDS_AS* cur = lds + (kb & 1) * kBufBytes;
        if (kb + 1 < nk)
            dma_k(lds + ((kb + 1) & 1) * kBufBytes, Kbh, a.bcol[br.k0 + kb0 + kb + 1], wave, lane);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const f32x4 x = key_tile(cur, t, kg, s16, q0, q1);
            if (P == kBMax) {
                m = fmaxf(fmaxf(m, x[0]), fmaxf(fmaxf(x[1], x[2]), x[3]));
                continue;
            }
            float w[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                w[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[e], a.scale_log2, -ms));
            if (P == kBWriteNorm) {
#pragma unroll
                for (int e = 0; e < 4; ++e) w[e] *= inv;
            }
            if (P == kBSum) {
                // Normalised mode divides by the sum of the exact weights.
                sum += (w[0] + w[1]) + (w[2] + w[3]);
                continue;
            }
            const uint32_t lo = to_bf16_pair(w[0], w[1]), hi = to_bf16_pair(w[2], w[3]);
            // Fused mode: c_i is over the weights as stored.
            if (P == kBWrite) sum += (bf16_lo(lo) + bf16_hi(lo)) + (bf16_lo(hi) + bf16_hi(hi));
            if (P == kBWrite || P == kBWriteNorm)
                *reinterpret_cast<u32x2*>(Arow + (int64_t)kb * kBlk + 16 * t + 4 * kg) =
                    u32x2{lo, hi};
        }
    }
    __syncthreads();   // every wave is done with the buffers
}

// acc + a.lo b.lo + a.hi b.hi for two packed bf16 pairs (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), acc, false);
}

__device__ __forceinline__ float quad_max(float x) {
    x = fmaxf(x, __shfl_xor(x, 16));
    return fmaxf(x, __shfl_xor(x, 32));
}

__device__ __forceinline__ float quad_sum(float x) {
    x += __shfl_xor(x, 16);
    return x + __shfl_xor(x, 32);
}

// Partial row maxima of the parts of the global query blocks (fused mode):
// pmax[(bh, gq, part)][row].
__global__ __launch_bounds__(kThreads)
void k_block_gmax(BlockArgs a) {
    __shared__ __align__(16) char lds_raw[2 * kBufBytes];
    char LDS_AS* lds = (char LDS_AS*)lds_raw;
    const int32_t per_bh = a.gblocks * a.gparts;
    const int32_t bh = (int32_t)blockIdx.x / per_bh, r = (int32_t)blockIdx.x % per_bh;
    const int32_t I = r / a.gparts, p = r % a.gparts;
    const int lane = __lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int kg = lane >> 4, s16 = lane & 15;
    const int32_t b = bh / a.H;
    const int32_t gr = a.num_graphs == 1 ? 0 : b;
    const int64_t n = a.n;
    const BlockRows br = block_rows(a, gr, I);
    const int32_t kb0 = kSplit * p, kb1 = min(br.nk, kb0 + kSplit);
    const int64_t row = (int64_t)I * kBlk + 16 * wave + s16;
    const uint16_t* Qbh = a.X + (int64_t)bh * n * kD;
    const uint16_t* Kbh = a.Y + (int64_t)bh * n * kD;
    const u32x4 q0 = load16(Qbh + row * kD + 8 * kg);
    const u32x4 q1 = load16(Qbh + row * kD + 32 + 8 * kg);
    float m = -INFINITY, sum = 0.0f;
    score_pass<kBMax>(a, br, kb0, kb1, Kbh, nullptr, lds, wave, lane, q0, q1, m, 0.0f, sum, 0.0f);
    m = quad_max(m);
    if (kg == 0)
        a.part[((int64_t)bh * a.gblocks + I) * a.gparts * kBlk + p * kBlk + 16 * wave + s16] = m;
}

__global__ __launch_bounds__(kThreads)
void k_block_scores(BlockArgs a) {
    __shared__ __align__(16) char lds_raw[2 * kBufBytes];
    char LDS_AS* lds = (char LDS_AS*)lds_raw;
    const DiffItem it = diff_item(blockIdx.x, a);
    if (!it.valid) return;
    const int lane = __lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int kg = lane >> 4, s16 = lane & 15;
    const int32_t b = it.bh / a.H, h = it.bh - b * a.H;
    const int32_t gr = a.num_graphs == 1 ? 0 : b;
    const int64_t n = a.n;
    const BlockRows br = block_rows(a, gr, it.I);
    const int64_t row = (int64_t)it.I * kBlk + 16 * wave + s16;
    const uint16_t* Qbh = a.X + (int64_t)it.bh * n * kD;
    const uint16_t* Kbh = a.Y + (int64_t)it.bh * n * kD;
    uint16_t* Arow = a.out + a_block_offset(a.slot_off, a.num_graphs, a.H, b, h) + br.row0 +
                     (int64_t)(row - (int64_t)it.I * kBlk) * br.nk * kBlk;
    const u32x4 q0 = load16(Qbh + row * kD + 8 * kg);
    const u32x4 q1 = load16(Qbh + row * kD + 32 + 8 * kg);
    float m = -INFINITY, sum = 0.0f;
    if (it.p >= 0) {
        // A part of a global query block (fused mode): the row maximum from
        // the parts' maxima, one writing pass over the part's key blocks,
        // its sum of stored weights into psum (after the maxima).
        const int32_t kb0 = kSplit * it.p, kb1 = min(br.nk, kb0 + kSplit);
        const float* pm = a.part + ((int64_t)it.bh * a.gblocks + it.I) * a.gparts * kBlk +
                          16 * wave + s16;
        for (int32_t p = 0; p < a.gparts; ++p) m = fmaxf(m, pm[p * kBlk]);
        score_pass<kBWrite>(a, br, kb0, kb1, Kbh, Arow + (int64_t)kb0 * kBlk, lds, wave, lane, q0,
                            q1, m, m * a.scale_log2, sum, 0.0f);
        sum = quad_sum(sum);
        float* ps = a.part + ((int64_t)a.total_parts +
                              ((int64_t)it.bh * a.gblocks + it.I) * a.gparts +
                              it.p) * kBlk;
        if (kg == 0) ps[16 * wave + s16] = sum;
        return;
    }
    // Shift: the row's own score (the diagonal block is among its key
    // blocks), at most the row maximum; rows whose weights reach 2^64 are
    // redone with the exact maximum.
    {
        const u32x4 k0 = load16(Kbh + row * kD + 8 * kg);
        const u32x4 k1 = load16(Kbh + row * kD + 32 + 8 * kg);
        float d = 0.0f;
#pragma unroll
        for (int u = 0; u < 4; ++u) d = dot2_bf16(q1[u], k1[u], dot2_bf16(q0[u], k0[u], d));
        m = quad_sum(d);
    }
    float ms = m * a.scale_log2;
    for (int attempt = 0; attempt < 2; ++attempt) {
        if (attempt == 1) {
            m = -INFINITY;
            score_pass<kBMax>(a, br, 0, br.nk, Kbh, Arow, lds, wave, lane, q0, q1, m, 0.0f, sum,
                              0.0f);
            m = quad_max(m);
            ms = m * a.scale_log2;
        }
        sum = 0.0f;
        if (a.normalized)
            score_pass<kBSum>(a, br, 0, br.nk, Kbh, Arow, lds, wave, lane, q0, q1, m, ms, sum,
                              0.0f);
        else
            score_pass<kBWrite>(a, br, 0, br.nk, Kbh, Arow, lds, wave, lane, q0, q1, m, ms, sum,
                                0.0f);
        sum = quad_sum(sum);
        if (attempt == 1 || !__syncthreads_or(!(sum < kSumLimit))) break;
    }
    if (a.normalized)
        score_pass<kBWriteNorm>(a, br, 0, br.nk, Kbh, Arow, lds, wave, lane, q0, q1, m, ms, sum,
                                1.0f / sum);
    else if (a.row_scale != nullptr && kg == 0)
        a.row_scale[(int64_t)it.bh * n + row] = 1.0f / sum;
}

// c_i of the global query blocks' rows from their parts' sums (in part
// order): one workgroup per (batch, head, global query block).
__global__ __launch_bounds__(kThreads)
void k_block_gsum(BlockArgs a) {
    const int32_t bh = (int32_t)blockIdx.x / a.gblocks, I = (int32_t)blockIdx.x % a.gblocks;
    const float* ps =
        a.part + ((int64_t)a.total_parts + ((int64_t)bh * a.gblocks + I) * a.gparts) * kBlk;
    for (int r = threadIdx.x; r < kBlk; r += kThreads) {
        float sum = 0.0f;
        for (int32_t p = 0; p < a.gparts; ++p) sum += ps[p * kBlk + r];
        a.row_scale[(int64_t)bh * a.n + (int64_t)I * kBlk + r] = 1.0f / sum;
    }
}

// ---------------------------------------------------------------------------
// Diffusion step.

__device__ __forceinline__ i16x4 tr_read(uint32_t addr) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LDS_AS*)(uintptr_t)addr);
}

// Direct loads of key block J of Z_k into `buf` in the diffusion layout
// (quarters permuted by key_row_code): in LDS block 2 w + j lane l writes
// 16-byte unit l % 8 of row 8 (2 w + j) + l / 8, which holds the row's
// logical unit (l % 8) ^ (2 (key_row_code(row) & 3)).
__device__ __forceinline__ void dma_z(char LDS_AS* buf, const uint16_t* Zbh, int32_t J, int wave,
                                      int lane) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int blk = 2 * wave + j;
        const uint32_t pr = (uint32_t)(blk * 8 + (lane >> 3));
        const uint32_t lu = (uint32_t)(lane & 7) ^ ((key_row_code(pr) & 3u) << 1);
        dma16(Zbh + ((int64_t)J * kBlk + pr) * kD + lu * 8, buf + blk * 1024);
    }
}

__global__ __launch_bounds__(kThreads)
void k_block_diffuse(BlockArgs a) {
    __shared__ __align__(128) char lds_raw[2 * kBufBytes];
    char LDS_AS* lds = (char LDS_AS*)lds_raw;
    const DiffItem it = diff_item(blockIdx.x, a);
    if (!it.valid) return;
    const int lane = __lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int kg = lane >> 4, s16 = lane & 15;
    const uint32_t a8 = 8u * (lane & 3), q4 = (lane >> 2) & 3;
    const int32_t b = it.bh / a.H, h = it.bh - b * a.H;
    const int32_t gr = a.num_graphs == 1 ? 0 : b;
    const int64_t n = a.n;
    const BlockRows br = block_rows(a, gr, it.I);
    const int64_t row = (int64_t)it.I * kBlk + 16 * wave + s16;   // W^T column of this lane
    const uint16_t* Zbh = a.Y + (int64_t)it.bh * n * kD;
    // List entries [kb0, kb1) of the query block's key blocks.
    const int32_t kb0 = it.p < 0 ? 0 : kSplit * it.p;
    const int32_t kb1 = it.p < 0 ? br.nk : min(br.nk, kb0 + kSplit);
    const uint16_t* Arow = a.X + a_block_offset(a.slot_off, a.num_graphs, a.H, b, h) + br.row0 +
                           (int64_t)(row - (int64_t)it.I * kBlk) * br.nk * kBlk +
                           (int64_t)kb0 * kBlk;
    // Transposed-read source rows of the two 32-key steps.
    uint32_t r1[2], r2[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        r1[ks] = a8 + (key_row_code(32u * ks + 8u * kg + q4) << 5);
        r2[ks] = a8 + (key_row_code(32u * ks + 8u * kg + 4u + q4) << 5);
    }
    f32x4 acc[kNB];
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    u32x4 w[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) w[ks] = load16(Arow + 32 * ks + 8 * kg);
    const int32_t nk = kb1 - kb0;
    dma_z(lds, Zbh, a.bcol[br.k0 + kb0], wave, lane);
    for (int32_t kb = 0; kb < nk; ++kb) {
        full_barrier();   // key block kb and its weights in, kb - 1 done by every wave
        const uint32_t base = lds_addr(lds + (kb & 1) * kBufBytes);
        u32x4 wn[2] = {w[0], w[1]};
        if (kb + 1 < nk) {
            dma_z(lds + ((kb + 1) & 1) * kBufBytes, Zbh, a.bcol[br.k0 + kb0 + kb + 1], wave, lane);
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                wn[ks] = load16(Arow + (int64_t)(kb + 1) * kBlk + 32 * ks + 8 * kg);
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
            for (int nb = 0; nb < kNB; ++nb) {
                const i16x4 lo = tr_read((base + r1[ks]) ^ ((uint32_t)nb << 5));
                const i16x4 hi = tr_read((base + r2[ks]) ^ ((uint32_t)nb << 5));
                const u32x2 l = __builtin_bit_cast(u32x2, lo), hh = __builtin_bit_cast(u32x2, hi);
                acc[nb] = mfma_bf16(u32x4{l[0], l[1], hh[0], hh[1]}, w[ks], acc[nb]);
            }
        }
        w[0] = wn[0];
        w[1] = wn[1];
    }
    if (it.p >= 0) {
        // A part of a global query block: fp32 partial sums, added later.
        float* dst = a.part + (((int64_t)it.bh * a.gblocks + it.I) * a.gparts + it.p) * kBlk * kD +
                     (int64_t)(16 * wave + s16) * kD + 4 * kg;
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb) *reinterpret_cast<f32x4*>(dst + 16 * nb) = acc[nb];
        return;
    }
    // Restart and store: lane holds channels 16 nb + 4 kg .. + 3 of its row.
    const float keep =
        a.row_scale != nullptr ? a.keep * a.row_scale[(int64_t)it.bh * n + row] : a.keep;
    const int64_t o = ((int64_t)it.bh * n + row) * kD + 4 * kg;
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) {
        const u32x2 v = *reinterpret_cast<const u32x2*>(a.V + o + 16 * nb);
        u32x2 z;
        z[0] = to_bf16_pair(keep * acc[nb][0] + a.restart * bf16_lo(v[0]),
                            keep * acc[nb][1] + a.restart * bf16_hi(v[0]));
        z[1] = to_bf16_pair(keep * acc[nb][2] + a.restart * bf16_lo(v[1]),
                            keep * acc[nb][3] + a.restart * bf16_hi(v[1]));
        *reinterpret_cast<u32x2*>(a.out + o + 16 * nb) = z;
    }
}

// Sum of the parts of each global query block (in part order), restart and
// store: one thread per output element, kBlk * kD / kThreads workgroups per
// (batch, head, global query block).
constexpr int kCombineGroups = kBlk * kD / kThreads;

__global__ __launch_bounds__(kThreads)
void k_block_combine(BlockArgs a) {
    const int32_t q = (int32_t)blockIdx.x / kCombineGroups;
    const int32_t bh = q / a.gblocks, I = q % a.gblocks;
    const int idx = ((int)blockIdx.x % kCombineGroups) * kThreads + (int)threadIdx.x;
    const int64_t n = a.n;
    const float* src = a.part + ((int64_t)bh * a.gblocks + I) * a.gparts * kBlk * kD + idx;
    float sum = 0.0f;
    for (int p = 0; p < a.gparts; ++p) sum += src[(int64_t)p * kBlk * kD];
    const int64_t row = (int64_t)I * kBlk + idx / kD;
    const int64_t o = ((int64_t)bh * n + row) * kD + idx % kD;
    const float keep =
        a.row_scale != nullptr ? a.keep * a.row_scale[(int64_t)bh * n + row] : a.keep;
    a.out[o] = (uint16_t)f32_to_bf16(keep * sum + a.restart * bf16_to_f32(a.V[o]));
}

// Global query blocks read every block: with more than kSplit key blocks
// they are split into parts of kSplit, unless the item and thread counts
// of the launches would then pass the int32 range (they run whole).
int32_t global_parts(const diffuser_graph& g, const attn_shape& s) {
    if (g.global_blocks == 0 || g.nblocks <= kSplit) return 0;
    const int64_t parts = (g.nblocks + kSplit - 1) / kSplit;
    const int64_t items = (int64_t)s.B * s.H * (g.global_blocks * parts + g.nblocks);
    if (items * kCombineGroups >= (1ll << 31)) return 0;
    return (int32_t)parts;
}

BlockArgs block_args(const diffuser_graph& g, const attn_shape& s) {
    BlockArgs a{};
    a.n = g.n;
    a.H = s.H;
    a.num_graphs = g.num_graphs;
    a.nblocks = (int32_t)g.nblocks;
    a.slot_off = g.d_slot_off;
    a.bptr = g.d_bptr;
    a.bcol = g.d_bcol;
    return a;
}

}  // namespace

size_t block_part_bytes(const diffuser_graph& g, const attn_shape& s) {
    return (size_t)s.B * s.H * g.global_blocks * global_parts(g, s) * kBlk * kD * sizeof(float);
}

bool fast_block_supported(const diffuser_graph& g, const attn_shape& s) {
    if (!g.blocked || g.block != kBlk || s.dtype != DIFFUSER_BF16 || s.d != kD) return false;
    if ((int64_t)s.B * s.H * g.nblocks >= (1ll << 31)) return false;
    for (int64_t x : g.slots)
        if (x >= (1ll << 31)) return false;
    return true;
}

hipError_t launch_block_scores(const diffuser_graph& g, const attn_shape& s, const void* Q,
                               const void* K, void* A, float* row_scale, float scale_log2,
                               bool normalized, float* part, hipStream_t st) {
    BlockArgs a = block_args(g, s);
    a.X = static_cast<const uint16_t*>(Q);
    a.Y = static_cast<const uint16_t*>(K);
    a.out = static_cast<uint16_t*>(A);
    a.row_scale = row_scale;
    a.scale_log2 = scale_log2;
    a.normalized = normalized ? 1 : 0;
    // The fused mode splits the global query blocks (as the diffusion step);
    // the normalised one keeps them whole.
    const bool split = !normalized && row_scale != nullptr && part != nullptr;
    a.gparts = split ? global_parts(g, s) : 0;
    a.gblocks = a.gparts > 0 ? g.global_blocks : 0;
    a.part = part;
    a.total_parts = s.B * s.H * a.gblocks * a.gparts;
    a.total = s.B * s.H * (a.gblocks * a.gparts + (a.nblocks - a.gblocks));
    a.per_xcd = (a.total + 7) / 8;
    if (a.gparts > 0)
        hipLaunchKernelGGL(k_block_gmax, dim3((unsigned)a.total_parts), dim3(kThreads), 0, st, a);
    hipLaunchKernelGGL(k_block_scores, dim3((unsigned)(8 * a.per_xcd)), dim3(kThreads), 0, st, a);
    if (a.gparts > 0)
        hipLaunchKernelGGL(k_block_gsum, dim3((unsigned)(s.B * s.H * a.gblocks)), dim3(kThreads), 0,
                           st, a);
    return hipGetLastError();
}

hipError_t launch_block_diffuse(const diffuser_graph& g, const attn_shape& s, const void* A,
                                const void* Zk, const void* V, void* Zn, const float* row_scale,
                                step_coefs k, float* part, hipStream_t st) {
    BlockArgs a = block_args(g, s);
    a.gparts = global_parts(g, s);
    a.gblocks = a.gparts > 0 ? g.global_blocks : 0;
    a.part = part;
    a.total = s.B * s.H * (a.gblocks * a.gparts + (a.nblocks - a.gblocks));
    a.per_xcd = (a.total + 7) / 8;
    a.X = static_cast<const uint16_t*>(A);
    a.Y = static_cast<const uint16_t*>(Zk);
    a.V = static_cast<const uint16_t*>(V);
    a.out = static_cast<uint16_t*>(Zn);
    a.row_scale = const_cast<float*>(row_scale);
    a.keep = k.keep;
    a.restart = k.restart;
    hipLaunchKernelGGL(k_block_diffuse, dim3((unsigned)(8 * a.per_xcd)), dim3(kThreads), 0, st, a);
    if (a.gparts > 0)
        hipLaunchKernelGGL(k_block_combine,
                           dim3((unsigned)(s.B * s.H * a.gblocks * kCombineGroups)),
                           dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace diffuser
