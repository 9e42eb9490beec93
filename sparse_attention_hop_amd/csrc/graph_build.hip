// Static token-graph builder: window u globals u random extras, one CSR per
// graph, ascending columns ("Diffuser" reading notes, section 2.2 connection
// table; "1.2.1 Static sparsity", section 1.1 eq. 5 and section 1.2 eq. 12;
// "038 BigBird", section 2, union neighbourhood). Random edges are seeded
// and input-independent ("1.2.1", section 2: static random edges are fixed
// before execution and reproducible from the seed).
//
// Kernels, one wavefront per row (or row block) where those are independent:
//   draw  : random extras of a row by rejection sampling on a counter-based
//           SplitMix64 stream, sorted into an ELL table, plus the row's edge
//           count and its row-segment slot count;
//   scan  : exclusive scan of per-row counts into int64 offsets (one block
//           per graph);
//   fill  : the sorted merge window u (G minus window) u random into the
//           ascending CSR, and the edge of every row-segment slot;
//   sched : the random schedule of each row block (count, then fill).
//
// Weight-slot layout (where the edge weights live in A). Every segment is a
// multiple of 8 slots, so it starts 16-byte aligned in bf16. A global row's
// segment holds its columns 0, 1, ... in order. Any other row's segment:
//   window : 8-column blocks from (lo & ~7) through the last window column
//            (hi, or i when causal); slot t is column (lo & ~7) + t when that
//            column lies in the window, else padding;
//   global : slot t < g is global G[t] unless G[t] lies in the window (or,
//            when causal, above i); padding to a multiple of 8;
//   random : (unscheduled graphs only) the row's random columns, ascending
//            (when causal, only those below the window), padded.
// Scheduled graphs hold the random edges after all row segments, in
// schedule order: for each row block (kRowBlock rows) and key chunk
// (kChunkRows keys) with random edges, the block's edges into that chunk by
// row, then column, two edges of one row per pair (an odd one out paired
// with a dummy), 16 pairs = kGroupSlots slots per group, the last group of
// a (block, chunk) padded with dummy pairs; pair p of a group owns slots
// 2p and 2p + 1. Padding and dummy slots carry row and column -1 and
// weight 0.
#include "internal.h"

namespace diffuser {
namespace {

constexpr int kWave = 64;
constexpr int kWavesPerBlock = 4;
constexpr int kMaxSampled = 1024;        // random budget held in LDS per row
constexpr int64_t kMaxDraws = 1ll << 20; // draws per row before giving up
constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

// SplitMix64 output function (Steele, Lea & Flood, OOPSLA 2014).
__device__ __forceinline__ uint64_t splitmix_mix(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

// Number of entries of the ascending array a[0..len) that are < x.
__device__ __forceinline__ int32_t count_less(const int32_t* a, int32_t len, int64_t x) {
    int32_t lo = 0, hi = len;
    while (lo < hi) {
        int32_t mid = (lo + hi) >> 1;
        if ((int64_t)a[mid] < x) lo = mid + 1; else hi = mid;
    }
    return lo;
}

__device__ __forceinline__ bool is_global(const int32_t* G, int32_t g, int64_t j) {
    int32_t k = count_less(G, g, j);
    return k < g && G[k] == j;
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// The member of rank t (0-based, ascending) of [a, b] minus the globals;
// the caller guarantees it exists.
__device__ __forceinline__ int64_t nth_outside_globals(const int32_t* G, int32_t g, int64_t a,
                                                       int64_t b, int64_t t) {
    const int32_t ga = count_less(G, g, a);
    int64_t lo = a + t, hi = b;   // the answer lies in [a + t, min(b, a + t + g)]
    if (hi > a + t + g) hi = a + t + g;
    while (lo < hi) {             // smallest j with |[a, j] \ G| >= t + 1
        const int64_t mid = (lo + hi) >> 1;
        const int64_t have = (mid - a + 1) - (count_less(G, g, mid + 1) - ga);
        if (have >= t + 1) hi = mid; else lo = mid + 1;
    }
    return lo;
}

__host__ __device__ __forceinline__ int64_t round8(int64_t x) { return (x + 7) & ~7ll; }

__global__ __launch_bounds__(kWave * kWavesPerBlock)
void k_draw(int64_t n, int32_t r, const int32_t* __restrict__ G, int32_t g, int32_t R,
            int32_t rnd_width, int32_t causal, int32_t scheduled, uint64_t seed, int32_t even,
            int32_t* __restrict__ deg,
            int32_t* __restrict__ slots, int32_t* __restrict__ rnd,
            int32_t* __restrict__ rnd_cnt, int32_t* __restrict__ status) {
    __shared__ int32_t taken[kWavesPerBlock][kMaxSampled];
    const int wave = threadIdx.x / kWave;
    const int lane = lane_id();
    const int64_t i = (int64_t)blockIdx.x * kWavesPerBlock + wave;
    const int64_t gr = blockIdx.y;
    if (i >= n) return;
    const int64_t row = gr * n + i;
    int32_t* out = rnd + row * (int64_t)rnd_width;

    if (is_global(G, g, i)) {
        if (lane == 0) {
            deg[row] = (int32_t)(causal ? i + 1 : n);
            slots[row] = (int32_t)round8(causal ? i + 1 : n);
            rnd_cnt[row] = 0;
        }
        return;
    }
    const int64_t lo = i - r < 0 ? 0 : i - r;
    const int64_t hi = i + r > n - 1 ? n - 1 : i + r;
    const int64_t wlen = hi - lo + 1;
    const int32_t g_before = count_less(G, g, lo);
    const int32_t g_in = count_less(G, g, hi + 1) - g_before;
    const int64_t pool = n - wlen - (g - g_in);

    int32_t m = 0;  // accepted random extras (wave-uniform)
    if (pool <= R) {
        // The whole pool: every position outside the window and the globals.
        for (int64_t base = 0; base < n; base += kWave) {
            const int64_t j = base + lane;
            const bool in_pool = j < n && (j < lo || j > hi) && !is_global(G, g, j);
            const uint64_t mask = __ballot(in_pool);
            const int32_t pos = m + __popcll(mask & ((1ull << lane) - 1));
            if (in_pool && pos < rnd_width) out[pos] = (int32_t)j;
            m += __popcll(mask);
        }
    } else if (even) {
        // Evenly spaced extras: pool members of rank q * pool / R, ascending.
        int32_t* list = taken[wave];
        const int64_t below_lo = lo - g_before;   // pool members left of the window
        for (int32_t q = lane; q < R; q += kWave) {
            const int64_t t = (int64_t)q * pool / R;
            const int64_t j = t < below_lo ? nth_outside_globals(G, g, 0, lo - 1, t)
                                           : nth_outside_globals(G, g, hi + 1, n - 1,
                                                                 t - below_lo);
            list[q] = (int32_t)j;
            if (q < rnd_width) out[q] = (int32_t)j;
        }
        m = R;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    } else {
        int32_t* list = taken[wave];
        const uint64_t ctr_row = ((uint64_t)(gr * n + i)) << 20;
        for (int64_t t0 = 0; m < R && t0 < kMaxDraws; t0 += kWave) {
            const int64_t t = t0 + lane;
            const uint64_t u = splitmix_mix(seed + kGamma * ((ctr_row | (uint64_t)t) + 1ull));
            const int64_t j = (int64_t)(((u >> 32) * (uint64_t)n) >> 32);
            bool ok = (j < lo || j > hi) && !is_global(G, g, j);
            for (int32_t q = 0; q < m; ++q) ok = ok && list[q] != (int32_t)j;
            uint64_t mask = __ballot(ok);
            // Accept in draw order; drop later repeats of an accepted value.
            while (mask != 0 && m < R) {
                const int l = __ffsll((unsigned long long)mask) - 1;
                const int32_t c = __shfl((int32_t)j, l);
                if (lane == 0) list[m] = c;
                ++m;
                mask &= ~__ballot((int32_t)j == c);
            }
            __builtin_amdgcn_wave_barrier();
        }
        if (m < R) {
            if (lane == 0) status[0] = 1;
            return;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // Rank sort of the distinct values into ascending order.
        for (int32_t e = lane; e < m; e += kWave) {
            const int32_t v = list[e];
            int32_t rank = 0;
            for (int32_t q = 0; q < m; ++q) rank += list[q] < v;
            if (rank < rnd_width) out[rank] = v;
        }
    }
    const int64_t wb0 = lo & ~7ll;
    if (!causal) {
        if (lane == 0) {
            rnd_cnt[row] = m;
            deg[row] = (int32_t)(wlen + (g - g_in) + m);
            slots[row] = (int32_t)((hi - wb0) / 8 * 8 + 8 + round8(g) + (scheduled ? 0 : round8(m)));
        }
        return;
    }
    // Causal: keep j <= i: the window part [lo, i], globals below lo, and
    // the random extras below lo (none lie inside the window).
    int32_t below = 0;
    if (pool <= R) {
        below = (int32_t)(lo - g_before);
    } else {
        const int32_t* list = taken[wave];
        int32_t c = 0;
        for (int32_t e = lane; e < m; e += kWave) c += list[e] < lo;
        for (int off = 32; off > 0; off >>= 1) c += __shfl_xor(c, off);
        below = c;
    }
    if (lane == 0) {
        rnd_cnt[row] = below;
        deg[row] = (int32_t)((i - lo + 1) + g_before + below);
        slots[row] = (int32_t)((i - wb0) / 8 * 8 + 8 + round8(g_before) +
                               (scheduled ? 0 : round8(below)));
    }
}

constexpr int kScanThreads = 1024;

__global__ __launch_bounds__(kScanThreads)
void k_scan(int64_t n, const int32_t* __restrict__ deg, int64_t* __restrict__ row_ptr,
            int64_t* __restrict__ max_deg) {
    // deg: [graphs][n] counts; row_ptr: [graphs][n + 1] exclusive offsets.
    __shared__ int64_t part[kScanThreads];
    __shared__ int64_t pmax[kScanThreads];
    const int64_t gr = blockIdx.x;
    const int32_t* d = deg + gr * n;
    int64_t* rp = row_ptr + gr * (n + 1);
    const int64_t chunk = (n + kScanThreads - 1) / kScanThreads;
    const int64_t b0 = threadIdx.x * chunk;
    const int64_t b1 = b0 + chunk < n ? b0 + chunk : n;
    int64_t s = 0, mx = 0;
    for (int64_t i = b0; i < b1; ++i) {
        s += d[i];
        mx = d[i] > mx ? d[i] : mx;
    }
    part[threadIdx.x] = s;
    pmax[threadIdx.x] = mx;
    __syncthreads();
    // Inclusive Hillis-Steele scan of the per-thread sums.
    for (int off = 1; off < kScanThreads; off <<= 1) {
        int64_t v = threadIdx.x >= off ? part[threadIdx.x - off] : 0;
        int64_t w = threadIdx.x >= off ? pmax[threadIdx.x - off] : 0;
        __syncthreads();
        part[threadIdx.x] += v;
        pmax[threadIdx.x] = pmax[threadIdx.x] > w ? pmax[threadIdx.x] : w;
        __syncthreads();
    }
    int64_t run = part[threadIdx.x] - s;
    for (int64_t i = b0; i < b1; ++i) {
        rp[i] = run;
        run += d[i];
    }
    if (threadIdx.x == kScanThreads - 1) {
        rp[n] = part[kScanThreads - 1];
        max_deg[gr] = pmax[kScanThreads - 1];
    }
}

__global__ __launch_bounds__(kWave * kWavesPerBlock)
void k_fill(int64_t n, int32_t r, const int32_t* __restrict__ G, int32_t g, int32_t rnd_width,
            int32_t causal, int32_t scheduled, const int64_t* __restrict__ row_ptr,
            const int64_t* __restrict__ col_off, const int64_t* __restrict__ seg_ptr,
            const int64_t* __restrict__ slot_off, const int32_t* __restrict__ rnd,
            const int32_t* __restrict__ rnd_cnt, int32_t* __restrict__ col_idx,
            int32_t* __restrict__ slot_col, int32_t* __restrict__ slot_row,
            int32_t* __restrict__ rslot, int4* __restrict__ row_info) {
    const int wave = threadIdx.x / kWave;
    const int lane = lane_id();
    const int64_t i = (int64_t)blockIdx.x * kWavesPerBlock + wave;
    const int64_t gr = blockIdx.y;
    if (i >= n) return;
    const int64_t row = gr * n + i;
    const int64_t* rp = row_ptr + gr * (n + 1);
    const int64_t* sp = seg_ptr + gr * (n + 1);
    int32_t* out = col_idx + col_off[gr] + rp[i];
    int32_t* sout = slot_col + slot_off[gr] + sp[i];
    int32_t* rout = slot_row + slot_off[gr] + sp[i];
    // Every store below is kept inside this row's entries.
    const int64_t deg = rp[i + 1] - rp[i];
    const int64_t nslot = sp[i + 1] - sp[i];
    const int64_t last = causal ? i : n - 1;

    if (is_global(G, g, i)) {
        for (int64_t j = lane; j < nslot; j += kWave) {
            if (j < deg) out[j] = (int32_t)j;
            sout[j] = j <= last ? (int32_t)j : -1;
            rout[j] = j <= last ? (int32_t)i : -1;
        }
        if (lane == 0) row_info[row] = make_int4((int32_t)sp[i], 0, -1, 0);
        return;
    }
    const int64_t lo = i - r < 0 ? 0 : i - r;
    const int64_t hi = i + r > n - 1 ? n - 1 : i + r;
    const int64_t wlen = hi - lo + 1;
    const int64_t wend = causal ? i : hi;
    const int64_t wb0 = lo & ~7ll;
    const int64_t wseg = (wend - wb0) / 8 * 8 + 8;
    const int32_t g_before = count_less(G, g, lo);
    const int32_t g_in = count_less(G, g, hi + 1) - g_before;
    const int64_t gseg = round8(causal ? g_before : g);
    const int32_t m = rnd_cnt[row];  // random columns kept in this row
    const int32_t* rr = rnd + row * (int64_t)rnd_width;
    const int32_t r_before = count_less(rr, m, lo);
    const int64_t woff = g_before + r_before;
    if (lane == 0) row_info[row] = make_int4((int32_t)sp[i], (int32_t)wb0, (int32_t)wseg, (int32_t)gseg);

    // Ascending CSR: (left extras) window (right extras).
    for (int64_t k = lane; k < wlen; k += kWave) {
        const int64_t j = lo + k;
        if (j <= last && woff + k < deg) out[woff + k] = (int32_t)j;
    }
    for (int32_t q = lane; q < g; q += kWave) {
        const int64_t p = G[q];
        if (p >= lo && p <= hi) continue;
        const bool right = p > hi;
        const int64_t pos = (q - (right ? g_in : 0)) + count_less(rr, m, p) + (right ? wlen : 0);
        if (p <= last && pos < deg) out[pos] = (int32_t)p;
    }
    for (int32_t q = lane; q < m; q += kWave) {
        const int64_t v = rr[q];
        const bool right = v > hi;
        const int64_t gx_less = count_less(G, g, v) - (right ? g_in : 0);
        const int64_t pos = q + gx_less + (right ? wlen : 0);
        if (v <= last && pos < deg) out[pos] = (int32_t)v;
    }
    // Row segment: window blocks, globals, then (unscheduled) randoms.
    for (int64_t t = lane; t < wseg && t < nslot; t += kWave) {
        const int64_t j = wb0 + t;
        const bool in = j >= lo && j <= wend;
        sout[t] = in ? (int32_t)j : -1;
        rout[t] = in ? (int32_t)i : -1;
    }
    for (int64_t t = lane; t < gseg && wseg + t < nslot; t += kWave) {
        int32_t c = -1;
        if (t < g) {
            const int64_t p = G[t];
            if ((p < lo || p > hi) && p <= last) c = (int32_t)p;
        }
        sout[wseg + t] = c;
        rout[wseg + t] = c >= 0 ? (int32_t)i : -1;
    }
    if (scheduled) return;
    int32_t* rs = rslot + row * (int64_t)rnd_width;
    for (int64_t t = lane; wseg + gseg + t < nslot; t += kWave) {
        sout[wseg + gseg + t] = t < m ? rr[t] : -1;
        rout[wseg + gseg + t] = t < m ? (int32_t)i : -1;
        if (t < m) rs[t] = (int32_t)(sp[i] + wseg + gseg + t);
    }
}

// Random schedule of one row block per wavefront (lanes 0..kRowBlock-1 own
// its rows). The block's rows are merged chunk by chunk in ascending key
// order; for each chunk with random edges every row contributes
// ceil(count / 2) pairs, the block ceil(pairs / 16) groups. kFill = false
// counts the groups; kFill = true writes them (group numbering from
// grp_ptr) plus the slots' edges and each random edge's slot.
struct SchedArgs {
    int64_t n;
    int32_t rnd_width, nrb;
    const int32_t* rnd;
    const int32_t* rnd_cnt;
    int32_t* counts;               // [graphs][nrb] (count pass)
    const int64_t* grp_ptr;        // [graphs][nrb + 1]
    const int64_t* grp_off;        // [graphs + 1]
    const int64_t* seg_ptr;        // [graphs][n + 1]
    const int64_t* slot_off;       // [graphs + 1]
    int32_t nchunks;
    int32_t* grp_cptr;             // [graphs][nrb][nchunks + 1]
    uint8_t* sched_row;            // [groups][16] pair rows
    uint16_t* sched_j;             // [groups][32] slot key rows (diffusion layout)
    uint16_t* sched_k;             // [groups][32] slot key rows (score layout)
    int32_t* slot_col;
    int32_t* slot_row;
    int32_t* rslot;
};

__device__ __forceinline__ int32_t wave_min(int32_t v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const int32_t o = __shfl_xor(v, off);
        v = o < v ? o : v;
    }
    return v;
}

// Position of slot s (0..31) of a group in the [32] key-row array: slot
// 8k + a is the low half of word 4k + a, slot 8k + 4 + a its high half.
__device__ __forceinline__ int32_t sched_j_index(int32_t s) {
    const int32_t k = s >> 3, a = s & 7;
    return 2 * (4 * k + (a & 3)) + (a >> 2);
}

template <bool kFill>
__global__ __launch_bounds__(kWave * kWavesPerBlock)
void k_sched(SchedArgs a) {
    const int wave = threadIdx.x / kWave;
    const int lane = lane_id();
    const int32_t rb = (int32_t)blockIdx.x * kWavesPerBlock + wave;
    const int64_t gr = blockIdx.y;
    if (rb >= a.nrb) return;
    const int64_t n = a.n;
    const int64_t i = (int64_t)rb * kRowBlock + lane;
    const bool own = lane < kRowBlock && i < n;
    const int64_t row = gr * n + (own ? i : 0);
    const int32_t cnt = own ? a.rnd_cnt[row] : 0;
    const int32_t* rr = a.rnd + row * (int64_t)a.rnd_width;
    int64_t grp = 0, gbase = 0, rand_base = 0, soff = 0;
    if (kFill) {
        gbase = a.grp_off[gr];
        grp = a.grp_ptr[gr * (a.nrb + 1) + rb];
        rand_base = a.seg_ptr[gr * (n + 1) + n];
        soff = a.slot_off[gr];
    }
    int64_t groups = 0;
    int32_t p = 0;
    int32_t filled = -1;   // chunk table entries 0..filled are written
    int32_t* cptr = kFill ? a.grp_cptr + (gr * a.nrb + rb) * (int64_t)(a.nchunks + 1) : nullptr;
    while (true) {
        const int32_t cur = p < cnt ? rr[p] / kChunkRows : INT32_MAX;
        const int32_t c = wave_min(cur);
        if (c == INT32_MAX) break;
        int32_t k = p;
        while (k < cnt && rr[k] / kChunkRows == c) ++k;
        const int32_t pairs = (k - p + 1) >> 1;
        // Exclusive prefix of the pair counts over the lanes.
        int32_t incl = pairs;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const int32_t o = __shfl_up(incl, off);
            if (lane >= off) incl += o;
        }
        const int32_t total = __shfl(incl, kWave - 1);
        const int32_t ng = (total + 15) / 16;
        if (kFill) {
            const int32_t pre = incl - pairs;
            const int64_t g0 = grp + groups;   // first group of this chunk (in graph)
            for (int32_t t = 0; t < pairs; ++t) {
                const int32_t pidx = pre + t;
                const int64_t gg = gbase + g0 + pidx / 16;
                const int32_t pig = pidx % 16;
                const bool lone = p + 2 * t + 1 >= k;   // second slot is a dummy
                a.sched_row[gg * 16 + pig] = (uint8_t)(lane | (lone ? 0x80 : 0));
                for (int h = 0; h < 2; ++h) {
                    const int32_t kk = p + 2 * t + h;
                    const bool real = kk < k;
                    const int32_t s = 2 * pig + h;
                    const int64_t slot = rand_base + (int64_t)kGroupSlots * (g0 + pidx / 16) + s;
                    const uint32_t jr = real ? (uint32_t)(rr[kk] - c * kChunkRows) : kZeroRow;
                    a.sched_j[gg * kGroupSlots + sched_j_index(s)] = (uint16_t)key_row_code(jr);
                    a.sched_k[gg * kGroupSlots + s] = (uint16_t)score_row_code(jr);
                    a.slot_col[soff + slot] = real ? rr[kk] : -1;
                    a.slot_row[soff + slot] = real ? (int32_t)i : -1;
                    if (real) a.rslot[row * (int64_t)a.rnd_width + kk] = (int32_t)slot;
                }
            }
            // Dummy pairs that pad the chunk's last group.
            for (int32_t pidx = total + lane; pidx < 16 * ng; pidx += kWave) {
                const int64_t gg = gbase + g0 + pidx / 16;
                const int32_t pig = pidx % 16;
                a.sched_row[gg * 16 + pig] = (uint8_t)0xFF;
                for (int h = 0; h < 2; ++h) {
                    const int32_t s = 2 * pig + h;
                    const int64_t slot = rand_base + (int64_t)kGroupSlots * (g0 + pidx / 16) + s;
                    a.sched_j[gg * kGroupSlots + sched_j_index(s)] = (uint16_t)key_row_code(kZeroRow);
                    a.sched_k[gg * kGroupSlots + s] = (uint16_t)score_row_code(kZeroRow);
                    a.slot_col[soff + slot] = -1;
                    a.slot_row[soff + slot] = -1;
                }
            }
            // Chunks filled + 1 .. c start at this chunk's first group.
            for (int32_t cc = filled + 1 + lane; cc <= c; cc += kWave) cptr[cc] = (int32_t)g0;
            filled = c;
        }
        groups += ng;
        p = k;
    }
    if (kFill)
        for (int32_t cc = filled + 1 + lane; cc <= a.nchunks; cc += kWave)
            cptr[cc] = (int32_t)(grp + groups);
    if (!kFill && lane == 0) a.counts[gr * a.nrb + rb] = (int32_t)groups;
}

}  // namespace

hipError_t launch_draw(const diffuser_graph& g, int32_t* deg, int32_t* slots, int32_t* status,
                       hipStream_t st) {
    dim3 grid((unsigned)((g.n + kWavesPerBlock - 1) / kWavesPerBlock), (unsigned)g.num_graphs);
    hipLaunchKernelGGL(k_draw, grid, dim3(kWave * kWavesPerBlock), 0, st, g.n, g.radius,
                       g.d_global, g.num_global, g.num_random, g.rnd_width, g.causal,
                       (int32_t)g.scheduled, g.seed, g.random_layout, deg, slots, g.d_rnd,
                       g.d_rnd_cnt, status);
    return hipGetLastError();
}

hipError_t launch_scan(int64_t n, int32_t num_graphs, const int32_t* counts, int64_t* offsets,
                       int64_t* max_count, hipStream_t st) {
    hipLaunchKernelGGL(k_scan, dim3((unsigned)num_graphs), dim3(kScanThreads), 0, st, n, counts,
                       offsets, max_count);
    return hipGetLastError();
}

hipError_t launch_fill(const diffuser_graph& g, hipStream_t st) {
    dim3 grid((unsigned)((g.n + kWavesPerBlock - 1) / kWavesPerBlock), (unsigned)g.num_graphs);
    hipLaunchKernelGGL(k_fill, grid, dim3(kWave * kWavesPerBlock), 0, st, g.n, g.radius,
                       g.d_global, g.num_global, g.rnd_width, g.causal, (int32_t)g.scheduled,
                       g.d_row_ptr, g.d_col_off, g.d_seg_ptr, g.d_slot_off, g.d_rnd,
                       g.d_rnd_cnt, g.d_col_idx, g.d_slot_col, g.d_slot_row, g.d_rslot,
                       reinterpret_cast<int4*>(g.d_row_info));
    return hipGetLastError();
}

static SchedArgs sched_args(const diffuser_graph& g) {
    SchedArgs a{};
    a.n = g.n;
    a.rnd_width = g.rnd_width;
    a.nrb = (int32_t)((g.n + kRowBlock - 1) / kRowBlock);
    a.rnd = g.d_rnd;
    a.rnd_cnt = g.d_rnd_cnt;
    a.grp_ptr = g.d_grp_ptr;
    a.grp_off = g.d_grp_off;
    a.seg_ptr = g.d_seg_ptr;
    a.slot_off = g.d_slot_off;
    a.nchunks = (int32_t)((g.n + kChunkRows - 1) / kChunkRows);
    a.grp_cptr = g.d_grp_cptr;
    a.sched_row = reinterpret_cast<uint8_t*>(g.d_sched_row);
    a.sched_j = reinterpret_cast<uint16_t*>(g.d_sched_j);
    a.sched_k = g.d_sched_k;
    a.slot_col = g.d_slot_col;
    a.slot_row = g.d_slot_row;
    a.rslot = g.d_rslot;
    return a;
}

hipError_t launch_sched_count(const diffuser_graph& g, int32_t* counts, hipStream_t st) {
    SchedArgs a = sched_args(g);
    a.counts = counts;
    dim3 grid((unsigned)((a.nrb + kWavesPerBlock - 1) / kWavesPerBlock), (unsigned)g.num_graphs);
    hipLaunchKernelGGL(k_sched<false>, grid, dim3(kWave * kWavesPerBlock), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_sched_fill(const diffuser_graph& g, hipStream_t st) {
    SchedArgs a = sched_args(g);
    dim3 grid((unsigned)((a.nrb + kWavesPerBlock - 1) / kWavesPerBlock), (unsigned)g.num_graphs);
    hipLaunchKernelGGL(k_sched<true>, grid, dim3(kWave * kWavesPerBlock), 0, st, a);
    return hipGetLastError();
}

}  // namespace diffuser
