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
            int32_t rnd_width, int32_t causal, int32_t apart, uint64_t seed, int32_t even,
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
            slots[row] = (int32_t)((hi - wb0) / 8 * 8 + 8 + round8(g) + (apart ? 0 : round8(m)));
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
                               (apart ? 0 : round8(below)));
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

// kOctet layout: slot_col / slot_row (and rslot, when given) of row i's
// positions in its row block's octet area; positions past its cnt random
// edges rr[0 .. cnt) are padding. A row i >= n (the last block's tail) has
// only padding.
__device__ void fill_octets(int64_t n, int64_t i, int32_t cnt, const int32_t* __restrict__ rr,
                            int64_t rand_base, const int64_t* __restrict__ roff,
                            const int32_t* __restrict__ oct, int32_t* __restrict__ scol,
                            int32_t* __restrict__ srow, int32_t* __restrict__ rs, int lane) {
    const int64_t rb = i / kRowBlock;
    const int32_t m = (int32_t)(i % kRowBlock);
    const int64_t base = rand_base + 128 * roff[rb];
    const int32_t noct = oct[rb];
    for (int32_t e = lane; e < 8 * noct; e += kWave) {
        const int64_t slot = base + ((int64_t)(e >> 3) * 16 + m) * 8 + (e & 7);
        const bool real = i < n && e < cnt;
        scol[slot] = real ? rr[e] : -1;
        srow[slot] = real ? (int32_t)i : -1;
        if (real) rs[e] = (int32_t)slot;
    }
}

__global__ __launch_bounds__(kWave * kWavesPerBlock)
void k_fill(int64_t n, int32_t r, const int32_t* __restrict__ G, int32_t g, int32_t rnd_width,
            int32_t causal, int32_t layout, int32_t nrb, const int64_t* __restrict__ rb_roff,
            const int32_t* __restrict__ rb_oct, const int64_t* __restrict__ row_ptr,
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
    const bool octet = layout == 2;
    int32_t* gcol = slot_col + slot_off[gr];
    int32_t* grow = slot_row + slot_off[gr];
    const int64_t* roff = rb_roff + gr * (nrb + 1);
    const int32_t* oct = rb_oct + gr * nrb;
    int32_t* rs = rslot + row * (int64_t)rnd_width;
    const int32_t* rr = rnd + row * (int64_t)rnd_width;
    // The last row's wave also writes the padding of the rows past n in
    // its block's octet area.
    if (octet && i == n - 1)
        for (int64_t v = n; v < (n + kRowBlock - 1) / kRowBlock * kRowBlock; ++v)
            fill_octets(n, v, 0, rr, sp[n], roff, oct, gcol, grow, rs, lane);

    if (is_global(G, g, i)) {
        for (int64_t j = lane; j < nslot; j += kWave) {
            if (j < deg) out[j] = (int32_t)j;
            sout[j] = j <= last ? (int32_t)j : -1;
            rout[j] = j <= last ? (int32_t)i : -1;
        }
        if (lane == 0) row_info[row] = make_int4((int32_t)sp[i], 0, -1, 0);
        if (octet) fill_octets(n, i, 0, rr, sp[n], roff, oct, gcol, grow, rs, lane);
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
    // Row segment: window blocks, globals, then (kRow layout) randoms.
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
    if (octet) fill_octets(n, i, m, rr, sp[n], roff, oct, gcol, grow, rs, lane);
    if (layout != 0) return;   // random weights outside the row segment
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
    int32_t octet;                 // kOctet layout (else kGroup)
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
    uint16_t* sched_off;           // [groups][16] (kOctet) first slot of each pair in its
                                   //   row block's octet area
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
    // kOctet: position e of this lane's row sits at slot 8 lane + (e / 8) *
    // 128 + e % 8 of the block's octet area.
    while (true) {
        const int32_t cur = p < cnt ? rr[p] / kChunkRows : INT32_MAX;
        const int32_t c = wave_min(cur);
        if (c == INT32_MAX) break;
        int32_t k = p;
        while (k < cnt && rr[k] / kChunkRows == c) ++k;
        // Pairs cover edge positions [p - lead, k): in the octet layout a
        // pair starts at an even position, so its two slots are one aligned
        // 4-byte word of the row's octet, and the odd edge that opens a
        // chunk is paired with a dummy before it.
        const int32_t lead = a.octet ? (p & 1) : 0;
        const int32_t pairs = k > p ? (k - p + lead + 1) >> 1 : 0;
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
                const int32_t e0 = p - lead + 2 * t;        // the pair's first position
                const bool first_dummy = e0 < p;
                const bool second_dummy = e0 + 1 >= k;
                a.sched_row[gg * 16 + pig] =
                    (uint8_t)(lane | (first_dummy ? 0x40 : 0) | (second_dummy ? 0x80 : 0));
                const int64_t gslot = rand_base + (int64_t)kGroupSlots * (g0 + pidx / 16);
                if (a.octet)
                    a.sched_off[gg * 16 + pig] =
                        (uint16_t)(8 * lane + (e0 >> 3) * 128 + (e0 & 7));
                for (int h = 0; h < 2; ++h) {
                    const int32_t kk = e0 + h;
                    const bool real = kk >= p && kk < k;
                    const int32_t s = 2 * pig + h;
                    const uint32_t jr = real ? (uint32_t)(rr[kk] - c * kChunkRows) : kZeroRow;
                    a.sched_j[gg * kGroupSlots + sched_j_index(s)] = (uint16_t)key_row_code(jr);
                    a.sched_k[gg * kGroupSlots + s] = (uint16_t)score_row_code(jr);
                    if (!a.octet) {
                        const int64_t slot = gslot + s;
                        a.slot_col[soff + slot] = real ? rr[kk] : -1;
                        a.slot_row[soff + slot] = real ? (int32_t)i : -1;
                        if (real) a.rslot[row * (int64_t)a.rnd_width + kk] = (int32_t)slot;
                    }
                }
            }
            // Dummy pairs that pad the chunk's last group.
            for (int32_t pidx = total + lane; pidx < 16 * ng; pidx += kWave) {
                const int64_t gg = gbase + g0 + pidx / 16;
                const int32_t pig = pidx % 16;
                a.sched_row[gg * 16 + pig] = (uint8_t)0xFF;
                const int64_t gslot = rand_base + (int64_t)kGroupSlots * (g0 + pidx / 16);
                // Group layout: the dummy pair's slots are padding, written 0.
                if (a.octet) a.sched_off[gg * 16 + pig] = 0;
                for (int h = 0; h < 2; ++h) {
                    const int32_t s = 2 * pig + h;
                    a.sched_j[gg * kGroupSlots + sched_j_index(s)] = (uint16_t)key_row_code(kZeroRow);
                    a.sched_k[gg * kGroupSlots + s] = (uint16_t)score_row_code(kZeroRow);
                    if (!a.octet) {
                        a.slot_col[soff + gslot + s] = -1;
                        a.slot_row[soff + gslot + s] = -1;
                    }
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


// Slot of key row k in the resident-slice layout of the diffusion step:
// bit 2 of the row is flipped when bit 3 is set (an involution on every
// aligned run of 16 rows), which puts the two 4-row halves of one
// transposed read on different LDS bank groups.
__host__ __device__ __forceinline__ uint32_t res_unit(uint32_t k) { return k ^ ((k >> 1) & 4u); }

// Random octets of every row block of a kOctet graph: ceil(most random
// edges of any of its rows / 8) (0 when every row is a global row).
__global__ void k_rb_oct(int64_t n, int32_t nrb, const int32_t* __restrict__ rnd_cnt,
                         int32_t* __restrict__ oct) {
    const int32_t rb = (int32_t)(blockIdx.x * blockDim.x + threadIdx.x);
    const int64_t gr = blockIdx.y;
    if (rb >= nrb) return;
    const int64_t r0 = (int64_t)rb * kRowBlock;
    const int64_t r1 = r0 + kRowBlock < n ? r0 + kRowBlock : n;
    int32_t mx = 0;
    for (int64_t i = r0; i < r1; ++i) mx = max(mx, rnd_cnt[gr * n + i]);
    oct[gr * nrb + rb] = (mx + 7) / 8;
}

// Key table of the resident-slice diffusion step, one thread per (row
// block, batch, lane): the lane's 8 entries (see diffuser_graph::d_rkey) in
// one 16-byte store.
__global__ void k_rkey(int64_t n, int32_t nrb, int32_t batches, int32_t rnd_width,
                       uint32_t n_pad, const int32_t* __restrict__ rnd,
                       const int32_t* __restrict__ rnd_cnt, uint16_t* __restrict__ rkey) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t gr = blockIdx.y;
    if (idx >= (int64_t)nrb * batches * kWave) return;
    const int32_t l = (int32_t)(idx % kWave);
    const int32_t b = (int32_t)((idx / kWave) % batches);
    const int64_t rb = idx / ((int64_t)kWave * batches);
    const int32_t kg = l >> 4, q = (l >> 2) & 3, j = l & 3;
    const int32_t o = kOctBatch * b + j;
    uint32_t w[8];
    for (int32_t t = 0; t < 4; ++t) {
        const int64_t i = rb * kRowBlock + 4 * t + ((kg + o) & 3);
        for (int32_t h = 0; h < 2; ++h) {
            const int32_t e = 8 * o + 4 * h + q;
            uint32_t k = n_pad;
            if (i < n) {
                const int64_t row = gr * n + i;
                if (e < rnd_cnt[row]) k = res_unit((uint32_t)rnd[row * rnd_width + e]);
            }
            w[2 * t + h] = k;
        }
    }
    uint4* out = reinterpret_cast<uint4*>(rkey) + gr * nrb * batches * kWave + idx;
    *out = make_uint4(w[0] | (w[1] << 16), w[2] | (w[3] << 16), w[4] | (w[5] << 16),
                      w[6] | (w[7] << 16));
}

// Per row block of every graph, for the resident-slice diffusion step's
// work split: its cost (band steps, global-column steps and 4 products per
// random octet, plus 2 for the restart and store; 0 when every row of the
// block is a global row) into cost.
__global__ void k_rb_cost(int64_t n, int32_t r, int32_t causal, int32_t g, int32_t nrb,
                          const int32_t* __restrict__ G, const int32_t* __restrict__ oct,
                          int32_t* __restrict__ cost) {
    const int32_t rb = (int32_t)(blockIdx.x * blockDim.x + threadIdx.x);
    const int64_t gr = blockIdx.y;
    if (rb >= nrb) return;
    const int64_t r0 = (int64_t)rb * kRowBlock;
    const int64_t r1 = r0 + kRowBlock < n ? r0 + kRowBlock : n;
    const int32_t gin = count_less(G, g, r1) - count_less(G, g, r0);
    int32_t c = 0;
    if (gin < r1 - r0) {
        const int64_t lo = (r0 - r < 0 ? 0 : r0 - r) & ~31ll;
        const int64_t hi = causal ? r1 - 1 : (r1 - 1 + r < n - 1 ? r1 - 1 + r : n - 1);
        c = (int32_t)(((hi - lo) >> 5) + 1 + ((g + 31) >> 5) + 4 * oct[gr * nrb + rb] + 2);
    }
    cost[gr * nrb + rb] = c;
}

}  // namespace

hipError_t launch_draw(const diffuser_graph& g, int32_t* deg, int32_t* slots, int32_t* status,
                       hipStream_t st) {
    dim3 grid((unsigned)((g.n + kWavesPerBlock - 1) / kWavesPerBlock), (unsigned)g.num_graphs);
    hipLaunchKernelGGL(k_draw, grid, dim3(kWave * kWavesPerBlock), 0, st, g.n, g.radius,
                       g.d_global, g.num_global, g.num_random, g.rnd_width, g.causal,
                       (int32_t)g.rand_apart(), g.seed, g.random_layout, deg, slots, g.d_rnd,
                       g.d_rnd_cnt, status);
    return hipGetLastError();
}

hipError_t launch_scan(int64_t n, int32_t num_graphs, const int32_t* counts, int64_t* offsets,
                       int64_t* max_count, hipStream_t st) {
    hipLaunchKernelGGL(k_scan, dim3((unsigned)num_graphs), dim3(kScanThreads), 0, st, n, counts,
                       offsets, max_count);
    return hipGetLastError();
}

// Long-row flags: row i of graph gr has seg_ptr[i + 1] - seg_ptr[i] slots
// in its segment plus, when the random slots lie apart, rnd_cnt of them.
__global__ void k_long_flags(int64_t n, const int64_t* __restrict__ seg_ptr,
                             const int32_t* __restrict__ rnd_cnt, int32_t* __restrict__ flags) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t gr = blockIdx.y;
    if (i >= n) return;
    const int64_t* sp = seg_ptr + gr * (n + 1);
    const int64_t len = sp[i + 1] - sp[i] + (rnd_cnt != nullptr ? rnd_cnt[gr * n + i] : 0);
    flags[gr * n + i] = len > kLongRow ? 1 : 0;
}

__global__ void k_long_fill(int64_t n, const int32_t* __restrict__ flags,
                            const int64_t* __restrict__ offsets,
                            const int64_t* __restrict__ long_off, int32_t* __restrict__ rows) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t gr = blockIdx.y;
    if (i >= n || flags[gr * n + i] == 0) return;
    rows[long_off[gr] + offsets[gr * (n + 1) + i]] = (int32_t)i;
}

hipError_t launch_long_flags(const diffuser_graph& g, int32_t* flags, hipStream_t st) {
    dim3 grid((unsigned)((g.n + 255) / 256), (unsigned)g.num_graphs);
    hipLaunchKernelGGL(k_long_flags, grid, dim3(256), 0, st, g.n, g.d_seg_ptr,
                       g.rand_apart() ? g.d_rnd_cnt : nullptr, flags);
    return hipGetLastError();
}

hipError_t launch_long_fill(const diffuser_graph& g, const int32_t* flags,
                            const int64_t* offsets, hipStream_t st) {
    dim3 grid((unsigned)((g.n + 255) / 256), (unsigned)g.num_graphs);
    hipLaunchKernelGGL(k_long_fill, grid, dim3(256), 0, st, g.n, flags, offsets, g.d_long_off,
                       g.d_long_rows);
    return hipGetLastError();
}

hipError_t launch_fill(const diffuser_graph& g, hipStream_t st) {
    dim3 grid((unsigned)((g.n + kWavesPerBlock - 1) / kWavesPerBlock), (unsigned)g.num_graphs);
    hipLaunchKernelGGL(k_fill, grid, dim3(kWave * kWavesPerBlock), 0, st, g.n, g.radius,
                       g.d_global, g.num_global, g.rnd_width, g.causal,
                       g.octet() ? 2 : g.grouped() ? 1 : 0,
                       (int32_t)((g.n + kRowBlock - 1) / kRowBlock), g.d_rb_roff, g.d_rb_oct,
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
    a.octet = g.octet() ? 1 : 0;
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
    a.sched_off = g.d_sched_off;
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

hipError_t launch_rb_octets(const diffuser_graph& g, int64_t* max_count, hipStream_t st) {
    const int32_t nrb = (int32_t)((g.n + kRowBlock - 1) / kRowBlock);
    dim3 grid((unsigned)((nrb + 255) / 256), (unsigned)g.num_graphs);
    hipLaunchKernelGGL(k_rb_oct, grid, dim3(256), 0, st, g.n, nrb, g.d_rnd_cnt, g.d_rb_oct);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_scan(nrb, g.num_graphs, g.d_rb_oct, g.d_rb_roff, max_count, st);
}

hipError_t launch_res_tables(const diffuser_graph& g, int32_t* cost_tmp, hipStream_t st) {
    const int32_t nrb = (int32_t)((g.n + kRowBlock - 1) / kRowBlock);
    hipError_t e;
    if (g.key_batches > 0) {
        const int64_t items = (int64_t)nrb * g.key_batches * kWave;
        dim3 grid((unsigned)((items + 255) / 256), (unsigned)g.num_graphs);
        hipLaunchKernelGGL(k_rkey, grid, dim3(256), 0, st, g.n, nrb, g.key_batches, g.rnd_width,
                           (uint32_t)res_npad(g.n), g.d_rnd, g.d_rnd_cnt, g.d_rkey);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    dim3 cgrid((unsigned)((nrb + 255) / 256), (unsigned)g.num_graphs);
    hipLaunchKernelGGL(k_rb_cost, cgrid, dim3(256), 0, st, g.n, g.radius, g.causal, g.num_global,
                       nrb, g.d_global, g.d_rb_oct, cost_tmp);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return launch_scan(nrb, g.num_graphs, cost_tmp, g.d_rb_cost, g.d_rb_cost_max, st);
}

}  // namespace diffuser
