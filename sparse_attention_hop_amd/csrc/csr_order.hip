// Edge weights in CSR order: the map from each weight slot to its edge's
// CSR position, and the two permutations between the weight-slot layout
// of A and CSR order. The weights are the edge-softmax values of the
// "Diffuser" notes (section 2.1, eqs. S.1-S.5) and the operator the
// diffusion step applies (section 2.4, eq. S.7); CSR order lists each row's
// edges by ascending column, the order in which the pages write the
// neighbourhood sums. The permutations only move element bits.
#include <hip/hip_runtime.h>

#include "internal.h"

namespace diffuser {
namespace {

constexpr int kThreads = 256;

// map[slot_off[gr] + s] = position within graph gr's CSR of slot s's edge
// (row_ptr[row] + rank of the column within the row), or -1 for padding.
// Columns within a CSR row ascend, so a binary search finds the rank.
__global__ __launch_bounds__(kThreads)
void k_slot_csr(int64_t n, const int64_t* __restrict__ slot_off,
                const int32_t* __restrict__ slot_row, const int32_t* __restrict__ slot_col,
                const int64_t* __restrict__ row_ptr, const int64_t* __restrict__ col_off,
                const int32_t* __restrict__ col_idx, int32_t* __restrict__ map) {
    const int32_t gr = blockIdx.y;
    const int64_t base = slot_off[gr];
    const int64_t len = slot_off[gr + 1] - base;
    const int64_t* rp = row_ptr + (int64_t)gr * (n + 1);
    const int32_t* ci = col_idx + col_off[gr];
    for (int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; s < len;
         s += (int64_t)gridDim.x * blockDim.x) {
        const int32_t j = slot_col[base + s];
        int32_t pos = -1;
        if (j >= 0) {
            const int32_t i = slot_row[base + s];
            const int64_t end = rp[i + 1];
            int64_t lo = rp[i], hi = end;  // first entry >= j lies in [lo, hi]
            while (lo < hi) {
                const int64_t mid = lo + ((hi - lo) >> 1);
                if (ci[mid] < j) lo = mid + 1;
                else hi = mid;
            }
            // Every slot's edge is in the CSR; a miss would leave the slot
            // unmapped rather than point at another edge.
            if (lo < end && ci[lo] == j) pos = (int32_t)lo;
        }
        map[base + s] = pos;
    }
}

// Start (in elements) of the (b, h) block of a per-graph array whose graph
// gr holds off[gr + 1] - off[gr] entries: the A layout's rule, with
// `off` the slot or the edge prefix sums.
__device__ __forceinline__ int64_t bh_block(const int64_t* off, int32_t num_graphs, int32_t H,
                                            int32_t b, int32_t h) {
    if (num_graphs == 1) return ((int64_t)b * H + h) * off[1];
    return (int64_t)H * off[b] + (int64_t)h * (off[b + 1] - off[b]);
}

// CSR-ordered weights from the slot layout: every valid slot's weight goes
// to its edge's CSR position (each edge owns one slot, so every CSR entry
// is written once).
template <typename E>
__global__ __launch_bounds__(kThreads)
void k_slots_to_csr(int32_t H, int32_t num_graphs, const int64_t* __restrict__ slot_off,
                    const int64_t* __restrict__ col_off, const int32_t* __restrict__ map,
                    const E* __restrict__ A, E* __restrict__ A_csr) {
    const int32_t bh = blockIdx.y;
    const int32_t b = bh / H, h = bh - b * H;
    const int32_t gr = num_graphs == 1 ? 0 : b;
    const int64_t len = slot_off[gr + 1] - slot_off[gr];
    const int32_t* m = map + slot_off[gr];
    const E* src = A + bh_block(slot_off, num_graphs, H, b, h);
    E* dst = A_csr + bh_block(col_off, num_graphs, H, b, h);
    for (int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; s < len;
         s += (int64_t)gridDim.x * blockDim.x) {
        const int32_t p = m[s];
        if (p >= 0) dst[p] = src[s];
    }
}

// Slot-layout weights from CSR order: each slot reads its edge's weight;
// padding slots get 0.
template <typename E>
__global__ __launch_bounds__(kThreads)
void k_csr_to_slots(int32_t H, int32_t num_graphs, const int64_t* __restrict__ slot_off,
                    const int64_t* __restrict__ col_off, const int32_t* __restrict__ map,
                    const E* __restrict__ A_csr, E* __restrict__ A) {
    const int32_t bh = blockIdx.y;
    const int32_t b = bh / H, h = bh - b * H;
    const int32_t gr = num_graphs == 1 ? 0 : b;
    const int64_t len = slot_off[gr + 1] - slot_off[gr];
    const int32_t* m = map + slot_off[gr];
    const E* src = A_csr + bh_block(col_off, num_graphs, H, b, h);
    E* dst = A + bh_block(slot_off, num_graphs, H, b, h);
    for (int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; s < len;
         s += (int64_t)gridDim.x * blockDim.x) {
        const int32_t p = m[s];
        dst[s] = p >= 0 ? src[p] : E(0);
    }
}

// Workgroups along the slots of one (b, h) block (or graph): enough to
// cover the longest graph, at most 1024.
unsigned slot_blocks(const diffuser_graph& g) {
    int64_t longest = 0;
    for (int64_t s : g.slots) longest = s > longest ? s : longest;
    const int64_t want = (longest + kThreads - 1) / kThreads;
    return (unsigned)(want < 1 ? 1 : want > 1024 ? 1024 : want);
}

}  // namespace

hipError_t launch_slot_csr(const diffuser_graph& g, int32_t* map, hipStream_t st) {
    hipLaunchKernelGGL(k_slot_csr, dim3(slot_blocks(g), (unsigned)g.num_graphs), dim3(kThreads),
                       0, st, g.n, g.d_slot_off, g.d_slot_row, g.d_slot_col, g.d_row_ptr,
                       g.d_col_off, g.d_col_idx, map);
    return hipGetLastError();
}

hipError_t launch_slots_csr_permute(const diffuser_graph& g, int32_t B, int32_t H, size_t es,
                                    const void* src, void* dst, bool to_csr, hipStream_t st) {
    const dim3 grid(slot_blocks(g), (unsigned)(B * H));
    if (es == 2) {
        if (to_csr)
            hipLaunchKernelGGL((k_slots_to_csr<uint16_t>), grid, dim3(kThreads), 0, st, H,
                               g.num_graphs, g.d_slot_off, g.d_col_off, g.d_slot_csr,
                               static_cast<const uint16_t*>(src), static_cast<uint16_t*>(dst));
        else
            hipLaunchKernelGGL((k_csr_to_slots<uint16_t>), grid, dim3(kThreads), 0, st, H,
                               g.num_graphs, g.d_slot_off, g.d_col_off, g.d_slot_csr,
                               static_cast<const uint16_t*>(src), static_cast<uint16_t*>(dst));
    } else if (es == 4) {
        if (to_csr)
            hipLaunchKernelGGL((k_slots_to_csr<uint32_t>), grid, dim3(kThreads), 0, st, H,
                               g.num_graphs, g.d_slot_off, g.d_col_off, g.d_slot_csr,
                               static_cast<const uint32_t*>(src), static_cast<uint32_t*>(dst));
        else
            hipLaunchKernelGGL((k_csr_to_slots<uint32_t>), grid, dim3(kThreads), 0, st, H,
                               g.num_graphs, g.d_slot_off, g.d_col_off, g.d_slot_csr,
                               static_cast<const uint32_t*>(src), static_cast<uint32_t*>(dst));
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace diffuser
