// Storage-type helpers for the compute kernels: 16-byte chunks of fp32 or
// bf16 rows, unpacked to fp32 registers; fp32 -> bf16 with
// round-to-nearest-even.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace diffuser {

struct bf16_t {
    uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Round to nearest, ties to even; NaN stays NaN (quiet bit set).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

template <typename T> struct chunk;

// fp32: 4 values per 16 bytes.
template <> struct chunk<float> {
    static constexpr int kElems = 4;
    __device__ __forceinline__ static void load(const float* p, float (&v)[4]) {
        const float4 x = *reinterpret_cast<const float4*>(p);
        v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
    }
    __device__ __forceinline__ static void store(float* p, const float (&v)[4]) {
        *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    }
    __device__ __forceinline__ static float load1(const float* p) { return *p; }
    __device__ __forceinline__ static float round(float v) { return v; }
    __device__ __forceinline__ static void store1(float* p, float v) { *p = v; }
};

// bf16: 8 values per 16 bytes.
template <> struct chunk<bf16_t> {
    static constexpr int kElems = 8;
    __device__ __forceinline__ static void load(const bf16_t* p, float (&v)[8]) {
        const uint4 x = *reinterpret_cast<const uint4*>(p);
        const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v[2 * k] = __uint_as_float(w[k] << 16);
            v[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
        }
    }
    __device__ __forceinline__ static void store(bf16_t* p, const float (&v)[8]) {
        uint32_t w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) w[k] = f32_to_bf16(v[2 * k]) | (f32_to_bf16(v[2 * k + 1]) << 16);
        *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
    }
    __device__ __forceinline__ static float load1(const bf16_t* p) {
        return bf16_to_f32(p->bits);
    }
    __device__ __forceinline__ static void store1(bf16_t* p, float v) {
        p->bits = (uint16_t)f32_to_bf16(v);
    }
    // The value as it reads back after a store.
    __device__ __forceinline__ static float round(float v) { return bf16_to_f32(f32_to_bf16(v)); }
};

// Offset (in elements) of the A block of (b, h) given the per-graph slot
// offsets: graphs are per batch element when num_graphs == B, else one
// graph serves every (b, h).
__device__ __forceinline__ int64_t a_block_offset(const int64_t* slot_off, int32_t num_graphs,
                                                  int32_t H, int32_t b, int32_t h) {
    if (num_graphs == 1) return ((int64_t)b * H + h) * slot_off[1];
    const int64_t slots_b = slot_off[b + 1] - slot_off[b];
    return (int64_t)H * slot_off[b] + (int64_t)h * slots_b;
}

// The weight slots of one row for the generic kernels: its row segment
// [seg_begin, seg_end) (columns from slot_col) followed by its scheduled
// random edges (slots from rslot, columns from rnd), if any.
struct RowSlots {
    int64_t seg_begin, seg_len;
    const int32_t* slot_col;   // the graph's slot columns
    const int32_t* rslot;      // this row's random slots (or null)
    const int32_t* rcol;       // this row's random columns
    int32_t rcnt;

    __device__ __forceinline__ int64_t count() const { return seg_len + rcnt; }
    // Slot and column of the row's k-th slot; column -1 marks padding.
    __device__ __forceinline__ int64_t slot(int64_t k, int32_t& col) const {
        if (k < seg_len) {
            col = slot_col[seg_begin + k];
            return seg_begin + k;
        }
        col = rcol[k - seg_len];
        return rslot[k - seg_len];
    }
};

// Row i and pair bh of wave `wave` in a 1-D grid of 8 per_xcd workgroups
// of kW waves (xcd_row_grid): XCD blk % 8 takes items [x per_xcd,
// (x + 1) per_xcd) of the (bh, block of kW rows) order, so each XCD's L2
// serves the rows of few (b, h) pairs. False past the last item or row.
template <int kW>
__device__ __forceinline__ bool xcd_row_item(int64_t n, int32_t BH, int wave, int64_t& i,
                                             int32_t& bh) {
    const int64_t per_xcd = gridDim.x >> 3;
    const int64_t item = (int64_t)(blockIdx.x & 7u) * per_xcd + (blockIdx.x >> 3);
    const int64_t nrb = (n + kW - 1) / kW;
    if (item >= (int64_t)BH * nrb) return false;
    bh = (int32_t)(item / nrb);
    i = (item - (int64_t)bh * nrb) * kW + wave;
    return i < n;
}

// Workgroups of that grid.
inline dim3 xcd_row_grid(int64_t n, int32_t BH, int kW) {
    const int64_t items = (int64_t)BH * ((n + kW - 1) / kW);
    return dim3((unsigned)(8 * ((items + 7) / 8)));
}

// Graph arrays the generic kernels read.
struct GenericGraph {
    int64_t n;
    int32_t num_graphs, rnd_width;
    const int64_t* seg_ptr;    // [graphs][n + 1]
    const int32_t* slot_col;   // [slots of all graphs]
    const int64_t* slot_off;   // [graphs + 1]
    const int32_t* rnd;        // [graphs][n][rnd_width] (scheduled graphs, else null)
    const int32_t* rnd_cnt;    // [graphs][n]
    const int32_t* rslot;      // [graphs][n][rnd_width]
    const int32_t* long_rows;  // rows with more than kLongRow slots, per graph from long_off
    const int64_t* long_off;   // [graphs + 1]

    __device__ __forceinline__ RowSlots row(int32_t gr, int64_t i) const {
        RowSlots r;
        const int64_t* sp = seg_ptr + (int64_t)gr * (n + 1);
        r.seg_begin = sp[i];
        r.seg_len = sp[i + 1] - sp[i];
        r.slot_col = slot_col + slot_off[gr];
        r.rcnt = 0;
        r.rslot = nullptr;
        r.rcol = nullptr;
        if (rslot != nullptr) {
            const int64_t row = (int64_t)gr * n + i;
            r.rcnt = rnd_cnt[row];
            r.rslot = rslot + row * rnd_width;
            r.rcol = rnd + row * rnd_width;
        }
        return r;
    }
};

}  // namespace diffuser
