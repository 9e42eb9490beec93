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

}  // namespace diffuser
