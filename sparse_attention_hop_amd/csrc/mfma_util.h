// Device helpers shared by the LDS-streamed MFMA kernels (bf16 storage,
// v_mfma_f32_16x16x32_bf16).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "vec.h"

#define LDS_AS __attribute__((address_space(3)))

namespace diffuser {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// D += A B for a 16 x 32 A (lane l: row l % 16, k = 8 (l / 16) .. + 7) and a
// 32 x 16 B (lane l: column l % 16, the same k); D lane l holds rows
// 4 (l / 16) .. + 3 of column l % 16.
__device__ __forceinline__ f32x4 mfma_bf16(const u32x4& a, const u32x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ u32x4 load16(const uint16_t* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

// Direct global-to-LDS load of 16 bytes per active lane: lane l writes its
// 16 bytes at lds + 16 l (lds wave-uniform, src 16-byte aligned).
__device__ __forceinline__ void dma16(const void* src, void LDS_AS* lds) {
    __builtin_amdgcn_global_load_lds(src, lds, 16, 0, 0);
}

// Raw buffer resource over `bytes` bytes from `base`: a load at a byte
// offset at or past the end returns zero, which masks a lane's load without
// a branch.
// The base and size are wave-uniform; they are read from the first lane so
// that the descriptor lives in scalar registers. readfirstlane returns a
// signed int: each half goes through an unsigned 32-bit variable, since a
// sign-extended low half would set every bit of the high half.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
    const uint64_t u = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
    const uint64_t b = ((uint64_t)hi << 32) | lo;
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(b), (short)0,
                                             (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

constexpr uint32_t kOutside = 0x80000000u;   // a byte offset past every buffer used here

// 16 (8) bytes at lane offset voff plus wave-uniform offset soff.
__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                         r, (int)voff, (int)__builtin_amdgcn_readfirstlane(soff), 0));
}
__device__ __forceinline__ u32x2 bload8(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                                         r, (int)voff, (int)__builtin_amdgcn_readfirstlane(soff), 0));
}

// Load of a wave-uniform int32 of read-only graph data through the scalar
// cache (the constant address space).
__device__ __forceinline__ int32_t uniform_load(const int32_t* p) {
    const uint64_t u = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
    return *reinterpret_cast<const __attribute__((address_space(4))) int32_t*>(
        ((uint64_t)hi << 32) | lo);
}

// Waits for this wave's outstanding loads (direct-to-LDS ones included)
// and LDS traffic, then for the whole workgroup. The explicit vmcnt(0)
// matters: a workgroup barrier by itself does not wait for loads, and a
// direct-to-LDS load has only written LDS once it is counted complete.
__device__ __forceinline__ void full_barrier() {
    __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0); expcnt not waited
    __syncthreads();
}

// Barrier for LDS traffic only: global loads in flight stay in flight.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Work item (batch-head pair, sub-item) of workgroup `blk`: XCD blk % 8
// runs position blk / 8 of its own list. When the pairs split evenly over
// the 8 XCDs (bh_per_xcd > 0), an XCD's list is its pairs' global-row
// items (sub < grow), which read every key and take longest, followed by
// their row tiles (sub >= grow); otherwise the lists are consecutive runs
// of (bh, sub) order.
struct WorkItem {
    int32_t bh, sub;
    bool valid;
};

__device__ __forceinline__ WorkItem work_item(uint32_t blk, int32_t per_xcd, int32_t total,
                                              int32_t grow, int32_t tiles, int32_t bh_per_xcd) {
    const int32_t x = (int32_t)(blk & 7u), pos = (int32_t)(blk >> 3);
    WorkItem w{0, 0, false};
    if (bh_per_xcd > 0) {
        const int32_t ng = bh_per_xcd * grow;
        if (pos < ng) {
            w.bh = x * bh_per_xcd + pos / grow;
            w.sub = pos % grow;
            w.valid = true;
        } else if (pos - ng < bh_per_xcd * tiles) {
            w.bh = x * bh_per_xcd + (pos - ng) / tiles;
            w.sub = grow + (pos - ng) % tiles;
            w.valid = true;
        }
        return w;
    }
    const int32_t item = x * per_xcd + pos;
    if (item >= total) return w;
    w.bh = item / (grow + tiles);
    w.sub = item - w.bh * (grow + tiles);
    w.valid = true;
    return w;
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two floats to bf16 (round to nearest even) in one v_cvt_pk_bf16_f32; lo
// in the low half.
__device__ __forceinline__ uint32_t to_bf16_pair(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// The two bf16 halves of a word as floats.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

}  // namespace diffuser
