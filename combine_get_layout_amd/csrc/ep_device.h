// ep_device.h -- device-side helpers shared by the gfx950 kernels of libep.
//
// Wave64 throughout: one wavefront = 64 lanes; a 16-byte vector per lane makes
// one wave-wide load or store move 1 KiB of contiguous memory.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ep.h"

namespace ep {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kBlockThreads = 256;             // 4 waves per workgroup
constexpr int kWavesPerBlock = kBlockThreads / kWave;

// 512 B data-as-flag blocks: 480 B payload (30 vectors) + 32 B flag (2 vectors).
constexpr int kChunkBytes = 512;
constexpr int kChunkPayload = 480;
constexpr int kChunkPayloadVecs = 30;
constexpr int kChunkVecs = 32;

// A chunked row is moved one wave-iteration (two 512 B blocks, 1 KiB) at a
// time: lanes 0-31 cover block 2*it, lanes 32-63 block 2*it + 1. Byte offset
// of this lane's 16-byte vector of iteration `it`.
__device__ __forceinline__ int64_t chunk_lane_offset(int it, int lane) {
    const int c = 2 * it + (lane >> 5);
    return (int64_t)c * kChunkBytes + (int64_t)(lane & 31) * 16;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }
__device__ __forceinline__ int wave_in_block() { return threadIdx.x / kWave; }

__device__ __forceinline__ u32x4 ld16(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
}
// Streaming store: receive rows and outputs are written once and not re-read
// by this kernel, so keep them from displacing reusable lines in L2/MALL.
__device__ __forceinline__ void st16_stream(void* p, u32x4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
// Streaming load: rows read exactly once by the kernel.
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ int readlane(int v, int lane) {
    return __builtin_amdgcn_readlane(v, lane);
}
__device__ __forceinline__ float readlane_f(float v, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// The workspace holds two error words: err[0] covers the current pass of
// calls (the layout calls clear it), err[1] every call since the last
// ep_clear_errors (nothing else clears it). A report sets the bits in both.
__device__ __forceinline__ void report(uint32_t* err, uint32_t bits) {
    atomicOr(reinterpret_cast<unsigned int*>(err), bits);
    atomicOr(reinterpret_cast<unsigned int*>(err) + 1, bits);
}

// Wait (one thread) until the device-scope word *flag equals `value`, at most
// `timeout` wall-clock ticks (the device's wall-clock rate, kHz / 1000 per us),
// sleeping between polls; false if it never did. Used by the persistent
// launches for their per-batch flags.
__device__ __forceinline__ bool wait_flag_bounded(const uint32_t* flag, uint32_t value, uint64_t timeout) {
    const uint64_t start = (uint64_t)wall_clock64();
    for (;;) {
        if (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == value) return true;
        if ((uint64_t)wall_clock64() - start > timeout) return false;
        __builtin_amdgcn_s_sleep(8);
    }
}

// bf16 bit pattern -> float (bf16 is the upper half of a binary32).
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }

// float -> bf16 bits, round to nearest even; NaN -> 0x7FC0.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    uint32_t r = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
    return ((u & 0x7FFFFFFFu) > 0x7F800000u) ? 0x7FC0u : r;
}

// Division by a divisor that is fixed for a launch, as one multiply-high
// instead of the ~40-instruction integer division sequence. With m =
// ceil(2^32 / d) = (2^32 + eps) / d, 0 <= eps < d, n * m / 2^32 = n / d +
// n * eps / (d * 2^32), so floor(n * m / 2^32) = floor(n / d) whenever
// n * eps < 2^32: for every n < 2^20 and d <= 4096 (ids, ranks and groups stay
// below 4096 here). d = 1 (m would be 2^32) passes n through.
struct FastDiv {
    uint32_t m;  // ceil(2^32 / d), or 0 for d == 1
    static FastDiv make(uint32_t d) {
        FastDiv f;
        f.m = d == 1 ? 0u : (uint32_t)(((1ull << 32) + d - 1) / d);
        return f;
    }
    __device__ __forceinline__ int operator()(int n) const {
        return m ? (int)__umulhi((uint32_t)n, m) : n;
    }
};

// Expert id check shared by the kernels: -1 = no expert, anything else outside
// [0, E) is an error and behaves as -1.
__device__ __forceinline__ bool expert_ok(int64_t e, int E) { return e >= 0 && e < E; }
__device__ __forceinline__ bool expert_bad(int64_t e, int E) { return e < -1 || e >= E; }

}  // namespace ep
