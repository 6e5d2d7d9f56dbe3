// Device helpers shared by the gfx950 kernels of libalhr (wave64 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace alhr {

constexpr int kWave = 64;
constexpr int kXcds = 8;   // MI355X: 8 accelerator complex dies, round-robin dispatch

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Keep the compiler from moving LDS accesses across this point; LDS traffic
// of one wave is processed in order by the hardware.
__device__ __forceinline__ void wave_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Workgroups are dispatched round-robin over the XCDs; remap the hardware
// block id so that a contiguous range of logical blocks lands on one XCD and
// shares its L2.  Requires gridDim.x % kXcds == 0.
__device__ __forceinline__ uint32_t xcd_logical_block()
{
    uint32_t b = blockIdx.x, g = gridDim.x;
    return (b % kXcds) * (g / kXcds) + b / kXcds;
}

__device__ __forceinline__ int popc64(uint64_t m) { return __popcll(m); }

__device__ __forceinline__ uint32_t mbcnt(uint64_t m)
{
    uint32_t lo = __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u);
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), lo);
}

__device__ __forceinline__ int wave_count(bool p) { return popc64(__ballot(p)); }

template <typename T> __device__ __forceinline__ T wave_max(T v)
{
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        T w = __shfl_xor(v, o);
        v = w > v ? w : v;
    }
    return v;
}

template <typename T> __device__ __forceinline__ T wave_min(T v)
{
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        T w = __shfl_xor(v, o);
        v = w < v ? w : v;
    }
    return v;
}

template <typename T> __device__ __forceinline__ T wave_sum(T v)
{
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) v += __shfl_xor(v, o);
    return v;
}

// Sum over aligned groups of G consecutive lanes (G a power of two <= 64);
// every lane of the group receives the group sum.
template <int G, typename T> __device__ __forceinline__ T group_sum(T v)
{
#pragma unroll
    for (int o = 1; o < G; o <<= 1) v += __shfl_xor(v, o);
    return v;
}

__device__ __forceinline__ int dot4_i8(int a, int b, int acc)
{
    return __builtin_amdgcn_sdot4(a, b, acc, false);
}

// int8 byte e of a packed word, sign-extended.
__device__ __forceinline__ int sbyte(int w, int e) { return (int)(int8_t)(w >> (8 * e)); }

}  // namespace alhr
