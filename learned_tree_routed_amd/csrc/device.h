// Device helpers shared by the gfx950 kernels of libalhr (wave64 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace alhr {

constexpr int kWave = 64;
constexpr int kXcds = 8;   // MI355X: 8 accelerator complex dies, round-robin dispatch

// The lane index, opaque to the optimiser: values derived from it are
// recomputed where they are used instead of being hoisted out of loops and
// held in vector registers for a kernel's whole run (which cost the
// persistent routing kernel two waves per SIMD).
__device__ __forceinline__ int lane_id()
{
    int l = __lane_id();
    asm volatile("" : "+v"(l));
    return l;
}

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

// Marks a value that is the same in every lane, so the compiler keeps it in
// a scalar register and branches on it with scalar code.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ uint32_t uniform(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_readfirstlane((int)v);
}

// ---- cross-lane reductions with DPP (no LDS traffic) ----------------------
// gfx9 DPP controls: quad_perm [1,0,3,2] = 0xB1, [2,3,0,1] = 0x4E,
// row_mirror = 0x140, row_half_mirror = 0x141.
template <int CTRL> __device__ __forceinline__ int dpp(int v)
{
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL> __device__ __forceinline__ float dppf(float v)
{
    return __int_as_float(dpp<CTRL>(__float_as_int(v)));
}

// Sum over aligned groups of G consecutive lanes (G in 1, 2, 4, 8, 16); every
// lane of the group receives the group sum.
template <int G> __device__ __forceinline__ int group_sum(int v)
{
    static_assert(G == 1 || G == 2 || G == 4 || G == 8 || G == 16, "group size");
    if constexpr (G >= 2) v += dpp<0xB1>(v);
    if constexpr (G >= 4) v += dpp<0x4E>(v);
    if constexpr (G >= 8) v += dpp<0x141>(v);
    if constexpr (G >= 16) v += dpp<0x140>(v);
    return v;
}

// Whole-wave reductions returning a wave-uniform value: butterfly within each
// 16-lane row by DPP (every lane then holds its row's result), then
// row_bcast:15 folds rows 0 and 2 into rows 1 and 3 and row_bcast:31 folds
// row 1 into rows 2 and 3, so lane 63 holds the result.  Rows left out by the
// row mask keep `id` as the DPP operand (the identity of op).
template <int CTRL, int ROWS> __device__ __forceinline__ int dpp_rows(int id, int v)
{
    return __builtin_amdgcn_update_dpp(id, v, CTRL, ROWS, 0xF, false);
}
template <typename Op> __device__ __forceinline__ int wave_reduce_i(int v, int id, Op op)
{
    v = op(v, dpp<0xB1>(v));
    v = op(v, dpp<0x4E>(v));
    v = op(v, dpp<0x141>(v));
    v = op(v, dpp<0x140>(v));
    v = op(v, dpp_rows<0x142, 0xA>(id, v));
    v = op(v, dpp_rows<0x143, 0xC>(id, v));
    return __builtin_amdgcn_readlane(v, 63);
}
template <typename Op> __device__ __forceinline__ float wave_reduce_f(float v, float id, Op op)
{
    v = op(v, dppf<0xB1>(v));
    v = op(v, dppf<0x4E>(v));
    v = op(v, dppf<0x141>(v));
    v = op(v, dppf<0x140>(v));
    v = op(v, __int_as_float(dpp_rows<0x142, 0xA>(__float_as_int(id), __float_as_int(v))));
    v = op(v, __int_as_float(dpp_rows<0x143, 0xC>(__float_as_int(id), __float_as_int(v))));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    return (uint32_t)wave_reduce_i((int)v, 0, [](int a, int b) { return (int)((uint32_t)a > (uint32_t)b ? a : b); });
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v)
{
    return (uint32_t)wave_reduce_i((int)v, -1, [](int a, int b) { return (int)((uint32_t)a < (uint32_t)b ? a : b); });
}
__device__ __forceinline__ int wave_max_i32(int v)
{
    return wave_reduce_i(v, (int)0x80000000, [](int a, int b) { return a > b ? a : b; });
}
__device__ __forceinline__ float wave_sum_f(float v)
{
    return wave_reduce_f(v, 0.0f, [](float a, float b) { return a + b; });
}

// Generic shuffle reduction, for the rare wider types.
template <typename T> __device__ __forceinline__ T wave_max(T v)
{
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        T w = __shfl_xor(v, o);
        v = w > v ? w : v;
    }
    return v;
}

// ---- tree table layout ----------------------------------------------------
// One pair's table is T * d * 4 bytes.  Heap row r (node (l, p) is row
// (T >> l) + p) of a level l > l16 is d int32 at byte r * 4d; rows of levels
// 1..l16 (r >= T >> l16) are d int16, packed densely after the int32 rows:
// byte (T >> l16) * 4d + (r - (T >> l16)) * 2d.
//
// Column order inside an int32 row: its d/4 16-byte slots form 4 blocks of
// LPR = d/16 slots, and the natural slot g = 2c + h (8-column chunk c, half
// h) is stored at slot (2 * (c / LPR) + h) * LPR + c % LPR.  Lane s of a row
// group (which holds the query for chunks s and LPR + s) then reads slots
// s, LPR + s, 2 LPR + s and 3 LPR + s, so each of its four loads covers one
// contiguous block of the row.  int16 rows keep the natural order: chunk c
// is slot c.
template <int D>
__host__ __device__ constexpr int wide_slot(int g)
{
    constexpr int LPR = D / 16;
    return (2 * ((g >> 1) / LPR) + (g & 1)) * LPR + (g >> 1) % LPR;
}

template <int D>
__device__ __forceinline__ const int32_t* tree_row32(const int32_t* pair_table, size_t r)
{
    return pair_table + r * D;
}
template <int D>
__device__ __forceinline__ const int32_t* tree_row16(const int32_t* pair_table, int T, int l16,
                                                     size_t r)
{
    const size_t b16 = (size_t)(T >> l16);
    return reinterpret_cast<const int32_t*>(reinterpret_cast<const char*>(pair_table) +
                                            b16 * 4 * D + (r - b16) * 2 * D);
}

// A global-memory base known to be the same in every lane: kept in scalar
// registers, so loads through it take the scalar-base form (SGPR base +
// 32-bit lane offset) and each lane computes only a 32-bit byte offset.
typedef const char __attribute__((address_space(1))) gbyte;

__device__ __forceinline__ gbyte* uniform_base(const void* p)
{
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<gbyte*>(((uint64_t)hi << 32) | lo);
}

// 16 bytes at byte offset `off` (16-byte aligned) from a uniform base.
typedef int gvec4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ int4 load16(gbyte* base, uint32_t off)
{
    const gvec4 v = *reinterpret_cast<const gvec4 __attribute__((address_space(1)))*>(base + off);
    return make_int4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ int dot4_i8(int a, int b, int acc)
{
    return __builtin_amdgcn_sdot4(a, b, acc, false);
}

// int8 byte e of a packed word, sign-extended.
__device__ __forceinline__ int sbyte(int w, int e) { return (int)(int8_t)(w >> (8 * e)); }

}  // namespace alhr
