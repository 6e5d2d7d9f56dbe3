// Decode-cache maintenance (openai-hub article "ALHR把注意力变成树搜索",
// section "ALHR是什么": one new token per step; tree of key sums from the
// ALHR README's opening paragraph).
//
// Append at position pos: the key and value rows are stored, the key is added
// to each of the L ancestor sums (node (l, pos >> l), l = 1..L) and to the
// running causal key sum.  One thread owns 4 columns of one pair, so the L
// read-modify-writes of a pair are independent 16-byte accesses issued
// back to back, and no two threads touch the same word.
#include "device.h"
#include "kernels.h"

namespace alhr {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxLevels = 20;   // T <= 2^20

__device__ __forceinline__ int pack16(int lo, int hi) { return (lo & 0xFFFF) | (hi << 16); }
__device__ __forceinline__ int lo16(int w) { return (int)(short)(w & 0xFFFF); }
__device__ __forceinline__ int hi16(int w) { return w >> 16; }

template <int D>
__global__ __launch_bounds__(kThreads) void k_append(const int8_t* __restrict__ k_new,
                                                     const float* __restrict__ v_new,
                                                     int8_t* __restrict__ K,
                                                     float* __restrict__ V,
                                                     int32_t* __restrict__ nodes,
                                                     int32_t* __restrict__ prefix, int P, int T,
                                                     int L, int l16, int pos)
{
    constexpr int C4 = D / 4;
    const int gid = blockIdx.x * kThreads + threadIdx.x;
    if (gid >= P * C4) return;
    const int pair = gid / C4, g = gid % C4;
    const int kw = reinterpret_cast<const int*>(k_new)[(size_t)pair * C4 + g];
    const int4 kv = make_int4(sbyte(kw, 0), sbyte(kw, 1), sbyte(kw, 2), sbyte(kw, 3));
    // key bytes of the even and the odd thread of this thread's pair g, g ^ 1
    // (C4 is even, so both belong to the same (batch, head) pair)
    const int kw_partner = __shfl_xor(kw, 1);
    const int kw_even = (g & 1) ? kw_partner : kw, kw_odd = (g & 1) ? kw : kw_partner;
    const size_t row = (size_t)pair * T + pos;
    reinterpret_cast<int*>(K)[row * C4 + g] = kw;
    reinterpret_cast<float4*>(V)[row * C4 + g] =
        reinterpret_cast<const float4*>(v_new)[(size_t)pair * C4 + g];
    // All L ancestor cells (and the running sum) are loaded before anything
    // is stored, so the loads are in flight together instead of one
    // dependent round trip per level.  Levels 1..l16 hold int16 rows, higher
    // levels int32.  No load or store sits in a branch (a branch around a
    // memory access makes the next one wait for it): every level is one
    // 16-byte load and one 16-byte store at a selected address.  At an int16
    // level, threads g and g ^ 1 share one 16-byte chunk (8 columns) and
    // both write the same updated chunk.  The level loop runs to kMaxLevels
    // with the level clamped to L, so it has no branch either: the extra
    // iterations re-read and re-write the root with the same value.
    int32_t* tree = nodes + (size_t)pair * T * D;
    int4* pre = reinterpret_cast<int4*>(prefix) + (size_t)pair * C4 + g;
    int4* cell_at[kMaxLevels];
    int4 cells[kMaxLevels];
#pragma unroll
    for (int i = 1; i <= kMaxLevels; ++i) {
        const int l = i < L ? i : L;
        const size_t r = (size_t)((T >> l) + (pos >> l));
        cell_at[i - 1] = l <= l16
            ? reinterpret_cast<int4*>(const_cast<int32_t*>(tree_row16<D>(tree, T, l16, r))) +
                  (g >> 1)
            : reinterpret_cast<int4*>(tree + r * D) + wide_slot<D>(g);
        cells[i - 1] = *cell_at[i - 1];
    }
    const int4 p = *pre;
#pragma unroll
    for (int i = 1; i <= kMaxLevels; ++i) {
        const int l = i < L ? i : L;
        const int4 c = cells[i - 1];
        const int4 wide = make_int4(c.x + kv.x, c.y + kv.y, c.z + kv.z, c.w + kv.w);
        const int4 narrow = make_int4(
            pack16(lo16(c.x) + sbyte(kw_even, 0), hi16(c.x) + sbyte(kw_even, 1)),
            pack16(lo16(c.y) + sbyte(kw_even, 2), hi16(c.y) + sbyte(kw_even, 3)),
            pack16(lo16(c.z) + sbyte(kw_odd, 0), hi16(c.z) + sbyte(kw_odd, 1)),
            pack16(lo16(c.w) + sbyte(kw_odd, 2), hi16(c.w) + sbyte(kw_odd, 3)));
        const bool nar = l <= l16;   // per-component select, no int4 temporary
        *cell_at[i - 1] = make_int4(nar ? narrow.x : wide.x, nar ? narrow.y : wide.y,
                                    nar ? narrow.z : wide.z, nar ? narrow.w : wide.w);
    }
    *pre = make_int4(p.x + kv.x, p.y + kv.y, p.z + kv.z, p.w + kv.w);
}

// prefix[pair] = sum of the maximal complete subtrees covering [0, n).
template <int D>
__global__ __launch_bounds__(kThreads) void k_prefix_from_tree(const int8_t* __restrict__ K,
                                                               const int32_t* __restrict__ nodes,
                                                               int32_t* __restrict__ prefix,
                                                               int P, int T, int L, int l16,
                                                               int n)
{
    constexpr int C4 = D / 4;
    const int gid = blockIdx.x * kThreads + threadIdx.x;
    if (gid >= P * C4) return;
    const int pair = gid / C4, g = gid % C4;
    int4 acc = make_int4(0, 0, 0, 0);
    for (int l = L; l >= 0; --l) {
        if (!((n >> l) & 1)) continue;
        const int start = n & ~((2 << l) - 1);
        if (l == 0) {
            const int kw =
                reinterpret_cast<const int*>(K)[((size_t)pair * T + start) * C4 + g];
            acc.x += sbyte(kw, 0);
            acc.y += sbyte(kw, 1);
            acc.z += sbyte(kw, 2);
            acc.w += sbyte(kw, 3);
        } else {
            const int32_t* tree = nodes + (size_t)pair * T * D;
            const size_t r = (size_t)((T >> l) + (start >> l));
            const int32_t* row = l <= l16 ? tree_row16<D>(tree, T, l16, r) : tree_row32<D>(tree, r);
            int4 v;
            if (l <= l16) {
                const int2 w = reinterpret_cast<const int2*>(row)[g];
                v = make_int4(lo16(w.x), hi16(w.x), lo16(w.y), hi16(w.y));
            } else {
                v = reinterpret_cast<const int4*>(row)[wide_slot<D>(g)];
            }
            acc.x += v.x;
            acc.y += v.y;
            acc.z += v.z;
            acc.w += v.w;
        }
    }
    reinterpret_cast<int4*>(prefix)[(size_t)pair * C4 + g] = acc;
}

unsigned blocks_for(int P, int d) { return (unsigned)(((size_t)P * (d / 4) + kThreads - 1) / kThreads); }

}  // namespace

hipError_t launch_append(const Shape& s, int pos, const int8_t* k_new, const float* v_new,
                         int8_t* K, float* V, int32_t* nodes, int32_t* prefix, hipStream_t st)
{
    const dim3 grid(blocks_for(s.P, s.d));
#define ALHR_APPEND(DD)                                                                        \
    hipLaunchKernelGGL((k_append<DD>), grid, dim3(kThreads), 0, st, k_new, v_new, K, V, nodes, \
                       prefix, s.P, s.T, s.L, s.l16, pos)
    switch (s.d) {
        case 16: ALHR_APPEND(16); break;
        case 32: ALHR_APPEND(32); break;
        case 64: ALHR_APPEND(64); break;
        case 128: ALHR_APPEND(128); break;
        case 256: ALHR_APPEND(256); break;
        default: return hipErrorInvalidValue;
    }
#undef ALHR_APPEND
    return hipGetLastError();
}

hipError_t launch_prefix_from_tree(const Shape& s, int n, const int8_t* K, const int32_t* nodes,
                                   int32_t* prefix, hipStream_t st)
{
    const dim3 grid(blocks_for(s.P, s.d));
#define ALHR_PREFIX(DD)                                                                       \
    hipLaunchKernelGGL((k_prefix_from_tree<DD>), grid, dim3(kThreads), 0, st, K, nodes, prefix, \
                       s.P, s.T, s.L, s.l16, n)
    switch (s.d) {
        case 16: ALHR_PREFIX(16); break;
        case 32: ALHR_PREFIX(32); break;
        case 64: ALHR_PREFIX(64); break;
        case 128: ALHR_PREFIX(128); break;
        case 256: ALHR_PREFIX(256); break;
        default: return hipErrorInvalidValue;
    }
#undef ALHR_PREFIX
    return hipGetLastError();
}

}  // namespace alhr
