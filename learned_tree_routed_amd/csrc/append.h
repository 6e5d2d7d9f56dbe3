// Decode append of one key and value row (openai-hub article
// "ALHR把注意力变成树搜索", section "ALHR是什么": one new token per step; tree
// of key sums from the ALHR README's opening paragraph), shared by the
// append kernel and the fused append + decode kernel.
//
// Thread g < d/4 of a pair owns 4 columns: it stores its part of the key and
// value rows at pos, adds the key to each of the L ancestor sums
// (node (l, pos >> l), l = 1..L) and to the running causal key sum.  Threads
// g and g ^ 1 must be adjacent lanes of one wave (they exchange key words).
#pragma once

#include "device.h"

namespace alhr {
namespace appendk {

constexpr int kMaxLevels = 20;   // T <= 2^20

__device__ __forceinline__ int pack16(int lo, int hi) { return (lo & 0xFFFF) | (hi << 16); }
__device__ __forceinline__ int lo16(int w) { return (int)(short)(w & 0xFFFF); }
__device__ __forceinline__ int hi16(int w) { return w >> 16; }

template <int D>
__device__ __forceinline__ void append_columns(int pair, int g, const int8_t* __restrict__ k_new,
                                               const float* __restrict__ v_new,
                                               int8_t* __restrict__ K, float* __restrict__ V,
                                               int32_t* __restrict__ nodes,
                                               int32_t* __restrict__ prefix, int T, int L,
                                               int l16, int pos)
{
    constexpr int C4 = D / 4;
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

// The append spread over NT threads of a workgroup (thread index tid < NT)
// for one pair, in two halves so that the caller's own loads can be in
// flight with these: load() reads the new key and this thread's ancestor
// cells, store() writes the cells with the key added.  No store comes before
// a load: a wave's loads and stores share one completion counter, so a
// store issued first would hold up the loads.  The key and value rows at pos
// are the caller's to store.  Thread tid owns column chunk
// g = tid % (d/4) at the levels lgrp + 1, lgrp + 1 + groups, ...
// (lgrp = tid / (d/4), groups = NT / (d/4)); threads g and g ^ 1 of a level
// group are adjacent lanes (d/4 is even and divides 64).  The running sum
// is not touched here: its owner forms S[pos] = S[pos-1] + k_new itself.
template <int D, int NT>
struct SpreadAppend {
    static constexpr int C4 = D / 4, NG = NT / C4;
    static constexpr int kPer = (kMaxLevels + NG - 1) / NG;   // levels per thread at most
    static_assert(NT % C4 == 0 && 64 % C4 == 0 && C4 % 2 == 0, "column chunks tile the waves");
    int4 cells[kPer];
    int kw;

    __device__ __forceinline__ static int4* cell(int32_t* tree, int T, int l16, int pos, int l,
                                                 int g)
    {
        const size_t r = (size_t)((T >> l) + (pos >> l));
        return l <= l16
            ? reinterpret_cast<int4*>(const_cast<int32_t*>(tree_row16<D>(tree, T, l16, r))) +
                  (g >> 1)
            : reinterpret_cast<int4*>(tree + r * D) + wide_slot<D>(g);
    }

    __device__ __forceinline__ void load(int tid, int pair, const int8_t* __restrict__ k_new,
                                         const int32_t* __restrict__ nodes, int T, int L, int l16,
                                         int pos)
    {
        const int g = tid % C4, lgrp = tid / C4;
        kw = reinterpret_cast<const int*>(k_new)[(size_t)pair * C4 + g];
        int32_t* tree = const_cast<int32_t*>(nodes) + (size_t)pair * T * D;
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            const int l0 = lgrp + 1 + k * NG;
            const int l = l0 < L ? l0 : L;   // clamped: extra cells re-read the root
            cells[k] = *cell(tree, T, l16, pos, l, g);
        }
    }

    __device__ __forceinline__ void store(int tid, int pair, int32_t* __restrict__ nodes, int T,
                                          int L, int l16, int pos) const
    {
        const int g = tid % C4, lgrp = tid / C4;
        const int4 kv = make_int4(sbyte(kw, 0), sbyte(kw, 1), sbyte(kw, 2), sbyte(kw, 3));
        // key bytes of the even and the odd thread of this thread's pair g, g ^ 1
        const int kw_partner = __shfl_xor(kw, 1);
        const int kw_even = (g & 1) ? kw_partner : kw, kw_odd = (g & 1) ? kw : kw_partner;
        int32_t* tree = nodes + (size_t)pair * T * D;
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            const int l0 = lgrp + 1 + k * NG;
            const int l = l0 < L ? l0 : L;
            const int4 c = cells[k];
            const int4 wide = make_int4(c.x + kv.x, c.y + kv.y, c.z + kv.z, c.w + kv.w);
            const int4 narrow = make_int4(
                pack16(lo16(c.x) + sbyte(kw_even, 0), hi16(c.x) + sbyte(kw_even, 1)),
                pack16(lo16(c.y) + sbyte(kw_even, 2), hi16(c.y) + sbyte(kw_even, 3)),
                pack16(lo16(c.z) + sbyte(kw_odd, 0), hi16(c.z) + sbyte(kw_odd, 1)),
                pack16(lo16(c.w) + sbyte(kw_odd, 2), hi16(c.w) + sbyte(kw_odd, 3)));
            const bool nar = l <= l16;
            // several threads may clamp to the root: only the one whose level is
            // really L (or, past L, none) writes it
            if (l0 <= L)
                *cell(tree, T, l16, pos, l, g) =
                    make_int4(nar ? narrow.x : wide.x, nar ? narrow.y : wide.y,
                              nar ? narrow.z : wide.z, nar ? narrow.w : wide.w);
        }
    }
};

}  // namespace appendk
}  // namespace alhr
