// Tree of key sums (ALHR README, opening paragraph and "Inference stage"),
// device code shared by the build launches and the fused preparation launch:
// node (l, p) = node (l-1, 2p) + node (l-1, 2p+1), with the key rows as
// level 0, stored in heap order (node (l, p) is row (T >> l) + p).
//
// Level-synchronous reduction in passes.  A pass takes a tile of rows of one
// level (int8 key rows for the first pass, tree rows after), and a workgroup
// reduces it through log2(tile) levels: the first level is summed straight
// from global memory, the later ones from an LDS copy of the level below.
// Every level of a tile is a contiguous block of rows, so all global writes
// are coalesced.  Tiles hold tile * d = 16384 elements, so the LDS level
// buffer is 32 KiB at every d.
//
// Storage: rows of levels 1..l16 (the levels whose sums fit int16 under the
// declared key bound) are d int16, packed densely after the int32 rows of
// the higher levels (see tree_row16).  Sums are formed in int32 either way.
#pragma once

#include "device.h"

namespace alhr {
namespace buildk {

constexpr int kBuildThreads = 256;
constexpr int kTileElems = 16384;

enum InKind { kInKeys = 0, kInI16 = 1, kInI32 = 2 };

__device__ __forceinline__ int pack16(int lo, int hi) { return (lo & 0xFFFF) | (hi << 16); }
__device__ __forceinline__ int lo16(int w) { return (int)(short)(w & 0xFFFF); }
__device__ __forceinline__ int hi16(int w) { return w >> 16; }

// Store 4 sums (columns 4g .. 4g+3, natural slot g) of heap row r of pair
// `pair_table`, int16 or int32 by level.
template <int D>
__device__ __forceinline__ void store_chunk(int32_t* __restrict__ pair_table, int T, int l16,
                                            size_t r, int g, int4 v, bool narrow)
{
    if (narrow)
        reinterpret_cast<int2*>(const_cast<int32_t*>(tree_row16<D>(pair_table, T, l16, r)))[g] =
            make_int2(pack16(v.x, v.y), pack16(v.z, v.w));
    else
        reinterpret_cast<int4*>(pair_table + r * D)[wide_slot<D>(g)] = v;
}

// Load 4 columns (natural slot g) of input row r (key row r, or heap row r
// of a tree level).
template <int D, int IN>
__device__ __forceinline__ int4 load_chunk(const void* __restrict__ in_pair, int T, int l16,
                                           size_t r, int g)
{
    if constexpr (IN == kInKeys) {
        const int w = reinterpret_cast<const int*>(in_pair)[r * (D / 4) + g];
        return make_int4(sbyte(w, 0), sbyte(w, 1), sbyte(w, 2), sbyte(w, 3));
    } else if constexpr (IN == kInI16) {
        const int2 w = reinterpret_cast<const int2*>(
            tree_row16<D>(reinterpret_cast<const int32_t*>(in_pair), T, l16, r))[g];
        return make_int4(lo16(w.x), hi16(w.x), lo16(w.y), hi16(w.y));
    } else {
        return reinterpret_cast<const int4*>(
            tree_row32<D>(reinterpret_cast<const int32_t*>(in_pair), r))[wide_slot<D>(g)];
    }
}

// One tile of a build pass: workgroup `blk` of the pass, kBuildThreads
// threads, `lvl` an LDS buffer of kTileElems / 2 int32.
template <int D, int IN>
__device__ __forceinline__ void build_tile(int blk, int4* lvl, const void* __restrict__ in,
                                           int32_t* __restrict__ nodes, int T, int in_level,
                                           int tile_rows, int tiles_per_pair, int levels, int l16)
{
    constexpr int C4 = D / 4;   // 4-column chunks of a row

    const int pair = blk / tiles_per_pair;
    const int tile = blk % tiles_per_pair;
    const int in_first = tile * tile_rows;   // first input row (index within its level)
    const void* in_pair = IN == kInKeys
        ? static_cast<const void*>(static_cast<const int8_t*>(in) + (size_t)pair * T * D)
        : static_cast<const void*>(static_cast<const int32_t*>(in) + (size_t)pair * T * D);
    int32_t* out_pair = nodes + (size_t)pair * T * D;
    const size_t in_row0 = (IN == kInKeys ? 0 : (size_t)(T >> in_level)) + in_first;

    // first output level: sums of input row pairs, read from global memory
    int rows = tile_rows / 2;
    int out_level = in_level + 1;
    {
        const size_t out_row0 = (size_t)(T >> out_level) + in_first / 2;
        const bool narrow = out_level <= l16;
        // every load of the level issued before the first sum (a tile's
        // first level is at most kTileElems / 8 chunks, kFirstPer per thread);
        // the loads are unconditional, chunks past the level re-reading its
        // last chunk, so that nothing separates them
        constexpr int kFirstPer = kTileElems / 2 / 4 / kBuildThreads;
        const int last = rows * C4 - 1;
        int4 a[kFirstPer], b[kFirstPer];
#pragma unroll
        for (int u = 0; u < kFirstPer; ++u) {
            const int c = min(threadIdx.x + u * kBuildThreads, last);
            const int j = c / C4, g = c % C4;
            a[u] = load_chunk<D, IN>(in_pair, T, l16, in_row0 + 2 * j, g);
            b[u] = load_chunk<D, IN>(in_pair, T, l16, in_row0 + 2 * j + 1, g);
        }
#pragma unroll
        for (int u = 0; u < kFirstPer; ++u) {
            const int c = threadIdx.x + u * kBuildThreads;
            if (c < rows * C4) {
                const int j = c / C4, g = c % C4;
                const int4 sum = make_int4(a[u].x + b[u].x, a[u].y + b[u].y, a[u].z + b[u].z,
                                           a[u].w + b[u].w);
                lvl[c] = sum;
                store_chunk<D>(out_pair, T, l16, out_row0 + j, g, sum, narrow);
            }
        }
    }
    // later levels from the LDS copy of the level below
    for (int k = 1; k < levels; ++k) {
        __syncthreads();
        rows >>= 1;
        ++out_level;
        const size_t out_row0 = (size_t)(T >> out_level) + (in_first >> (k + 1));
        const bool narrow = out_level <= l16;
        constexpr int kMaxPer = kTileElems / 4 / 4 / kBuildThreads;   // chunks per thread, level 2
        int4 acc[kMaxPer > 0 ? kMaxPer : 1];
        int nmine = 0;
#pragma unroll
        for (int u = 0; u < (kMaxPer > 0 ? kMaxPer : 1); ++u) {
            const int c = threadIdx.x + u * kBuildThreads;
            if (c < rows * C4) {
                const int j = c / C4, g = c % C4;
                const int4 a = lvl[(2 * j) * C4 + g], b = lvl[(2 * j + 1) * C4 + g];
                acc[u] = make_int4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
                nmine = u + 1;
            }
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < (kMaxPer > 0 ? kMaxPer : 1); ++u) {
            const int c = threadIdx.x + u * kBuildThreads;
            if (u < nmine) {
                const int j = c / C4, g = c % C4;
                lvl[c] = acc[u];
                store_chunk<D>(out_pair, T, l16, out_row0 + j, g, acc[u], narrow);
            }
        }
    }
}

// Tiling of the pass that starts at level in_level: tile rows, levels per
// tile and tiles per pair.
struct BuildPass {
    int tile, levels, tiles;
};
__host__ __device__ inline BuildPass build_pass_plan(int T, int d, int in_level)
{
    const int avail = T >> in_level;
    const int tile = avail < kTileElems / d ? avail : kTileElems / d;
    int levels = 0;
    while ((1 << levels) < tile) ++levels;
    return BuildPass{tile, levels, avail / tile};
}

}  // namespace buildk
}  // namespace alhr
