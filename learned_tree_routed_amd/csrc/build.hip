// Tree of key sums (ALHR README, opening paragraph and "Inference stage"):
// node (l, p) = node (l-1, 2p) + node (l-1, 2p+1), with the key rows as
// level 0, stored in heap order (node (l, p) is row (T >> l) + p).
//
// Level-synchronous reduction in passes.  A pass takes a tile of rows of one
// level (int8 key rows for the first pass, int32 tree rows after), and a
// workgroup reduces it through log2(tile) levels: the first level is summed
// straight from global memory, the later ones from an LDS copy of the level
// below.  Every level of a tile is a contiguous block of rows, so all global
// writes are coalesced 16-byte stores.  Tiles hold tile * d = 16384 elements,
// so the LDS level buffer is 32 KiB at every d.
#include "device.h"
#include "kernels.h"

namespace alhr {
namespace {

constexpr int kBuildThreads = 256;
constexpr int kTileElems = 16384;

template <int D, bool FROM_KEYS>
__global__ __launch_bounds__(kBuildThreads) void k_build_pass(const void* __restrict__ in,
                                                              int32_t* __restrict__ nodes, int T,
                                                              int in_level, int tile_rows,
                                                              int tiles_per_pair, int levels)
{
    constexpr int C4 = D / 4;   // 16-byte chunks of an int32 row
    __shared__ int4 lvl[kTileElems / 2 / 4];

    const int pair = blockIdx.x / tiles_per_pair;
    const int tile = blockIdx.x % tiles_per_pair;
    const size_t pair_row0 = (size_t)pair * T;
    const int in_first = tile * tile_rows;   // first input row (index within its level)

    // first output level: sums of input row pairs, read from global memory
    int rows = tile_rows / 2;
    int out_level = in_level + 1;
    {
        const size_t out_row0 = pair_row0 + (size_t)(T >> out_level) + in_first / 2;
        for (int c = threadIdx.x; c < rows * C4; c += kBuildThreads) {
            const int j = c / C4, g = c % C4;
            int4 sum;
            if constexpr (FROM_KEYS) {
                const int* k = reinterpret_cast<const int*>(in);
                const size_t r0 = (pair_row0 + in_first + 2 * j) * (D / 4);
                const int a = k[r0 + g], b = k[r0 + D / 4 + g];
                sum.x = sbyte(a, 0) + sbyte(b, 0);
                sum.y = sbyte(a, 1) + sbyte(b, 1);
                sum.z = sbyte(a, 2) + sbyte(b, 2);
                sum.w = sbyte(a, 3) + sbyte(b, 3);
            } else {
                const int4* n = reinterpret_cast<const int4*>(in);
                const size_t r0 = (pair_row0 + (size_t)(T >> in_level) + in_first + 2 * j) * C4;
                const int4 a = n[r0 + g], b = n[r0 + C4 + g];
                sum = make_int4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
            }
            lvl[c] = sum;
            reinterpret_cast<int4*>(nodes)[(out_row0 + j) * C4 + g] = sum;
        }
    }
    // later levels from the LDS copy of the level below
    for (int k = 1; k < levels; ++k) {
        __syncthreads();
        rows >>= 1;
        ++out_level;
        const size_t out_row0 = pair_row0 + (size_t)(T >> out_level) + (in_first >> (k + 1));
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
                reinterpret_cast<int4*>(nodes)[(out_row0 + j) * C4 + g] = acc[u];
            }
        }
    }
}

template <int D>
hipError_t build_d(const Shape& s, const int8_t* K, int32_t* nodes, hipStream_t st)
{
    int in_level = 0;
    while (in_level < s.L) {
        const int avail = s.T >> in_level;
        const int tile = avail < kTileElems / D ? avail : kTileElems / D;
        int levels = 0;
        while ((1 << levels) < tile) ++levels;
        const int tiles = avail / tile;
        const dim3 grid((unsigned)(s.P * tiles));
        if (in_level == 0)
            hipLaunchKernelGGL((k_build_pass<D, true>), grid, dim3(kBuildThreads), 0, st,
                               (const void*)K, nodes, s.T, in_level, tile, tiles, levels);
        else
            hipLaunchKernelGGL((k_build_pass<D, false>), grid, dim3(kBuildThreads), 0, st,
                               (const void*)nodes, nodes, s.T, in_level, tile, tiles, levels);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        in_level += levels;
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_build(const Shape& s, const int8_t* K, int32_t* nodes, hipStream_t st)
{
    switch (s.d) {
        case 16: return build_d<16>(s, K, nodes, st);
        case 32: return build_d<32>(s, K, nodes, st);
        case 64: return build_d<64>(s, K, nodes, st);
        case 128: return build_d<128>(s, K, nodes, st);
        case 256: return build_d<256>(s, K, nodes, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace alhr
