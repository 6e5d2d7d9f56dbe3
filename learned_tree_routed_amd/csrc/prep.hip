// Tree build and budget prediction in two shared launches.  The two steps
// are independent (both read only the key rows, the predictor also the
// queries), so each launch carries the workgroups of one build pass and of
// one predictor pass side by side, and neither step waits on the other:
//   launch 1: build pass from the key rows  +  predictor chunk totals;
//   launch 2: the next build pass (if any)  +  predictor final pass;
// further build passes (T above the two passes' levels) follow on their own.
// A workgroup takes one role by its block index (uniform over the
// workgroup); the LDS of the two roles is a union.  Results equal those of
// alhr_build_tree and alhr_predict_budget, which run the same device code.
#include "build_impl.h"
#include "kernels.h"
#include "predict_impl.h"

namespace alhr {
namespace {

using namespace buildk;
using namespace predictk;
static_assert(kBuildThreads == kChunk, "one workgroup size for both roles");

template <int D>
union FirstLds {
    int4 lvl[kTileElems / 2 / 4];
    ChunksLds<D> pc;
};

template <int D>
union SecondLds {
    int4 lvl[kTileElems / 2 / 4];
    FinalLds<D> pf;
};

template <int D>
__global__ __launch_bounds__(kChunk) void k_prep_first(const int8_t* __restrict__ K,
                                                       int32_t* __restrict__ nodes,
                                                       const int8_t* __restrict__ W,
                                                       int32_t* __restrict__ tot, int T,
                                                       int tile_rows, int tiles_per_pair,
                                                       int levels, int l16, int nc, int nbuild)
{
    __shared__ FirstLds<D> sm;
    if ((int)blockIdx.x < nbuild)
        build_tile<D, kInKeys>(blockIdx.x, sm.lvl, K, nodes, T, 0, tile_rows, tiles_per_pair,
                               levels, l16);
    else
        predict_chunks_block<D>(blockIdx.x - nbuild, sm.pc, K, W, tot, T, nc);
}

template <int D, int IN>
__global__ __launch_bounds__(kChunk) void k_prep_second(
    int32_t* __restrict__ nodes, int in_level, int tile_rows, int tiles_per_pair, int levels,
    int l16, const int8_t* __restrict__ Q, const int8_t* __restrict__ K,
    const int8_t* __restrict__ W, const int32_t* __restrict__ tot, int32_t* __restrict__ budget,
    int T, int nc, int kpc, int cap, int nbuild)
{
    __shared__ SecondLds<D> sm;
    if ((int)blockIdx.x < nbuild)
        build_tile<D, IN>(blockIdx.x, sm.lvl, nodes, nodes, T, in_level, tile_rows,
                          tiles_per_pair, levels, l16);
    else
        predict_final_block<D>(blockIdx.x - nbuild, sm.pf, Q, K, W, tot, budget, T, nc, kpc, cap);
}

template <int D>
hipError_t prep_d(const Shape& s, const int8_t* Q, const int8_t* K, const int8_t* W,
                  int32_t* nodes, int32_t* budget, void* ws, hipStream_t st)
{
    int32_t* tot = static_cast<int32_t*>(ws);
    const int npred = s.P * (int)chunks_per_pair(s.T);
    const BuildPass b1 = build_pass_plan(s.T, D, 0);
    const int nb1 = s.P * b1.tiles;
    hipLaunchKernelGGL((k_prep_first<D>), dim3((unsigned)(nb1 + npred)), dim3(kChunk), 0, st, K,
                       nodes, W, tot, s.T, b1.tile, b1.tiles, b1.levels, s.l16, s.n_classes, nb1);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    int level = b1.levels;
    BuildPass b2{1, 0, 0};
    int nb2 = 0;
    if (level < s.L) {
        b2 = build_pass_plan(s.T, D, level);
        nb2 = s.P * b2.tiles;
    }
    const dim3 grid2((unsigned)(nb2 + npred));
    if (nb2 == 0 || level <= s.l16)
        hipLaunchKernelGGL((k_prep_second<D, kInI16>), grid2, dim3(kChunk), 0, st, nodes, level,
                           b2.tile, b2.tiles, b2.levels, s.l16, Q, K, W, (const int32_t*)tot,
                           budget, s.T, s.n_classes, s.keys_per_class, s.max_budget, nb2);
    else
        hipLaunchKernelGGL((k_prep_second<D, kInI32>), grid2, dim3(kChunk), 0, st, nodes, level,
                           b2.tile, b2.tiles, b2.levels, s.l16, Q, K, W, (const int32_t*)tot,
                           budget, s.T, s.n_classes, s.keys_per_class, s.max_budget, nb2);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    level += b2.levels;
    return level < s.L ? launch_build_from(s, K, nodes, level, st) : hipSuccess;
}

}  // namespace

hipError_t launch_prep(const Shape& s, const int8_t* Q, const int8_t* K, const int8_t* W,
                       int32_t* nodes, int32_t* budget, void* ws, hipStream_t st)
{
    switch (s.d) {
        case 16: return prep_d<16>(s, Q, K, W, nodes, budget, ws, st);
        case 32: return prep_d<32>(s, Q, K, W, nodes, budget, ws, st);
        case 64: return prep_d<64>(s, Q, K, W, nodes, budget, ws, st);
        case 128: return prep_d<128>(s, Q, K, W, nodes, budget, ws, st);
        case 256: return prep_d<256>(s, Q, K, W, nodes, budget, ws, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace alhr
