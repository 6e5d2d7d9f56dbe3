// Tree of key sums (ALHR README, opening paragraph and "Inference stage"):
// the level-synchronous build passes of build_impl.h, one launch per pass.
#include "build_impl.h"
#include "kernels.h"

namespace alhr {
namespace {

using namespace buildk;

template <int D, int IN>
__global__ __launch_bounds__(kBuildThreads) void k_build_pass(const void* __restrict__ in,
                                                              int32_t* __restrict__ nodes, int T,
                                                              int in_level, int tile_rows,
                                                              int tiles_per_pair, int levels,
                                                              int l16)
{
    __shared__ int4 lvl[kTileElems / 2 / 4];
    build_tile<D, IN>(blockIdx.x, lvl, in, nodes, T, in_level, tile_rows, tiles_per_pair, levels,
                      l16);
}

template <int D>
hipError_t build_d(const Shape& s, const int8_t* K, int32_t* nodes, int in_level, hipStream_t st)
{
    while (in_level < s.L) {
        const BuildPass bp = build_pass_plan(s.T, D, in_level);
        const dim3 grid((unsigned)(s.P * bp.tiles));
        if (in_level == 0)
            hipLaunchKernelGGL((k_build_pass<D, kInKeys>), grid, dim3(kBuildThreads), 0, st,
                               (const void*)K, nodes, s.T, in_level, bp.tile, bp.tiles, bp.levels,
                               s.l16);
        else if (in_level <= s.l16)
            hipLaunchKernelGGL((k_build_pass<D, kInI16>), grid, dim3(kBuildThreads), 0, st,
                               (const void*)nodes, nodes, s.T, in_level, bp.tile, bp.tiles,
                               bp.levels, s.l16);
        else
            hipLaunchKernelGGL((k_build_pass<D, kInI32>), grid, dim3(kBuildThreads), 0, st,
                               (const void*)nodes, nodes, s.T, in_level, bp.tile, bp.tiles,
                               bp.levels, s.l16);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        in_level += bp.levels;
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_build_from(const Shape& s, const int8_t* K, int32_t* nodes, int in_level,
                             hipStream_t st)
{
    switch (s.d) {
        case 16: return build_d<16>(s, K, nodes, in_level, st);
        case 32: return build_d<32>(s, K, nodes, in_level, st);
        case 64: return build_d<64>(s, K, nodes, in_level, st);
        case 128: return build_d<128>(s, K, nodes, in_level, st);
        case 256: return build_d<256>(s, K, nodes, in_level, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_build(const Shape& s, const int8_t* K, int32_t* nodes, hipStream_t st)
{
    return launch_build_from(s, K, nodes, 0, st);
}

}  // namespace alhr
