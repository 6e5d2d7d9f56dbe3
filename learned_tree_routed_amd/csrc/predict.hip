// Budget predictor (ALHR README, "Inference stage"; caps in "Results and
// Variables"): the two launches of predict_impl.h.
#include "kernels.h"
#include "predict_impl.h"

namespace alhr {
namespace {

using namespace predictk;

template <int D>
__global__ __launch_bounds__(kChunk) void k_predict_chunks(const int8_t* __restrict__ K,
                                                           const int8_t* __restrict__ W,
                                                           int32_t* __restrict__ tot, int T, int nc)
{
    __shared__ ChunksLds<D> sm;
    predict_chunks_block<D>(blockIdx.x, sm, K, W, tot, T, nc);
}

template <int D>
__global__ __launch_bounds__(kChunk) void k_predict_final(const int8_t* __restrict__ Q,
                                                          const int8_t* __restrict__ K,
                                                          const int8_t* __restrict__ W,
                                                          const int32_t* __restrict__ tot,
                                                          int32_t* __restrict__ budget, int T,
                                                          int nc, int kpc, int cap)
{
    __shared__ FinalLds<D> sm;
    predict_final_block<D>(blockIdx.x, sm, Q, K, W, tot, budget, T, nc, kpc, cap);
}

template <int D>
hipError_t predict_d(const Shape& s, const int8_t* Q, const int8_t* K, const int8_t* W,
                     int32_t* budget, void* ws, hipStream_t st)
{
    const int nch = (int)chunks_per_pair(s.T);
    int32_t* tot = static_cast<int32_t*>(ws);
    const dim3 grid((unsigned)(s.P * nch));
    hipLaunchKernelGGL((k_predict_chunks<D>), grid, dim3(kChunk), 0, st, K, W, tot, s.T,
                       s.n_classes);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_predict_final<D>), grid, dim3(kChunk), 0, st, Q, K, W,
                       (const int32_t*)tot, budget, s.T, s.n_classes, s.keys_per_class,
                       s.max_budget);
    return hipGetLastError();
}

}  // namespace

size_t predict_ws_bytes(const Shape& s)
{
    const size_t b = (size_t)s.P * chunks_per_pair(s.T) * kMaxClasses * sizeof(int32_t);
    return (b + 255) / 256 * 256;
}

hipError_t launch_predict(const Shape& s, const int8_t* Q, const int8_t* K, const int8_t* W,
                          int32_t* budget, void* ws, hipStream_t st)
{
    switch (s.d) {
        case 16: return predict_d<16>(s, Q, K, W, budget, ws, st);
        case 32: return predict_d<32>(s, Q, K, W, budget, ws, st);
        case 64: return predict_d<64>(s, Q, K, W, budget, ws, st);
        case 128: return predict_d<128>(s, Q, K, W, budget, ws, st);
        case 256: return predict_d<256>(s, Q, K, W, budget, ws, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace alhr
