// Decode-cache maintenance (openai-hub article "ALHR把注意力变成树搜索",
// section "ALHR是什么": one new token per step; tree of key sums from the
// ALHR README's opening paragraph).
//
// Append at position pos (append.h): the key and value rows are stored, the
// key is added to each of the L ancestor sums and to the running causal key
// sum, one thread per 4 columns of a pair.
#include "append.h"
#include "device.h"
#include "kernels.h"

namespace alhr {
namespace {

constexpr int kThreads = 256;
using appendk::hi16;
using appendk::lo16;

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
    appendk::append_columns<D>(gid / C4, gid % C4, k_new, v_new, K, V, nodes, prefix, T, L, l16,
                               pos);
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
