// Budget predictor, device code shared by the predictor launches and the
// fused preparation launch (ALHR README "Inference stage"; caps in "Results and
// Variables"): z_c(t) = W[c][0:d] . Q[t] + W[c][d:2d] . S[t] with the causal
// key sum S[t] = sum_{j<=t} K[j]; budget = min(kpc * (first argmax + 1), cap).
//
// S[t] is never formed.  Because the map is linear, W_s . S[t] is the
// inclusive scan over j <= t of u[j][c] = W_s[c] . K[j], which is exact in
// int32 under the declared bounds.  Two passes per call:
//   1. per chunk of 256 positions, the chunk totals of u (int32 workspace);
//   2. per chunk, the offsets from earlier chunks, an in-LDS scan of u over
//      the chunk, the query term W_q . Q[t] and the argmax.
// The dot products use the packed int8 dot instruction (4 MACs per op); at
// 2 * d MACs per class and query this is far too small to pay for MFMA.
#pragma once

#include "device.h"

namespace alhr {
namespace predictk {

constexpr int kChunk = 256;        // positions per workgroup (one per thread)
constexpr int kMaxClasses = 32;

__host__ __device__ inline size_t chunks_per_pair(int T) { return (size_t)((T + kChunk - 1) / kChunk); }

// u[c] = W_s[c] . k for every class; W staged in LDS as words.
template <int D>
__device__ __forceinline__ void class_dots(const int* __restrict__ kw, const int* __restrict__ wl,
                                           int nc, int col0, int (&u)[kMaxClasses])
{
#pragma unroll
    for (int c = 0; c < kMaxClasses; ++c) {
        int acc = 0;
        if (c < nc) {
            // 16-byte LDS reads (broadcast: every thread reads the same class row)
            const int4* w = reinterpret_cast<const int4*>(wl + c * (D / 2) + col0);
#pragma unroll
            for (int i = 0; i < D / 16; ++i) {
                const int4 v = w[i];
                acc = dot4_i8(kw[4 * i + 0], v.x, acc);
                acc = dot4_i8(kw[4 * i + 1], v.y, acc);
                acc = dot4_i8(kw[4 * i + 2], v.z, acc);
                acc = dot4_i8(kw[4 * i + 3], v.w, acc);
            }
        }
        u[c] = acc;
    }
}

template <int D>
__device__ __forceinline__ void stage_weights(const int8_t* __restrict__ W, int nc, int* wl)
{
    const int* w = reinterpret_cast<const int*>(W);
    for (int i = threadIdx.x; i < nc * (D / 2); i += kChunk) wl[i] = w[i];
}

// Chunk totals: by linearity the sum over the chunk of W_s[c] . K[t] is
// W_s[c] . (sum over the chunk of K[t]), so the chunk's key rows are summed
// per column first (coalesced dword loads, one LDS reduction) and then dotted
// with each class row: D loads per position instead of 32 class dots.  Exact
// in int32 under the declared bounds, like every other order of this sum.
template <int D>
struct ChunksLds {
    int part[kChunk / (D / 4)][D + 1];
    int colsum[D];
};

// Workgroup `blk` (kChunk threads) of the chunk-totals pass.
template <int D>
__device__ __forceinline__ void predict_chunks_block(int blk, ChunksLds<D>& sm,
                                                     const int8_t* __restrict__ K,
                                                     const int8_t* __restrict__ W,
                                                     int32_t* __restrict__ tot, int T, int nc)
{
    constexpr int C4 = D / 4, RG = kChunk / C4;   // dword columns, row groups
    auto& part = sm.part;
    auto& colsum = sm.colsum;
    const int nch = (int)chunks_per_pair(T);
    const int pair = blk / nch, chunk = blk % nch;
    const int g = threadIdx.x % C4, rg = threadIdx.x / C4;
    const int* kr = reinterpret_cast<const int*>(K) + (size_t)pair * T * C4;
    int a0 = 0, a1 = 0, a2 = 0, a3 = 0;
    for (int r = rg; r < kChunk; r += RG) {
        const int t = chunk * kChunk + r;
        if (t < T) {
            const int w = kr[(size_t)t * C4 + g];
            a0 += sbyte(w, 0);
            a1 += sbyte(w, 1);
            a2 += sbyte(w, 2);
            a3 += sbyte(w, 3);
        }
    }
    part[rg][4 * g + 0] = a0;
    part[rg][4 * g + 1] = a1;
    part[rg][4 * g + 2] = a2;
    part[rg][4 * g + 3] = a3;
    __syncthreads();
    for (int j = threadIdx.x; j < D; j += kChunk) {
        int acc = 0;
        for (int k = 0; k < RG; ++k) acc += part[k][j];
        colsum[j] = acc;
    }
    __syncthreads();
    if (threadIdx.x < nc) {
        const int8_t* ws = W + (size_t)threadIdx.x * 2 * D + D;
        int acc = 0;
        for (int j = 0; j < D; ++j) acc += (int)ws[j] * colsum[j];
        tot[((size_t)pair * nch + chunk) * kMaxClasses + threadIdx.x] = acc;
    }
}

template <int D>
struct FinalLds {
    __align__(16) int wl[kMaxClasses * D / 2];
    int us[kChunk][kMaxClasses + 1];
    int off[kChunk / 32][kMaxClasses + 1];
    int segoff[kChunk / 32][kMaxClasses + 1];
    int base[kChunk / 32][kMaxClasses + 1];
};

// Workgroup `blk` (kChunk threads) of the final pass.
template <int D>
__device__ __forceinline__ void predict_final_block(int blk, FinalLds<D>& sm,
                                                    const int8_t* __restrict__ Q,
                                                    const int8_t* __restrict__ K,
                                                    const int8_t* __restrict__ W,
                                                    const int32_t* __restrict__ tot,
                                                    int32_t* __restrict__ budget, int T, int nc,
                                                    int kpc, int cap)
{
    int* const wl = sm.wl;
    auto& us = sm.us;
    auto& off = sm.off;
    auto& segoff = sm.segoff;
    auto& base = sm.base;
    const int nch = (int)chunks_per_pair(T);
    const int pair = blk / nch, chunk = blk % nch;
    stage_weights<D>(W, nc, wl);
    {   // offset from earlier chunks: thread (lane-group, class) takes a strided share
        const int c = threadIdx.x % kMaxClasses, grp = threadIdx.x / kMaxClasses;
        int acc = 0;
        for (int k = grp; k < chunk; k += kChunk / kMaxClasses)
            acc += tot[((size_t)pair * nch + k) * kMaxClasses + c];
        off[grp][c] = acc;
    }
    __syncthreads();
    const int t = chunk * kChunk + threadIdx.x;
    const bool live = t < T;
    int u[kMaxClasses];
    if (live) {
        int kw[D / 4];
        const int* kr = reinterpret_cast<const int*>(K + ((size_t)pair * T + t) * D);
#pragma unroll
        for (int i = 0; i < D / 4; ++i) kw[i] = kr[i];
        class_dots<D>(kw, wl, nc, D / 4, u);
    } else {
#pragma unroll
        for (int c = 0; c < kMaxClasses; ++c) u[c] = 0;
    }
#pragma unroll
    for (int c = 0; c < kMaxClasses; ++c) us[threadIdx.x][c] = u[c];
    __syncthreads();
    {   // inclusive scan within each 32-position segment, per class
        const int c = threadIdx.x % kMaxClasses, seg = threadIdx.x / kMaxClasses;
        int acc = 0;
        for (int j = 0; j < 32; ++j) {
            acc += us[seg * 32 + j][c];
            us[seg * 32 + j][c] = acc;
        }
        segoff[seg][c] = acc;
    }
    __syncthreads();
    {   // per (segment, class): everything before the segment (earlier chunks
        // and earlier segments of this chunk)
        const int c = threadIdx.x % kMaxClasses, seg = threadIdx.x / kMaxClasses;
        int acc = 0;
        for (int g = 0; g < kChunk / kMaxClasses; ++g) acc += off[g][c];
        for (int s2 = 0; s2 < seg; ++s2) acc += segoff[s2][c];
        base[seg][c] = acc;
    }
    __syncthreads();
    if (!live) return;
    const int seg = threadIdx.x / 32;
    int qw[D / 4];
    const int* qr = reinterpret_cast<const int*>(Q + ((size_t)pair * T + t) * D);
#pragma unroll
    for (int i = 0; i < D / 4; ++i) qw[i] = qr[i];
    int best = 0, best_z = 0;
    for (int c = 0; c < nc; ++c) {
        int z = us[threadIdx.x][c] + base[seg][c];
        const int4* w = reinterpret_cast<const int4*>(wl + c * (D / 2));
#pragma unroll
        for (int i = 0; i < D / 16; ++i) {
            const int4 v = w[i];
            z = dot4_i8(qw[4 * i + 0], v.x, z);
            z = dot4_i8(qw[4 * i + 1], v.y, z);
            z = dot4_i8(qw[4 * i + 2], v.z, z);
            z = dot4_i8(qw[4 * i + 3], v.w, z);
        }
        if (c == 0 || z > best_z) {
            best = c;
            best_z = z;
        }
    }
    const int b = kpc * (best + 1);
    budget[(size_t)pair * T + t] = b < cap ? b : cap;
}

}  // namespace predictk
}  // namespace alhr
