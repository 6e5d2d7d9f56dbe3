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
// In pass 2 the class dots of a chunk are two small matrix products,
// [positions x d] . [d x classes] for the key rows against W_s and for the
// query rows against W_q, on the int8 matrix cores (v_mfma_i32_32x32x32_i8,
// exact int32 accumulation): a wave's 64 positions take 2 tiles x d / 32
// steps per product instead of 32 classes x d / 4 packed dot instructions
// per position.
#pragma once

#include "device.h"

namespace alhr {
namespace predictk {

constexpr int kChunk = 256;        // positions per workgroup (one per thread)
constexpr int kMaxClasses = 32;

__host__ __device__ inline size_t chunks_per_pair(int T) { return (size_t)((T + kChunk - 1) / kChunk); }

typedef int v16i_mfma __attribute__((ext_vector_type(16)));
typedef int v4i_mfma __attribute__((ext_vector_type(4)));

// 16 bytes at byte b of an int8 row, or zero.
__device__ __forceinline__ v4i_mfma chunk16(const int8_t* __restrict__ row, int b, bool ok)
{
    return ok ? *reinterpret_cast<const v4i_mfma*>(row + b) : (v4i_mfma){0, 0, 0, 0};
}

// The class dots of one wave's 64 positions t0 .. t0 + 63 on the int8 matrix
// cores, as 32 x 32 tiles C[i][c] = X[t0 + 32 j + i] . W[c][part]: u[j] for
// the key rows against W_s (bytes D .. 2D of a class row), v[j] for the query
// rows against W_q (bytes 0 .. D), rows t >= T and classes c >= nc giving 0.
// Operands: lane l holds row (l % 32) and class (l % 32), bytes 16 (l / 32)
// .. +15 of each 32-byte step of the row (zero past D); on return element r
// of lane l is C[8 (r / 4) + 4 (l / 32) + r % 4][l % 32].  A step's operands
// are loaded by load() and multiplied by mma(), so that the caller can have
// the loads of the first steps in flight together with its own.  All 64 lanes
// must be active.
template <int D>
struct ClassTiles {
    static constexpr int kSteps = (D + 31) / 32;
    static constexpr int kEarly = kSteps < 2 ? kSteps : 2;   // steps loaded up front
    struct Ops {
        v4i_mfma ws, wq, k0, k1, q0, q1;
    };
    const int8_t* Kr;   // this lane's row of the first tile in the key rows
    const int8_t* Qr;   // the same row in the query rows
    const int8_t* Wr;   // this lane's class row of W
    bool t0ok, t1ok, cok;
    int half;

    __device__ __forceinline__ ClassTiles(const int8_t* __restrict__ Kp,
                                          const int8_t* __restrict__ Qp, int t0, int T,
                                          const int8_t* __restrict__ W, int nc)
    {
        const int lane = lane_id(), col = lane & 31;
        half = lane >> 5;
        t0ok = t0 + col < T;
        t1ok = t0 + 32 + col < T;
        cok = col < nc;
        Kr = Kp + (size_t)(t0 + col) * D;
        Qr = Qp + (size_t)(t0 + col) * D;
        Wr = W + (size_t)col * 2 * D;
    }

    __device__ __forceinline__ void load(Ops& o, int ks) const
    {
        const int b = 32 * ks + 16 * half;
        const bool in = D >= 32 || b < D;
        constexpr size_t R1 = (size_t)32 * D;   // the second tile's rows
        o.ws = chunk16(Wr + D, b, in && cok);
        o.wq = chunk16(Wr, b, in && cok);
        o.k0 = chunk16(Kr, b, in && t0ok);
        o.k1 = chunk16(Kr + R1, b, in && t1ok);
        o.q0 = chunk16(Qr, b, in && t0ok);
        o.q1 = chunk16(Qr + R1, b, in && t1ok);
    }

    static __device__ __forceinline__ void mma(const Ops& o, v16i_mfma (&u)[2],
                                               v16i_mfma (&v)[2])
    {
        u[0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(o.k0, o.ws, u[0], 0, 0, 0);
        u[1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(o.k1, o.ws, u[1], 0, 0, 0);
        v[0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(o.q0, o.wq, v[0], 0, 0, 0);
        v[1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(o.q1, o.wq, v[1], 0, 0, 0);
    }
};

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
    // the thread's kChunk / RG = C4 rows, up to 16 loads in flight at a time
    constexpr int NR = kChunk / RG, NB = NR < 16 ? NR : 16;
    int a0 = 0, a1 = 0, a2 = 0, a3 = 0;
#pragma unroll
    for (int r0 = 0; r0 < NR; r0 += NB) {
        int w[NB];
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const int t = chunk * kChunk + rg + (r0 + i) * RG;
            w[i] = t < T ? kr[(size_t)t * C4 + g] : 0;
        }
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            a0 += sbyte(w[i], 0);
            a1 += sbyte(w[i], 1);
            a2 += sbyte(w[i], 2);
            a3 += sbyte(w[i], 3);
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
    auto& us = sm.us;
    auto& off = sm.off;
    auto& segoff = sm.segoff;
    auto& base = sm.base;
    const int nch = (int)chunks_per_pair(T);
    const int pair = blk / nch, chunk = blk % nch;
    const int t = chunk * kChunk + threadIdx.x;
    const bool live = t < T;
    const int lane = lane_id(), w64 = threadIdx.x - lane;   // the wave's first position
    // class-dot operands of the first steps, in flight with the loads below
    const ClassTiles<D> ct(K + (size_t)pair * T * D, Q + (size_t)pair * T * D,
                           chunk * kChunk + w64, T, W, nc);
    typename ClassTiles<D>::Ops early[ClassTiles<D>::kEarly];
#pragma unroll
    for (int ks = 0; ks < ClassTiles<D>::kEarly; ++ks) ct.load(early[ks], ks);
    {   // offset from earlier chunks: thread (lane-group, class) takes a strided
        // share, eight loads in flight at a time; the first eight (all of
        // them up to 64 chunks) outside any loop, so that they share one wait
        // with the loads above
        constexpr int G = kChunk / kMaxClasses;
        const int c = threadIdx.x % kMaxClasses, grp = threadIdx.x / kMaxClasses;
        const int32_t* const tp = tot + (size_t)pair * nch * kMaxClasses + c;
        int tv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            tv[j] = grp + G * j < chunk ? tp[(size_t)(grp + G * j) * kMaxClasses] : 0;
        int acc = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc += tv[j];
        if (chunk > 8 * G) {   // uniform over the workgroup
            for (int k0 = grp + 8 * G; k0 < chunk; k0 += 8 * G) {
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    tv[j] = k0 + G * j < chunk ? tp[(size_t)(k0 + G * j) * kMaxClasses] : 0;
#pragma unroll
                for (int j = 0; j < 8; ++j) acc += tv[j];
            }
        }
        off[grp][c] = acc;
    }
    // u[t][c] = W_s[c] . K[t] into LDS; v[t][c] = W_q[c] . Q[t] kept for later
    v16i_mfma u[2], v[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) u[j] = v[j] = (v16i_mfma){};
#pragma unroll
    for (int ks = 0; ks < ClassTiles<D>::kEarly; ++ks) ClassTiles<D>::mma(early[ks], u, v);
#pragma unroll
    for (int ks = ClassTiles<D>::kEarly; ks < ClassTiles<D>::kSteps; ++ks) {
        typename ClassTiles<D>::Ops o;
        ct.load(o, ks);
        ClassTiles<D>::mma(o, u, v);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            us[w64 + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)][lane & 31] = u[i][r];
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
    // the query term W_q[c] . Q[t], added in place: each (position, class)
    // of this wave's rows belongs to one lane, and the scan above is done
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            us[w64 + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)][lane & 31] += v[i][r];
    __syncthreads();
    if (!live) return;
    const int seg = threadIdx.x / 32;
    int best = 0, best_z = 0;
    for (int c = 0; c < nc; ++c) {
        const int z = us[threadIdx.x][c] + base[seg][c];
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
