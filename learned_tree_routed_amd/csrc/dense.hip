// Dense causal softmax attention on the same int8 Q/K and fp32 V: the dense
// baseline the ALHR README's result tables compare against ("Dense
// Baseline(Teacher)" rows), and the optimised dense kernel the openai-hub
// article asks the comparison to use (section "接下来最该验证的不是更高压缩比").
// O[t] = sum_{j <= t} softmax_j(scale * Q[t] . K[j]) V[j].
//
// A workgroup of 4 waves takes 4 consecutive blocks of 32 queries of one
// pair and streams 32-key blocks up to the last block's diagonal with an
// online (running max) softmax.  Each key block is staged once in LDS for the
// 4 waves (K rows as they are, V transposed to d-major rows), double
// buffered: the global loads of the next block are issued before the current
// block's products.  Both products run on the matrix cores:
//  * S^T = K_blk . Q_blk^T with v_mfma_i32_32x32x16_i8 (exact int32 scores);
//    computing the transpose puts one query in each lane column, so the
//    per-query max and sum need one cross-half exchange per block;
//  * O^T += V_blk^T . P^T with v_mfma_f32_32x32x16_bf16 in three products:
//    P and V are each split into a bf16 head and a bf16 tail (x = hi + lo up
//    to 2^-18 |x|), and hi.hi + lo.hi + hi.lo is accumulated in fp32; the
//    dropped lo.lo term and the split residuals leave |p v| 3 * 2^-18 short at
//    most, so each output is within 1.2e-5 * max |v| of the fp32 result
//    (tolerance 1e-4).  The B operand is the lane's own probabilities: the 8
//    k-slots of step s are its accumulator elements 8s .. 8s + 7, keys
//    16s + 8g + 4 half + b for slot 4g + b, and V is staged with each d row's
//    keys permuted to that order, so the A operand is one 16-byte read.
// MFMA 32x32 layouts (checked on gfx950): A lane l holds row l%32 (int8 and
// bf16: k = 8*(l/32)..+7), B lane l holds column l%32 with the same k, and C
// element r of lane l is row 8*(r/4) + 4*(l/32) + r%4, column l%32.
#include <climits>

#include "device.h"
#include "kernels.h"

namespace alhr {
namespace {

typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 bf8 __attribute__((ext_vector_type(8)));

constexpr int kBlk = 32;
constexpr int kDenseWaves = 4;
constexpr int kThreads = kDenseWaves * kWave;

__device__ __forceinline__ int key_row_of(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// One staged key block: K rows (D bytes, padded to keep 16-byte rows
// aligned) and V transposed to d-major rows of bf16 heads and tails,
// vh[c][pos(j)] + vl[c][pos(j)] = V[k0 + j][c], where pos swaps bits 2 and 3
// of the key index (the k-slot order of the bf16 products); rows are padded
// to 40 entries so that 8 lanes' 16-byte reads hit distinct banks.
template <int D>
struct DenseTile {
    static constexpr int kKs = D + 16;
    static constexpr int kVs = 40;
    int8_t k[kBlk][kKs];
    uint32_t vh[D][kVs / 2];   // packed bf16 pairs
    uint32_t vl[D][kVs / 2];
};

__device__ __forceinline__ int vt_pos(int j) { return (j & ~12) | ((j & 4) << 1) | ((j & 8) >> 1); }

// The global loads of one key block, one or more 16-byte chunks per thread:
// K: 2D chunks (row j = chunk / (D/16), chunk column c = chunk % (D/16)),
// V: 4D pairs of chunks (rows 2q and 2q + 1, q = pair % 16, float4 column
// c = pair / 16), so a thread writes whole packed bf16 pairs.
template <int D>
struct DenseStage {
    static constexpr int kKc = (2 * D + kThreads - 1) / kThreads;
    static constexpr int kVc = (4 * D + kThreads - 1) / kThreads;
    int4 k[kKc];
    float4 v0[kVc], v1[kVc];
};

template <int D>
__device__ __forceinline__ void dense_load(DenseStage<D>& st, const int8_t* __restrict__ Kp,
                                           const float* __restrict__ Vp, int k0, int T)
{
    const int t = threadIdx.x;
#pragma unroll
    for (int u = 0; u < DenseStage<D>::kKc; ++u) {
        const int ch = t + kThreads * u;
        if (ch < 2 * D) {
            const int j = ch / (D / 16), c = ch % (D / 16);
            const int row = k0 + j < T ? k0 + j : T - 1;   // rows past T: finite stand-ins
            st.k[u] = reinterpret_cast<const int4*>(Kp + (size_t)row * D)[c];
        }
    }
#pragma unroll
    for (int u = 0; u < DenseStage<D>::kVc; ++u) {
        const int ch = t + kThreads * u;
        if (ch < 4 * D) {
            const int q = ch % (kBlk / 2), c = ch / (kBlk / 2);
            const int r0 = k0 + 2 * q < T ? k0 + 2 * q : T - 1;   // rows past T: finite stand-ins
            const int r1 = k0 + 2 * q + 1 < T ? k0 + 2 * q + 1 : T - 1;
            st.v0[u] = reinterpret_cast<const float4*>(Vp + (size_t)r0 * D)[c];
            st.v1[u] = reinterpret_cast<const float4*>(Vp + (size_t)r1 * D)[c];
        }
    }
}

// bf16 head and tail of x and y, each pair packed (x in the low half)
__device__ __forceinline__ void split_pair(float x, float y, uint32_t& hi, uint32_t& lo)
{
    const __bf16 hx = (__bf16)x, hy = (__bf16)y;   // round to nearest even
    const __bf16 lx = (__bf16)(x - (float)hx), ly = (__bf16)(y - (float)hy);
    hi = (uint32_t)__builtin_bit_cast(uint16_t, hx) | ((uint32_t)__builtin_bit_cast(uint16_t, hy) << 16);
    lo = (uint32_t)__builtin_bit_cast(uint16_t, lx) | ((uint32_t)__builtin_bit_cast(uint16_t, ly) << 16);
}

template <int D>
__device__ __forceinline__ void dense_store(const DenseStage<D>& st, DenseTile<D>& tile)
{
    const int t = threadIdx.x;
#pragma unroll
    for (int u = 0; u < DenseStage<D>::kKc; ++u) {
        const int ch = t + kThreads * u;
        if (ch < 2 * D) {
            const int j = ch / (D / 16), c = ch % (D / 16);
            *reinterpret_cast<int4*>(&tile.k[j][16 * c]) = st.k[u];
        }
    }
#pragma unroll
    for (int u = 0; u < DenseStage<D>::kVc; ++u) {
        const int ch = t + kThreads * u;
        if (ch < 4 * D) {
            const int q = ch % (kBlk / 2), c = ch / (kBlk / 2);
            const int w = vt_pos(2 * q) >> 1;   // keys 2q, 2q + 1 stay adjacent
            const float a[4] = {st.v0[u].x, st.v0[u].y, st.v0[u].z, st.v0[u].w};
            const float b[4] = {st.v1[u].x, st.v1[u].y, st.v1[u].z, st.v1[u].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                uint32_t hi, lo;
                split_pair(a[e], b[e], hi, lo);
                tile.vh[4 * c + e][w] = hi;
                tile.vl[4 * c + e][w] = lo;
            }
        }
    }
}

// The running-maximum slack: the maximum a query's probabilities are taken
// against moves only when a block's maximum exceeds it by more than this
// (natural-log units), so exp() of a logit never exceeds e^8 and the
// accumulators are rescaled a few times per query instead of on most blocks.
// Every choice of the reference maximum gives the same softmax.
constexpr float kMaxSlack = 8.0f;

// 2^x by the hardware instruction alone (v_exp_f32, about 1 ulp): every
// argument here is at most the slack above (the probabilities) or at most 0
// (the rescaling factor, -inf on the first block giving 0), so the range
// handling a general exp2f wraps around it is not needed; results below the
// normal range are weights too small to move a sum that includes 1.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// One key block's product for the wave: S^T on the int8 matrix cores, the
// online softmax update and O^T += V^T P^T.  MASK: the block holds keys past
// a query of the wave (its diagonal) or past T.
template <int D, bool MASK>
__device__ __forceinline__ void dense_block(const DenseTile<D>& tl, int k0, int qrow, int T,
                                            float c1, const int64_t (&qb_op)[D / 16],
                                            v16f (&acc)[D / 32], float& m, float& lsum)
{
    constexpr int NT = D / 32, NK = D / 16;
    const int lane = lane_id(), col = lane & 31, half = lane >> 5;
    v16i sc = (v16i){};
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
        const int64_t ka = *reinterpret_cast<const int64_t*>(&tl.k[col][16 * kk + 8 * half]);
        sc = __builtin_amdgcn_mfma_i32_32x32x16_i8(ka, qb_op[kk], sc, 0, 0, 0);
    }
    bool ok[16];
    int smax = INT_MIN;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int key = k0 + key_row_of(r, lane);
        ok[r] = !MASK || (key <= qrow && key < T);
        const int v = ok[r] ? sc[r] : INT_MIN;
        smax = v > smax ? v : smax;
    }
    const int so = __shfl_xor(smax, 32);
    smax = so > smax ? so : smax;   // a real score: key k0 <= every query of the block
    // logits scale * s in log2 units: c1 = scale * log2(e)
    const float mb = (float)smax * c1;
    const float mn = mb > m + kMaxSlack * 1.44269504f ? mb : m;
    if (__ballot(mn != m) != 0ull) {
        const float corr = exp2_hw(m - mn);   // 1 where unchanged, 0 on the first block
        lsum *= corr;
#pragma unroll
        for (int i = 0; i < NT; ++i) acc[i] *= corr;
        m = mn;
    }
    float p[16];
    float ps = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        p[r] = exp2_hw(__builtin_fmaf((float)sc[r], c1, -m));
        if (MASK) p[r] = ok[r] ? p[r] : 0.0f;
        ps += p[r];
    }
    lsum += ps;
    // B operands: step s takes the lane's p[8s .. 8s + 7] (keys 16s + 8g +
    // 4 half + b for k-slot 4g + b) as bf16 heads and tails
    uint32_t ph[8], pl[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) split_pair(p[2 * r], p[2 * r + 1], ph[r], pl[r]);
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
        const bf8 bh = __builtin_bit_cast(bf8, make_uint4(ph[4 * s2], ph[4 * s2 + 1], ph[4 * s2 + 2], ph[4 * s2 + 3]));
        const bf8 bl = __builtin_bit_cast(bf8, make_uint4(pl[4 * s2], pl[4 * s2 + 1], pl[4 * s2 + 2], pl[4 * s2 + 3]));
#pragma unroll
        for (int i = 0; i < NT; ++i) {
            // keys 16 s2 + 8 half .. + 7 of the permuted row: one 16-byte read each
            const bf8 ah = __builtin_bit_cast(bf8, *reinterpret_cast<const uint4*>(&tl.vh[32 * i + col][8 * s2 + 4 * half]));
            const bf8 al = __builtin_bit_cast(bf8, *reinterpret_cast<const uint4*>(&tl.vl[32 * i + col][8 * s2 + 4 * half]));
            acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bh, acc[i], 0, 0, 0);
            acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bh, acc[i], 0, 0, 0);
            acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bl, acc[i], 0, 0, 0);
        }
    }
}

template <int D>
__global__ __launch_bounds__(kThreads) void k_dense(const int8_t* __restrict__ Q,
                                                    const int8_t* __restrict__ K,
                                                    const float* __restrict__ V,
                                                    float* __restrict__ O, int P, int T,
                                                    float scale)
{
    constexpr int NT = D / 32;    // 32-wide output tiles along d
    constexpr int NK = D / 16;    // int8 MFMA steps along d
    __shared__ DenseTile<D> tiles[2];
    const int lane = lane_id(), wv = threadIdx.x / kWave;
    const int nqb = (T + kBlk - 1) / kBlk;
    const int ngr = (nqb + kDenseWaves - 1) / kDenseWaves;
    const int w = (int)xcd_logical_block();
    if (w >= P * ngr) return;                      // uniform over the workgroup
    const int pair = w / ngr;
    const int gr = ngr - 1 - w % ngr;              // long (late) query groups first
    const int qb = gr * kDenseWaves + wv;          // this wave's query block (may be >= nqb)
    const int kb_end = min(gr * kDenseWaves + kDenseWaves - 1, nqb - 1);   // uniform
    const int q0 = qb * kBlk;
    const int8_t* Qp = Q + (size_t)pair * T * D;
    const int8_t* Kp = K + (size_t)pair * T * D;
    const float* Vp = V + (size_t)pair * T * D;
    const int col = lane & 31, half = lane >> 5;
    const int qrow = q0 + col;
    const int qload = qrow < T ? qrow : T - 1;

    int64_t qb_op[NK];                         // B operand: Q^T, this lane's query column
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
        qb_op[kk] = *reinterpret_cast<const int64_t*>(Qp + (size_t)qload * D + 16 * kk + 8 * half);

    v16f acc[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) acc[i] = (v16f){};
    float m = -INFINITY, lsum = 0.0f;   // m: reference maximum in log2 units
    const float c1 = scale * 1.44269504f;

    DenseStage<D> st;
    dense_load<D>(st, Kp, Vp, 0, T);
    dense_store<D>(st, tiles[0]);
    __syncthreads();
    // this wave's key blocks are 0 .. qb (its diagonal); the workgroup's go on
    // to kb_end, and every wave takes part in staging all of them
    const int kb_mine = qb < nqb ? qb : -1;
    int kb = 0;
    for (; kb <= kb_mine; ++kb) {
        const bool more = kb < kb_end;
        if (more) dense_load<D>(st, Kp, Vp, (kb + 1) * kBlk, T);
        const int k0 = kb * kBlk;
        if (kb == qb || k0 + kBlk > T)
            dense_block<D, true>(tiles[kb & 1], k0, qrow, T, c1, qb_op, acc, m, lsum);
        else
            dense_block<D, false>(tiles[kb & 1], k0, qrow, T, c1, qb_op, acc, m, lsum);
        if (more) dense_store<D>(st, tiles[(kb + 1) & 1]);
        __syncthreads();
    }
    for (; kb <= kb_end; ++kb) {
        if (kb < kb_end) {
            dense_load<D>(st, Kp, Vp, (kb + 1) * kBlk, T);
            dense_store<D>(st, tiles[(kb + 1) & 1]);
        }
        __syncthreads();
    }
    if (qb >= nqb) return;
    const float ltot = lsum + __shfl_xor(lsum, 32);
    const float inv = 1.0f / ltot;
    if (qrow < T) {
        float* orow = O + ((size_t)pair * T + qrow) * D;
#pragma unroll
        for (int i = 0; i < NT; ++i)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d0 = 32 * i + 8 * g + 4 * half;
                *reinterpret_cast<float4*>(orow + d0) =
                    make_float4(acc[i][4 * g] * inv, acc[i][4 * g + 1] * inv,
                                acc[i][4 * g + 2] * inv, acc[i][4 * g + 3] * inv);
            }
    }
}

}  // namespace

hipError_t launch_dense(const Shape& s, const int8_t* Q, const int8_t* K, const float* V, float* O,
                        hipStream_t st)
{
    // one workgroup per group of kDenseWaves query blocks of a pair
    const uint64_t groups = (uint64_t)s.P * (((s.T + kBlk - 1) / kBlk + kDenseWaves - 1) / kDenseWaves);
    const uint64_t blocks = (groups + kXcds - 1) / kXcds * kXcds;
    const dim3 grid((unsigned)blocks), block(kThreads);
    switch (s.d) {
        case 32: hipLaunchKernelGGL((k_dense<32>), grid, block, 0, st, Q, K, V, O, s.P, s.T, s.scale); break;
        case 64: hipLaunchKernelGGL((k_dense<64>), grid, block, 0, st, Q, K, V, O, s.P, s.T, s.scale); break;
        case 128: hipLaunchKernelGGL((k_dense<128>), grid, block, 0, st, Q, K, V, O, s.P, s.T, s.scale); break;
        case 256: hipLaunchKernelGGL((k_dense<256>), grid, block, 0, st, Q, K, V, O, s.P, s.T, s.scale); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace alhr
