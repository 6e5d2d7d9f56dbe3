// Dense causal softmax attention on the same int8 Q/K and fp32 V: the dense
// baseline the ALHR README's result tables compare against ("Dense
// Baseline(Teacher)" rows), and the optimised dense kernel the openai-hub
// article asks the comparison to use (section "接下来最该验证的不是更高压缩比").
// O[t] = sum_{j <= t} softmax_j(scale * Q[t] . K[j]) V[j].
//
// One wave per block of 32 queries, streaming 32-key blocks up to the
// diagonal with an online (running max) softmax.  Both products run on the
// matrix cores:
//  * S^T = K_blk . Q_blk^T with v_mfma_i32_32x32x16_i8 (exact int32 scores);
//    computing the transpose puts one query in each lane column, so the
//    per-query max and sum need one cross-half exchange per block;
//  * O^T += V_blk^T . P^T with v_mfma_f32_32x32x2_f32: the probabilities stay
//    fp32 (tolerance 1e-4 against an fp64 reference), and the B operand of
//    step r is the lane's own accumulator element r, so P never moves.
// MFMA 32x32 layouts (checked on gfx950): A lane l holds row l%32 (int8: k =
// 8*(l/32)..+7; f32: k = l/32), B lane l holds column l%32 with the same k,
// and C element r of lane l is row 8*(r/4) + 4*(l/32) + r%4, column l%32.
#include "device.h"
#include "kernels.h"

namespace alhr {
namespace {

typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kBlk = 32;
constexpr int kDenseWaves = 4;

__device__ __forceinline__ int key_row_of(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

template <int D>
__global__ __launch_bounds__(kDenseWaves * kWave) void k_dense(
    const int8_t* __restrict__ Q, const int8_t* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, int P, int T, float scale)
{
    constexpr int NT = D / 32;    // 32-wide output tiles along d
    constexpr int NK = D / 16;    // int8 MFMA steps along d
    const int lane = lane_id();
    const int nqb = (T + kBlk - 1) / kBlk;
    const int w = uniform((int)(xcd_logical_block() * kDenseWaves + threadIdx.x / kWave));
    if (w >= P * nqb) return;
    const int pair = w / nqb;
    const int qb = nqb - 1 - w % nqb;        // long (late) query blocks first
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
    float m = -INFINITY, lsum = 0.0f;

    for (int kb = 0; kb <= qb; ++kb) {
        const int k0 = kb * kBlk;
        const int krow = k0 + col < T ? k0 + col : T - 1;
        v16i s = (v16i){};
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
            const int64_t ka =
                *reinterpret_cast<const int64_t*>(Kp + (size_t)krow * D + 16 * kk + 8 * half);
            s = __builtin_amdgcn_mfma_i32_32x32x16_i8(ka, qb_op[kk], s, 0, 0, 0);
        }
        float p[16];
        float mb = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = k0 + key_row_of(r, lane);
            const bool ok = key <= qrow && key < T;
            p[r] = ok ? (float)s[r] * scale : -INFINITY;
            mb = p[r] > mb ? p[r] : mb;
        }
        const float mo = __shfl_xor(mb, 32);
        mb = mo > mb ? mo : mb;
        const float mn = m > mb ? m : mb;      // finite: key k0 <= every query of the block
        const float corr = __expf(m - mn);
        float ps = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            p[r] = __expf(p[r] - mn);
            ps += p[r];
        }
        lsum = lsum * corr + ps;
        m = mn;
#pragma unroll
        for (int i = 0; i < NT; ++i) acc[i] *= corr;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = k0 + key_row_of(r, lane);
            const int vrow = key < T ? key : T - 1;
            const float* vr = Vp + (size_t)vrow * D + col;
#pragma unroll
            for (int i = 0; i < NT; ++i)
                acc[i] = __builtin_amdgcn_mfma_f32_32x32x2f32(vr[32 * i], p[r], acc[i], 0, 0, 0);
        }
    }
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
    const uint64_t waves = (uint64_t)s.P * ((s.T + kBlk - 1) / kBlk);
    uint64_t blocks = (waves + kDenseWaves - 1) / kDenseWaves;
    blocks = (blocks + kXcds - 1) / kXcds * kXcds;
    const dim3 grid((unsigned)blocks), block(kDenseWaves * kWave);
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
