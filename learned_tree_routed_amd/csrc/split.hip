// Query/key splitter (ALHR README, "Inference stage": the layer input is
// split into queries and keys before the tree is built; "Training stage":
// the splitter is one of the two trained functions).  Per token, two
// bias-free linear maps of the int8 input row with exact int32 accumulation,
// requantised to int8 by a round-half-up right shift and a symmetric clamp.
//
// As a matrix product: C = X . W^T with X int8 [M = batch * T, d_model] and
// W int8 [N = 2 * heads * d, d_model] (row o = output feature o), on
// v_mfma_i32_32x32x32_i8.  A workgroup of 8 waves owns a 128 x 256 tile of C
// (each wave 64 x 64 = 2 x 2 MFMA tiles), so a block of X rows is read by
// half as many workgroups as with square tiles.  K is staged through two LDS
// buffers 64 bytes at a time with 16-byte coalesced loads: the next stage's
// global loads are in flight in registers while the current stage's MFMAs
// run, so each stage costs one barrier and no exposed load latency.  The
// epilogue requantises in registers, transposes the int8 tile through LDS
// and writes 16-byte chunks straight into the [batch, heads, T, d] layout of
// Q and K (a chunk is 16 consecutive features of one head, since d >= 16).
#include "device.h"
#include "kernels.h"

namespace alhr {
namespace {

typedef int v16i __attribute__((ext_vector_type(16)));
typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kSplitThreads = 512;
constexpr int kBM = 128, kBN = 256, kBK = 64;
constexpr int kInRow = kBK + 16;     // padded LDS row of a staged operand (bytes)
constexpr int kOutRow = kBN + 16;    // padded LDS row of the int8 output tile

struct SplitStage {
    int8_t x[kBM * kInRow];
    int8_t w[kBN * kInRow];
};

struct SplitLds {
    union {
        SplitStage in[2];
        int8_t out[kBM * kOutRow];
    };
};

// This thread's 16-byte chunks of X (one) and of W (two) for the stage at
// k0 (rows r = c / 4 for c = tid (+ 512 for W); chunk c % 4), zero outside.
struct StageRegs {
    int4 x[1], w[2];
};

__device__ __forceinline__ void load_stage(StageRegs& g, const int8_t* __restrict__ X,
                                           const int8_t* __restrict__ W, int m0, int n0, int k0,
                                           int M, int N, int dm, int tid)
{
    {
        const int r = tid >> 2, kk = k0 + 16 * (tid & 3);
        g.x[0] = make_int4(0, 0, 0, 0);
        if (m0 + r < M && kk < dm) g.x[0] = *reinterpret_cast<const int4*>(X + (size_t)(m0 + r) * dm + kk);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int c = tid + i * kSplitThreads;
        const int r = c >> 2, kk = k0 + 16 * (c & 3);
        g.w[i] = make_int4(0, 0, 0, 0);
        if (n0 + r < N && kk < dm) g.w[i] = *reinterpret_cast<const int4*>(W + (size_t)(n0 + r) * dm + kk);
    }
}

__device__ __forceinline__ void store_stage(SplitStage& st, const StageRegs& g, int tid)
{
    *reinterpret_cast<int4*>(st.x + (tid >> 2) * kInRow + 16 * (tid & 3)) = g.x[0];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int c = tid + i * kSplitThreads;
        *reinterpret_cast<int4*>(st.w + (c >> 2) * kInRow + 16 * (c & 3)) = g.w[i];
    }
}

__global__ __launch_bounds__(kSplitThreads) __attribute__((amdgpu_waves_per_eu(4))) void k_split(
    const int8_t* __restrict__ X, const int8_t* __restrict__ W, int8_t* __restrict__ Q,
    int8_t* __restrict__ K, int M, int N, int dm, int T, int H, int d, int shift, int qclamp,
    int kclamp)
{
    __shared__ __align__(16) SplitLds sm;
    const int tid = threadIdx.x, lane = lane_id(), wv = tid / kWave;
    const int nbn = (N + kBN - 1) / kBN, nbm = (M + kBM - 1) / kBM;
    // logical tiles in XCD-major order: the nbn tiles that share one X row
    // block run on one XCD and read it through one L2
    const int lb = (int)xcd_logical_block();
    if (lb >= nbm * nbn) return;   // grid padding, uniform over the workgroup
    const int bm = lb / nbn, bn = lb % nbn;
    const int m0 = bm * kBM, n0 = bn * kBN;
    const int wm = (wv >> 2) * 64, wn = (wv & 3) * 64;        // this wave's 64 x 64 sub-tile
    const int col = lane & 31, half = lane >> 5;
    const int stages = (dm + kBK - 1) / kBK;

    v16i acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = (v16i){};

    StageRegs g;
    load_stage(g, X, W, m0, n0, 0, M, N, dm, tid);
    store_stage(sm.in[0], g, tid);
    __syncthreads();
    for (int s = 0; s < stages; ++s) {
        const bool more = s + 1 < stages;
        if (more) load_stage(g, X, W, m0, n0, (s + 1) * kBK, M, N, dm, tid);
        const SplitStage& st = sm.in[s & 1];
#pragma unroll
        for (int ks = 0; ks < kBK / 32; ++ks) {
            // A operand: token row (l % 32), bytes 16 * (l / 32) .. +15 of this
            // 32-byte k step; B operand: feature column (l % 32), same bytes
            v4i a[2], b[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                a[i] = *reinterpret_cast<const v4i*>(st.x + (wm + 32 * i + col) * kInRow + 32 * ks + 16 * half);
                b[i] = *reinterpret_cast<const v4i*>(st.w + (wn + 32 * i + col) * kInRow + 32 * ks + 16 * half);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        if (more) store_stage(sm.in[(s + 1) & 1], g, tid);
        __syncthreads();
    }

    // requantise: element r of a lane is C[8 (r / 4) + 4 (l / 32) + r % 4][l % 32]
    const int HD = H * d;
    const int half_step = shift >= 1 ? 1 << (shift - 1) : 0;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int o = n0 + wn + 32 * j + col;
        const int c = o >= HD ? kclamp : qclamp;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                int v = (acc[i][j][r] + half_step) >> shift;   // arithmetic: floor
                v = v > c ? c : (v < -c ? -c : v);
                const int row = wm + 32 * i + 8 * (r >> 2) + 4 * half + (r & 3);
                sm.out[row * kOutRow + wn + 32 * j + col] = (int8_t)v;
            }
    }
    __syncthreads();

    // 16-byte chunks: row = token, 16 consecutive features of one head
#pragma unroll
    for (int i = 0; i < kBM * kBN / 16 / kSplitThreads; ++i) {
        const int c = tid + i * kSplitThreads;
        const int row = c / (kBN / 16), cc = c % (kBN / 16);
        const int m = m0 + row, o = n0 + 16 * cc;
        if (m >= M || o >= N) continue;
        const bool is_key = o >= HD;
        const int f = is_key ? o - HD : o;
        const int h = f / d, jj = f % d;
        const int b = m / T, t = m % T;
        int8_t* dst = (is_key ? K : Q) + (((size_t)b * H + h) * T + t) * d + jj;
        *reinterpret_cast<int4*>(dst) = *reinterpret_cast<const int4*>(sm.out + row * kOutRow + 16 * cc);
    }
}

}  // namespace

hipError_t launch_split(const SplitShape& s, const int8_t* X, const int8_t* W, int8_t* Q,
                        int8_t* K, hipStream_t st)
{
    const int M = s.batch * s.T, N = 2 * s.heads * s.d;
    const unsigned tiles = (unsigned)(((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN));
    const unsigned blocks = (tiles + kXcds - 1) / kXcds * kXcds;   // a multiple of the XCD count
    hipLaunchKernelGGL(k_split, dim3(blocks), dim3(kSplitThreads), 0, st, X, W, Q, K, M, N,
                       s.d_model, s.T, s.heads, s.d, s.shift, s.qclamp, s.kclamp);
    return hipGetLastError();
}

}  // namespace alhr
