// Device-side twin of the host input generator in synth/__init__.py: the
// same SplitMix64 counters (Steele, Lea & Flood, OOPSLA 2014), the same
// packing of (seed, stream, b, h, t, i) and the same integer maps, so every
// element equals its host value bit for bit.  This library holds no step of
// the ALHR method; it only fills caller-owned device arrays with seeded
// synthetic inputs, which is needed where they are too large to copy from
// the host (a 2^17-position cache of 64 x 16 heads).
//
// Output rows of one (b, h) pair are written at
//   out[((b * H + h) * row_stride + (t - t0)) * d + i],  t0 <= t < t0 + nt.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;
enum : uint64_t { kCentre = 0, kCluster = 1, kKnoise = 2, kSrc = 3, kQnoise = 4, kVal = 5, kW = 6 };

__device__ __forceinline__ uint64_t mix64(uint64_t x)
{
    uint64_t z = x + 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

__device__ __forceinline__ uint64_t pack(uint64_t seed, uint64_t stream, uint64_t b, uint64_t h,
                                         uint64_t t, uint64_t i)
{
    return (seed << 56) | (stream << 52) | (b << 44) | (h << 36) | (t << 16) | i;
}

__device__ __forceinline__ int64_t uniform(uint64_t x, int64_t lo, int64_t hi)
{
    return lo + (int64_t)(((x >> 32) * (uint64_t)(hi - lo + 1)) >> 32);
}

__device__ __forceinline__ int key_elem(uint64_t seed, uint64_t b, uint64_t h, uint64_t t, uint64_t i)
{
    const int64_t cl = uniform(mix64(pack(seed, kCluster, b, h, t, 0)), 0, 63);
    const int64_t centre = uniform(mix64(pack(seed, kCentre, b, h, (uint64_t)cl, i)), -6, 6);
    const int64_t noise = uniform(mix64(pack(seed, kKnoise, b, h, t, i)), -2, 2);
    return (int)(centre + noise);
}

struct Grid {
    int B, H, d, t0, nt;
    int64_t row_stride;
    __device__ void coords(uint64_t e, uint64_t& b, uint64_t& h, uint64_t& t, uint64_t& i,
                           uint64_t& dst) const
    {
        i = e % (uint64_t)d;
        uint64_t r = e / (uint64_t)d;
        const uint64_t tt = r % (uint64_t)nt;
        r /= (uint64_t)nt;
        h = r % (uint64_t)H;
        b = r / (uint64_t)H;
        t = (uint64_t)t0 + tt;
        dst = ((b * (uint64_t)H + h) * (uint64_t)row_stride + tt) * (uint64_t)d + i;
    }
    __host__ __device__ uint64_t total() const { return (uint64_t)B * H * nt * d; }
};

__global__ __launch_bounds__(kThreads) void k_keys(uint64_t seed, Grid g, int8_t* out)
{
    const uint64_t n = g.total();
    for (uint64_t e = (uint64_t)blockIdx.x * kThreads + threadIdx.x; e < n;
         e += (uint64_t)gridDim.x * kThreads) {
        uint64_t b, h, t, i, dst;
        g.coords(e, b, h, t, i, dst);
        out[dst] = (int8_t)key_elem(seed, b, h, t, i);
    }
}

__global__ __launch_bounds__(kThreads) void k_queries(uint64_t seed, Grid g, int8_t* out)
{
    const uint64_t n = g.total();
    for (uint64_t e = (uint64_t)blockIdx.x * kThreads + threadIdx.x; e < n;
         e += (uint64_t)gridDim.x * kThreads) {
        uint64_t b, h, t, i, dst;
        g.coords(e, b, h, t, i, dst);
        const uint64_t x = mix64(pack(seed, kSrc, b, h, t, 0));
        const uint64_t src = ((x >> 32) * t) >> 32;   // uniform in [0, t-1]; 0 at t = 0
        const int k = key_elem(seed, b, h, src, i);
        const int64_t noise = uniform(mix64(pack(seed, kQnoise, b, h, t, i)), -1, 1);
        out[dst] = (int8_t)(k + noise);
    }
}

__global__ __launch_bounds__(kThreads) void k_values(uint64_t seed, Grid g, float* out)
{
    const uint64_t n = g.total();
    for (uint64_t e = (uint64_t)blockIdx.x * kThreads + threadIdx.x; e < n;
         e += (uint64_t)gridDim.x * kThreads) {
        uint64_t b, h, t, i, dst;
        g.coords(e, b, h, t, i, dst);
        int64_t acc = 0;
        for (uint64_t k = 0; k < 3; ++k) {
            const uint64_t x = mix64(pack(seed, kVal, b, h, t, 4 * i + k));
            for (int m = 0; m < 4; ++m) acc += (int64_t)((x >> (16 * m)) & 0xFFFFu);
        }
        out[dst] = (float)(2 * acc - 12 * 65535) * (1.0f / 131072.0f);
    }
}

__global__ __launch_bounds__(kThreads) void k_uniform(uint64_t seed, uint64_t stream, int lo,
                                                      int hi, Grid g, int8_t* out)
{
    const uint64_t n = g.total();
    for (uint64_t e = (uint64_t)blockIdx.x * kThreads + threadIdx.x; e < n;
         e += (uint64_t)gridDim.x * kThreads) {
        uint64_t b, h, t, i, dst;
        g.coords(e, b, h, t, i, dst);
        out[dst] = (int8_t)uniform(mix64(pack(seed, stream, b, h, t, i)), lo, hi);
    }
}

__global__ __launch_bounds__(kThreads) void k_weights(uint64_t seed, int nc, int d, int8_t* out)
{
    const int e = blockIdx.x * kThreads + threadIdx.x;
    if (e >= nc * 2 * d) return;
    const int c = e / (2 * d), i = e % (2 * d);
    out[e] = (int8_t)uniform(mix64(pack(seed, kW, 0, 0, (uint64_t)c, (uint64_t)i)), -4, 4);
}

bool grid_ok(int seed, int B, int H, int d, int t0, int nt, int64_t row_stride)
{
    return seed >= 0 && seed < 256 && B > 0 && B <= 256 && H > 0 && H <= 256 && d > 0 &&
           d <= 256 && t0 >= 0 && nt >= 0 && (int64_t)t0 + nt <= (1 << 20) && row_stride >= nt;
}

unsigned blocks(uint64_t n)
{
    const uint64_t b = (n + kThreads - 1) / kThreads;
    return (unsigned)(b < 65536 * 4 ? (b ? b : 1) : 65536 * 4);
}

}  // namespace

extern "C" {

// Each call returns 0 on success, -1 on a bad argument (nothing launched) and
// -3 on a launch failure.  Generation runs asynchronously on `stream`.

#define SYNTH_GRID_CHECK()                                                     \
    if (!grid_ok(seed, B, H, d, t0, nt, row_stride) || !out) return -1;        \
    const Grid g{B, H, d, t0, nt, row_stride};                                 \
    if (g.total() == 0) return 0

// Clustered keys in [-8, 8]: centre[cluster(t)] + noise.
int alhr_synth_keys(int seed, int B, int H, int d, int t0, int nt, int64_t row_stride,
                    int8_t* out, void* stream)
{
    SYNTH_GRID_CHECK();
    hipLaunchKernelGGL(k_keys, dim3(blocks(g.total())), dim3(kThreads), 0, (hipStream_t)stream,
                       (uint64_t)seed, g, out);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

// Queries in [-9, 9]: a noisy copy of the key at a random earlier position.
int alhr_synth_queries(int seed, int B, int H, int d, int t0, int nt, int64_t row_stride,
                       int8_t* out, void* stream)
{
    SYNTH_GRID_CHECK();
    hipLaunchKernelGGL(k_queries, dim3(blocks(g.total())), dim3(kThreads), 0,
                       (hipStream_t)stream, (uint64_t)seed, g, out);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

// Values: centred Irwin-Hall sum of twelve 16-bit uniforms, scaled by 2^-17.
int alhr_synth_values(int seed, int B, int H, int d, int t0, int nt, int64_t row_stride,
                      float* out, void* stream)
{
    SYNTH_GRID_CHECK();
    hipLaunchKernelGGL(k_values, dim3(blocks(g.total())), dim3(kThreads), 0, (hipStream_t)stream,
                       (uint64_t)seed, g, out);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

// Uniform int8 in [lo, hi] from stream `stream_id`.
int alhr_synth_uniform_i8(int seed, int stream_id, int lo, int hi, int B, int H, int d, int t0,
                          int nt, int64_t row_stride, int8_t* out, void* stream)
{
    if (stream_id < 0 || stream_id > 15 || lo > hi || lo < -128 || hi > 127) return -1;
    SYNTH_GRID_CHECK();
    hipLaunchKernelGGL(k_uniform, dim3(blocks(g.total())), dim3(kThreads), 0,
                       (hipStream_t)stream, (uint64_t)seed, (uint64_t)stream_id, lo, hi, g, out);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

// Predictor weights int8 [n_classes, 2d] in [-4, 4].
int alhr_synth_weights(int seed, int n_classes, int d, int8_t* out, void* stream)
{
    if (seed < 0 || seed > 255 || n_classes < 1 || n_classes > 4096 || d < 1 || d > 256 || !out)
        return -1;
    const int n = n_classes * 2 * d;
    hipLaunchKernelGGL(k_weights, dim3((n + kThreads - 1) / kThreads), dim3(kThreads), 0,
                       (hipStream_t)stream, (uint64_t)seed, n_classes, d, out);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // extern "C"
