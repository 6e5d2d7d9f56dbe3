// Internal launch interface between the C ABI layer and the gfx950 kernels.
// Every launcher assumes its arguments were validated by the ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace alhr {

struct Shape {
    int P;            // batch * heads pairs
    int T;            // positions per pair (power of two)
    int L;            // log2(T)
    int d;            // head dimension
    int window;
    int n_classes;
    int keys_per_class;
    int max_budget;
    float scale;
    bool mul24;       // every scored tree node fits a signed 24-bit multiply
    int l16;          // tree levels 1..l16 are stored as int16 rows (kmax * 2^l <= 32767)
};

// Scratch for the predictor: one int32 per (pair, chunk, class).
size_t predict_ws_bytes(const Shape& s);

hipError_t launch_build(const Shape& s, const int8_t* K, int32_t* nodes, hipStream_t st);
// The build passes from tree level in_level up (in_level = 0: from the keys).
hipError_t launch_build_from(const Shape& s, const int8_t* K, int32_t* nodes, int in_level,
                             hipStream_t st);
// Tree build and budget prediction sharing their launches (prep.hip); ws as
// for launch_predict.
hipError_t launch_prep(const Shape& s, const int8_t* Q, const int8_t* K, const int8_t* W,
                       int32_t* nodes, int32_t* budget, void* ws, hipStream_t st);

hipError_t launch_predict(const Shape& s, const int8_t* Q, const int8_t* K, const int8_t* W,
                          int32_t* budget, void* ws, hipStream_t st);

// O == nullptr: routing only (score, if not null, receives q . K[j] of the
// selected keys); stats != nullptr: write per-query load counts instead.
hipError_t launch_route(const Shape& s, const int8_t* Q, const int8_t* K, const float* V,
                        const int32_t* nodes, const int32_t* budget, int fixed_budget,
                        int32_t* idx, int32_t* count, float* O, int32_t* stats, int32_t* score,
                        hipStream_t st);

hipError_t launch_attend(const Shape& s, const int8_t* Q, const int8_t* K, const float* V,
                         const int32_t* idx, const int32_t* count, float* O, hipStream_t st);

hipError_t launch_prefix_from_tree(const Shape& s, int n, const int8_t* K, const int32_t* nodes,
                                   int32_t* prefix, hipStream_t st);

hipError_t launch_append(const Shape& s, int pos, const int8_t* k_new, const float* v_new,
                         int8_t* K, float* V, int32_t* nodes, int32_t* prefix, hipStream_t st);

// k_new == nullptr: decode step only (the pair's rows are already appended);
// otherwise append k_new / v_new at pos first, in the same launch.  The
// decode-only path reads K, V, nodes and prefix without writing them.
hipError_t launch_decode(const Shape& s, int pos, const int8_t* q_new, const int8_t* k_new,
                         const float* v_new, int8_t* K, float* V, int32_t* nodes,
                         int32_t* prefix, const int8_t* W, int fixed_budget, int32_t* budget,
                         int32_t* idx, int32_t* count, float* O, hipStream_t st);

hipError_t launch_dense(const Shape& s, const int8_t* Q, const int8_t* K, const float* V, float* O,
                        hipStream_t st);

struct SplitShape {
    int batch, heads, T, d, d_model, shift, qclamp, kclamp;
};

hipError_t launch_split(const SplitShape& s, const int8_t* X, const int8_t* W, int8_t* Q,
                        int8_t* K, hipStream_t st);

}  // namespace alhr
