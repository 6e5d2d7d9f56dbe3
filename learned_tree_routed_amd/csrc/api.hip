// C ABI of libalhr: argument validation on the host, then kernel launches on
// the caller's stream.  Every check runs before the first HIP call, so a
// rejected call touches neither the device nor the outputs.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "../../include/alhr.h"
#include "kernels.h"

namespace {

thread_local std::string g_last_error;

alhr_status fail(alhr_status st, const char* fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

alhr_status ok()
{
    g_last_error.clear();
    return ALHR_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

#define ALHR_NEED_PTR(p)                                                                  \
    do {                                                                                  \
        if (!(p)) return fail(ALHR_ERR_ARG, "%s: argument '%s' is NULL", fn, #p);         \
        if (!aligned16(p))                                                                \
            return fail(ALHR_ERR_ARG, "%s: argument '%s' is not 16-byte aligned", fn, #p); \
    } while (0)

// Levels whose node sums fit int16: largest l <= L with kmax * 2^l <= 32767.
int int16_levels(int kmax, int L)
{
    int l = 0;
    while (l < L && (int64_t)kmax * ((int64_t)2 << l) <= 32767) ++l;
    return l;
}

alhr_status check_config(const char* fn, const alhr_config* c, alhr::Shape* s)
{
    if (!c) return fail(ALHR_ERR_ARG, "%s: cfg is NULL", fn);
    if (c->batch < 1 || c->heads < 1)
        return fail(ALHR_ERR_ARG, "%s: batch (%d) and heads (%d) must be >= 1", fn, c->batch,
                    c->heads);
    if ((int64_t)c->batch * c->heads > 65536)
        return fail(ALHR_ERR_ARG, "%s: batch * heads = %lld exceeds 65536", fn,
                    (long long)c->batch * c->heads);
    if (c->T < 2 || c->T > (1 << 20) || (c->T & (c->T - 1)))
        return fail(ALHR_ERR_ARG, "%s: T = %d must be a power of two in [2, 2^20]", fn, c->T);
    if (c->d < 1 || c->d % 16)
        return fail(ALHR_ERR_ARG, "%s: d = %d must be a positive multiple of 16", fn, c->d);
    if (c->d != 16 && c->d != 32 && c->d != 64 && c->d != 128 && c->d != 256)
        return fail(ALHR_ERR_UNSUPPORTED, "%s: d = %d is not built (16, 32, 64, 128, 256)", fn,
                    c->d);
    if (c->window < 1) return fail(ALHR_ERR_ARG, "%s: window = %d must be >= 1", fn, c->window);
    if (c->n_classes < 1 || c->n_classes > 32)
        return fail(ALHR_ERR_ARG, "%s: n_classes = %d must be in [1, 32]", fn, c->n_classes);
    if (c->keys_per_class < 1)
        return fail(ALHR_ERR_ARG, "%s: keys_per_class = %d must be >= 1", fn,
                    c->keys_per_class);
    if (c->max_budget < 1 || c->max_budget > 128)
        return fail(ALHR_ERR_ARG, "%s: max_budget = %d must be in [1, 128]", fn, c->max_budget);
    if (c->kmax < 0 || c->kmax > 127 || c->qmax < 0 || c->qmax > 127 || c->wmax < 0 ||
        c->wmax > 127)
        return fail(ALHR_ERR_ARG, "%s: kmax, qmax, wmax must be in [0, 127]", fn);
    if (!std::isfinite(c->scale)) return fail(ALHR_ERR_ARG, "%s: scale is not finite", fn);
    const int64_t lim = (int64_t)1 << 31;
    const int64_t T = c->T, d = c->d;
    if ((int64_t)c->kmax * T >= lim)
        return fail(ALHR_ERR_OVERFLOW, "%s: kmax * T = %lld reaches 2^31 (node sums)", fn,
                    (long long)(c->kmax * T));
    if ((int64_t)c->qmax * c->kmax * d * (T / 2) >= lim)
        return fail(ALHR_ERR_OVERFLOW, "%s: qmax * kmax * d * T/2 = %lld reaches 2^31 (scores)",
                    fn, (long long)((int64_t)c->qmax * c->kmax * d * (T / 2)));
    if ((int64_t)c->wmax * d * (c->qmax + (int64_t)c->kmax * T) >= lim)
        return fail(ALHR_ERR_OVERFLOW, "%s: wmax * d * (qmax + kmax * T) reaches 2^31 (logits)",
                    fn);
    if (s) {
        s->P = c->batch * c->heads;
        s->T = c->T;
        int L = 0;
        while ((1 << L) < c->T) ++L;
        s->L = L;
        s->d = c->d;
        s->window = c->window;
        s->n_classes = c->n_classes;
        s->keys_per_class = c->keys_per_class;
        s->max_budget = c->max_budget;
        s->scale = c->scale;
        // every scored node has at most T/2 keys: its entries fit 24 signed bits?
        s->mul24 = (int64_t)c->kmax * (T / 2) < ((int64_t)1 << 23);
        s->l16 = int16_levels(c->kmax, L);
    }
    return ALHR_OK;
}

alhr_status check_fixed(const char* fn, const alhr_config* c, const int32_t* budget, int32_t fb)
{
    if (!budget && (fb < 1 || fb > c->max_budget))
        return fail(ALHR_ERR_ARG, "%s: fixed_budget = %d must be in [1, max_budget = %d]", fn,
                    fb, c->max_budget);
    if (budget && !aligned16(budget))
        return fail(ALHR_ERR_ARG, "%s: argument 'budget' is not 16-byte aligned", fn);
    return ALHR_OK;
}

alhr_status device_status(const char* fn, hipError_t e)
{
    if (e != hipSuccess)
        return fail(ALHR_ERR_DEVICE, "%s: %s (%s)", fn, hipGetErrorName(e), hipGetErrorString(e));
    return ok();
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

size_t workspace_bytes(const alhr::Shape& s) { return alhr::predict_ws_bytes(s); }

alhr_status check_ws(const char* fn, const alhr::Shape& s, const void* ws, size_t ws_bytes)
{
    const size_t need = workspace_bytes(s);
    if (!ws || ws_bytes < need || !aligned16(ws))
        return fail(ALHR_ERR_WORKSPACE, "%s: workspace of %zu bytes needed (got %zu%s%s)", fn,
                    need, ws_bytes, ws ? "" : ", NULL", ws && !aligned16(ws) ? ", misaligned" : "");
    return ALHR_OK;
}

}  // namespace

extern "C" {

int32_t alhr_version(void) { return 100; }

const char* alhr_status_string(alhr_status s)
{
    switch (s) {
        case ALHR_OK: return "ALHR_OK";
        case ALHR_ERR_ARG: return "ALHR_ERR_ARG: invalid argument";
        case ALHR_ERR_OVERFLOW: return "ALHR_ERR_OVERFLOW: declared bounds overflow int32";
        case ALHR_ERR_DEVICE: return "ALHR_ERR_DEVICE: HIP runtime or launch failure";
        case ALHR_ERR_UNSUPPORTED: return "ALHR_ERR_UNSUPPORTED: configuration not built";
        case ALHR_ERR_WORKSPACE: return "ALHR_ERR_WORKSPACE: workspace missing or too small";
    }
    return "unknown alhr_status";
}

const char* alhr_last_error(void) { return g_last_error.c_str(); }

int32_t alhr_tree_int16_levels(const alhr_config* cfg)
{
    alhr::Shape s;
    if (check_config("alhr_tree_int16_levels", cfg, &s) != ALHR_OK) return -1;
    return s.l16;
}

size_t alhr_workspace_bytes(const alhr_config* cfg)
{
    alhr::Shape s;
    if (check_config("alhr_workspace_bytes", cfg, &s) != ALHR_OK) return 0;
    return workspace_bytes(s);
}

alhr_status alhr_build_tree(const alhr_config* cfg, const int8_t* K, int32_t* nodes,
                            void* stream)
{
    const char* fn = "alhr_build_tree";
    alhr::Shape s;
    if (alhr_status st = check_config(fn, cfg, &s)) return st;
    ALHR_NEED_PTR(K);
    ALHR_NEED_PTR(nodes);
    (void)hipGetLastError();
    return device_status(fn, alhr::launch_build(s, K, nodes, as_stream(stream)));
}

alhr_status alhr_predict_budget(const alhr_config* cfg, const int8_t* Q, const int8_t* K,
                                const int8_t* W, int32_t* budget, void* ws, size_t ws_bytes,
                                void* stream)
{
    const char* fn = "alhr_predict_budget";
    alhr::Shape s;
    if (alhr_status st = check_config(fn, cfg, &s)) return st;
    ALHR_NEED_PTR(Q);
    ALHR_NEED_PTR(K);
    ALHR_NEED_PTR(W);
    ALHR_NEED_PTR(budget);
    if (alhr_status st = check_ws(fn, s, ws, ws_bytes)) return st;
    (void)hipGetLastError();
    return device_status(fn, alhr::launch_predict(s, Q, K, W, budget, ws,
                                                  as_stream(stream)));
}

alhr_status alhr_prepare(const alhr_config* cfg, const int8_t* Q, const int8_t* K,
                         const int8_t* W, int32_t* nodes, int32_t* budget, void* ws,
                         size_t ws_bytes, void* stream)
{
    const char* fn = "alhr_prepare";
    alhr::Shape s;
    if (alhr_status st = check_config(fn, cfg, &s)) return st;
    ALHR_NEED_PTR(K);
    ALHR_NEED_PTR(nodes);
    if (W) {
        ALHR_NEED_PTR(Q);
        ALHR_NEED_PTR(W);
        ALHR_NEED_PTR(budget);
        if (alhr_status st = check_ws(fn, s, ws, ws_bytes)) return st;
    }
    (void)hipGetLastError();
    hipStream_t st = as_stream(stream);
    return device_status(fn, W ? alhr::launch_prep(s, Q, K, W, nodes, budget, ws, st)
                               : alhr::launch_build(s, K, nodes, st));
}

static alhr_status route_common(const char* fn, const alhr_config* cfg, const int8_t* Q,
                                const int8_t* K, const float* V, const int32_t* nodes,
                                const int32_t* budget, int32_t fixed_budget, int32_t* idx,
                                int32_t* count, float* O, int32_t* stats, int32_t* score,
                                bool attend, void* stream)
{
    alhr::Shape s;
    if (alhr_status st = check_config(fn, cfg, &s)) return st;
    ALHR_NEED_PTR(Q);
    ALHR_NEED_PTR(K);
    ALHR_NEED_PTR(nodes);
    ALHR_NEED_PTR(idx);
    ALHR_NEED_PTR(count);
    if (attend) {
        ALHR_NEED_PTR(V);
        ALHR_NEED_PTR(O);
    }
    if (alhr_status st = check_fixed(fn, cfg, budget, fixed_budget)) return st;
    if (score && !aligned16(score))
        return fail(ALHR_ERR_ARG, "%s: argument 'score' is not 16-byte aligned", fn);
    (void)hipGetLastError();
    return device_status(fn, alhr::launch_route(s, Q, K, attend ? V : nullptr, nodes, budget,
                                                fixed_budget, idx, count, attend ? O : nullptr,
                                                stats, score, as_stream(stream)));
}

alhr_status alhr_route(const alhr_config* cfg, const int8_t* Q, const int8_t* K,
                       const int32_t* nodes, const int32_t* budget, int32_t fixed_budget,
                       int32_t* idx, int32_t* count, int32_t* score, void* stream)
{
    return route_common("alhr_route", cfg, Q, K, nullptr, nodes, budget, fixed_budget, idx,
                        count, nullptr, nullptr, score, false, stream);
}

alhr_status alhr_route_stats(const alhr_config* cfg, const int8_t* Q, const int8_t* K,
                             const int32_t* nodes, const int32_t* budget, int32_t fixed_budget,
                             int32_t* idx, int32_t* count, int32_t* stats, void* stream)
{
    const char* fn = "alhr_route_stats";
    ALHR_NEED_PTR(stats);
    return route_common(fn, cfg, Q, K, nullptr, nodes, budget, fixed_budget, idx, count,
                        nullptr, stats, nullptr, false, stream);
}

alhr_status alhr_sparse_attend(const alhr_config* cfg, const int8_t* Q, const int8_t* K,
                               const float* V, const int32_t* idx, const int32_t* count,
                               float* O, void* stream)
{
    const char* fn = "alhr_sparse_attend";
    alhr::Shape s;
    if (alhr_status st = check_config(fn, cfg, &s)) return st;
    ALHR_NEED_PTR(Q);
    ALHR_NEED_PTR(K);
    ALHR_NEED_PTR(V);
    ALHR_NEED_PTR(idx);
    ALHR_NEED_PTR(count);
    ALHR_NEED_PTR(O);
    (void)hipGetLastError();
    return device_status(fn, alhr::launch_attend(s, Q, K, V, idx, count, O, as_stream(stream)));
}

alhr_status alhr_route_attend(const alhr_config* cfg, const int8_t* Q, const int8_t* K,
                              const float* V, const int32_t* nodes, const int32_t* budget,
                              int32_t fixed_budget, int32_t* idx, int32_t* count, float* O,
                              void* stream)
{
    return route_common("alhr_route_attend", cfg, Q, K, V, nodes, budget, fixed_budget, idx,
                        count, O, nullptr, nullptr, true, stream);
}

}  // extern "C"

namespace {

// The checks and launches of alhr_forward.  ws == nullptr with W given means
// the library's own scratch array (alhr_forward_noalloc, below).
alhr_status forward_impl(const char* fn, const alhr_config* cfg, const int8_t* Q,
                         const int8_t* K, const float* V, const int8_t* W, int32_t fixed_budget,
                         int32_t* nodes, int32_t* budget, int32_t* idx, int32_t* count, float* O,
                         void* ws, size_t ws_bytes, bool own_scratch, void* stream);

}  // namespace

extern "C" {

alhr_status alhr_forward(const alhr_config* cfg, const int8_t* Q, const int8_t* K,
                         const float* V, const int8_t* W, int32_t fixed_budget, int32_t* nodes,
                         int32_t* budget, int32_t* idx, int32_t* count, float* O, void* ws,
                         size_t ws_bytes, void* stream)
{
    return forward_impl("alhr_forward", cfg, Q, K, V, W, fixed_budget, nodes, budget, idx, count,
                        O, ws, ws_bytes, false, stream);
}

alhr_status alhr_forward_noalloc(const alhr_config* cfg, const int8_t* Q, const int8_t* K,
                                 const float* V, const int8_t* W, int32_t fixed_budget,
                                 int32_t* nodes, int32_t* budget, int32_t* idx, int32_t* count,
                                 float* O, void* stream)
{
    return forward_impl("alhr_forward_noalloc", cfg, Q, K, V, W, fixed_budget, nodes, budget, idx,
                        count, O, nullptr, 0, true, stream);
}

}  // extern "C"

// ---- the scratch array of alhr_forward_noalloc -------------------------------
// A file-scope device array that every GPU the library runs on holds until the
// process ends (each at its own address).  Host code never passes `scratch`
// itself to a kernel or copy: on the host the name is a stand-in, not a device
// address.  The device address comes from hipGetSymbolAddress, taken once per
// device on the entry point's first call there (that device current) and kept.
namespace {

constexpr size_t kScratchBytes = (size_t)4 << 20;
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch`, in *out; the device the stream
// belongs to must be the current one.
alhr_status scratch_on_current_device(const char* fn, hipStream_t st, void** out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return device_status(fn, e);
    if (dev < 0 || dev >= kMaxDevices)
        return fail(ALHR_ERR_UNSUPPORTED, "%s: device %d beyond the %d devices served", fn, dev,
                    kMaxDevices);
    if (st) {
        hipDevice_t sdev = -1;
        e = hipStreamGetDevice(st, &sdev);
        if (e != hipSuccess) return device_status(fn, e);
        if ((int)sdev != dev)
            return fail(ALHR_ERR_ARG, "%s: the stream belongs to device %d, the current device "
                                      "is %d", fn, (int)sdev, dev);
    }
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return device_status(fn, e);
        if (!p) return fail(ALHR_ERR_DEVICE, "%s: no device address for the scratch array", fn);
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return ALHR_OK;
}

alhr_status forward_impl(const char* fn, const alhr_config* cfg, const int8_t* Q,
                         const int8_t* K, const float* V, const int8_t* W, int32_t fixed_budget,
                         int32_t* nodes, int32_t* budget, int32_t* idx, int32_t* count, float* O,
                         void* ws, size_t ws_bytes, bool own_scratch, void* stream)
{
    alhr::Shape s;
    if (alhr_status st = check_config(fn, cfg, &s)) return st;
    ALHR_NEED_PTR(Q);
    ALHR_NEED_PTR(K);
    ALHR_NEED_PTR(V);
    ALHR_NEED_PTR(nodes);
    ALHR_NEED_PTR(idx);
    ALHR_NEED_PTR(count);
    ALHR_NEED_PTR(O);
    if (W) {
        if (!aligned16(W)) return fail(ALHR_ERR_ARG, "%s: argument 'W' is not 16-byte aligned", fn);
        if (!budget)
            return fail(ALHR_ERR_ARG, "%s: 'budget' must be given when W is (it holds the "
                                      "predicted budgets)", fn);
        if (!aligned16(budget))
            return fail(ALHR_ERR_ARG, "%s: argument 'budget' is not 16-byte aligned", fn);
        if (own_scratch) {
            if (workspace_bytes(s) > kScratchBytes)
                return fail(ALHR_ERR_WORKSPACE, "%s: this shape needs %zu bytes of predictor "
                                                "scratch, beyond the %zu bytes of the library's "
                                                "array (batch * heads * ceil(T / 256) must not "
                                                "exceed 32768); use alhr_forward with a workspace",
                            fn, workspace_bytes(s), kScratchBytes);
        } else if (alhr_status st = check_ws(fn, s, ws, ws_bytes)) {
            return st;
        }
    } else if (fixed_budget < 1 || fixed_budget > cfg->max_budget) {
        return fail(ALHR_ERR_ARG, "%s: fixed_budget = %d must be in [1, max_budget = %d]", fn,
                    fixed_budget, cfg->max_budget);
    }
    hipStream_t st = as_stream(stream);
    (void)hipGetLastError();
    if (W && own_scratch) {
        if (alhr_status r = scratch_on_current_device(fn, st, &ws)) return r;
    }
    // tree and budgets share their launches (alhr_prepare)
    hipError_t e = W ? alhr::launch_prep(s, Q, K, W, nodes, budget, ws, st)
                     : alhr::launch_build(s, K, nodes, st);
    if (e == hipSuccess)
        e = alhr::launch_route(s, Q, K, V, nodes, W ? budget : nullptr, fixed_budget, idx, count,
                               O, nullptr, nullptr, st);
    return device_status(fn, e);
}

}  // namespace

extern "C" {

alhr_status alhr_dense_attend(const alhr_config* cfg, const int8_t* Q, const int8_t* K,
                              const float* V, float* O, void* stream)
{
    const char* fn = "alhr_dense_attend";
    alhr::Shape s;
    if (alhr_status st = check_config(fn, cfg, &s)) return st;
    if (cfg->d < 32)
        return fail(ALHR_ERR_UNSUPPORTED, "%s: d = %d is not built for the dense kernel (32, 64, "
                                          "128, 256)", fn, cfg->d);
    if ((int64_t)s.P * s.T >= ((int64_t)1 << 31))   // one launch of 2 * P * T work-items
        return fail(ALHR_ERR_UNSUPPORTED, "%s: batch * heads * T must stay below 2^31", fn);
    ALHR_NEED_PTR(Q);
    ALHR_NEED_PTR(K);
    ALHR_NEED_PTR(V);
    ALHR_NEED_PTR(O);
    (void)hipGetLastError();
    return device_status(fn, alhr::launch_dense(s, Q, K, V, O, as_stream(stream)));
}

alhr_status alhr_split_qk(const alhr_split_config* cfg, const int8_t* X, const int8_t* W,
                          int8_t* Q, int8_t* K, void* stream)
{
    const char* fn = "alhr_split_qk";
    if (!cfg) return fail(ALHR_ERR_ARG, "%s: cfg is NULL", fn);
    const alhr_split_config& c = *cfg;
    if (c.batch < 1 || c.heads < 1)
        return fail(ALHR_ERR_ARG, "%s: batch = %d and heads = %d must be >= 1", fn, c.batch, c.heads);
    if (c.T < 1 || c.T > (1 << 20)) return fail(ALHR_ERR_ARG, "%s: T = %d outside [1, 2^20]", fn, c.T);
    if (c.d != 16 && c.d != 32 && c.d != 64 && c.d != 128 && c.d != 256)
        return fail(ALHR_ERR_UNSUPPORTED, "%s: d = %d is not built (16, 32, 64, 128, 256)", fn, c.d);
    if (c.d_model < 16 || c.d_model > 16384 || c.d_model % 16)
        return fail(ALHR_ERR_ARG, "%s: d_model = %d must be a multiple of 16 in [16, 16384]", fn,
                    c.d_model);
    if (c.shift < 0 || c.shift > 30) return fail(ALHR_ERR_ARG, "%s: shift = %d outside [0, 30]", fn, c.shift);
    if (c.qclamp < 1 || c.qclamp > 127 || c.kclamp < 1 || c.kclamp > 127)
        return fail(ALHR_ERR_ARG, "%s: qclamp = %d, kclamp = %d must be in [1, 127]", fn, c.qclamp,
                    c.kclamp);
    const int64_t wide = std::max<int64_t>(c.d_model, (int64_t)c.heads * c.d);
    if ((int64_t)c.batch * c.T * wide >= ((int64_t)1 << 31))
        return fail(ALHR_ERR_ARG, "%s: batch * T * max(d_model, heads * d) must stay below 2^31", fn);
    ALHR_NEED_PTR(X);
    ALHR_NEED_PTR(W);
    ALHR_NEED_PTR(Q);
    ALHR_NEED_PTR(K);
    const alhr::SplitShape s{c.batch, c.heads, c.T, c.d, c.d_model, c.shift, c.qclamp, c.kclamp};
    (void)hipGetLastError();
    return device_status(fn, alhr::launch_split(s, X, W, Q, K, as_stream(stream)));
}

alhr_status alhr_prefix_from_tree(const alhr_config* cfg, int32_t n, const int8_t* K,
                                  const int32_t* nodes, int32_t* prefix, void* stream)
{
    const char* fn = "alhr_prefix_from_tree";
    alhr::Shape s;
    if (alhr_status st = check_config(fn, cfg, &s)) return st;
    if (n < 0 || n > cfg->T) return fail(ALHR_ERR_ARG, "%s: n = %d must be in [0, T]", fn, n);
    ALHR_NEED_PTR(K);
    ALHR_NEED_PTR(nodes);
    ALHR_NEED_PTR(prefix);
    (void)hipGetLastError();
    return device_status(fn, alhr::launch_prefix_from_tree(s, n, K, nodes, prefix,
                                                           as_stream(stream)));
}

alhr_status alhr_append(const alhr_config* cfg, int32_t pos, const int8_t* k_new,
                        const float* v_new, int8_t* K, float* V, int32_t* nodes, int32_t* prefix,
                        void* stream)
{
    const char* fn = "alhr_append";
    alhr::Shape s;
    if (alhr_status st = check_config(fn, cfg, &s)) return st;
    if (pos < 0 || pos >= cfg->T) return fail(ALHR_ERR_ARG, "%s: pos = %d outside [0, T)", fn, pos);
    ALHR_NEED_PTR(k_new);
    ALHR_NEED_PTR(v_new);
    ALHR_NEED_PTR(K);
    ALHR_NEED_PTR(V);
    ALHR_NEED_PTR(nodes);
    ALHR_NEED_PTR(prefix);
    (void)hipGetLastError();
    return device_status(fn, alhr::launch_append(s, pos, k_new, v_new, K, V, nodes, prefix,
                                                 as_stream(stream)));
}

static alhr_status decode_common(const char* fn, const alhr_config* cfg, int32_t pos,
                                 const int8_t* q_new, const int8_t* k_new, const float* v_new,
                                 const int8_t* K, const float* V, const int32_t* nodes,
                                 const int32_t* prefix, const int8_t* W, int32_t fixed_budget,
                                 int32_t* budget, int32_t* idx, int32_t* count, float* O,
                                 bool append, void* stream)
{
    alhr::Shape s;
    if (alhr_status st = check_config(fn, cfg, &s)) return st;
    if (pos < 0 || pos >= cfg->T) return fail(ALHR_ERR_ARG, "%s: pos = %d outside [0, T)", fn, pos);
    ALHR_NEED_PTR(q_new);
    if (append) {
        ALHR_NEED_PTR(k_new);
        ALHR_NEED_PTR(v_new);
        ALHR_NEED_PTR(prefix);
    }
    ALHR_NEED_PTR(K);
    ALHR_NEED_PTR(V);
    ALHR_NEED_PTR(nodes);
    ALHR_NEED_PTR(idx);
    ALHR_NEED_PTR(count);
    ALHR_NEED_PTR(O);
    if (W) {
        ALHR_NEED_PTR(prefix);
        if (!aligned16(W)) return fail(ALHR_ERR_ARG, "%s: argument 'W' is not 16-byte aligned", fn);
    } else if (fixed_budget < 1 || fixed_budget > cfg->max_budget) {
        return fail(ALHR_ERR_ARG, "%s: fixed_budget = %d must be in [1, max_budget = %d]", fn,
                    fixed_budget, cfg->max_budget);
    }
    if (budget && !aligned16(budget))
        return fail(ALHR_ERR_ARG, "%s: argument 'budget' is not 16-byte aligned", fn);
    (void)hipGetLastError();
    // the decode-only path reads K, V, nodes and prefix and never writes them
    return device_status(fn, alhr::launch_decode(s, pos, q_new, append ? k_new : nullptr,
                                                 append ? v_new : nullptr,
                                                 const_cast<int8_t*>(K), const_cast<float*>(V),
                                                 const_cast<int32_t*>(nodes),
                                                 const_cast<int32_t*>(prefix), W, fixed_budget,
                                                 budget, idx, count, O, as_stream(stream)));
}

alhr_status alhr_decode_step(const alhr_config* cfg, int32_t pos, const int8_t* q_new,
                             const int8_t* K, const float* V, const int32_t* nodes,
                             const int32_t* prefix, const int8_t* W, int32_t fixed_budget,
                             int32_t* budget, int32_t* idx, int32_t* count, float* O,
                             void* stream)
{
    return decode_common("alhr_decode_step", cfg, pos, q_new, nullptr, nullptr, K, V, nodes,
                         prefix, W, fixed_budget, budget, idx, count, O, false, stream);
}

alhr_status alhr_append_decode(const alhr_config* cfg, int32_t pos, const int8_t* k_new,
                               const float* v_new, const int8_t* q_new, int8_t* K, float* V,
                               int32_t* nodes, int32_t* prefix, const int8_t* W,
                               int32_t fixed_budget, int32_t* budget, int32_t* idx,
                               int32_t* count, float* O, void* stream)
{
    return decode_common("alhr_append_decode", cfg, pos, q_new, k_new, v_new, K, V, nodes,
                         prefix, W, fixed_budget, budget, idx, count, O, true, stream);
}

}  // extern "C"
