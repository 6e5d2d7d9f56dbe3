/*
 * alhr.h - C ABI of the ALHR tree-attention inference path for AMD Instinct
 * MI355X (gfx950).
 *
 * ALHR (Adaptive Learnable Hierarchical Routing) summarises the keys of each
 * (batch, head) pair in a static binary tree whose nodes hold the sum of the
 * key vectors beneath them; a budget predictor maps each query and the
 * causal key sum to a key budget; the query takes its own and neighbouring
 * keys, then descends the causal part of the tree along the branches with
 * the higher q . node_sum score until the budget is filled, and finally runs
 * softmax attention over only the selected keys.
 * Sources: the ALHR README ("Adaptive learnable Hierarchical routing:
 * sub-quadratic tree attention ... (beta)"), sections "Inference stage",
 * "Training stage" (causality) and "Results and Variables" (caps of 96 keys
 * and 32 budget classes); decode use from the openai-hub article
 * "ALHR把注意力变成树搜索", section "ALHR是什么".
 *
 * Conventions shared by every call
 * --------------------------------
 * Pointers.  Every array argument is DEVICE memory owned by the caller; the
 * library never allocates or frees device memory, and keeps no state between
 * calls.  Scratch space is passed explicitly as (ws, ws_bytes), at least
 * alhr_workspace_bytes() bytes; its contents need no initialisation and are
 * not meaningful between calls, and two calls that may run at the same time
 * (different streams) must not share one.  Array base pointers must be
 * 16-byte aligned.  `stream` is a hipStream_t passed as void* (NULL = the
 * null stream).  Calls are asynchronous: results are valid once the caller
 * synchronises `stream`.
 *
 * Layouts (row-major, d contiguous; P = batch * heads pairs):
 *   Q, K   int8  [batch, heads, T, d]     queries / keys
 *   V, O   fp32  [batch, heads, T, d]     values / attention output
 *   W      int8  [n_classes, 2d]          predictor weights: columns [0, d)
 *                                         multiply the query, [d, 2d) the
 *                                         causal key sum; shared by all pairs
 *   nodes  int32 [batch, heads, T, d]     tree of key sums in heap order:
 *          node (level l >= 1, index p), covering keys [p*2^l, (p+1)*2^l),
 *          is row (T >> l) + p; row 1 is the root; row 0 is never written;
 *          the children of row i are rows 2i and 2i+1, and a row number
 *          h >= T stands for key row h - T.  Compact encoding: with
 *          l16 = alhr_tree_int16_levels(cfg) (the levels whose sums
 *          provably fit int16: kmax * 2^l <= 32767) and b = T >> l16, a row
 *          i < b (levels above l16) holds d int32 at byte offset 4*d*i of
 *          the pair's table, and a row i >= b (levels 1..l16) holds d int16
 *          at byte offset 4*d*b + 2*d*(i - b), packed densely; the last
 *          2*d*(T - b) bytes of the table are left untouched.  The buffer
 *          size is T * d * 4 bytes per pair either way.  Column order: an
 *          int16 row is in natural order; an int32 row's d/4 16-byte slots
 *          (slot g = columns 4g .. 4g+3) are block-interleaved: with
 *          m = d/16, slot g is stored at slot
 *          (2 * ((g/2) / m) + g%2) * m + (g/2) % m  (identity at d = 16),
 *          which lets the scoring kernels read every row with contiguous
 *          loads.  Callers treat `nodes` as opaque and fill it with
 *          alhr_build_tree / alhr_append.
 *   budget int32 [batch, heads, T]        keys asked for by each query
 *   idx    int32 [batch, heads, T, max_budget]   selected key positions,
 *          ascending, padded with -1
 *   count  int32 [batch, heads, T]        number of selected keys, C_t
 *
 * Errors.  Every argument check runs on the host before any launch; a call
 * that fails a check returns its code and writes nothing.  Launch failures
 * return ALHR_ERR_DEVICE.  alhr_last_error() gives a thread-local message
 * for the last non-OK status.  No C++ exception crosses this interface.
 * Calls on different streams do not share state and may run concurrently.
 *
 * Exactness.  Keys and queries are small integers, so node sums, scores and
 * predictor logits are exact int32 values as long as the declared bounds
 * hold: the library rejects (ALHR_ERR_OVERFLOW) a configuration for which
 *   kmax * T                           >= 2^31   (node sums),
 *   qmax * kmax * d * (T / 2)          >= 2^31   (scores; the root is never
 *                                                 scored, its halves are),
 *   wmax * d * (qmax + kmax * T)       >= 2^31   (predictor logits).
 * The bounds are declared, not measured: data outside them give undefined
 * (wrong, not unsafe) results.
 */
#ifndef ALHR_H
#define ALHR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum alhr_status {
    ALHR_OK = 0,
    ALHR_ERR_ARG = -1,          /* null pointer, bad size or bad parameter   */
    ALHR_ERR_OVERFLOW = -2,     /* bounds do not guarantee exact int32 sums  */
    ALHR_ERR_DEVICE = -3,       /* a HIP call or kernel launch failed        */
    ALHR_ERR_UNSUPPORTED = -4,  /* valid, but not built (e.g. this d)        */
    ALHR_ERR_WORKSPACE = -5     /* workspace missing or too small            */
} alhr_status;

typedef struct alhr_config {
    int32_t batch;           /* B >= 1 (decode: number of sequences)         */
    int32_t heads;           /* H >= 1; batch * heads <= 65536                */
    int32_t T;               /* positions = tree capacity: a power of two,
                                2 <= T <= 2^20                                */
    int32_t d;               /* head dimension: 16, 32, 64, 128 or 256        */
    int32_t window;          /* neighbour window w >= 1: key t and the w-1
                                keys before it                                */
    int32_t n_classes;       /* budget classes, 1..32                          */
    int32_t keys_per_class;  /* budget = keys_per_class * (class + 1), >= 1   */
    int32_t max_budget;      /* cap on the budget and row stride of idx,
                                1..128                                         */
    int32_t kmax, qmax, wmax;/* declared bounds on |K|, |Q|, |W| (0..127)     */
    float scale;             /* softmax scale, normally fl32(1/sqrt(d))       */
} alhr_config;

/* Number of tree levels stored as int16 rows (see `nodes` above), or -1 if
 * cfg is invalid. */
int32_t alhr_tree_int16_levels(const alhr_config *cfg);

/* Bytes of scratch (ws) that alhr_predict_budget / alhr_prepare /
 * alhr_forward need: the predictor's per-chunk class totals (a multiple of
 * 256; 0 if cfg is invalid). */
size_t alhr_workspace_bytes(const alhr_config *cfg);

/* Tree of key sums (README, opening paragraph and "Inference stage": one
 * static binary tree per layer over the key matrix, each branch keyed by the
 * sum of the keys beneath it).  Reads K, writes every row 1..T-1 of nodes. */
alhr_status alhr_build_tree(const alhr_config *cfg, const int8_t *K,
                            int32_t *nodes, void *stream);

/* Budget predictor (README "Inference stage"; caps in "Results and
 * Variables"): z_c = W[c][0:d] . Q[t] + W[c][d:2d] . S[t] with the causal
 * prefix S[t] = sum_{j<=t} K[j]; budget[t] = min(keys_per_class *
 * (argmax_c z_c + 1), max_budget), ties to the lowest class.  Needs
 * ws_bytes >= alhr_workspace_bytes(cfg). */
alhr_status alhr_predict_budget(const alhr_config *cfg, const int8_t *Q,
                                const int8_t *K, const int8_t *W,
                                int32_t *budget, void *ws, size_t ws_bytes,
                                void *stream);

/* alhr_build_tree followed by alhr_predict_budget (same citations, same
 * results, same argument rules), with the two steps sharing their launches:
 * they are independent, so each launch runs one build pass beside one
 * predictor pass.  W NULL: the tree only (budget and ws are then unused and
 * may be NULL).  alhr_forward prepares this way. */
alhr_status alhr_prepare(const alhr_config *cfg, const int8_t *Q,
                         const int8_t *K, const int8_t *W, int32_t *nodes,
                         int32_t *budget, void *ws, size_t ws_bytes,
                         void *stream);

/* Routing (README "Inference stage" and "Training stage"): for each query t
 * with budget B_t (budget[t], or fixed_budget when budget is NULL; array
 * values outside [1, max_budget] are clamped into it): C_t = min(B_t, t+1)
 * keys; the n_t = min(window, C_t) keys t, t-1, ...; then a beam of width
 * r_t = C_t - n_t descends from the maximal complete subtrees covering
 * [0, t+1-n_t), expanding every internal beam node each round and keeping
 * the r_t best nodes by (q . node_sum descending, first position ascending).
 * Writes idx and count; score (nullable) int32 [batch, heads, T, max_budget]
 * receives q . K[j] for each selected j in idx order and 0 in the padding. */
alhr_status alhr_route(const alhr_config *cfg, const int8_t *Q,
                       const int8_t *K, const int32_t *nodes,
                       const int32_t *budget, int32_t fixed_budget,
                       int32_t *idx, int32_t *count, int32_t *score,
                       void *stream);

/* Per-query load counts of the routing step (README "Inference stage"), for
 * byte accounting: stats is int32 [batch, heads, T, 4] = (int32 tree rows
 * loaded, int16 tree rows loaded, key rows loaded by the descent, selected
 * keys C); the neighbour key rows are min(window, C).  Arguments as for
 * alhr_route without score; idx and count are written as by alhr_route. */
alhr_status alhr_route_stats(const alhr_config *cfg, const int8_t *Q,
                             const int8_t *K, const int32_t *nodes,
                             const int32_t *budget, int32_t fixed_budget,
                             int32_t *idx, int32_t *count, int32_t *stats,
                             void *stream);

/* Sparse attention over selected keys (README "Inference stage"): for each
 * query, a_j = fl32(fl32(Q[t] . K[j]) * scale) over j in idx[t][0..count[t]),
 * and O[t] = sum_j softmax(a)_j V[j], in fp32.  count values are clamped to
 * [0, max_budget]; positions outside [0, T) are left out of the softmax; a
 * query with no valid position gets O[t] = 0. */
alhr_status alhr_sparse_attend(const alhr_config *cfg, const int8_t *Q,
                               const int8_t *K, const float *V,
                               const int32_t *idx, const int32_t *count,
                               float *O, void *stream);

/* Fused routing + attention in one pass per query (README "Inference
 * stage": the descent's keys, then attention over them; the openai-hub
 * article, section "判断：方向对，但离“大模型可用”还有两道关", on dedicated
 * kernels and batched routing).  Same results as alhr_route followed by
 * alhr_sparse_attend; the leaf scores found by the descent are reused as
 * logits. */
alhr_status alhr_route_attend(const alhr_config *cfg, const int8_t *Q,
                              const int8_t *K, const float *V,
                              const int32_t *nodes, const int32_t *budget,
                              int32_t fixed_budget, int32_t *idx,
                              int32_t *count, float *O, void *stream);

/* The whole prefill path of the README's "Inference stage": build the tree,
 * predict budgets (W != NULL; else every query uses fixed_budget), route and
 * attend.  budget (nullable) receives the predicted budgets.  ws as for
 * alhr_predict_budget (unused when W is NULL). */
alhr_status alhr_forward(const alhr_config *cfg, const int8_t *Q,
                         const int8_t *K, const float *V, const int8_t *W,
                         int32_t fixed_budget, int32_t *nodes,
                         int32_t *budget, int32_t *idx, int32_t *count,
                         float *O, void *ws, size_t ws_bytes, void *stream);

/* alhr_forward for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.  The
 * same arguments, checks and results as alhr_forward, without (ws,
 * ws_bytes): the predictor's scratch is an array of 4 MiB that the library
 * holds on each GPU it runs on until the process ends, so batch * heads *
 * ceil(T / 256) must not exceed 32768 when W is given (ALHR_ERR_WORKSPACE
 * otherwise).  Nothing is allocated or freed.  Every call on one GPU uses
 * that GPU's array: calls that may overlap on one GPU (different streams)
 * race and must not be issued.  The stream must belong to the current
 * device (ALHR_ERR_ARG otherwise). */
alhr_status alhr_forward_noalloc(const alhr_config *cfg, const int8_t *Q,
                                 const int8_t *K, const float *V,
                                 const int8_t *W, int32_t fixed_budget,
                                 int32_t *nodes, int32_t *budget,
                                 int32_t *idx, int32_t *count, float *O,
                                 void *stream);

/* Decode cache set-up: prefix[b, h] = sum_{j < n} K[j] (int32 [batch, heads,
 * d]) read from the tree as the sum of the maximal complete subtrees
 * covering [0, n); 0 <= n <= T (n = 0 gives zeros). */
alhr_status alhr_prefix_from_tree(const alhr_config *cfg, int32_t n,
                                  const int8_t *K, const int32_t *nodes,
                                  int32_t *prefix, void *stream);

/* Decode append at position pos, the same for every pair (openai-hub
 * article, "ALHR是什么": one new token at a time): K[pos] = k_new,
 * V[pos] = v_new, nodes(l, pos >> l) += k_new for every level l >= 1, and
 * prefix += k_new (so prefix holds S[pos] afterwards).  k_new int8 and v_new
 * fp32 are [batch, heads, d].  Precondition: key rows >= pos are zero and
 * nodes is the tree of those keys (rebuilding after appends gives the same
 * table). */
alhr_status alhr_append(const alhr_config *cfg, int32_t pos,
                        const int8_t *k_new, const float *v_new, int8_t *K,
                        float *V, int32_t *nodes, int32_t *prefix,
                        void *stream);

/* Decode step (openai-hub article, section "ALHR是什么": one new token at a
 * time, routed through the cached tree; README "Inference stage" for the
 * steps): route and attend the single query q_new (int8 [batch, heads, d])
 * at position pos of every pair, after alhr_append(pos).  The budget comes
 * from W and prefix (= S[pos]) when W != NULL, else fixed_budget.
 * Outputs are per pair: budget (nullable) int32 [batch, heads], idx int32
 * [batch, heads, max_budget], count int32 [batch, heads], O fp32 [batch,
 * heads, d]. */
alhr_status alhr_decode_step(const alhr_config *cfg, int32_t pos,
                             const int8_t *q_new, const int8_t *K,
                             const float *V, const int32_t *nodes,
                             const int32_t *prefix, const int8_t *W,
                             int32_t fixed_budget, int32_t *budget,
                             int32_t *idx, int32_t *count, float *O,
                             void *stream);

/* Append and decode step in one launch: alhr_append(pos, k_new, v_new)
 * followed by alhr_decode_step(pos, q_new), with the same arguments, layouts,
 * results and error codes (prefix is required).  Each (batch, head) pair's
 * workgroup appends its own key and value rows while it predicts and routes:
 * the route reads only subtrees of [0, pos + 1 - n) and the key rows below
 * pos (the new key itself from k_new), none of which the append changes, and
 * the predictor forms the new running sum itself; so no pair waits for another, and this saves the
 * second launch of every token step (openai-hub article
 * "ALHR把注意力变成树搜索", section "ALHR是什么": one new token per step). */
alhr_status alhr_append_decode(const alhr_config *cfg, int32_t pos,
                               const int8_t *k_new, const float *v_new,
                               const int8_t *q_new, int8_t *K, float *V,
                               int32_t *nodes, int32_t *prefix, const int8_t *W,
                               int32_t fixed_budget, int32_t *budget,
                               int32_t *idx, int32_t *count, float *O,
                               void *stream);

/* Dense causal softmax attention over every past key, the baseline the
 * README's result tables compare against (dense teacher rows) and the
 * optimised dense kernel the openai-hub article asks comparisons to use:
 * O[t] = sum_{j <= t} softmax_j(scale * Q[t] . K[j]) V[j], fp32 output.
 * Scores are exact int32; the P.V product is formed from bf16 heads and
 * tails of P and V (three matrix-core products, fp32 accumulation), so each
 * output is within 3 * 2^-18 * max|V| of the fp32 result.
 * Uses batch, heads, T, d and scale of cfg (d = 32, 64, 128 or 256; other
 * built sizes, and batch * heads * T >= 2^31, return ALHR_ERR_UNSUPPORTED);
 * the routing fields are checked as for the other calls but not used. */
alhr_status alhr_dense_attend(const alhr_config *cfg, const int8_t *Q,
                              const int8_t *K, const float *V, float *O,
                              void *stream);

/* Query/key splitter: the step before the tree that turns the layer input
 * into queries and keys (README "Inference stage", first paragraph; the
 * splitter is one of the two trained functions, README "Training stage").
 * The pages give no formula; the function computed is, for every token
 * m = b*T + t and output feature o < 2*heads*d,
 *   acc = sum_i X[m][i] * W[o][i]                 (exact int32)
 *   v   = clamp(floor((acc + half) / 2^shift), -c, c)
 * with half = 2^(shift-1) (0 when shift = 0), i.e. round half up, and
 * c = qclamp for o < heads*d, kclamp otherwise.  Feature o = h*d + j is
 * written to Q[b][h][t][j]; feature heads*d + h*d + j to K[b][h][t][j].
 *   X  int8 [batch, T, d_model]         input rows
 *   W  int8 [2 * heads * d, d_model]    weight rows, queries then keys
 *   Q, K int8 [batch, heads, T, d]      outputs (the layout of the tree path)
 * Checks: batch, heads >= 1; 1 <= T <= 2^20; d in {16, 32, 64, 128, 256};
 * d_model a multiple of 16 in [16, 16384] (so |acc| < 2^31 for any int8
 * input); 0 <= shift <= 30; 1 <= qclamp, kclamp <= 127; batch * T *
 * max(d_model, heads * d) < 2^31; pointers non-NULL and 16-byte aligned.
 * The outputs satisfy |Q| <= qclamp and |K| <= kclamp, the bounds to declare
 * as qmax / kmax in the alhr_config of the tree path. */
typedef struct alhr_split_config {
    int32_t batch;
    int32_t heads;
    int32_t T;
    int32_t d;          /* head dimension of Q and K                          */
    int32_t d_model;    /* input row length                                   */
    int32_t shift;      /* requantisation right shift                         */
    int32_t qclamp;     /* |Q| <= qclamp                                      */
    int32_t kclamp;     /* |K| <= kclamp                                      */
} alhr_split_config;

alhr_status alhr_split_qk(const alhr_split_config *cfg, const int8_t *X,
                          const int8_t *W, int8_t *Q, int8_t *K, void *stream);

/* Static text for a status code. */
const char *alhr_status_string(alhr_status status);

/* Thread-local detail of the last non-OK status on this thread ("" if none). */
const char *alhr_last_error(void);

/* Library ABI version (major * 100 + minor). */
int32_t alhr_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ALHR_H */
