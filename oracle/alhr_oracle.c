/*
 * ALHR tree-attention oracle: a plain, slow, single-threaded CPU version of
 * what the inference path computes, written for reading, not for speed.
 *
 * TEST INFRASTRUCTURE ONLY.  It is loaded by the test suite, by the smoke
 * check and by the benchmark's CPU-baseline leg, and by nothing else.  It
 * shares no code, header, table or helper with the GPU library.
 *
 * Sources.  "README" below is the ALHR project page (Adaptive learnable
 * Hierarchical routing: sub-quadratic tree attention ... (beta)); "news" is
 * the openai-hub article "ALHR把注意力变成树搜索".
 *   - tree of key sums, fixed binary topology: README opening paragraph and
 *     "Inference stage" (tree built once per layer over the key matrix);
 *     news, section "ALHR是什么" (topology fixed, path per query).
 *   - budget predictor on (query, global key sum) giving a leaf group:
 *     README "Inference stage"; caps of 96 keys and 32 classes: README
 *     "Results and Variables".
 *   - probe of the query's own key and its neighbours, then descent along
 *     the more similar branches, as many as keys are still missing:
 *     README "Inference stage".
 *   - causality by treating the branches that hold only past keys as the
 *     whole tree: README "Training stage" (last paragraph).
 *   - plain dot-product softmax attention over the keys found:
 *     README "Inference stage".
 *   - decode, one token at a time: news, section "ALHR是什么".
 *   - the query/key splitter that turns the layer input into queries and
 *     keys before the tree is built, one of the two trained functions:
 *     README "Inference stage" (first paragraph) and "Training stage"
 *     (last paragraph).
 *
 * Readings where the pages leave a step open (each listed with its reason
 * in the design notes): positional leaves; node value = raw sum; branch
 * similarity = q . node_sum; the predictor's global sum is the inclusive
 * causal prefix; predictor = bias-free linear map of [q; S_t] with argmax
 * ties to the lowest class, budget = keys_per_class * (class + 1) capped;
 * neighbours = the window t, t-1, ... taken unconditionally; the descent
 * covers [0, t+1-n) with maximal complete subtrees and runs a beam of width
 * r = C - n in which every internal node expands each round and leaves stay
 * and compete; order = score descending, then start position ascending;
 * the splitter = two bias-free linear maps of each token's input row (one
 * for the queries, one for the keys, heads side by side), requantised to
 * int8 by a rounding right shift and a symmetric clamp.
 *
 * Arithmetic.  Every integer quantity (node sums, prefix sums, scores,
 * predictor logits) is an exact int64.  An attention logit is the fp32
 * product of the score (exact in fp32) and the fp32 scale; the softmax and
 * the weighted sum are computed in fp64 and rounded to fp32 once at the end.
 *
 * Layout of the tree table (per (batch, head) pair, T = 2^L positions):
 * node (level l, index p) covers keys [p*2^l, (p+1)*2^l); for l >= 1 it is
 * row (T >> l) + p of an int64 [T][d] table whose row 0 is unused; level-0
 * nodes are the key rows themselves.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>

#define REF_OK 0
#define REF_ERR_ARG (-1)
#define REF_ERR_NOMEM (-2)

typedef struct {
    int64_t cover_internal;   /* cover roots that are tree nodes (level >= 1) */
    int64_t cover_leaf;       /* cover roots that are single keys (level 0)   */
    int64_t child_internal;   /* expanded children at level >= 1              */
    int64_t child_leaf;       /* expanded children at level 0                 */
    int64_t rounds;           /* beam expansion rounds                         */
    int64_t neighbours;       /* n_t                                          */
    int64_t count;            /* C_t                                          */
    int64_t cover_by_level[24];   /* cover roots per level                    */
    int64_t child_by_level[24];   /* expanded children per level              */
} alhr_ref_route_stats;

static int is_pow2(int64_t x) { return x >= 2 && (x & (x - 1)) == 0; }

static int log2i(int64_t x)
{
    int l = 0;
    while ((1LL << l) < x) ++l;
    return l;
}

/* ---------------------------------------------------------------- O1 ---- */
/* Tree of key sums: node(l, p) = node(l-1, 2p) + node(l-1, 2p+1), built
 * bottom-up from the key rows (README, opening paragraph: every branch is
 * keyed by the sum of the key vectors under it). */
int alhr_ref_build_tree(int32_t T, int32_t d, const int8_t *K, int64_t *nodes)
{
    if (!is_pow2(T) || d < 1 || !K || !nodes) return REF_ERR_ARG;
    int L = log2i(T);
    memset(nodes, 0, sizeof(int64_t) * (size_t)d);          /* row 0 unused */
    for (int l = 1; l <= L; ++l) {
        int64_t count = (int64_t)T >> l;
        for (int64_t p = 0; p < count; ++p) {
            int64_t row = count + p;
            int64_t *out = nodes + row * d;
            for (int i = 0; i < d; ++i) {
                int64_t left, right;
                if (l == 1) {
                    left = K[(2 * p) * d + i];
                    right = K[(2 * p + 1) * d + i];
                } else {
                    left = nodes[(2 * row) * d + i];
                    right = nodes[(2 * row + 1) * d + i];
                }
                out[i] = left + right;
            }
        }
    }
    return REF_OK;
}

/* ---------------------------------------------------------------- O2 ---- */
/* Inclusive causal prefix of the keys, S[t] = sum_{j <= t} K[j]: the
 * predictor's "global sum" read causally (README "Inference stage" with the
 * causality rule of "Training stage"). */
int alhr_ref_prefix(int32_t T, int32_t d, const int8_t *K, int64_t *S)
{
    if (T < 1 || d < 1 || !K || !S) return REF_ERR_ARG;
    for (int i = 0; i < d; ++i) S[i] = K[i];
    for (int64_t t = 1; t < T; ++t)
        for (int i = 0; i < d; ++i)
            S[t * d + i] = S[(t - 1) * d + i] + K[t * d + i];
    return REF_OK;
}

/* ---------------------------------------------------------------- O3 ---- */
/* Budget predictor: z_c = W[c][0:d] . q + W[c][d:2d] . S_t; the class is the
 * first argmax; the leaf group asks for keys_per_class * (class + 1) keys,
 * capped at max_budget (README "Inference stage"; caps in "Results and
 * Variables").  Returns the budget, or a negative code. */
int32_t alhr_ref_budget(int32_t d, const int8_t *q, const int64_t *s,
                        const int8_t *W, int32_t n_classes,
                        int32_t keys_per_class, int32_t max_budget,
                        int64_t *logits)
{
    if (d < 1 || !q || !s || !W || n_classes < 1 || keys_per_class < 1 || max_budget < 1)
        return REF_ERR_ARG;
    int32_t best = 0;
    int64_t best_z = 0;
    for (int32_t c = 0; c < n_classes; ++c) {
        const int8_t *w = W + (int64_t)c * 2 * d;
        int64_t z = 0;
        for (int i = 0; i < d; ++i) z += (int64_t)w[i] * q[i];
        for (int i = 0; i < d; ++i) z += (int64_t)w[d + i] * s[i];
        if (logits) logits[c] = z;
        if (c == 0 || z > best_z) { best = c; best_z = z; }
    }
    int64_t b = (int64_t)keys_per_class * (best + 1);
    return (int32_t)(b < max_budget ? b : max_budget);
}

/* ---------------------------------------------------------- O4 .. O8 ---- */
typedef struct {
    int64_t score;
    int32_t level;
    int64_t start;   /* first key position the node covers */
} ref_node;

/* The total order of the descent: higher score first, then lower start.
 * Candidates are disjoint, so starts are distinct and the order is total. */
static int node_before(const void *pa, const void *pb)
{
    const ref_node *a = (const ref_node *)pa, *b = (const ref_node *)pb;
    if (a->score != b->score) return a->score > b->score ? -1 : 1;
    if (a->start != b->start) return a->start < b->start ? -1 : 1;
    return 0;
}

static int64_t dot_q_key(int32_t d, const int8_t *q, const int8_t *k)
{
    int64_t s = 0;
    for (int i = 0; i < d; ++i) s += (int64_t)q[i] * k[i];
    return s;
}

/* sigma(x) = q . N(x) for node (level, start) */
static int64_t score_node(int32_t T, int32_t d, const int8_t *q, const int8_t *K,
                          const int64_t *nodes, int32_t level, int64_t start)
{
    if (level == 0) return dot_q_key(d, q, K + start * d);
    int64_t row = ((int64_t)T >> level) + (start >> level);
    const int64_t *n = nodes + row * d;
    int64_t s = 0;
    for (int i = 0; i < d; ++i) s += (int64_t)q[i] * n[i];
    return s;
}

typedef struct { int64_t pos; int64_t score; } ref_pick;

static int pick_by_pos(const void *pa, const void *pb)
{
    const ref_pick *a = (const ref_pick *)pa, *b = (const ref_pick *)pb;
    return (a->pos > b->pos) - (a->pos < b->pos);
}

/* Route query t with budget B_t.  Writes the selected key positions to
 * idx[0..C) in ascending order and -1 to idx[C..cap); score (nullable) gets
 * q . K[j] for each selected j (0 in padding).  Returns C_t >= 1, or a
 * negative code. */
int32_t alhr_ref_route(int32_t T, int32_t d, int32_t window, int32_t t,
                       int32_t budget, const int8_t *q, const int8_t *K,
                       const int64_t *nodes, int32_t cap, int32_t *idx,
                       int64_t *score, alhr_ref_route_stats *st)
{
    if (!is_pow2(T) || d < 1 || window < 1 || t < 0 || t >= T || budget < 1 ||
        !q || !K || !nodes || !idx || cap < 1)
        return REF_ERR_ARG;
    int L = log2i(T);

    /* O4: the number of keys and the neighbour window */
    int64_t C = budget < (int64_t)t + 1 ? budget : (int64_t)t + 1;
    int64_t n = window < C ? window : C;
    if (cap < C) return REF_ERR_ARG;
    int64_t r = C - n;
    int64_t m = (int64_t)t + 1 - n;          /* descent domain [0, m) */

    ref_pick *picked = (ref_pick *)malloc(sizeof(ref_pick) * (size_t)C);
    if (!picked) return REF_ERR_NOMEM;
    int64_t npicked = 0;
    for (int64_t j = t - n + 1; j <= t; ++j) {
        picked[npicked].pos = j;
        picked[npicked].score = dot_q_key(d, q, K + j * d);
        ++npicked;
    }
    if (st) {
        memset(st, 0, sizeof(*st));
        st->neighbours = n;
        st->count = C;
    }

    if (r > 0) {
        /* O6: cover [0, m) with maximal complete subtrees, largest first */
        ref_node *beam = (ref_node *)malloc(sizeof(ref_node) * (size_t)(2 * r + L + 2));
        ref_node *cand = (ref_node *)malloc(sizeof(ref_node) * (size_t)(2 * r + L + 2));
        if (!beam || !cand) { free(beam); free(cand); free(picked); return REF_ERR_NOMEM; }
        int64_t nb = 0, a = 0;
        for (int l = L; l >= 0; --l) {
            if ((m >> l) & 1) {
                beam[nb].level = l;
                beam[nb].start = a;
                beam[nb].score = score_node(T, d, q, K, nodes, l, a);
                if (st) {
                    if (l > 0) st->cover_internal++; else st->cover_leaf++;
                    st->cover_by_level[l]++;
                }
                ++nb;
                a += (int64_t)1 << l;
            }
        }
        /* O7: the beam keeps the best min(r, |candidates|) nodes */
        qsort(beam, (size_t)nb, sizeof(ref_node), node_before);
        if (nb > r) nb = r;
        for (;;) {
            int any_internal = 0;
            for (int64_t i = 0; i < nb; ++i) any_internal |= beam[i].level > 0;
            if (!any_internal) break;
            int64_t nc = 0;
            for (int64_t i = 0; i < nb; ++i) {
                if (beam[i].level == 0) {
                    cand[nc++] = beam[i];
                    continue;
                }
                int32_t cl = beam[i].level - 1;
                for (int side = 0; side < 2; ++side) {
                    int64_t cs = beam[i].start + (int64_t)side * ((int64_t)1 << cl);
                    cand[nc].level = cl;
                    cand[nc].start = cs;
                    cand[nc].score = score_node(T, d, q, K, nodes, cl, cs);
                    if (st) {
                        if (cl > 0) st->child_internal++; else st->child_leaf++;
                        st->child_by_level[cl]++;
                    }
                    ++nc;
                }
            }
            qsort(cand, (size_t)nc, sizeof(ref_node), node_before);
            nb = nc < r ? nc : r;
            memcpy(beam, cand, sizeof(ref_node) * (size_t)nb);
            if (st) st->rounds++;
        }
        /* R_t: the starts of the final (all-leaf) beam; |R_t| = r */
        for (int64_t i = 0; i < nb; ++i) {
            picked[npicked].pos = beam[i].start;
            picked[npicked].score = beam[i].score;
            ++npicked;
        }
        free(beam);
        free(cand);
    }
    if (npicked != C) { free(picked); return REF_ERR_ARG; }

    /* O8: ascending positions, -1 padding */
    qsort(picked, (size_t)npicked, sizeof(ref_pick), pick_by_pos);
    for (int64_t i = 0; i < cap; ++i) {
        idx[i] = i < C ? (int32_t)picked[i].pos : -1;
        if (score) score[i] = i < C ? picked[i].score : 0;
    }
    free(picked);
    return (int32_t)C;
}

/* ---------------------------------------------------------------- O9 ---- */
/* Softmax attention over the selected keys (README "Inference stage"):
 * the logit of key j is a_j = fl32(fl32(q . K[j]) * scale), i.e. the exact
 * integer score rounded to fp32 (exact while |q . K[j]| < 2^24, which the
 * int8 inputs guarantee for d <= 256) times the fp32 scale, rounded to fp32;
 * then out = sum_j e^{a_j - max} V[j] / sum_j e^{a_j - max} in fp64, rounded
 * to fp32 once.  `scale` must be an fp32 value (it is converted exactly). */
int alhr_ref_attend(int32_t d, int32_t C, const int32_t *idx, const int8_t *q,
                    const int8_t *K, const float *V, double scale, float *out)
{
    if (d < 1 || C < 1 || !idx || !q || !K || !V || !out) return REF_ERR_ARG;
    const float scale32 = (float)scale;
    if ((double)scale32 != scale) return REF_ERR_ARG;
    double *a = (double *)malloc(sizeof(double) * (size_t)C);
    double *acc = (double *)calloc((size_t)d, sizeof(double));
    if (!a || !acc) { free(a); free(acc); return REF_ERR_NOMEM; }
    double mx = -INFINITY;
    for (int32_t j = 0; j < C; ++j) {
        const float s32 = (float)dot_q_key(d, q, K + (int64_t)idx[j] * d);
        const float a32 = s32 * scale32;
        a[j] = (double)a32;
        if (a[j] > mx) mx = a[j];
    }
    double z = 0.0;
    for (int32_t j = 0; j < C; ++j) {
        double w = exp(a[j] - mx);
        z += w;
        const float *v = V + (int64_t)idx[j] * d;
        for (int i = 0; i < d; ++i) acc[i] += w * (double)v[i];
    }
    for (int i = 0; i < d; ++i) out[i] = (float)(acc[i] / z);
    free(a);
    free(acc);
    return REF_OK;
}

/* ------------------------------------------------------ one (b, h) pair -- */
/* Build + prefix + (budget) + route + attend for the queries ts[0..nt) of one
 * pair (all T queries when ts is NULL, then nt must be T).  W == NULL selects
 * the fixed budget.  Outputs are indexed by the position in ts. */
int alhr_ref_pair_forward(int32_t T, int32_t d, int32_t window,
                          int32_t n_classes, int32_t keys_per_class,
                          int32_t max_budget, double scale,
                          const int8_t *Q, const int8_t *K, const float *V,
                          const int8_t *W, int32_t fixed_budget,
                          const int32_t *ts, int32_t nt,
                          int64_t *nodes, int64_t *S,
                          int32_t *budget, int32_t cap, int32_t *idx,
                          int32_t *count, float *O,
                          alhr_ref_route_stats *stats)
{
    if (!ts && nt != T) return REF_ERR_ARG;
    int rc = alhr_ref_build_tree(T, d, K, nodes);
    if (rc) return rc;
    if (W) {
        rc = alhr_ref_prefix(T, d, K, S);
        if (rc) return rc;
    }
    for (int32_t k = 0; k < nt; ++k) {
        int32_t t = ts ? ts[k] : k;
        if (t < 0 || t >= T) return REF_ERR_ARG;
        const int8_t *q = Q + (int64_t)t * d;
        int32_t b = W ? alhr_ref_budget(d, q, S + (int64_t)t * d, W, n_classes,
                                        keys_per_class, max_budget, NULL)
                      : fixed_budget;
        if (b < 1) return REF_ERR_ARG;
        if (budget) budget[k] = b;
        int32_t *row = idx + (int64_t)k * cap;
        int32_t c = alhr_ref_route(T, d, window, t, b, q, K, nodes, cap, row, NULL,
                                   stats ? stats + k : NULL);
        if (c < 1) return c < 0 ? c : REF_ERR_ARG;
        if (count) count[k] = c;
        rc = alhr_ref_attend(d, c, row, q, K, V, scale, O + (int64_t)k * d);
        if (rc) return rc;
    }
    return REF_OK;
}

/* --------------------------------------------------------------- O10 ---- */
/* Decode append at position p: store the key and value rows, add the key to
 * each ancestor sum, and advance the prefix from S[p-1] to S[p].  Requires
 * that rows >= p hold zeros (the table is O1 of the zero-padded keys). */
int alhr_ref_append(int32_t T, int32_t d, int32_t p, const int8_t *k_new,
                    const float *v_new, int8_t *K, float *V, int64_t *nodes,
                    int64_t *prefix)
{
    if (!is_pow2(T) || d < 1 || p < 0 || p >= T || !k_new || !K || !nodes) return REF_ERR_ARG;
    int L = log2i(T);
    memcpy(K + (int64_t)p * d, k_new, (size_t)d);
    if (V && v_new) memcpy(V + (int64_t)p * d, v_new, sizeof(float) * (size_t)d);
    for (int l = 1; l <= L; ++l) {
        int64_t row = ((int64_t)T >> l) + ((int64_t)p >> l);
        for (int i = 0; i < d; ++i) nodes[row * d + i] += k_new[i];
    }
    if (prefix)
        for (int i = 0; i < d; ++i) prefix[i] += k_new[i];
    return REF_OK;
}

/* Budgets of every query of one pair: O2 then O3 for t = 0..T-1. */
int alhr_ref_pair_budgets(int32_t T, int32_t d, const int8_t *Q, const int8_t *K,
                          const int8_t *W, int32_t n_classes, int32_t keys_per_class,
                          int32_t max_budget, int64_t *S, int32_t *budget)
{
    int rc = alhr_ref_prefix(T, d, K, S);
    if (rc) return rc;
    for (int64_t t = 0; t < T; ++t) {
        int32_t b = alhr_ref_budget(d, Q + t * d, S + t * d, W, n_classes, keys_per_class,
                                    max_budget, NULL);
        if (b < 1) return REF_ERR_ARG;
        budget[t] = b;
    }
    return REF_OK;
}

/* ---------------------------------------------------------------------
 * Query/key splitter (README "Inference stage": the layer input is split
 * into queries and keys, then the tree is built over the keys; "Training
 * stage": the splitter is trained with the budget predictor).  The pages
 * give no formula; the reading here is the usual per-token projection:
 *   acc_o(b, t) = sum_i X[b][t][i] * W[o][i]            (exact int64)
 * for output feature o < 2*heads*d, where rows o = h*d + j of W give query
 * feature j of head h and rows heads*d + h*d + j give key feature j of head
 * h.  Each accumulator is requantised to int8 by
 *   requant(acc) = clamp(floor((acc + half) / 2^shift), -c, c),
 *   half = 2^(shift-1) for shift >= 1, 0 for shift = 0,
 * i.e. round half up, with c = qclamp for queries and kclamp for keys.
 * X is int8 [batch][T][d_model]; W int8 [2*heads*d][d_model]; Q and K are
 * written as int8 [batch][heads][T][d].
 * --------------------------------------------------------------------- */
static int64_t floor_div_pow2(int64_t a, int shift)
{
    const int64_t m = (int64_t)1 << shift;
    int64_t q = a / m;                   /* truncates toward zero */
    if (a % m != 0 && a < 0) q -= 1;     /* step down to the floor */
    return q;
}

int64_t alhr_ref_requant(int64_t acc, int32_t shift, int32_t clamp)
{
    const int64_t half = shift >= 1 ? ((int64_t)1 << (shift - 1)) : 0;
    int64_t v = floor_div_pow2(acc + half, shift);
    if (v > clamp) v = clamp;
    if (v < -clamp) v = -clamp;
    return v;
}

int alhr_ref_split_qk(int32_t batch, int32_t heads, int32_t T, int32_t d,
                      int32_t d_model, int32_t shift, int32_t qclamp,
                      int32_t kclamp, const int8_t *X, const int8_t *W,
                      int8_t *Q, int8_t *K)
{
    if (batch < 1 || heads < 1 || T < 1 || d < 1 || d_model < 1 || shift < 0 ||
        shift > 30 || qclamp < 1 || qclamp > 127 || kclamp < 1 || kclamp > 127)
        return REF_ERR_ARG;
    const int64_t HD = (int64_t)heads * d;
    for (int64_t b = 0; b < batch; ++b)
        for (int64_t t = 0; t < T; ++t) {
            const int8_t *x = X + (b * T + t) * d_model;
            for (int64_t o = 0; o < 2 * HD; ++o) {
                const int8_t *w = W + o * d_model;
                int64_t acc = 0;
                for (int64_t i = 0; i < d_model; ++i) acc += (int64_t)x[i] * w[i];
                const int is_key = o >= HD;
                const int64_t f = is_key ? o - HD : o;   /* h*d + j */
                const int64_t h = f / d, j = f % d;
                const int64_t dst = ((b * heads + h) * T + t) * d + j;
                const int64_t v = alhr_ref_requant(acc, shift, is_key ? kclamp : qclamp);
                if (is_key) K[dst] = (int8_t)v; else Q[dst] = (int8_t)v;
            }
        }
    return REF_OK;
}
