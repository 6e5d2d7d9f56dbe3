// Routing and sparse attention, one wavefront per query (ALHR README,
// "Inference stage" and "Training stage"; decode use from the openai-hub
// article "ALHR把注意力变成树搜索", section "ALHR是什么").
//
// Per query t with budget B: C = min(B, t+1) keys, the n = min(w, C)
// neighbours t-n+1..t, and a beam of width r = C - n over the maximal
// complete subtrees covering [0, m), m = t+1-n.  Each round expands every
// internal beam node into its two children and keeps the r best candidates
// by (q . node_sum desc, first position asc); leaves stay in the beam and
// compete.  The loop ends when the beam holds only leaves.
//
// Mapping to gfx950:
//  * scoring: a tree row is split over d/16 lanes (16 columns each): an
//    int16 row (levels 1..l16) is two 16-byte loads and eight v_dot2 per
//    lane, an int32 row (the few top levels) four loads and sixteen 24-bit
//    multiplies, a key row one load and four v_dot4; DPP adds finish the row.
//    64 / (d/16) rows are scored per pass.
//  * only the left child of an expanded node is loaded: the right child's
//    score is the parent's minus the left's (exact in integers), which
//    halves the gathered tree bytes.  The children's keys are derived from
//    the parent's key, and the child's heap row is (T + start) >> level.
//  * selection: candidates are 64-bit keys (biased score | inverted start |
//    level), up to 4 per lane; the r-th best score is found by a bitwise
//    threshold search over wave ballot counts, written in scalar assembly
//    (ties at the threshold by a second search on the start), then a ballot
//    prefix compacts the winners in slot order, so the beam stays sorted by
//    position and the final picks need no sort.
//  * beam, candidates and the final picks live in a 4.5 KiB per-wave LDS
//    block.
//  * attention reuses the leaf scores as logits: fp32 softmax, then a gather
//    of the C value rows with d/4 lanes per row (16 B each), four rows per
//    lane group in flight.
#include "append.h"
#include "device.h"
#include "kernels.h"

namespace alhr {
namespace {

constexpr int kMaxBudget = 128;
constexpr int kSlots = 256;             // 2 * (kMaxBudget - 1) candidates fit
// Waves (queries) per workgroup of the prefill routing and attention kernels.
// A build option only so that the same queries can be run at other launch
// geometries (the results must not depend on it); 4 is the product setting.
#ifndef ALHR_ROUTE_WAVES_PER_BLOCK
#define ALHR_ROUTE_WAVES_PER_BLOCK 4
#endif
constexpr int kWavesPerBlock = ALHR_ROUTE_WAVES_PER_BLOCK;
static_assert(kWavesPerBlock == 1 || kWavesPerBlock == 2 || kWavesPerBlock == 4 ||
                  kWavesPerBlock == 8,
              "1, 2, 4 or 8 waves per workgroup");
constexpr int kThreads = kWavesPerBlock * kWave;
constexpr int kMaxClasses = 32;

struct WaveLds {
    uint64_t beam[kMaxBudget];
    uint64_t cand[kSlots];
    int32_t pos[kMaxBudget];
    int32_t score[kMaxBudget];
    float w[kMaxBudget];
};

// ---- candidate keys: larger key = better node ----------------------------
__device__ __forceinline__ uint64_t make_key(int score, int start, int level)
{
    const uint32_t hi = (uint32_t)score ^ 0x80000000u;
    const uint32_t lo = ((uint32_t)(0xFFFFF - start) << 5) | (uint32_t)level;
    return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ int key_score(uint64_t k) { return (int)((uint32_t)(k >> 32) ^ 0x80000000u); }
__device__ __forceinline__ int key_start(uint64_t k) { return 0xFFFFF - (int)((uint32_t)k >> 5); }

// ---- the query in registers, in the two column layouts used for scoring ---
// Lane s of a row group (LPR = d / 16 lanes per row) holds the columns of the
// two 8-column chunks c = k * LPR + s (k < 2) as packed int16 pairs, and the
// 16 columns 16s .. 16s + 15 as packed int8 (for key rows).
template <int D>
struct QueryRegs {
    int qh[8];    // columns 8c + 2j, 8c + 2j + 1 of chunk c = k*LPR + s in qh[4k + j]
    int qp[4];    // key-row columns 16*s .. 16*s + 15, packed int8
};

template <int D>
__device__ __forceinline__ void load_query(const int8_t* __restrict__ q, int s, QueryRegs<D>& r)
{
    constexpr int LPR = D / 16;
    const int* qw = reinterpret_cast<const int*>(q);
    const int4 p = reinterpret_cast<const int4*>(q)[s];
    r.qp[0] = p.x;
    r.qp[1] = p.y;
    r.qp[2] = p.z;
    r.qp[3] = p.w;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int c = k * LPR + s;
        const int w0 = qw[2 * c], w1 = qw[2 * c + 1];
        r.qh[4 * k + 0] = (sbyte(w0, 0) & 0xFFFF) | (sbyte(w0, 1) << 16);
        r.qh[4 * k + 1] = (sbyte(w0, 2) & 0xFFFF) | (sbyte(w0, 3) << 16);
        r.qh[4 * k + 2] = (sbyte(w1, 0) & 0xFFFF) | (sbyte(w1, 1) << 16);
        r.qh[4 * k + 3] = (sbyte(w1, 2) & 0xFFFF) | (sbyte(w1, 3) << 16);
    }
}

__device__ __forceinline__ int lo16(int w) { return (int)(short)(w & 0xFFFF); }
__device__ __forceinline__ int hi16(int w) { return w >> 16; }

typedef short v2s __attribute__((ext_vector_type(2)));
__device__ __forceinline__ int dot2_i16(int a, int b, int acc)
{
    return __builtin_amdgcn_sdot2(__builtin_bit_cast(v2s, a), __builtin_bit_cast(v2s, b), acc, false);
}

template <bool MUL24>
__device__ __forceinline__ int imul(int a, int b)
{
    if constexpr (MUL24) return __mul24(a, b);
    else return a * b;
}

// q . node for node (level, start) of one pair; every lane of the row's
// group receives the full score.  Inactive lanes contribute 0.  Tree rows of
// levels 1..l16 are int16 (packed after the int32 rows, see tree_row16),
// higher levels int32, level 0 is the key row.
template <int D, bool MUL24>
__device__ __forceinline__ int score_node(const int32_t* __restrict__ nodes_pair,
                                          const int8_t* __restrict__ keys_pair, int T, int l16,
                                          int level, int start, bool active, int s,
                                          const QueryRegs<D>& q)
{
    constexpr int LPR = D / 16;
    // per-pair tables are under 2^30 bytes: 32-bit byte offsets from a
    // wave-uniform base (the scalar-base load form)
    gbyte* nbase = uniform_base(nodes_pair);
    gbyte* kbase = uniform_base(keys_pair);
    const uint32_t b16 = (uint32_t)T >> l16;
    int acc = 0;
    if (active) {
        const uint32_t r = ((uint32_t)T >> level) + ((uint32_t)start >> level);   // heap row
        if (level > l16) {
            // int32 row (block-interleaved, see wide_slot): block j = 2k + h
            // holds at slot s the columns 8c + 4h .. 8c + 4h + 3 of chunk
            // c = k * LPR + s, i.e. the query pairs qh[2j], qh[2j + 1].  The
            // pairs are unpacked here (these are the few top levels).
            const uint32_t row = r * (uint32_t)(4 * D);
            int4 v[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) v[j] = load16(nbase, row + 16u * (uint32_t)(j * LPR + s));
            // an opaque copy keeps the unpacking here instead of letting it
            // be hoisted out of the descent loop into 16 live registers
            int qh[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                qh[j] = q.qh[j];
                asm volatile("" : "+v"(qh[j]));
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                acc += imul<MUL24>(lo16(qh[2 * j]), v[j].x);
                acc += imul<MUL24>(hi16(qh[2 * j]), v[j].y);
                acc += imul<MUL24>(lo16(qh[2 * j + 1]), v[j].z);
                acc += imul<MUL24>(hi16(qh[2 * j + 1]), v[j].w);
            }
        } else if (level > 0) {
            // int16 row (the layout of tree_row16): chunk c is 16-byte slot c
            const uint32_t row = b16 * (uint32_t)(4 * D) + (r - b16) * (uint32_t)(2 * D);
            int4 v[2];
#pragma unroll
            for (int k = 0; k < 2; ++k) v[k] = load16(nbase, row + 16u * (uint32_t)(k * LPR + s));
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                acc = dot2_i16(q.qh[4 * k + 0], v[k].x, acc);
                acc = dot2_i16(q.qh[4 * k + 1], v[k].y, acc);
                acc = dot2_i16(q.qh[4 * k + 2], v[k].z, acc);
                acc = dot2_i16(q.qh[4 * k + 3], v[k].w, acc);
            }
        } else {
            const int4 v = load16(kbase, (uint32_t)start * (uint32_t)D + 16u * (uint32_t)s);
            acc = dot4_i8(q.qp[0], v.x, acc);
            acc = dot4_i8(q.qp[1], v.y, acc);
            acc = dot4_i8(q.qp[2], v.z, acc);
            acc = dot4_i8(q.qp[3], v.w, acc);
        }
    }
    return group_sum<LPR>(acc);
}

// Left-child scoring inside the descent, from ts = T + start: the child's
// heap row is r = ts >> level (exact: start is a multiple of 2^level).  The
// lane-dependent parts of the byte offsets are computed
// once per query: o16 = 2d * (T >> l16) + 16 s (an int16 row r starts at
// 2d * (r + (T >> l16)) in the packed layout), okey = 16 s - T d (key row
// r - T starts at d * (r - T); the sum wraps modulo 2^32 to the exact
// offset).  A row group is active or inactive as a whole and an inactive
// group's sum is never used, so its lanes return whatever they hold.
// The int16 rows (the common case) are tested first.  The first product of
// each chain is written with saturation, which keeps it in the three-operand
// form (no separate clear of the accumulator); no partial sum can saturate,
// since every |q . node| is below 2^31 by the host's overflow check.
__device__ __forceinline__ int dot2_i16_first(int a, int b)
{
    return __builtin_amdgcn_sdot2(__builtin_bit_cast(v2s, a), __builtin_bit_cast(v2s, b), 0, true);
}
__device__ __forceinline__ int dot4_i8_first(int a, int b)
{
    return __builtin_amdgcn_sdot4(a, b, 0, true);
}
template <int D, bool MUL24>
__device__ __forceinline__ int score_row(gbyte* nbase, gbyte* nbase_hi, gbyte* kbase, uint32_t ts,
                                         int level, int l16, bool active, int s, uint32_t o16,
                                         uint32_t okey, const QueryRegs<D>& q)
{
    constexpr int LPR = D / 16;
    int acc = (int)ts;   // any value: see above
    if (active) {
        // ts = T + start; the heap row is ts >> level (level < 31 when active)
        __builtin_assume(level >= 0 && level < 31);
        const uint32_t r = ts >> (uint32_t)level;
        if ((uint32_t)(level - 1) < (uint32_t)l16) {
            const uint32_t off = r * (uint32_t)(2 * D) + o16;
            const int4 v0 = load16(nbase, off), v1 = load16(nbase_hi, off);
            acc = dot2_i16_first(q.qh[0], v0.x);
            acc = dot2_i16(q.qh[1], v0.y, acc);
            acc = dot2_i16(q.qh[2], v0.z, acc);
            acc = dot2_i16(q.qh[3], v0.w, acc);
            acc = dot2_i16(q.qh[4], v1.x, acc);
            acc = dot2_i16(q.qh[5], v1.y, acc);
            acc = dot2_i16(q.qh[6], v1.z, acc);
            acc = dot2_i16(q.qh[7], v1.w, acc);
        } else if (level == 0) {
            const int4 v = load16(kbase, r * (uint32_t)D + okey);
            acc = dot4_i8_first(q.qp[0], v.x);
            acc = dot4_i8(q.qp[1], v.y, acc);
            acc = dot4_i8(q.qp[2], v.z, acc);
            acc = dot4_i8(q.qp[3], v.w, acc);
        } else {
            const uint32_t row = r * (uint32_t)(4 * D);
            int4 v[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) v[j] = load16(nbase, row + 16u * (uint32_t)(j * LPR + s));
            int qh[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                qh[j] = q.qh[j];
                asm volatile("" : "+v"(qh[j]));
            }
            acc = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                acc += imul<MUL24>(lo16(qh[2 * j]), v[j].x);
                acc += imul<MUL24>(hi16(qh[2 * j]), v[j].y);
                acc += imul<MUL24>(lo16(qh[2 * j + 1]), v[j].z);
                acc += imul<MUL24>(hi16(qh[2 * j + 1]), v[j].w);
            }
        }
    }
    return group_sum<LPR>(acc);
}

// A threshold x in [0, span] that selects the `need` largest values rel over
// the wave (NS values per lane; zeros never count for x >= 1): bits are
// decided from the most significant down, x | bit being kept when at least
// `need` values reach it.  The search stops early once exactly `need` values
// reach x, since {rel >= x} is then the answer; otherwise it ends at the
// largest x with at least `need` values >= x (ties at x are the caller's).
// x = 0 is returned when no x >= 1 qualifies.  Wave-uniform.
//
// The loop is written out in scalar code: per bit one s_or, NS compares
// (v_cmp into SGPR pairs), NS population counts, a compare-select and the two
// exits, about half the scalar instructions the compiler makes of it.  All
// lanes must be active (every caller runs with a full wave).
#define ALHR_BS_HEAD "1:\n s_or_b32 %[c], %[x], %[bit]\n"
#define ALHR_BS_CMP(J) "v_cmp_le_u32_e64 %[m" #J "], %[c], %[r" #J "]\n"
#define ALHR_BS_CNT(J) "s_bcnt1_i32_b64 %[t" #J "], %[m" #J "]\n"
#define ALHR_BS_TAIL(T)                                                                 \
    "s_cmp_ge_i32 " T ", %[need]\n s_cselect_b32 %[x], %[c], %[x]\n"                    \
    "s_cmp_eq_u32 " T ", %[need]\n s_cbranch_scc1 2f\n"                                 \
    "s_lshr_b32 %[bit], %[bit], 1\n s_cbranch_scc1 1b\n 2:\n"
template <int NS>
__device__ __forceinline__ uint32_t bit_search(const uint32_t (&rel)[NS], uint32_t span, int need)
{
    static_assert(NS >= 1 && NS <= 4, "slots per lane");
    uint32_t x = 0u;
    if (span == 0u) return x;
    uint32_t bit = 0x80000000u >> __builtin_clz(span);
    uint32_t c, t0, t1, t2, t3;
    uint64_t m0, m1, m2, m3;
    if constexpr (NS == 1) {
        asm volatile(ALHR_BS_HEAD ALHR_BS_CMP(0) ALHR_BS_CNT(0) ALHR_BS_TAIL("%[t0]")
                     : [x] "+s"(x), [bit] "+s"(bit), [c] "=&s"(c), [t0] "=&s"(t0), [m0] "=&s"(m0)
                     : [r0] "v"(rel[0]), [need] "s"(need)
                     : "scc");
    } else if constexpr (NS == 2) {
        asm volatile(ALHR_BS_HEAD ALHR_BS_CMP(0) ALHR_BS_CMP(1) ALHR_BS_CNT(0) ALHR_BS_CNT(1)
                     "s_add_u32 %[t0], %[t0], %[t1]\n" ALHR_BS_TAIL("%[t0]")
                     : [x] "+s"(x), [bit] "+s"(bit), [c] "=&s"(c), [t0] "=&s"(t0),
                       [t1] "=&s"(t1), [m0] "=&s"(m0), [m1] "=&s"(m1)
                     : [r0] "v"(rel[0]), [r1] "v"(rel[1]), [need] "s"(need)
                     : "scc");
    } else if constexpr (NS == 3) {
        asm volatile(ALHR_BS_HEAD ALHR_BS_CMP(0) ALHR_BS_CMP(1) ALHR_BS_CMP(2) ALHR_BS_CNT(0)
                     ALHR_BS_CNT(1) ALHR_BS_CNT(2)
                     "s_add_u32 %[t0], %[t0], %[t1]\n s_add_u32 %[t0], %[t0], %[t2]\n"
                     ALHR_BS_TAIL("%[t0]")
                     : [x] "+s"(x), [bit] "+s"(bit), [c] "=&s"(c), [t0] "=&s"(t0),
                       [t1] "=&s"(t1), [t2] "=&s"(t2), [m0] "=&s"(m0), [m1] "=&s"(m1),
                       [m2] "=&s"(m2)
                     : [r0] "v"(rel[0]), [r1] "v"(rel[1]), [r2] "v"(rel[2]), [need] "s"(need)
                     : "scc");
    } else {
        asm volatile(ALHR_BS_HEAD ALHR_BS_CMP(0) ALHR_BS_CMP(1) ALHR_BS_CMP(2) ALHR_BS_CMP(3)
                     ALHR_BS_CNT(0) ALHR_BS_CNT(1) ALHR_BS_CNT(2) ALHR_BS_CNT(3)
                     "s_add_u32 %[t0], %[t0], %[t1]\n s_add_u32 %[t2], %[t2], %[t3]\n"
                     "s_add_u32 %[t0], %[t0], %[t2]\n" ALHR_BS_TAIL("%[t0]")
                     : [x] "+s"(x), [bit] "+s"(bit), [c] "=&s"(c), [t0] "=&s"(t0),
                       [t1] "=&s"(t1), [t2] "=&s"(t2), [t3] "=&s"(t3), [m0] "=&s"(m0),
                       [m1] "=&s"(m1), [m2] "=&s"(m2), [m3] "=&s"(m3)
                     : [r0] "v"(rel[0]), [r1] "v"(rel[1]), [r2] "v"(rel[2]), [r3] "v"(rel[3]),
                       [need] "s"(need)
                     : "scc");
    }
    return x;
}
#undef ALHR_BS_HEAD
#undef ALHR_BS_CMP
#undef ALHR_BS_CNT
#undef ALHR_BS_TAIL

// The kept keys k[j] (slot lane + 64 j) for which pick(high word, low word)
// holds, compacted into beam[0, ...) in slot order; returns their number and
// sets `inner` when one of them is internal.  Each caller passes its own
// predicate, evaluated here on an opaque copy of the key: a lane flag
// computed in an earlier block would be rebuilt through a vector register
// for the ballot.  All lanes are active.
template <int NS, typename Pick>
__device__ __forceinline__ int compact_kept(const uint64_t (&k)[NS], uint64_t* beam, bool& inner,
                                            Pick pick)
{
    int base = 0;
    uint64_t internal = 0ull;
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        uint64_t kk = k[j];
        asm("" : "+v"(kk));
        const uint32_t hi = (uint32_t)(kk >> 32), lo = (uint32_t)kk;
        const bool sel = pick(hi, lo);
        const uint64_t msk = __ballot(sel);
        if (sel) beam[base + (int)mbcnt(msk)] = kk;
        base += popc64(msk);
        uint64_t deep;   // lanes whose key has level > 0 (a 32-bit test on the low word)
        asm("v_cmp_ne_u32_e64 %0, 0, %1" : "=s"(deep) : "v"(lo & 31u));
        internal |= msk & deep;
    }
    inner = internal != 0ull;
    return base;
}

// Keep the best min(r, #non-empty) keys of cand[0, n) in beam[0, ...), in
// slot order, and return how many were kept; `inner` tells whether any kept
// node is internal.  NS slots per lane (n <= 64 * NS).  A slot is empty when
// its high word is 0: a real key's high word is its score with the sign bit
// flipped, and a score of -2^31 cannot occur (the host's overflow check keeps
// every |q . node| below 2^31), so the low word of an empty slot is free.
template <int NS>
__device__ int select_best_ns(const uint64_t* cand, int n, int r, uint64_t* beam, bool& inner)
{
    const int lane = lane_id();
    uint64_t k[NS];
    uint32_t h[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        // every slot index is below kSlots, so the read needs no guard;
        // slots past n are then cleared
        const int sl = lane + kWave * j;
        const uint64_t v = cand[sl];
        const uint32_t keep = (uint32_t)0 - (uint32_t)(sl < n);
        k[j] = ((uint64_t)((uint32_t)(v >> 32) & keep) << 32) | ((uint32_t)v & keep);
        h[j] = (uint32_t)(k[j] >> 32);
    }
    int nvalid = 0;
#pragma unroll
    for (int j = 0; j < NS; ++j) nvalid += wave_count(h[j] != 0u);
    if (nvalid <= r)
        return compact_kept<NS>(k, beam, inner, [](uint32_t hk, uint32_t) { return hk != 0u; });
    // empty slots read 0, below every real key: they drop out of the maximum,
    // and h - 1 wraps them to the top for the minimum
    uint32_t mx = 0u, mn1 = 0xFFFFFFFFu;
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        mx = h[j] > mx ? h[j] : mx;
        mn1 = h[j] - 1u < mn1 ? h[j] - 1u : mn1;
    }
    mx = uniform(wave_max_u32(mx));
    const uint32_t mn = uniform(wave_min_u32(mn1)) + 1u;
    // largest threshold with at least r scores >= it: a bitwise search, most
    // significant bit first, over the scores relative to the minimum (empty
    // slots read 0 and never reach a candidate threshold >= 1)
    uint32_t rel[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) rel[j] = (h[j] > mn ? h[j] : mn) - mn;
    const uint32_t lo = mn + bit_search<NS>(rel, mx - mn, r);
    // lo >= mn >= 1, so every test against lo below passes real keys only
    int gt = 0, eq = 0;
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        gt += wave_count(h[j] > lo);
        eq += wave_count(h[j] == lo);
    }
    const int need = r - gt;
    if (need == eq)
        return compact_kept<NS>(k, beam, inner, [lo](uint32_t hk, uint32_t) { return hk >= lo; });
    // ties at the threshold: keep the `need` lowest starts (largest low words)
    uint32_t l[NS];
    uint32_t lmx = 0u, lmn = 0xFFFFFFFFu;
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        l[j] = (uint32_t)k[j];
        if (h[j] == lo) {
            lmx = l[j] > lmx ? l[j] : lmx;
            lmn = l[j] < lmn ? l[j] : lmn;
        }
    }
    lmx = wave_max_u32(lmx);
    lmn = wave_min_u32(lmn);
    uint32_t lrel[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) lrel[j] = h[j] == lo ? l[j] - lmn : 0u;
    const uint32_t a = uniform(lmn) + bit_search<NS>(lrel, uniform(lmx) - uniform(lmn), need);
    return compact_kept<NS>(k, beam, inner, [lo, a](uint32_t hk, uint32_t lk) {
        return hk > lo || (hk == lo && lk >= a);
    });
}

__device__ __forceinline__ int select_best(const uint64_t* cand, int n, int r, uint64_t* beam,
                                           bool& inner)
{
    if (n <= kWave) return select_best_ns<1>(cand, n, r, beam, inner);
    if (n <= 2 * kWave) return select_best_ns<2>(cand, n, r, beam, inner);
    if (n <= 3 * kWave) return select_best_ns<3>(cand, n, r, beam, inner);
    return select_best_ns<4>(cand, n, r, beam, inner);
}

struct RouteCounts {
    int tree_rows;     // int32 tree rows loaded
    int tree16_rows;   // int16 tree rows loaded
    int key_rows;      // key rows loaded by the descent
};

// Route query t of one pair.  On return sm.pos[0, C) holds the selected
// positions in ascending order and sm.score[0, C) their q . K scores.
template <int D, bool MUL24, bool STATS>
__device__ int route_query(const int32_t* __restrict__ nodes_pair,
                           const int8_t* __restrict__ keys_pair, int T, int L, int l16, int t,
                           int B, int window, const QueryRegs<D>& q, WaveLds& sm,
                           RouteCounts& cnt)
{
    constexpr int LPR = D / 16, RPG = kWave / LPR;
    const int lane = lane_id();
    const int s = lane % LPR, g = lane / LPR;
    const int C = uniform(B < t + 1 ? B : t + 1);
    const int n = uniform(window < C ? window : C);
    const int r = C - n;
    const int m = t + 1 - n;

    // neighbours m..t go to slots r.. (they follow every routed key, which is
    // < m).  Up to RPG of them (the usual window) are loaded first, with no
    // branch (inactive lanes read key row t), and scored after the cover's
    // rows are requested, so the two loads overlap.
    int4 nv = make_int4(0, 0, 0, 0);
    const bool near_one_pass = n <= RPG;
    if (near_one_pass)
        nv = load16(uniform_base(keys_pair),
                    (uint32_t)(g < n ? m + g : t) * (uint32_t)D + 16u * (uint32_t)s);
    auto finish_neighbours = [&]() {
        if (near_one_pass) {
            int acc = dot4_i8(q.qp[0], nv.x, 0);
            acc = dot4_i8(q.qp[1], nv.y, acc);
            acc = dot4_i8(q.qp[2], nv.z, acc);
            acc = dot4_i8(q.qp[3], nv.w, acc);
            const int sc = group_sum<LPR>(acc);
            if (g < n && s == 0) {
                sm.pos[r + g] = m + g;
                sm.score[r + g] = sc;
            }
            return;
        }
        for (int base = 0; base < n; base += RPG) {
            const int k = base + g;
            const bool act = k < n;
            const int sc = score_node<D, MUL24>(nodes_pair, keys_pair, T, l16, 0, m + k, act, s, q);
            if (act && s == 0) {
                sm.pos[r + k] = m + k;
                sm.score[r + k] = sc;
            }
        }
    };
    if (r == 0) {
        finish_neighbours();
        wave_sync();
        return C;
    }

    // cover of [0, m): bit b of m set -> node (b, start = m with bits <= b
    // cleared).  Slot L-1-b puts the cover in ascending start order; children
    // of beam entry i go to slots 2i and 2i+1 and the selection compacts in
    // slot order, so the beam stays sorted by start in every round.
    for (int base = 0; base < L; base += RPG) {
        const int b = base + g;
        const bool act = b < L && ((m >> b) & 1);
        const int start = act ? (m & ~((2 << b) - 1)) : 0;
        const int sc = score_node<D, MUL24>(nodes_pair, keys_pair, T, l16, b, start, act, s, q);
        if (STATS) {
            cnt.tree_rows += wave_count(act && s == 0 && b > l16);
            cnt.tree16_rows += wave_count(act && s == 0 && b > 0 && b <= l16);
            cnt.key_rows += wave_count(act && s == 0 && b == 0);
        }
        if (b < L && s == 0) sm.cand[L - 1 - b] = act ? make_key(sc, start, b) : 0ull;
    }
    finish_neighbours();
    wave_sync();
    bool inner;
    int nb = select_best(sm.cand, L, r, sm.beam, inner);
    wave_sync();

    // the descent's loop invariants (see score_row)
    gbyte* nbase = uniform_base(nodes_pair);
    gbyte* nbase_hi = nbase + 16 * LPR;   // second 16-byte chunk of an int16 row
    gbyte* kbase = uniform_base(keys_pair);
    const uint32_t o16 = (uint32_t)(2 * D) * ((uint32_t)T >> l16) + 16u * (uint32_t)s;
    const uint32_t okey = 16u * (uint32_t)s - (uint32_t)T * (uint32_t)D;
    const uint32_t tstart = (uint32_t)T + 0xFFFFFu;   // T + start = tstart - (lo >> 5)
    while (inner) {
        const int ng = nb - g;   // entry i = base + g is below nb iff base < ng
        for (int base = 0; base < nb; base += RPG) {
            // i < 128 = kMaxBudget (base < nb <= 127 is a multiple of RPG,
            // which divides 128): entries past nb are read and their two
            // candidate slots (< 2 * kMaxBudget) written, but never used
            const int i = base + g;
            const uint64_t key = sm.beam[i];
            const uint32_t lo = (uint32_t)key, hi = (uint32_t)(key >> 32);
            const int lv = (int)(lo & 31u);
            const bool expand = base < ng && lv > 0;
            const int cl = lv - 1;
            const int left = score_row<D, MUL24>(nbase, nbase_hi, kbase, tstart - (lo >> 5), cl, l16,
                                                 expand, s, o16, okey, q);
            if (STATS) {
                cnt.tree_rows += wave_count(expand && s == 0 && cl > l16);
                cnt.tree16_rows += wave_count(expand && s == 0 && cl > 0 && cl <= l16);
                cnt.key_rows += wave_count(expand && s == 0 && cl == 0);
            }
            // children from the parent key: the left child keeps the start
            // and has level lv - 1 (low word - 1); the right child starts
            // 2^cl later (low word - 1 - 32 * 2^cl) and scores parent - left
            // (biased high word - left).  A node that is not expanded keeps
            // its key and leaves an empty slot (high word 0).  Every lane of
            // the row group stores the same two keys.
            const uint32_t c0hi = expand ? (uint32_t)left ^ 0x80000000u : hi;
            const uint32_t c1hi = expand ? hi - (uint32_t)left : 0u;
            const uint32_t c1lo = lo - 1u - (32u << ((uint32_t)cl & 31u));
            sm.cand[2 * i] = ((uint64_t)c0hi << 32) | (lo - (uint32_t)expand);
            sm.cand[2 * i + 1] = ((uint64_t)c1hi << 32) | c1lo;
        }
        wave_sync();
        nb = select_best(sm.cand, 2 * nb, r, sm.beam, inner);
        wave_sync();
    }

    // the r routed keys, already in ascending position order
    for (int i = lane; i < r; i += kWave) {
        const uint64_t k = sm.beam[i];
        sm.pos[i] = key_start(k);
        sm.score[i] = key_score(k);
    }
    wave_sync();
    return C;
}

__device__ __forceinline__ void write_selection(const WaveLds& sm, int C, int max_budget,
                                                int32_t* __restrict__ idx_row,
                                                int32_t* __restrict__ count_out)
{
    const int lane = lane_id();
    for (int c = lane; c < max_budget; c += kWave) idx_row[c] = c < C ? sm.pos[c] : -1;
    if (lane == 0) *count_out = C;
}

// q . K[j] of the selected keys in idx order, 0 in the padding.
__device__ __forceinline__ void write_scores(const WaveLds& sm, int C, int max_budget,
                                             int32_t* __restrict__ score_row)
{
    for (int c = lane_id(); c < max_budget; c += kWave) score_row[c] = c < C ? sm.score[c] : 0;
}

// The attention logit fl32(score * scale), rounded on its own: never fused
// with the subtraction of the maximum that follows it.
__device__ __forceinline__ float logit(float score, float scale)
{
#pragma clang fp contract(off)
    return score * scale;
}

// softmax over sm.score[0, C) * scale and the weighted sum of value rows,
// returned per lane (see store_output).
// Positions outside [0, T) (possible only in caller-supplied index sets,
// CHECK = true) are left out of the softmax and never loaded; with none left
// the output is 0.  Routed sets (CHECK = false) hold valid positions only.
template <int D, bool CHECK>
__device__ float4 attend_selected(WaveLds& sm, int C, int T, float scale,
                                  const float* __restrict__ values_pair)
{
    constexpr int LPV = D / 4, RPV = kWave / LPV;
    const int lane = lane_id();
    const bool ok0 = lane < C && (!CHECK || (unsigned)sm.pos[lane] < (unsigned)T);
    const bool ok1 = lane + kWave < C && (!CHECK || (unsigned)sm.pos[lane + kWave] < (unsigned)T);
    // the largest logit is fl32(fl32(largest score) * scale): rounding to
    // fp32 and multiplying by the positive scale are both monotone, so the
    // maximum is taken on the integer scores (slots kMaxBudget = 2 * 64)
    const int s0 = ok0 ? sm.score[lane] : (int)0x80000000;
    const int s1 = ok1 ? sm.score[lane + kWave] : (int)0x80000000;
    const float mx = logit((float)wave_max_i32(s0 > s1 ? s0 : s1), scale);
    const float e0 = ok0 ? __expf(logit((float)s0, scale) - mx) : 0.0f;
    const float e1 = ok1 ? __expf(logit((float)s1, scale) - mx) : 0.0f;
    if (lane < C) sm.w[lane] = e0;
    if (lane + kWave < C) sm.w[lane + kWave] = e1;
    const float z = wave_sum_f(e0 + e1);
    wave_sync();
    const int cv = lane % LPV, rv = lane / LPV;
    gbyte* vbase = uniform_base(values_pair);   // a pair's values are under 2^30 bytes
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    // kU rows per lane group in flight: their loads are issued before the
    // first use.  A slot past C (or, CHECK, holding a position outside
    // [0, T)) reads a valid stand-in row and adds nothing: its row is
    // replaced by zeros and its weight is a finite softmax weight (or 0), so
    // even a non-finite stand-in row leaves the sum unchanged.
    constexpr int kU = 4;
    int c0 = 0;
    if constexpr (!CHECK) {
        // routed sets: the whole blocks of kU * RPV slots need no tests
        for (; c0 + kU * RPV <= C; c0 += kU * RPV) {
            int4 vi[kU];
            float wt[kU];
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                const int c = c0 + u * RPV + rv;
                wt[u] = sm.w[c];
                vi[u] = load16(vbase, (uint32_t)sm.pos[c] * (uint32_t)(4 * D) + 16u * (uint32_t)cv);
            }
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                acc.x += wt[u] * __int_as_float(vi[u].x);
                acc.y += wt[u] * __int_as_float(vi[u].y);
                acc.z += wt[u] * __int_as_float(vi[u].z);
                acc.w += wt[u] * __int_as_float(vi[u].w);
            }
        }
    }
    for (; c0 < C; c0 += kU * RPV) {
        int4 vi[kU];
        float wt[kU];
        bool ok[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int c = c0 + u * RPV + rv;
            const int cc = c < C ? c : 0;   // slot 0 holds a selected position (C >= 1)
            const int j = sm.pos[cc];
            ok[u] = c < C && (!CHECK || (unsigned)j < (unsigned)T);
            wt[u] = sm.w[cc];
            const uint32_t row = CHECK ? (ok[u] ? (uint32_t)j : 0u) : (uint32_t)j;
            vi[u] = load16(vbase, row * (uint32_t)(4 * D) + 16u * (uint32_t)cv);
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            if (!ok[u]) {
                if (CHECK) wt[u] = 0.0f;
                vi[u] = make_int4(0, 0, 0, 0);
            }
            acc.x += wt[u] * __int_as_float(vi[u].x);
            acc.y += wt[u] * __int_as_float(vi[u].y);
            acc.z += wt[u] * __int_as_float(vi[u].z);
            acc.w += wt[u] * __int_as_float(vi[u].w);
        }
    }
#pragma unroll
    for (int o = LPV; o < kWave; o <<= 1) {
        acc.x += __shfl_xor(acc.x, o);
        acc.y += __shfl_xor(acc.y, o);
        acc.z += __shfl_xor(acc.z, o);
        acc.w += __shfl_xor(acc.w, o);
    }
    const float inv = z > 0.0f ? 1.0f / z : 0.0f;
    return make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
}

// Every lane holds the output columns 4 (lane % (d/4)) .. + 3 after
// attend_selected; the first d/4 lanes store the row.
template <int D>
__device__ __forceinline__ void store_output(float* __restrict__ out, float4 o)
{
    const int lane = lane_id();
    if (lane < D / 4) reinterpret_cast<float4*>(out)[lane] = o;
}

// ---- prefill: one wave per (pair, t), expensive (late) queries first -----
struct RouteArgs {
    const int8_t* Q;
    const int8_t* K;
    const float* V;
    const int32_t* nodes;
    const int32_t* budget;   // nullable: fixed_budget for every query
    int32_t* idx;
    int32_t* count;
    float* O;                // ATTEND
    int32_t* stats;          // STATS
    int32_t* score;          // nullable, routing without attention only
    int fixed_budget, P, T, L, l16, window, max_budget;
    int interleave;          // see k_route
    float scale;
    uint64_t q0, nq;         // the launch covers queries [q0, q0 + nq)
};

// Query gw of the launch order is pair gw >> L at position T-1 - (gw mod T):
// pair-major, and within a pair from t = T-1 down (the late queries, whose
// covers are deepest, start first).
template <int D, bool MUL24, bool ATTEND, bool STATS>
__device__ __forceinline__ void route_one(const RouteArgs& a, uint64_t gw, WaveLds& sm)
{
    const int T = a.T;
    const uint32_t pair = uniform((uint32_t)(gw >> a.L));
    const int t = uniform(T - 1 - (int)((uint32_t)gw & (uint32_t)(T - 1)));
    const size_t qrow = (size_t)pair * T + t;
    QueryRegs<D> q;
    load_query<D>(a.Q + qrow * D, lane_id() % (D / 16), q);
    // budgets outside [1, max_budget] are clamped: the beam and idx rows hold max_budget
    int B = uniform(a.budget ? a.budget[qrow] : a.fixed_budget);
    B = B < 1 ? 1 : (B > a.max_budget ? a.max_budget : B);
    RouteCounts cnt{0, 0, 0};
    const int C = route_query<D, MUL24, STATS>(a.nodes + (size_t)pair * T * D,
                                                a.K + (size_t)pair * T * D, T, a.L, a.l16, t, B,
                                                a.window, q, sm, cnt);
    write_selection(sm, C, a.max_budget, a.idx + qrow * a.max_budget, a.count + qrow);
    if (STATS && lane_id() == 0) {
        a.stats[qrow * 4 + 0] = cnt.tree_rows;
        a.stats[qrow * 4 + 1] = cnt.tree16_rows;
        a.stats[qrow * 4 + 2] = cnt.key_rows;
        a.stats[qrow * 4 + 3] = C;
    }
    if constexpr (!ATTEND && !STATS) {
        if (a.score) write_scores(sm, C, a.max_budget, a.score + qrow * a.max_budget);
    }
    if constexpr (ATTEND)
        store_output<D>(a.O + qrow * D,
                        attend_selected<D, false>(sm, C, T, a.scale, a.V + (size_t)pair * T * D));
}

// Which queries each XCD runs (workgroups are dealt round-robin to the 8 XCDs,
// each with its own L2).  With at least kPairsPerXcd pairs per XCD, every XCD
// takes one contiguous range of queries, i.e. whole pairs, whose rows then stay
// in its L2; the budgets of the pairs in a range average out.  With fewer,
// the pairs' budgets (nearly constant within a pair for a predictor dominated
// by the key sum, and different between pairs) would leave the XCDs unequally
// loaded - the launch lasts as long as its busiest XCD - so consecutive
// workgroups go to consecutive XCDs instead: every XCD takes an equal share of
// every pair, at the price of each L2 holding every pair's rows in turn (the
// openai-hub article, section "次二次复杂度成立，需要满足三个前提", on GPU
// utilisation under divergent tree search).  A fixed budget is the same for
// every pair, so there the contiguous ranges keep their L2 locality.
constexpr int kPairsPerXcd = 8;

template <int D, bool MUL24, bool ATTEND, bool STATS>
__global__ __launch_bounds__(kThreads) void k_route(const RouteArgs a)
{
    __shared__ WaveLds smem[kWavesPerBlock];
    const int wid = uniform((int)(threadIdx.x / kWave));
    const uint64_t blk = a.interleave ? blockIdx.x : xcd_logical_block();
    const uint64_t lw = blk * kWavesPerBlock + wid;
    if (lw >= a.nq) return;
    route_one<D, MUL24, ATTEND, STATS>(a, a.q0 + lw, smem[wid]);
}

// ---- attention over given index sets -------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void k_attend(const int8_t* __restrict__ Q,
                                                     const int8_t* __restrict__ K,
                                                     const float* __restrict__ V,
                                                     const int32_t* __restrict__ idx,
                                                     const int32_t* __restrict__ count,
                                                     float* __restrict__ O, int P, int T,
                                                     int max_budget, float scale, uint64_t q0,
                                                     uint64_t nq)
{
    constexpr int LPR = D / 16, RPG = kWave / LPR;
    __shared__ WaveLds smem[kWavesPerBlock];
    const int wid = threadIdx.x / kWave;
    const uint64_t lw = (uint64_t)xcd_logical_block() * kWavesPerBlock + wid;
    if (lw >= nq) return;
    const uint64_t gw = q0 + lw;   // query index over all P * T (launches cover ranges)
    const int pair = (int)(gw / (uint64_t)T);
    const int t = (int)(gw % (uint64_t)T);
    const size_t qrow = (size_t)pair * T + t;
    const int lane = lane_id(), s = lane % LPR, g = lane / LPR;
    QueryRegs<D> q;
    load_query<D>(Q + qrow * D, s, q);
    WaveLds& sm = smem[wid];
    // caller-supplied sets: count is clamped to [0, max_budget], positions
    // outside [0, T) are skipped
    int C = count[qrow];
    C = C < 0 ? 0 : (C > max_budget ? max_budget : C);
    const int8_t* keys_pair = K + (size_t)pair * T * D;
    for (int base = 0; base < C; base += RPG) {
        const int c = base + g;
        const int j = c < C ? idx[qrow * max_budget + c] : -1;
        const bool act = c < C && (unsigned)j < (unsigned)T;
        const int sc = score_node<D, false>(nullptr, keys_pair, T, 0, 0, act ? j : 0, act, s, q);
        if (c < C && s == 0) {
            sm.pos[c] = j;
            sm.score[c] = sc;
        }
    }
    wave_sync();
    store_output<D>(O + qrow * D, attend_selected<D, true>(sm, C, T, scale, V + (size_t)pair * T * D));
}

// ---- decode: one workgroup per pair, query at position pos ---------------
// Decode has one query per (sequence, head) and step, so the grid is small
// and each query's chain of dependent steps decides the latency: budget,
// cover of [0, m), about log2(T) descent rounds, attention.  A workgroup of
// kDecodeWaves waves serves one query.
//
// The first phase runs three independent parts side by side: waves 0-3
// predict the budget and (fused append) store the new key and value rows and
// add the key to its ancestors; waves 4-7 score the cover roots and the
// window of neighbours.  None needs another's result: the cover roots, and
// every node below them, lie in [0, m) with m <= pos, so the append changes
// none of them; the window is scored for the widest n it can have before
// the budget is known (whenever r > 0 the cover's m is that window's); and
// the predictor forms S[pos] itself.  Each descent round then has wave 0
// select the beam between two barriers while every wave scores a share of
// the round's rows (kDecodeWaves x 64 / (d/16) rows per pass, two passes
// loaded together), and all waves share the value gather.
constexpr int kDecodeWaves = 8;
constexpr int kPredictWaves = 4;
constexpr int kPredictThreads = kPredictWaves * kWave;
constexpr int kCoverWaves = kDecodeWaves - kPredictWaves;

struct BlockShared {
    WaveLds sm;
    float4 red[kDecodeWaves][kWave];   // per-wave partial output rows
    uint64_t pbest[kPredictWaves];      // per-wave best (logit, class) key
    int nsc[kMaxBudget];                // window scores, positions t+1-nw .. t
    int4 snew[256 / 4];                 // S[pos] with the new key added (d <= 256)
    int nb, inner;
    float z;
};

// The budget predictor (ALHR README, "Inference stage": a linear layer on the
// query and the causal key sum, argmax over the budget classes) for one
// decode query, spread over threads u < kPredictThreads: thread u takes
// class c = u / TPC and the 16-column chunks p, p + TPC, ... (p = u % TPC)
// of both halves of the class row [Wq | Ws] against [q; S].  The logit is
// summed over the class's TPC lanes and each wave keeps its best key (larger
// logit, then lower class) in pbest.  With APPEND the stored running sum is
// S[pos-1] and S = S[pos-1] + k_new; class 0's threads leave S in snew, for
// the caller to store once no thread reads the old sum.  All sums are int32
// (two's complement), so the order of the additions does not change a logit.
// With APPEND the same threads also form q . k_new, the window score of
// position t (its key row is not stored yet), into nsc[nw - 1].
template <int D>
struct PredictSplit {
    static constexpr int TPC = D / 16 < 8 ? D / 16 : 8;   // threads per class
    static constexpr int CPT = D / 16 / TPC;                // chunks per thread
};

template <int D, bool APPEND>
__device__ __forceinline__ void predict_block(int u, const int8_t* __restrict__ qp,
                                              const int32_t* __restrict__ pre,
                                              const int8_t* __restrict__ kn,
                                              const int8_t* __restrict__ W, int nc, int nw,
                                              BlockShared& bs)
{
    constexpr int TPC = PredictSplit<D>::TPC, CPT = PredictSplit<D>::CPT;
    static_assert(kMaxClasses * TPC <= kPredictThreads, "one class per thread group");
    const int c = u / TPC, p = u % TPC;
    const bool act = c < nc;
    const int8_t* wrow = W + (size_t)(act ? c : 0) * 2 * D;   // inactive: class 0, unused
    int z = 0, self = 0;
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
        const int ch = p + k * TPC;   // columns 16 ch .. 16 ch + 15
        const int4 wq = reinterpret_cast<const int4*>(wrow)[ch];
        const int4 ws = reinterpret_cast<const int4*>(wrow + D)[ch];
        const int4 qq = reinterpret_cast<const int4*>(qp)[ch];
        int4 sv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) sv[e] = reinterpret_cast<const int4*>(pre)[4 * ch + e];
        if constexpr (APPEND) {
            const int4 kk = reinterpret_cast<const int4*>(kn)[ch];
            const int kw[4] = {kk.x, kk.y, kk.z, kk.w};
#pragma unroll
            for (int e = 0; e < 4; ++e)
                sv[e] = make_int4(sv[e].x + sbyte(kw[e], 0), sv[e].y + sbyte(kw[e], 1),
                                  sv[e].z + sbyte(kw[e], 2), sv[e].w + sbyte(kw[e], 3));
            self = dot4_i8(qq.x, kk.x, self);
            self = dot4_i8(qq.y, kk.y, self);
            self = dot4_i8(qq.z, kk.z, self);
            self = dot4_i8(qq.w, kk.w, self);
        }
        z = dot4_i8(wq.x, qq.x, z);
        z = dot4_i8(wq.y, qq.y, z);
        z = dot4_i8(wq.z, qq.z, z);
        z = dot4_i8(wq.w, qq.w, z);
        const int wsw[4] = {ws.x, ws.y, ws.z, ws.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            z += sbyte(wsw[e], 0) * sv[e].x;
            z += sbyte(wsw[e], 1) * sv[e].y;
            z += sbyte(wsw[e], 2) * sv[e].z;
            z += sbyte(wsw[e], 3) * sv[e].w;
            if (APPEND && c == 0) bs.snew[4 * ch + e] = sv[e];
        }
    }
    z = group_sum<TPC>(z);
    if constexpr (APPEND) {
        self = group_sum<TPC>(self);
        if (u == 0) bs.nsc[nw - 1] = self;
    }
    const uint64_t key = act && p == 0 ? (((uint64_t)((uint32_t)z ^ 0x80000000u) << 32) |
                                          (uint32_t)(kMaxClasses - c))
                                       : 0ull;
    const uint64_t best = wave_max(key);
    if (lane_id() == 0) bs.pbest[u / kWave] = best;
}

// q . k_new into nsc[nw - 1] when no predictor runs (fixed budget with
// APPEND): the threads u < TPC of the predictor's split, class 0's.
template <int D>
__device__ __forceinline__ void own_score(int u, const int8_t* __restrict__ qp,
                                          const int8_t* __restrict__ kn, int nw, BlockShared& bs)
{
    constexpr int TPC = PredictSplit<D>::TPC, CPT = PredictSplit<D>::CPT;
    if (u >= TPC) return;   // whole groups of TPC lanes: the sum below stays inside them
    int self = 0;
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
        const int ch = u + k * TPC;
        const int4 qq = reinterpret_cast<const int4*>(qp)[ch];
        const int4 kk = reinterpret_cast<const int4*>(kn)[ch];
        self = dot4_i8(qq.x, kk.x, self);
        self = dot4_i8(qq.y, kk.y, self);
        self = dot4_i8(qq.z, kk.z, self);
        self = dot4_i8(qq.w, kk.w, self);
    }
    self = group_sum<TPC>(self);
    if (u == 0) bs.nsc[nw - 1] = self;
}

__device__ __forceinline__ int budget_from_best(const BlockShared& bs, int kpc, int cap)
{
    uint64_t best = bs.pbest[0];
#pragma unroll
    for (int w = 1; w < kPredictWaves; ++w) best = bs.pbest[w] > best ? bs.pbest[w] : best;
    const int cls = kMaxClasses - (int)(uint32_t)best;
    const int b = kpc * (cls + 1);
    return b < cap ? b : cap;
}

// q . node with every kind of row loaded at once and no branch: four 16-byte
// loads from the tree table (an int32 row uses all four, an int16 row the
// first two) and one from the key rows.  Slots a node does not use read row
// 0 of their table (allocated; its value is discarded).  The first phase's rows are of mixed kinds (cover roots at
// every level, window keys); this way they cost one memory round trip, not
// one per kind.  Inactive lanes give 0.
template <int D, bool MUL24>
__device__ __forceinline__ int score_node_flat(gbyte* nbase, gbyte* kbase, int T, int l16,
                                               int level, int start, bool active, int s,
                                               const QueryRegs<D>& q)
{
    constexpr int LPR = D / 16;
    const uint32_t b16 = (uint32_t)T >> l16;
    const uint32_t r = ((uint32_t)T >> level) + ((uint32_t)start >> level);
    const bool k32 = active && level > l16;
    const bool k16 = active && level > 0 && level <= l16;
    const bool kk = active && level == 0;
    const uint32_t o32 = r * (uint32_t)(4 * D);
    const uint32_t o16 = b16 * (uint32_t)(4 * D) + (r - b16) * (uint32_t)(2 * D);
    int4 v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t slot = 16u * (uint32_t)(j * LPR + s);
        const uint32_t off = k32 ? o32 + slot : ((k16 && j < 2) ? o16 + slot : slot);
        v[j] = load16(nbase, off);
    }
    const int4 vk = load16(kbase, kk ? (uint32_t)start * (uint32_t)D + 16u * (uint32_t)s
                                     : 16u * (uint32_t)s);
    int qh[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        qh[j] = q.qh[j];
        asm volatile("" : "+v"(qh[j]));
    }
    int a32 = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        a32 += imul<MUL24>(lo16(qh[2 * j]), v[j].x);
        a32 += imul<MUL24>(hi16(qh[2 * j]), v[j].y);
        a32 += imul<MUL24>(lo16(qh[2 * j + 1]), v[j].z);
        a32 += imul<MUL24>(hi16(qh[2 * j + 1]), v[j].w);
    }
    int a16 = 0;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        a16 = dot2_i16(q.qh[4 * k + 0], v[k].x, a16);
        a16 = dot2_i16(q.qh[4 * k + 1], v[k].y, a16);
        a16 = dot2_i16(q.qh[4 * k + 2], v[k].z, a16);
        a16 = dot2_i16(q.qh[4 * k + 3], v[k].w, a16);
    }
    int ak = dot4_i8(q.qp[0], vk.x, 0);
    ak = dot4_i8(q.qp[1], vk.y, ak);
    ak = dot4_i8(q.qp[2], vk.z, ak);
    ak = dot4_i8(q.qp[3], vk.w, ak);
    const int acc = k32 ? a32 : (k16 ? a16 : (kk ? ak : 0));
    return group_sum<LPR>(acc);
}

// The cover roots of [0, ms) (candidate slots L-1-b, an empty key where bit
// b of ms is clear) and the window positions ms .. t (scores in nsc), with
// ms = t + 1 - nw, over the threads v < kCoverWaves * 64 of waves 4-7.  With
// APPEND, position t (whose key row is not stored yet) is left to the
// predictor's threads (nw - 1 window positions here).
template <int D, bool MUL24, bool APPEND>
__device__ __forceinline__ void cover_block(int v, const int32_t* __restrict__ nodes_pair,
                                            const int8_t* __restrict__ keys_pair, int T, int L,
                                            int l16, int t, int nw, const QueryRegs<D>& q,
                                            BlockShared& bs)
{
    constexpr int LPR = D / 16, RPG = kWave / LPR, RPC = RPG * kCoverWaves;
    const int lane = lane_id(), s = lane % LPR, e0 = (v / kWave) * RPG + lane / LPR;
    const int ms = t + 1 - nw;
    const int nwin = APPEND ? nw - 1 : nw;
    gbyte* nbase = uniform_base(nodes_pair);
    gbyte* kbase = uniform_base(keys_pair);
    for (int base = 0; base < L + nwin; base += RPC) {
        const int j = base + e0;
        const bool cov = j < L;
        const bool act_cov = cov && ((ms >> j) & 1);
        const int k = j - L;
        const bool act_win = !cov && k < nwin;
        const int level = act_cov ? j : 0;
        const int start = act_cov ? (ms & ~((2 << j) - 1)) : (act_win ? ms + k : 0);
        const int sc = score_node_flat<D, MUL24>(nbase, kbase, T, l16, level, start,
                                                 act_cov || act_win, s, q);
        if (lane % LPR == 0) {
            if (cov) bs.sm.cand[L - 1 - j] = act_cov ? make_key(sc, start, j) : 0ull;
            else if (act_win) bs.nsc[k] = sc;
        }
    }
}

// Left children of two beam entries per row group, when none of the wave's
// rows is an int32 row: an int16 row (two loads) or a key row (one) per
// entry, every load of both entries issued before any is used, so a round
// whose beam needs two block passes waits for memory once.  Loads are masked
// per lane by the row kind (a lane that loads nothing issues no address).
// Offsets as in score_row.
template <int D>
__device__ __forceinline__ void score_two_rows(gbyte* nbase, gbyte* nbase_hi, gbyte* kbase,
                                               uint32_t ts0, int cl0, bool x0, uint32_t ts1,
                                               int cl1, bool x1, int l16, uint32_t o16,
                                               uint32_t okey, const QueryRegs<D>& q, int& left0,
                                               int& left1)
{
    constexpr int LPR = D / 16;
    const uint32_t ts[2] = {ts0, ts1};
    const int cl[2] = {cl0, cl1};
    const bool ex[2] = {x0, x1};
    int4 a[2], b[2], c[2];
    bool k16[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        k16[i] = ex[i] && (uint32_t)(cl[i] - 1) < (uint32_t)l16;
        const bool kk = ex[i] && cl[i] == 0;
        const uint32_t off16 = (ts[i] >> (uint32_t)(cl[i] & 31)) * (uint32_t)(2 * D) + o16;
        const uint32_t offk = ts[i] * (uint32_t)D + okey;
        a[i] = make_int4(0, 0, 0, 0);
        b[i] = a[i];
        c[i] = a[i];
        if (k16[i]) {
            a[i] = load16(nbase, off16);
            b[i] = load16(nbase_hi, off16);
        }
        if (kk) c[i] = load16(kbase, offk);
    }
    int left[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        int h = dot2_i16_first(q.qh[0], a[i].x);
        h = dot2_i16(q.qh[1], a[i].y, h);
        h = dot2_i16(q.qh[2], a[i].z, h);
        h = dot2_i16(q.qh[3], a[i].w, h);
        h = dot2_i16(q.qh[4], b[i].x, h);
        h = dot2_i16(q.qh[5], b[i].y, h);
        h = dot2_i16(q.qh[6], b[i].z, h);
        h = dot2_i16(q.qh[7], b[i].w, h);
        int k = dot4_i8_first(q.qp[0], c[i].x);
        k = dot4_i8(q.qp[1], c[i].y, k);
        k = dot4_i8(q.qp[2], c[i].z, k);
        k = dot4_i8(q.qp[3], c[i].w, k);
        left[i] = group_sum<LPR>(k16[i] ? h : k);
    }
    left0 = left[0];
    left1 = left[1];
}

// The children of beam entry i (as in route_query; an empty slot, high word
// 0, for a node kept as it is); every lane of the row group stores the same
// two keys.
__device__ __forceinline__ void write_children(uint64_t* cand, int i, uint64_t key, bool expand,
                                               int left)
{
    const uint32_t lo = (uint32_t)key, hi = (uint32_t)(key >> 32);
    const int cl = (int)(lo & 31u) - 1;
    const uint32_t c0hi = expand ? (uint32_t)left ^ 0x80000000u : hi;
    const uint32_t c1hi = expand ? hi - (uint32_t)left : 0u;
    const uint32_t c1lo = lo - 1u - (32u << ((uint32_t)cl & 31u));
    cand[2 * i] = ((uint64_t)c0hi << 32) | (lo - (uint32_t)expand);
    cand[2 * i + 1] = ((uint64_t)c1hi << 32) | c1lo;
}

// The beam descent of one decode query from the cover candidates cand[0, L)
// (written by cover_block) to r routed keys, which end in slots 0 .. r-1 of
// pos / score in ascending position order.
template <int D, bool MUL24>
__device__ void descend_block(const int32_t* __restrict__ nodes_pair,
                              const int8_t* __restrict__ keys_pair, int T, int L, int l16, int r,
                              const QueryRegs<D>& q, BlockShared& bs)
{
    constexpr int LPR = D / 16, RPG = kWave / LPR, RPB = RPG * kDecodeWaves;
    WaveLds& sm = bs.sm;
    const int lane = lane_id(), wv = threadIdx.x / kWave;
    const int s = lane % LPR, e0 = wv * RPG + lane / LPR;
    // the descent's loop invariants (see score_row)
    gbyte* nbase = uniform_base(nodes_pair);
    gbyte* nbase_hi = nbase + 16 * LPR;
    gbyte* kbase = uniform_base(keys_pair);
    const uint32_t o16 = (uint32_t)(2 * D) * ((uint32_t)T >> l16) + 16u * (uint32_t)s;
    const uint32_t okey = 16u * (uint32_t)s - (uint32_t)T * (uint32_t)D;
    const uint32_t tstart = (uint32_t)T + 0xFFFFFu;
    int ncand = L;
    for (;;) {
        if (wv == 0) {
            wave_sync();
            bool inner;
            const int nb = select_best(sm.cand, ncand, r, sm.beam, inner);
            if (lane == 0) {
                bs.nb = nb;
                bs.inner = inner;
            }
        }
        __syncthreads();
        const int nb = uniform(bs.nb);
        if (!uniform(bs.inner)) break;
        for (int base = 0; base < nb; base += 2 * RPB) {
            // entries i0 = base + e0 and i1 = i0 + RPB of this row group
            const int i0 = base + e0, i1 = i0 + RPB;
            const bool v0 = i0 < nb, v1 = i1 < nb;
            const uint64_t key0 = sm.beam[v0 ? i0 : 0], key1 = sm.beam[v1 ? i1 : 0];
            const int cl0 = (int)((uint32_t)key0 & 31u) - 1, cl1 = (int)((uint32_t)key1 & 31u) - 1;
            const bool x0 = v0 && cl0 >= 0, x1 = v1 && cl1 >= 0;
            const uint32_t ts0 = tstart - ((uint32_t)key0 >> 5), ts1 = tstart - ((uint32_t)key1 >> 5);
            // the wave's second entries exist; none of its rows is an int32 row
            const bool second = __ballot(v1) != 0ull;
            const bool wide = __ballot((x0 && cl0 > l16) || (x1 && cl1 > l16)) != 0ull;
            int left0, left1 = 0;
            if (second && !wide) {
                score_two_rows<D>(nbase, nbase_hi, kbase, ts0, cl0, x0, ts1, cl1, x1, l16, o16,
                                  okey, q, left0, left1);
            } else {
                left0 = score_row<D, MUL24>(nbase, nbase_hi, kbase, ts0, cl0, l16, x0, s, o16,
                                            okey, q);
                if (second)
                    left1 = score_row<D, MUL24>(nbase, nbase_hi, kbase, ts1, cl1, l16, x1, s, o16,
                                                okey, q);
            }
            if (v0) write_children(sm.cand, i0, key0, x0, left0);
            if (v1) write_children(sm.cand, i1, key1, x1, left1);
        }
        ncand = 2 * nb;
        __syncthreads();
    }
    // the beam is in ascending position order
    for (int i = threadIdx.x; i < r; i += kDecodeWaves * kWave) {
        const uint64_t k = sm.beam[i];
        sm.pos[i] = key_start(k);
        sm.score[i] = key_score(k);
    }
}

// Softmax weights by wave 0, the value gather shared by every wave, partial
// rows summed through LDS.
template <int D>
__device__ void attend_block(BlockShared& bs, int C, int T, float scale,
                             const float* __restrict__ values_pair, float* __restrict__ out)
{
    constexpr int LPV = D / 4, RPV = kWave / LPV, RPB = RPV * kDecodeWaves;
    WaveLds& sm = bs.sm;
    const int lane = lane_id(), wv = threadIdx.x / kWave;
    if (wv == 0) {
        const bool ok0 = lane < C && (unsigned)sm.pos[lane] < (unsigned)T;
        const bool ok1 = lane + kWave < C && (unsigned)sm.pos[lane + kWave] < (unsigned)T;
        // the maximum on the integer scores, as in attend_selected
        const int s0 = ok0 ? sm.score[lane] : (int)0x80000000;
        const int s1 = ok1 ? sm.score[lane + kWave] : (int)0x80000000;
        const float mx = logit((float)wave_max_i32(s0 > s1 ? s0 : s1), scale);
        const float e0 = ok0 ? __expf(logit((float)s0, scale) - mx) : 0.0f;
        const float e1 = ok1 ? __expf(logit((float)s1, scale) - mx) : 0.0f;
        if (lane < C) sm.w[lane] = e0;
        if (lane + kWave < C) sm.w[lane + kWave] = e1;
        const float z = wave_sum_f(e0 + e1);
        if (lane == 0) bs.z = z;
    }
    __syncthreads();
    const int cv = lane % LPV, rv = lane / LPV;
    gbyte* vbase = uniform_base(values_pair);   // a pair's values are under 2^30 bytes
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    // as in attend_selected: kU rows in flight per lane group, slots past C
    // or holding a position outside [0, T) add nothing
    constexpr int kU = 4;
    for (int c0 = wv * RPV + rv; c0 < C; c0 += kU * RPB) {
        int4 vi[kU];
        float wt[kU];
        bool ok[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int c = c0 + u * RPB;
            const int cc = c < kMaxBudget ? c : kMaxBudget - 1;
            const int j = sm.pos[cc];
            ok[u] = c < C && (unsigned)j < (unsigned)T;
            wt[u] = sm.w[cc];
            vi[u] = load16(vbase, (ok[u] ? (uint32_t)j : 0u) * (uint32_t)(4 * D) + 16u * (uint32_t)cv);
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            if (!ok[u]) {
                wt[u] = 0.0f;
                vi[u] = make_int4(0, 0, 0, 0);
            }
            acc.x += wt[u] * __int_as_float(vi[u].x);
            acc.y += wt[u] * __int_as_float(vi[u].y);
            acc.z += wt[u] * __int_as_float(vi[u].z);
            acc.w += wt[u] * __int_as_float(vi[u].w);
        }
    }
#pragma unroll
    for (int o = LPV; o < kWave; o <<= 1) {
        acc.x += __shfl_xor(acc.x, o);
        acc.y += __shfl_xor(acc.y, o);
        acc.z += __shfl_xor(acc.z, o);
        acc.w += __shfl_xor(acc.w, o);
    }
    if (rv == 0) bs.red[wv][cv] = acc;
    __syncthreads();
    if (wv == 0 && lane < LPV) {
        float4 t = bs.red[0][lane];
#pragma unroll
        for (int w = 1; w < kDecodeWaves; ++w) {
            const float4 u = bs.red[w][lane];
            t.x += u.x;
            t.y += u.y;
            t.z += u.z;
            t.w += u.w;
        }
        const float inv = bs.z > 0.0f ? 1.0f / bs.z : 0.0f;
        reinterpret_cast<float4*>(out)[lane] = make_float4(t.x * inv, t.y * inv, t.z * inv, t.w * inv);
    }
}

// One workgroup per pair: the first phase (budget and append on waves 0-3,
// cover and window on waves 4-7, see above), then the descent, then the
// attention.  With APPEND the new key and value rows are stored at pos, the
// key is added to the pair's ancestor sums (append.h) and the running sum
// becomes S[pos]; the attention reads the value row at pos after several
// workgroup barriers, which make the workgroup's global writes visible to its
// own reads (one CU, workgroup-scope release and acquire).  Only the pair's
// own rows are touched, so workgroups stay independent.
template <int D, bool MUL24, bool APPEND>
__global__ __launch_bounds__(kDecodeWaves * kWave) __attribute__((amdgpu_num_sgpr(80), amdgpu_waves_per_eu(D >= 256 ? 4 : 8))) void k_decode(
    const int8_t* __restrict__ q_new, const int8_t* __restrict__ k_new,
    const float* __restrict__ v_new, int8_t* __restrict__ K, float* __restrict__ V,
    int32_t* __restrict__ nodes, int32_t* __restrict__ prefix,
    const int8_t* __restrict__ W, int fixed_budget, int32_t* __restrict__ budget_out,
    int32_t* __restrict__ idx, int32_t* __restrict__ count, float* __restrict__ O, int P, int T,
    int L, int l16, int pos, int window, int nc, int kpc, int max_budget, float scale)
{
    __shared__ BlockShared bs;
    const uint32_t pair = xcd_logical_block();
    if (pair >= (uint32_t)P) return;   // uniform over the workgroup
    const int lane = lane_id(), wv = threadIdx.x / kWave;
    const int s = lane % (D / 16);
    const int8_t* qp = q_new + (size_t)pair * D;
    const int8_t* kn = APPEND ? k_new + (size_t)pair * D : nullptr;
    int32_t* pre = prefix + (size_t)pair * D;
    const int32_t* nodes_pair = nodes + (size_t)pair * T * D;
    const int8_t* keys_pair = K + (size_t)pair * T * D;
    const int t = pos;
    int nw = window < max_budget ? window : max_budget;
    nw = nw < t + 1 ? nw : t + 1;
    if (wv < kPredictWaves) {
        const int u = threadIdx.x;
        appendk::SpreadAppend<D, kPredictThreads> app;
        if constexpr (APPEND) app.load(u, (int)pair, k_new, nodes, T, L, l16, pos);
        if (W) predict_block<D, APPEND>(u, qp, pre, kn, W, nc, nw, bs);
        else if (APPEND) own_score<D>(u, qp, kn, nw, bs);
        if constexpr (APPEND) app.store(u, (int)pair, nodes, T, L, l16, pos);
    } else {
        const int v = threadIdx.x - kPredictThreads;
        // the new key and value rows at pos (stored after the cover's loads)
        int kw = 0;
        float4 vv = make_float4(0.f, 0.f, 0.f, 0.f);
        if (APPEND && v < D / 4) {
            kw = reinterpret_cast<const int*>(kn)[v];
            vv = reinterpret_cast<const float4*>(v_new + (size_t)pair * D)[v];
        }
        QueryRegs<D> q;
        load_query<D>(qp, s, q);
        cover_block<D, MUL24, APPEND>(v, nodes_pair, keys_pair, T, L, l16, t, nw, q, bs);
        if (APPEND && v < D / 4) {
            const size_t row = (size_t)pair * T + pos;
            reinterpret_cast<int*>(K)[row * (D / 4) + v] = kw;
            reinterpret_cast<float4*>(V)[row * (D / 4) + v] = vv;
        }
    }
    // the query in registers for the descent (loaded after the first phase,
    // whose parts hold enough registers of their own)
    QueryRegs<D> q;
    load_query<D>(qp, s, q);
    __syncthreads();
    if constexpr (APPEND) {
        // the running sum becomes S[pos]: the predictor's (left in LDS), or,
        // without a predictor, formed here
        if (W) {
            if (threadIdx.x < D / 4) reinterpret_cast<int4*>(pre)[threadIdx.x] = bs.snew[threadIdx.x];
        } else if (threadIdx.x < D / 4) {
            const int kw = reinterpret_cast<const int*>(kn)[threadIdx.x];
            int4* p4 = reinterpret_cast<int4*>(pre) + threadIdx.x;
            const int4 p = *p4;
            *p4 = make_int4(p.x + sbyte(kw, 0), p.y + sbyte(kw, 1), p.z + sbyte(kw, 2),
                            p.w + sbyte(kw, 3));
        }
    }
    const int B = uniform(W ? budget_from_best(bs, kpc, max_budget) : fixed_budget);
    if (threadIdx.x == 0 && budget_out) budget_out[pair] = B;
    const int C = uniform(B < t + 1 ? B : t + 1);
    const int n = uniform(window < C ? window : C);
    const int r = C - n;
    const int m = t + 1 - n;
    // neighbours m .. t are the last n window positions; they go to slots r..
    if ((int)threadIdx.x < n) {
        bs.sm.pos[r + threadIdx.x] = m + (int)threadIdx.x;
        bs.sm.score[r + threadIdx.x] = bs.nsc[nw - n + (int)threadIdx.x];
    }
    if (r > 0) descend_block<D, MUL24>(nodes_pair, keys_pair, T, L, l16, r, q, bs);
    __syncthreads();
    if (wv == 0) write_selection(bs.sm, C, max_budget, idx + (size_t)pair * max_budget, count + pair);
    attend_block<D>(bs, C, T, scale, V + (size_t)pair * T * D, O + (size_t)pair * D);
}

// One wave per query, and a dispatch's work-item count is 32-bit: launches
// cover at most kQueriesPerLaunch queries each (2^30 work-items).
constexpr uint64_t kQueriesPerLaunch = (uint64_t)1 << 24;

unsigned grid_for_waves(uint64_t waves)
{
    uint64_t blocks = (waves + kWavesPerBlock - 1) / kWavesPerBlock;
    blocks = (blocks + kXcds - 1) / kXcds * kXcds;   // xcd_logical_block needs a multiple
    return (unsigned)blocks;
}

template <int D, bool MUL24, bool ATTEND, bool STATS>
hipError_t launch_one(const RouteArgs& a, hipStream_t st)
{
    hipLaunchKernelGGL((k_route<D, MUL24, ATTEND, STATS>), dim3(grid_for_waves(a.nq)),
                       dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

template <int D, bool MUL24>
hipError_t route_d(const Shape& s, const int8_t* Q, const int8_t* K, const float* V,
                   const int32_t* nodes, const int32_t* budget, int fixed_budget, int32_t* idx,
                   int32_t* count, float* O, int32_t* stats, int32_t* score, hipStream_t st)
{
    RouteArgs a{Q, K, V, nodes, budget, idx, count, O, stats, score, fixed_budget, s.P, s.T,
                s.L, s.l16, s.window, s.max_budget, 0, s.scale, 0, 0};
    const uint64_t total = (uint64_t)s.P * s.T;
    for (uint64_t q0 = 0; q0 < total; q0 += kQueriesPerLaunch) {
        a.q0 = q0;
        a.nq = total - q0 < kQueriesPerLaunch ? total - q0 : kQueriesPerLaunch;
        a.interleave = budget != nullptr && a.nq < (uint64_t)kXcds * kPairsPerXcd * s.T;
        hipError_t e;
        if (stats) e = launch_one<D, MUL24, false, true>(a, st);
        else if (O) e = launch_one<D, MUL24, true, false>(a, st);
        else e = launch_one<D, MUL24, false, false>(a, st);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int D>
hipError_t route_dispatch(const Shape& s, const int8_t* Q, const int8_t* K, const float* V,
                          const int32_t* nodes, const int32_t* budget, int fixed_budget,
                          int32_t* idx, int32_t* count, float* O, int32_t* stats, int32_t* score,
                          hipStream_t st)
{
    return s.mul24 ? route_d<D, true>(s, Q, K, V, nodes, budget, fixed_budget, idx, count, O,
                                      stats, score, st)
                   : route_d<D, false>(s, Q, K, V, nodes, budget, fixed_budget, idx, count, O,
                                       stats, score, st);
}

template <int D>
hipError_t decode_d(const Shape& s, int pos, const int8_t* q_new, const int8_t* k_new,
                    const float* v_new, int8_t* K, float* V, int32_t* nodes, int32_t* prefix,
                    const int8_t* W, int fixed_budget, int32_t* budget, int32_t* idx,
                    int32_t* count, float* O, hipStream_t st)
{
    const dim3 grid((unsigned)((s.P + kXcds - 1) / kXcds * kXcds));
#define ALHR_DECODE(MUL, APP)                                                                     \
    hipLaunchKernelGGL((k_decode<D, MUL, APP>), grid, dim3(kDecodeWaves * kWave), 0, st, q_new,    \
                       k_new, v_new, K, V, nodes, prefix, W, fixed_budget, budget, idx, count, O, \
                       s.P, s.T, s.L, s.l16, pos, s.window, s.n_classes, s.keys_per_class,      \
                       s.max_budget, s.scale)
    const bool append = k_new != nullptr;
    if (s.mul24) {
        if (append) ALHR_DECODE(true, true);
        else ALHR_DECODE(true, false);
    } else {
        if (append) ALHR_DECODE(false, true);
        else ALHR_DECODE(false, false);
    }
#undef ALHR_DECODE
    return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const Shape& s, const int8_t* Q, const int8_t* K, const float* V,
                        const int32_t* nodes, const int32_t* budget, int fixed_budget,
                        int32_t* idx, int32_t* count, float* O, int32_t* stats, int32_t* score,
                        hipStream_t st)
{
#define ALHR_RD(DD)                                                                              \
    return route_dispatch<DD>(s, Q, K, V, nodes, budget, fixed_budget, idx, count, O, stats,    \
                              score, st)
    switch (s.d) {
        case 16: ALHR_RD(16);
        case 32: ALHR_RD(32);
        case 64: ALHR_RD(64);
        case 128: ALHR_RD(128);
        case 256: ALHR_RD(256);
        default: return hipErrorInvalidValue;
    }
#undef ALHR_RD
}

hipError_t launch_attend(const Shape& s, const int8_t* Q, const int8_t* K, const float* V,
                         const int32_t* idx, const int32_t* count, float* O, hipStream_t st)
{
    const uint64_t total = (uint64_t)s.P * s.T;
    for (uint64_t q0 = 0; q0 < total; q0 += kQueriesPerLaunch) {
        const uint64_t nq = total - q0 < kQueriesPerLaunch ? total - q0 : kQueriesPerLaunch;
        const dim3 grid(grid_for_waves(nq));
#define ALHR_ATTEND(DD)                                                                           \
    hipLaunchKernelGGL((k_attend<DD>), grid, dim3(kThreads), 0, st, Q, K, V, idx, count, O, s.P,  \
                       s.T, s.max_budget, s.scale, q0, nq)
        switch (s.d) {
            case 16: ALHR_ATTEND(16); break;
            case 32: ALHR_ATTEND(32); break;
            case 64: ALHR_ATTEND(64); break;
            case 128: ALHR_ATTEND(128); break;
            case 256: ALHR_ATTEND(256); break;
            default: return hipErrorInvalidValue;
        }
#undef ALHR_ATTEND
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_decode(const Shape& s, int pos, const int8_t* q_new, const int8_t* k_new,
                         const float* v_new, int8_t* K, float* V, int32_t* nodes,
                         int32_t* prefix, const int8_t* W, int fixed_budget, int32_t* budget,
                         int32_t* idx, int32_t* count, float* O, hipStream_t st)
{
#define ALHR_DD(DD)                                                                               \
    return decode_d<DD>(s, pos, q_new, k_new, v_new, K, V, nodes, prefix, W, fixed_budget, budget, \
                        idx, count, O, st)
    switch (s.d) {
        case 16: ALHR_DD(16);
        case 32: ALHR_DD(32);
        case 64: ALHR_DD(64);
        case 128: ALHR_DD(128);
        case 256: ALHR_DD(256);
        default: return hipErrorInvalidValue;
    }
#undef ALHR_DD
}

}  // namespace alhr
