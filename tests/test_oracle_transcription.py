"""A second, literal transcription of the routed-attention steps, written
straight from the method's definitions in plain Python (node sums taken as
sums over their key ranges, the causal prefix as a running sum, the beam as a
sort of candidates by (score descending, first position ascending)), run on
every query of small inputs and required to equal the C oracle exactly
(budgets, index sets, counts) and to 1e-6 in the attention output.

This is a cross-check of the oracle's code, not one of its pins: it shares
the oracle's reading of the pages and would share a misreading.  The pins in
test_oracle_pins.py tie the oracle to facts fixed independently of it.

Definitions followed (ALHR README, "Inference stage"; the causal rule of its
"Training stage"; the budget classes of "Results and Variables"):
  node(l, p)   = sum of K[p 2^l .. (p+1) 2^l - 1]
  S[t]         = sum of K[0..t]
  budget       = min(kpc * (c* + 1), cap), c* the lowest class of largest
                 W[c] . [Q[t]; S[t]]  (or the fixed budget)
  C = min(budget, t + 1), n = min(window, C): keys t, t-1, .., t-n+1
  r = C - n routed keys from [0, m), m = t + 1 - n: cover of [0, m) by the
  set bits of m, beam of width r, every internal beam node replaced by its two
  children each round, leaves kept, best r by (q . node desc, start asc)
  attention: softmax of fl32(fl32(q . k) * scale) over the set, V averaged
"""
import math

import numpy as np
import pytest

import oracle


def transcribe(Q, K, V, W, fixed_budget, window, kpc, cap, scale):
    T, d = K.shape
    Ki, Qi = K.astype(np.int64), Q.astype(np.int64)
    S = np.cumsum(Ki, axis=0)

    def node(level, start):
        return Ki[start:start + (1 << level)].sum(axis=0)

    budgets, counts = [], []
    idx = np.full((T, cap), -1, dtype=np.int64)
    O = np.zeros((T, d), dtype=np.float32)
    for t in range(T):
        if W is None:
            B = fixed_budget
        else:
            Wi = W.astype(np.int64)
            z = [int(Wi[c, :d] @ Qi[t] + Wi[c, d:] @ S[t]) for c in range(W.shape[0])]
            B = min(kpc * (z.index(max(z)) + 1), cap)
        C = min(B, t + 1)
        n = min(window, C)
        r = C - n
        chosen = [t - i for i in range(n)]
        if r > 0:
            m = t + 1 - n
            cover, a = [], 0
            for level in range(m.bit_length() - 1, -1, -1):
                if (m >> level) & 1:
                    cover.append((level, a))
                    a += 1 << level

            def order(x):
                return (-int(Qi[t] @ node(*x)), x[1])

            beam = sorted(cover, key=order)[:r]
            while any(level > 0 for level, _ in beam):
                cand = []
                for level, start in beam:
                    if level == 0:
                        cand.append((level, start))
                    else:
                        cand += [(level - 1, start), (level - 1, start + (1 << (level - 1)))]
                beam = sorted(cand, key=order)[:r]
            chosen += [start for _, start in beam]
        chosen.sort()
        assert len(chosen) == C and len(set(chosen)) == C
        budgets.append(B)
        counts.append(C)
        idx[t, :C] = chosen
        logits = [float(np.float32(np.float32(int(Qi[t] @ Ki[j])) * np.float32(scale)))
                  for j in chosen]
        top = max(logits)
        e = [math.exp(x - top) for x in logits]
        acc = np.zeros(d, dtype=np.float64)
        for w, j in zip(e, chosen):
            acc += w * V[j].astype(np.float64)
        O[t] = (acc / sum(e)).astype(np.float32)
    return np.array(budgets), idx, np.array(counts), O


def inputs(seed, T, d, kind):
    r = np.random.default_rng(seed)
    K = r.integers(-4, 5, size=(T, d)).astype(np.int8)
    Q = r.integers(-4, 5, size=(T, d)).astype(np.int8)
    V = r.standard_normal((T, d)).astype(np.float32)
    if kind == "zero_query":
        Q[:] = 0
    elif kind == "planted":
        # a few keys far above the rest, queries copied from them
        K = r.integers(-1, 2, size=(T, d)).astype(np.int8)
        hot = r.choice(T, size=max(1, T // 8), replace=False)
        K[hot] = 8
        Q = np.ones((T, d), dtype=np.int8) * 2
    return Q, K, V


CASES = [
    # T, d, window, fixed budget (0 = predictor), kind
    (8, 16, 1, 3, "uniform"),
    (8, 16, 4, 16, "uniform"),
    (16, 16, 2, 5, "uniform"),
    (16, 16, 4, 0, "uniform"),
    (32, 16, 1, 7, "zero_query"),
    (32, 16, 4, 12, "planted"),
    (32, 32, 2, 0, "uniform"),
    (64, 16, 4, 16, "uniform"),
    (64, 16, 1, 1, "uniform"),
    (64, 16, 3, 0, "planted"),
]


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("case", CASES, ids=["T%d_d%d_w%d_b%d_%s" % c for c in CASES])
def test_oracle_equals_transcription_on_every_query(case, seed):
    T, d, window, fb, kind = case
    Q, K, V = inputs(1000 * seed + T + d + window, T, d, kind)
    W = None
    if fb == 0:
        W = np.random.default_rng(seed + 77).integers(-4, 5, size=(32, 2 * d)).astype(np.int8)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    kpc, cap = 3, 96
    b, idx, cnt, O = transcribe(Q, K, V, W, fb, window, kpc, cap, scale)
    ref = oracle.pair_forward(Q, K, V, W=W, fixed_budget=fb, window=window,
                              keys_per_class=kpc, max_budget=cap, scale=scale)
    if W is not None:
        np.testing.assert_array_equal(ref["budget"], b)
    np.testing.assert_array_equal(ref["count"], cnt)
    np.testing.assert_array_equal(ref["idx"], idx)
    np.testing.assert_allclose(ref["O"], O, rtol=0, atol=1e-6)
