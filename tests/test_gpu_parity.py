"""GPU parity: every entry point of libalhr, called through the C ABI (the
ctypes binding), against the CPU oracle on the same seeded inputs.

Bars: tree rows, budgets, selected index sets and counts bit-exact; the fp32
attention output within max-abs 1e-4 of the oracle's fp64 result rounded to
fp32.  Small cases are compared element by element for every query; the
full-size workloads are compared on sampled queries (each the oracle routes
one by one), with the tree and the budgets compared in full.
"""
import sys

import numpy as np
import pytest

import oracle
import synth
from synth.workloads import WORKLOADS, Workload, host_inputs
from tree_layout import decode_tree

pytestmark = pytest.mark.gpu
ATOL = 1e-4


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    return torch, torch.device("cuda:0")


def to_dev(torch, dev, *arrays):
    return [None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev)
            for a in arrays]


def run_forward(torch, dev, w: Workload, Q, K, V, W, cfg=None, fixed=None):
    import learned_tree_routed_amd as alhr
    cfg = cfg or w.config()
    q, k, v, wt = to_dev(torch, dev, Q, K, V, W)
    fb = fixed if fixed is not None else w.fixed_budget
    say("alhr_forward", w.name, "B%d H%d T%d d%d" % (cfg.batch, cfg.heads, cfg.T, cfg.d),
        "fixed" if wt is None else "predictor")
    out = alhr.alhr_forward(cfg, q, k, v, wt, fixed_budget=fb)
    torch.cuda.synchronize()
    return {k2: (None if t is None else t.cpu().numpy()) for k2, t in out.items()}


def check_pair(w, cfg, Q, K, V, W, out, b, h, ts=None, fixed=None):
    fb = fixed if fixed is not None else w.fixed_budget
    ref = oracle.pair_forward(Q[b, h], K[b, h], V[b, h], W=W, fixed_budget=fb,
                              window=cfg.window, keys_per_class=cfg.keys_per_class,
                              max_budget=cfg.max_budget, scale=cfg.scale, ts=ts)
    sel = slice(None) if ts is None else np.asarray(ts)
    if W is not None:
        np.testing.assert_array_equal(out["budget"][b, h][sel], ref["budget"])
    np.testing.assert_array_equal(out["count"][b, h][sel], ref["count"])
    np.testing.assert_array_equal(out["idx"][b, h][sel], ref["idx"])
    err = np.abs(out["O"][b, h][sel] - ref["O"]).max()
    assert err <= ATOL, "pair (%d, %d): max |O - oracle| = %g" % (b, h, err)
    return ref


def check_nodes(out_nodes, K, b, h, cfg):
    import learned_tree_routed_amd as alhr
    ref = oracle.build_tree(K[b, h])
    got = decode_tree(out_nodes[b, h], alhr.alhr_tree_int16_levels(cfg))
    np.testing.assert_array_equal(got[1:], ref[1:])


# ------------------------------------------------------------ full parity --
def test_tiny_every_query(torch_dev):
    torch, dev = torch_dev
    w = WORKLOADS["tiny"]
    Q, K, V, W = host_inputs(w)
    out = run_forward(torch, dev, w, Q, K, V, W)
    check_nodes(out["nodes"], K, 0, 0, w.config())
    check_pair(w, w.config(), Q, K, V, W, out, 0, 0)


def test_t1k_every_query(torch_dev):
    torch, dev = torch_dev
    w = WORKLOADS["t1k"]
    Q, K, V, W = host_inputs(w)
    out = run_forward(torch, dev, w, Q, K, V, W)
    cfg = w.config()
    for b in range(w.B):
        for h in range(w.H):
            check_nodes(out["nodes"], K, b, h, cfg)
            np.testing.assert_array_equal(out["budget"][b, h], oracle.pair_budgets(Q[b, h], K[b, h], W))
    for b, h in [(0, 0), (3, 5), (7, 7), (5, 2)]:
        check_pair(w, cfg, Q, K, V, W, out, b, h)


# ------------------------------------------------------- sampled, full size --
def sample_ts(T, rng, n=384):
    ts = set(rng.choice(T, size=min(n, T), replace=False).tolist())
    ts |= set(range(min(8, T))) | set(range(T - 8, T))
    return np.array(sorted(ts), dtype=np.int32)


@pytest.mark.parametrize("name", ["t4k", "t16k"])
def test_full_size_sampled(torch_dev, name):
    torch, dev = torch_dev
    w = WORKLOADS[name]
    Q, K, V, W = host_inputs(w)
    out = run_forward(torch, dev, w, Q, K, V, W)
    cfg = w.config()
    rng = np.random.default_rng(w.seed)
    for b in range(w.B):
        for h in range(w.H):
            check_nodes(out["nodes"], K, b, h, cfg)
            np.testing.assert_array_equal(out["budget"][b, h], oracle.pair_budgets(Q[b, h], K[b, h], W))
            check_pair(w, cfg, Q, K, V, W, out, b, h, ts=sample_ts(w.T, rng, 192))
    # every query: size = min(budget, t+1), ascending, own key included, -1 padding
    t = np.arange(w.T)
    C = out["count"]
    np.testing.assert_array_equal(C, np.minimum(out["budget"], t + 1))
    idx = out["idx"]
    pad = np.arange(w.max_budget)[None, None, None, :] >= C[..., None]
    assert np.all(idx[pad] == -1)
    assert np.all(idx[..., 0] >= 0)
    last = np.take_along_axis(idx, (C - 1)[..., None], axis=-1)[..., 0]
    np.testing.assert_array_equal(last, np.broadcast_to(t, last.shape))


@pytest.mark.parametrize("name", ["t4k", "t16k"])
def test_full_size_every_query(torch_dev, name):
    """Every query of the full workload (131072 at t4k and at t16k), launched
    as the benchmark times it (alhr_prepare, then alhr_route_attend with the
    predictor's budgets), against the oracle run on every query of every
    pair: budgets, index sets and counts bit-exact, outputs within 1e-4."""
    import learned_tree_routed_amd as alhr
    torch, dev = torch_dev
    w = WORKLOADS[name]
    Q, K, V, W = host_inputs(w)
    cfg = w.config()
    q, k, v, wt = to_dev(torch, dev, Q, K, V, W)
    say("alhr_prepare + alhr_route_attend, every query of", name)
    nodes, budget = alhr.alhr_prepare(cfg, q, k, wt)
    idx, count, O = alhr.alhr_route_attend(cfg, q, k, v, nodes, budget)
    torch.cuda.synchronize()
    bud, idx, count, O = (t.cpu().numpy() for t in (budget, idx, count, O))
    worst = 0.0
    for b in range(w.B):
        for h in range(w.H):
            ref = oracle.pair_forward(Q[b, h], K[b, h], V[b, h], W=W, window=cfg.window,
                                      keys_per_class=cfg.keys_per_class,
                                      max_budget=cfg.max_budget, scale=cfg.scale)
            np.testing.assert_array_equal(bud[b, h], ref["budget"], err_msg="(%d, %d)" % (b, h))
            np.testing.assert_array_equal(count[b, h], ref["count"], err_msg="(%d, %d)" % (b, h))
            np.testing.assert_array_equal(idx[b, h], ref["idx"], err_msg="(%d, %d)" % (b, h))
            worst = max(worst, float(np.abs(O[b, h] - ref["O"]).max()))
    assert worst <= ATOL, worst
    say("  max |O - oracle| over every query: %.3g" % worst)


# ------------------------------------------------------- entry-point paths --
def test_unfused_path_equals_fused(torch_dev):
    import learned_tree_routed_amd as alhr
    torch, dev = torch_dev
    w = WORKLOADS["t1k"]
    Q, K, V, W = host_inputs(w, B=2, H=4)
    cfg = w.config(batch=2, heads=4)
    q, k, v, wt = to_dev(torch, dev, Q, K, V, W)
    say("build / predict / route / attend separately, t1k B2 H4")
    nodes = alhr.alhr_build_tree(cfg, k)
    bud = alhr.alhr_predict_budget(cfg, q, k, wt)
    idx, cnt = alhr.alhr_route(cfg, q, k, nodes, bud)
    O1 = alhr.alhr_sparse_attend(cfg, q, k, v, idx, cnt)
    idx2, cnt2, O2 = alhr.alhr_route_attend(cfg, q, k, v, nodes, bud)
    full = alhr.alhr_forward(cfg, q, k, v, wt)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2) and torch.equal(cnt, cnt2)
    assert torch.equal(idx, full["idx"]) and torch.equal(bud, full["budget"])
    l16 = alhr.alhr_tree_int16_levels(cfg)
    for b in range(2):
        for h in range(4):
            np.testing.assert_array_equal(decode_tree(nodes[b, h].cpu().numpy(), l16),
                                          decode_tree(full["nodes"][b, h].cpu().numpy(), l16))
    assert (O1 - O2).abs().max().item() <= 1e-6
    assert torch.equal(O2, full["O"])
    out = {"budget": bud.cpu().numpy(), "count": cnt.cpu().numpy(), "idx": idx.cpu().numpy(),
           "O": O1.cpu().numpy()}
    check_pair(w, cfg, Q, K, V, W, out, 1, 3)


@pytest.mark.parametrize("name", ["t1k", "t4k"])
def test_route_stats_match_oracle_counts(torch_dev, name):
    import learned_tree_routed_amd as alhr
    torch, dev = torch_dev
    w = WORKLOADS[name]
    Q, K, V, W = host_inputs(w, B=1, H=2)
    cfg = w.config(batch=1, heads=2)
    q, k, wt = to_dev(torch, dev, Q, K, W)
    say("alhr_route_stats %s B1 H2" % name)
    nodes = alhr.alhr_build_tree(cfg, k)
    bud = alhr.alhr_predict_budget(cfg, q, k, wt)
    idx, cnt, st = alhr.alhr_route_stats(cfg, q, k, nodes, bud)
    idx_r, _ = alhr.alhr_route(cfg, q, k, nodes, bud)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx_r)
    st = st.cpu().numpy()
    L = w.T.bit_length() - 1
    l16 = alhr.alhr_tree_int16_levels(cfg)
    assert l16 == min(11, L)   # kmax = 8: 8 * 2^11 = 16384 fits int16, 8 * 2^12 does not
    ref = oracle.pair_forward(Q[0, 1], K[0, 1], V[0, 1], W=W, scale=cfg.scale, with_stats=True)
    for t in range(w.T):
        s = ref["stats"][t]
        # only left children are loaded; the right child's score is derived
        rows = [s["cover_by_level"][l] + s["child_by_level"][l] // 2 for l in range(24)]
        assert st[0, 1, t, 0] == sum(rows[l16 + 1:])
        assert st[0, 1, t, 1] == sum(rows[1:l16 + 1])
        assert st[0, 1, t, 2] == rows[0] == s["cover_leaf"] + s["child_leaf"] // 2
        assert st[0, 1, t, 3] == s["count"]


ROUTE_SCORE_CASES = [
    # few pairs per XCD (queries dealt to the XCDs in turn) and eight or more
    # (contiguous ranges per XCD), and a query count (1 x 5 x 16 = 80) that is
    # not a multiple of 32 (a block's four waves times the eight XCDs)
    Workload("score_t1k_b8h8", 2, 8, 8, 1024, 64, "clustered"),
    Workload("score_t16", 7, 1, 5, 16, 64, "clustered"),
    Workload("score_t4k_b1h3", 3, 1, 3, 4096, 64, "clustered"),
]


@pytest.mark.parametrize("w", ROUTE_SCORE_CASES, ids=[c.name for c in ROUTE_SCORE_CASES])
def test_route_scores_and_fused_path(torch_dev, w):
    """alhr_route's score output holds q . K[j] of every selected key in idx
    order and 0 in the padding (checked against the oracle's scores on
    sampled queries of two pairs); routing alone, routing with scores and the
    fused route + attend give the same index sets."""
    import learned_tree_routed_amd as alhr
    torch, dev = torch_dev
    Q, K, V, W = host_inputs(w)
    cfg = w.config()
    q, k, v, wt = to_dev(torch, dev, Q, K, V, W)
    say("alhr_route with scores", w.name, "B%d H%d T%d" % (w.B, w.H, w.T))
    nodes, bud = alhr.alhr_prepare(cfg, q, k, wt)
    i0, c0 = alhr.alhr_route(cfg, q, k, nodes, bud)
    i1, c1, sc = alhr.alhr_route(cfg, q, k, nodes, bud, with_score=True)
    i2, c2, O2 = alhr.alhr_route_attend(cfg, q, k, v, nodes, bud)
    torch.cuda.synchronize()
    assert torch.equal(i0, i1) and torch.equal(c0, c1)
    assert torch.equal(i0, i2) and torch.equal(c0, c2)
    idx, cnt, sc = (t.cpu().numpy() for t in (i1, c1, sc))
    ts = np.unique(np.r_[0, 1, 5, w.T // 2 + 3, w.T - 1, np.arange(0, w.T, max(1, w.T // 32))])
    ts = ts[ts < w.T].astype(np.int32)
    for (b, h) in ((0, 0), (w.B - 1, w.H - 1)):
        ref_nodes = oracle.build_tree(K[b, h])
        S = np.cumsum(K[b, h].astype(np.int64), axis=0)
        for t in ts:
            bt, _ = oracle.budget(Q[b, h, t], S[t], W)
            ridx, rsc, rc, _ = oracle.route(t, bt, Q[b, h, t], K[b, h], ref_nodes, cfg.window,
                                            cfg.max_budget)
            assert cnt[b, h, t] == rc
            np.testing.assert_array_equal(idx[b, h, t], ridx)
            np.testing.assert_array_equal(sc[b, h, t], rsc)
    check_pair(w, cfg, Q, K, V, W, {"budget": bud.cpu().numpy(), "idx": idx, "count": cnt,
                                    "O": O2.cpu().numpy()}, w.B - 1, w.H - 1, ts=ts)


def test_repeat_runs_are_bit_identical(torch_dev):
    """Ten runs of every prefill entry point on the same inputs give identical
    outputs (no race decides a result)."""
    import learned_tree_routed_amd as alhr
    torch, dev = torch_dev
    w = WORKLOADS["t4k"]
    Q, K, V, W = host_inputs(w, B=1, H=4)
    cfg = w.config(batch=1, heads=4)
    q, k, v, wt = to_dev(torch, dev, Q, K, V, W)
    say("repeat alhr_forward / alhr_route / alhr_sparse_attend x10, t4k B1 H4")
    first = alhr.alhr_forward(cfg, q, k, v, wt)
    r0 = alhr.alhr_route(cfg, q, k, first["nodes"], first["budget"], with_score=True)
    a0 = alhr.alhr_sparse_attend(cfg, q, k, v, first["idx"], first["count"])
    for _ in range(9):
        again = alhr.alhr_forward(cfg, q, k, v, wt)
        r1 = alhr.alhr_route(cfg, q, k, again["nodes"], again["budget"], with_score=True)
        a1 = alhr.alhr_sparse_attend(cfg, q, k, v, again["idx"], again["count"])
        torch.cuda.synchronize()
        for key in ("budget", "idx", "count", "O"):
            assert torch.equal(first[key], again[key]), key
        assert all(torch.equal(x, y) for x, y in zip(r0, r1))
        assert torch.equal(a0, a1)


def test_two_streams_at_once(torch_dev):
    """Two alhr_forward calls on two streams at the same time, each with its
    own outputs and workspace (the library keeps no state between calls): both
    equal a call alone on the default stream."""
    import learned_tree_routed_amd as alhr
    torch, dev = torch_dev
    w = WORKLOADS["t1k"]
    Q, K, V, W = host_inputs(w, B=2, H=4)
    cfg = w.config(batch=2, heads=4)
    q, k, v, wt = to_dev(torch, dev, Q, K, V, W)
    say("alhr_forward on two streams at once, t1k B2 H4")
    alone = alhr.alhr_forward(cfg, q, k, v, wt)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]   # default priority
    outs = []
    for st in streams:
        with torch.cuda.stream(st):
            outs.append(alhr.alhr_forward(cfg, q, k, v, wt))
    torch.cuda.synchronize()
    l16 = alhr.alhr_tree_int16_levels(cfg)
    ref_nodes = alone["nodes"].cpu().numpy()
    for out in outs:
        for key in ("budget", "idx", "count", "O"):
            assert torch.equal(out[key], alone[key]), key
        # the stored rows (the tail of a compact table is never written)
        got = out["nodes"].cpu().numpy()
        for b in range(2):
            for h in range(4):
                np.testing.assert_array_equal(decode_tree(got[b, h], l16)[1:],
                                              decode_tree(ref_nodes[b, h], l16)[1:])


def test_launch_geometry_does_not_change_results(torch_dev):
    """The same pairs computed by different waves, blocks and XCDs: alone in a
    B1 H8 launch (fewer than 8 pairs per XCD: queries dealt to the XCDs in
    turn), and as pairs 9..16 of a B9 H8 launch of 72 pairs (contiguous
    ranges per XCD, other block and wave positions).  Every output of those
    pairs is identical."""
    import learned_tree_routed_amd as alhr
    torch, dev = torch_dev
    base = WORKLOADS["t1k"]
    w8 = Workload("geom8", base.seed, 1, 8, base.T, base.d, base.kind)
    w72 = Workload("geom72", base.seed, 9, 8, base.T, base.d, base.kind)
    Q8, K8, V8, W = host_inputs(w8)
    Q72, K72, V72, _ = host_inputs(w72)
    # put the 8 pairs of the small launch at batch row 1 of the large one
    for a, b in ((Q72, Q8), (K72, K8), (V72, V8)):
        a[1] = b[0]
    say("launch geometry: B1 H8 vs rows of B9 H8, T1024")
    small = run_forward(torch, dev, w8, Q8, K8, V8, W)
    large = run_forward(torch, dev, w72, Q72, K72, V72, W)
    for key in ("budget", "idx", "count", "O"):
        np.testing.assert_array_equal(small[key][0], large[key][1], err_msg=key)
    l16 = alhr.alhr_tree_int16_levels(w8.config())
    for h in range(8):
        np.testing.assert_array_equal(decode_tree(small["nodes"][0, h], l16)[1:],
                                      decode_tree(large["nodes"][1, h], l16)[1:])


@pytest.mark.parametrize("waves", [2, 8])
def test_waves_per_workgroup_do_not_change_results(torch_dev, monkeypatch, waves):
    """The prefill routing and attention kernels built with 2 or 8 queries per
    workgroup instead of 4 (libalhr_wpb2.so, libalhr_wpb8.so): identical
    budgets, index sets, counts, scores and outputs for alhr_forward,
    alhr_route and alhr_sparse_attend, at 64 pairs (contiguous query ranges
    per XCD) and at 4 pairs (queries dealt to the XCDs in turn)."""
    import learned_tree_routed_amd as alhr
    torch, dev = torch_dev
    variant = alhr.load_geometry_variant(waves)
    for name, B, H in (("t1k", 8, 8), ("t4k", 1, 4)):
        w = WORKLOADS[name]
        Q, K, V, W = host_inputs(w, B=B, H=H)
        cfg = w.config(batch=B, heads=H)
        q, k, v, wt = to_dev(torch, dev, Q, K, V, W)

        def run():
            f = alhr.alhr_forward(cfg, q, k, v, wt)
            r = alhr.alhr_route(cfg, q, k, f["nodes"], f["budget"], with_score=True)
            a = alhr.alhr_sparse_attend(cfg, q, k, v, f["idx"], f["count"])
            torch.cuda.synchronize()
            return [f[x] for x in ("budget", "idx", "count", "O")] + list(r) + [a]

        say("libalhr.so (4 waves per workgroup)", name, "B%d H%d" % (B, H))
        ref = run()
        say("libalhr_wpb%d.so" % waves, name, "B%d H%d" % (B, H))
        with monkeypatch.context() as m:
            m.setattr(alhr, "_lib", variant)
            got = run()
        for i, (a, b) in enumerate(zip(ref, got)):
            assert torch.equal(a, b), (name, i)


def test_sparse_attend_skips_invalid_caller_indices(torch_dev):
    """Caller-supplied index sets with positions outside [0, T) (negative, or
    T and beyond) and counts outside [0, max_budget]: the count is clamped,
    invalid positions are left out of the softmax, and the output equals the
    oracle's attention over the valid positions (0 when none is valid)."""
    import learned_tree_routed_amd as alhr
    torch, dev = torch_dev
    w = Workload("attend_invalid", 31, 1, 2, 512, 64, "clustered")
    Q, K, V, _ = host_inputs(w)
    cfg = w.config(max_budget=32)
    rng = np.random.default_rng(31)
    T, mb = w.T, cfg.max_budget
    idx = rng.integers(0, T, size=(1, 2, T, mb)).astype(np.int32)
    bad = rng.random(size=idx.shape) < 0.25
    idx[bad] = rng.choice(np.array([-1, -7, T, T + 5, 1 << 30, -(1 << 30)], dtype=np.int32),
                          size=int(bad.sum()))
    cnt = rng.integers(-3, mb + 8, size=(1, 2, T)).astype(np.int32)
    idx[0, 0, 7, :] = -1            # a query with no valid position at all
    cnt[0, 0, 7] = 5
    q, k, v, ti, tc = to_dev(torch, dev, Q, K, V, idx, cnt)
    say("alhr_sparse_attend with invalid caller indices, T512 d64")
    O = alhr.alhr_sparse_attend(cfg, q, k, v, ti, tc)
    torch.cuda.synchronize()
    O = O.cpu().numpy()
    worst = 0.0
    for h in range(2):
        for t in range(T):
            c = int(np.clip(cnt[0, h, t], 0, mb))
            sel = idx[0, h, t, :c]
            sel = sel[(sel >= 0) & (sel < T)]
            if len(sel) == 0:
                assert not O[0, h, t].any(), (h, t)
                continue
            ref = oracle.attend(sel, Q[0, h, t], K[0, h], V[0, h], cfg.scale)
            worst = max(worst, float(np.abs(O[0, h, t] - ref).max()))
    assert worst <= ATOL, worst


def test_route_d64_two_cover_passes_at_2_17(torch_dev):
    """d = 64 at T = 2^17 (B1 H8, the length sweep's top point).  A wave
    scores 16 rows per pass at d = 64 and the cover of [0, m) has a root on
    every set bit of m, levels 0..16 here, so every query with m >= 2^16 takes
    a second cover pass for its level-16 root.  Sampled queries of two pairs
    (the first and last, m = 2^16 exactly, the m below T with the most set
    bits, random) against the oracle."""
    import learned_tree_routed_amd as alhr
    from synth import device as sd
    from synth.workloads import pair_keys, pair_query_rows, pair_value_rows
    torch, dev = torch_dev
    T, d = 1 << 17, 64
    w = Workload("t2e17", 8, 1, 8, T, d, "clustered")
    cfg = w.config()
    shape = (1, 8, T, d)
    K = sd.keys_(torch.empty(shape, dtype=torch.int8, device=dev), w.seed)
    Qd = sd.queries_(torch.empty(shape, dtype=torch.int8, device=dev), w.seed)
    V = sd.values_(torch.empty(shape, dtype=torch.float32, device=dev), w.seed)
    W = synth.predictor_weights(w.seed, w.n_classes, d)
    say("alhr_forward B1 H8 T2^17 d64 (two cover passes)")
    out = alhr.alhr_forward(cfg, Qd, K, V, torch.from_numpy(W).to(dev))
    torch.cuda.synchronize()
    # t = m + 3 when the window holds 4 keys; m = 2^17 - 5 has 15 set bits
    many = [m + 3 for m in range(T - 64, T - 3) if bin(m).count("1") >= 15]
    rng = np.random.default_rng(w.seed)
    ts = np.unique(np.r_[0, 1, 2, 3, 4, 65535, 65538, 65539, 65540, T - 2, T - 1, many,
                         rng.integers(1 << 16, T, 48)]).astype(np.int32)
    for h in (0, 5):
        Kp = pair_keys(w, 0, h)
        Qp = pair_query_rows(w, 0, h, np.arange(T))
        Vp = pair_value_rows(w, 0, h, np.arange(T))
        ref = oracle.pair_forward(Qp, Kp, Vp, W=W, window=cfg.window, scale=cfg.scale, ts=ts)
        np.testing.assert_array_equal(out["budget"][0, h].cpu().numpy()[ts], ref["budget"])
        np.testing.assert_array_equal(out["count"][0, h].cpu().numpy()[ts], ref["count"])
        np.testing.assert_array_equal(out["idx"][0, h].cpu().numpy()[ts], ref["idx"])
        err = np.abs(out["O"][0, h].cpu().numpy()[ts] - ref["O"]).max()
        assert err <= ATOL, (h, err)


def random_config(i):
    """The i-th seeded random small configuration: shapes, window, budget
    mode and the magnitude of the int8 queries and keys (which sets how many
    tree levels are stored as int16)."""
    rng = np.random.default_rng(9000 + i)
    d = int(rng.choice([16, 32, 64, 128, 256]))
    a = int(rng.choice([1, 3, 8, 31, 127]))
    T = 1 << int(rng.integers(1, 10 if a == 127 else 11))
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
    window = int(rng.integers(1, 10))
    max_budget = int(rng.integers(3, 129))
    if rng.random() < 0.5:
        mode = dict(fixed=int(rng.integers(1, max_budget + 1)), n_classes=32, kpc=3)
    else:
        mode = dict(fixed=0, n_classes=int(rng.integers(1, 33)), kpc=int(rng.integers(1, 5)))
    return rng, dict(B=B, H=H, T=T, d=d, a=a, window=window, max_budget=max_budget, **mode)


@pytest.mark.parametrize("i", range(16))
def test_random_configs_every_query(torch_dev, i):
    """Seeded random small configurations (T = 2 .. 1024, d = 16 .. 256,
    windows 1 .. 9, fixed or predicted budgets with 1 .. 32 classes of 1 .. 4
    keys, budgets up to 128, |Q|, |K| up to 1 .. 127): the tree, budgets,
    index sets and counts bit-exact and the outputs within 1e-4 of the oracle
    on every query of every pair."""
    import learned_tree_routed_amd as alhr
    torch, dev = torch_dev
    rng, c = random_config(i)
    B, H, T, d, a = c["B"], c["H"], c["T"], c["d"], c["a"]
    Q = rng.integers(-a, a + 1, size=(B, H, T, d)).astype(np.int8)
    K = rng.integers(-a, a + 1, size=(B, H, T, d)).astype(np.int8)
    V = rng.standard_normal(size=(B, H, T, d)).astype(np.float32)
    W = None if c["fixed"] else rng.integers(-4, 5, size=(c["n_classes"], 2 * d)).astype(np.int8)
    cfg = alhr.Config(batch=B, heads=H, T=T, d=d, window=c["window"], n_classes=c["n_classes"],
                      keys_per_class=c["kpc"], max_budget=c["max_budget"], kmax=a, qmax=a, wmax=4)
    w = Workload("random%d" % i, 0, B, H, T, d, "uniform", fixed_budget=c["fixed"],
                 window=c["window"], n_classes=c["n_classes"], keys_per_class=c["kpc"],
                 max_budget=c["max_budget"])
    say("random config", i, c)
    out = run_forward(torch, dev, w, Q, K, V, W, cfg=cfg)
    for b in range(B):
        for h in range(H):
            check_nodes(out["nodes"], K, b, h, cfg)
            check_pair(w, cfg, Q, K, V, W, out, b, h)


# ---------------------------------------------------------------- edges ---
EDGE_CASES = [
    # name, T, d, window, fixed budget (0 = predictor), max_budget, kind
    ("T2", 2, 16, 4, 2, 96, "uniform"),
    ("T4_w1_b1", 4, 16, 1, 1, 96, "uniform"),
    ("T8_w1", 8, 32, 1, 5, 96, "uniform"),
    ("window_over_budget", 64, 32, 40, 16, 96, "uniform"),
    ("budget_128", 512, 16, 4, 128, 128, "uniform"),
    ("budget_127_w1", 512, 32, 1, 127, 128, "uniform"),
    ("d128", 256, 128, 4, 37, 96, "uniform"),
    ("d256", 128, 256, 4, 50, 96, "uniform"),
    ("d16_predictor", 512, 16, 4, 0, 96, "clustered"),
    ("d128_predictor", 1024, 128, 4, 0, 96, "clustered"),
    ("d32_predictor_w2", 2048, 32, 2, 0, 96, "clustered"),
]


@pytest.mark.parametrize("case", EDGE_CASES, ids=[c[0] for c in EDGE_CASES])
def test_edge_cases_every_query(torch_dev, case):
    torch, dev = torch_dev
    name, T, d, window, fb, mb, kind = case
    w = Workload(name, 11, 2, 2, T, d, kind, fixed_budget=fb, window=window, max_budget=mb)
    Q, K, V, W = host_inputs(w)
    cfg = w.config()
    out = run_forward(torch, dev, w, Q, K, V, W, cfg=cfg)
    for b in range(2):
        for h in range(2):
            check_nodes(out["nodes"], K, b, h, cfg)
            check_pair(w, cfg, Q, K, V, W, out, b, h)


def test_zero_query_and_planted_keys(torch_dev):
    """All-tie queries (order falls to position) and planted keys, on the GPU."""
    torch, dev = torch_dev
    T, d = 512, 64
    w = Workload("planted", 12, 1, 2, T, d, "uniform", fixed_budget=24)
    rng = np.random.default_rng(5)
    Q = np.zeros((1, 2, T, d), np.int8)
    K = rng.integers(-4, 5, size=(1, 2, T, d)).astype(np.int8)
    Q[0, 1] = rng.integers(1, 5, size=(T, d))
    K[0, 1] = 0
    planted = rng.choice(T, size=40, replace=False)
    K[0, 1, planted] = rng.integers(1, 5, size=(40, d))
    V = synth.values(12, 1, 2, d, 0, T)
    out = run_forward(torch, dev, w, Q, K, V, None)
    cfg = w.config()
    for h in range(2):
        check_pair(w, cfg, Q, K, V, None, out, 0, h)
    t = T - 1
    sel = out["idx"][0, 0, t, :24]
    np.testing.assert_array_equal(sel[:20], np.arange(20))   # ties: lowest positions


def test_wide_int32_path(torch_dev):
    """Bounds that rule out 24-bit multiplies (kmax * T/2 >= 2^23) take the
    full 32-bit scoring path; same parity bar on sampled queries."""
    import learned_tree_routed_amd as alhr
    torch, dev = torch_dev
    T, d = 1 << 18, 16
    rng = np.random.default_rng(6)
    K = rng.integers(-127, 128, size=(1, 1, T, d)).astype(np.int8)
    Q = rng.integers(-4, 5, size=(1, 1, T, d)).astype(np.int8)
    V = synth.values(13, 1, 1, d, 0, T)
    w = Workload("wide", 13, 1, 1, T, d, "uniform", fixed_budget=40)
    cfg = w.config(kmax=127, qmax=4)
    assert cfg.kmax * (T // 2) >= 1 << 23
    out = run_forward(torch, dev, w, Q, K, V, None, cfg=cfg)
    check_nodes(out["nodes"], K, 0, 0, cfg)
    ts = sample_ts(T, np.random.default_rng(1), 256)
    check_pair(w, cfg, Q, K, V, None, out, 0, 0, ts=ts)


def test_budget_array_values_are_clamped(torch_dev):
    import learned_tree_routed_amd as alhr
    torch, dev = torch_dev
    w = WORKLOADS["tiny"]
    Q, K, V, _ = host_inputs(w)
    cfg = w.config()
    q, k, v = to_dev(torch, dev, Q, K, V)
    nodes = alhr.alhr_build_tree(cfg, k)
    raw = np.full((1, 1, w.T), 7, np.int32)
    raw[0, 0, ::3] = 0
    raw[0, 0, 1::3] = 500
    say("alhr_route with out-of-range budgets (clamped)")
    idx, cnt = alhr.alhr_route(cfg, q, k, nodes, torch.from_numpy(raw).to(dev))
    torch.cuda.synchronize()
    clamped = np.clip(raw, 1, cfg.max_budget)[0, 0]
    np.testing.assert_array_equal(cnt.cpu().numpy()[0, 0], np.minimum(clamped, np.arange(w.T) + 1))


def test_invalid_arguments_rejected_on_device(torch_dev):
    import learned_tree_routed_amd as alhr
    torch, dev = torch_dev
    cfg = alhr.Config(batch=1, heads=1, T=64, d=32)
    k = torch.zeros((1, 1, 64, 32), dtype=torch.int8, device=dev)
    nodes = alhr.alhr_build_tree(cfg, k)
    with pytest.raises(alhr.AlhrError) as e:
        alhr.alhr_route(cfg, k, k, nodes, None, fixed_budget=0)
    assert e.value.status == -1
    bad = alhr.Config(batch=1, heads=1, T=64, d=48)
    with pytest.raises(alhr.AlhrError) as e:
        alhr.alhr_build_tree(bad, torch.zeros((1, 1, 64, 48), dtype=torch.int8, device=dev))
    assert e.value.status == -4


# ------------------------------------------------------- dense baseline ---
def dense_oracle_rows(Q, K, V, scale, ts):
    """The oracle's attention over all past keys for the queries ts."""
    return np.stack([oracle.attend(np.arange(t + 1, dtype=np.int32), Q[t], K, V, scale) for t in ts])


@pytest.mark.parametrize("T,d", [(16, 32), (64, 32), (256, 64), (128, 128), (64, 256), (1024, 64)])
def test_dense_attention_every_query(torch_dev, T, d):
    import learned_tree_routed_amd as alhr
    torch, dev = torch_dev
    w = Workload("dense", 21, 2, 2, T, d, "clustered")
    Q, K, V, _ = host_inputs(w)
    cfg = w.config()
    q, k, v = to_dev(torch, dev, Q, K, V)
    say("alhr_dense_attend B2 H2 T%d d%d" % (T, d))
    O = alhr.alhr_dense_attend(cfg, q, k, v)
    torch.cuda.synchronize()
    O = O.cpu().numpy()
    for b in range(2):
        for h in range(2):
            ref = dense_oracle_rows(Q[b, h], K[b, h], V[b, h], cfg.scale, range(T))
            err = np.abs(O[b, h] - ref).max()
            assert err <= ATOL, "pair (%d, %d): max |O - oracle| = %g" % (b, h, err)


@pytest.mark.parametrize("i", range(8))
def test_dense_attention_random_configs(torch_dev, i):
    """Seeded random shapes for the dense baseline (T = 4 .. 1024, d = 32 ..
    256, 1 .. 3 pairs, |Q|, |K| up to 127, N(0, 1) values): every query
    within 1e-4 of the oracle's attention over all past keys."""
    import learned_tree_routed_amd as alhr
    torch, dev = torch_dev
    rng = np.random.default_rng(6000 + i)
    d = int(rng.choice([32, 64, 128, 256]))
    T = 1 << int(rng.integers(2, 11))
    a = int(rng.choice([1, 4, 31, 127]))
    B, H = 1, int(rng.integers(1, 4))
    Q = rng.integers(-a, a + 1, size=(B, H, T, d)).astype(np.int8)
    K = rng.integers(-a, a + 1, size=(B, H, T, d)).astype(np.int8)
    V = rng.standard_normal(size=(B, H, T, d)).astype(np.float32)
    cfg = alhr.Config(batch=B, heads=H, T=T, d=d, kmax=a, qmax=a)
    q, k, v = to_dev(torch, dev, Q, K, V)
    say("alhr_dense_attend random config", i, "H%d T%d d%d |q|,|k| <= %d" % (H, T, d, a))
    O = alhr.alhr_dense_attend(cfg, q, k, v)
    torch.cuda.synchronize()
    O = O.cpu().numpy()
    for h in range(H):
        ref = dense_oracle_rows(Q[0, h], K[0, h], V[0, h], cfg.scale, range(T))
        err = np.abs(O[0, h] - ref).max()
        assert err <= ATOL, "head %d: max |O - oracle| = %g" % (h, err)


def test_dense_attention_full_size_sampled(torch_dev):
    import learned_tree_routed_amd as alhr
    torch, dev = torch_dev
    w = WORKLOADS["t16k"]
    Q, K, V, _ = host_inputs(w)
    cfg = w.config()
    q, k, v = to_dev(torch, dev, Q, K, V)
    say("alhr_dense_attend t16k")
    O = alhr.alhr_dense_attend(cfg, q, k, v)
    torch.cuda.synchronize()
    O = O.cpu().numpy()
    rng = np.random.default_rng(3)
    for h in (0, 3, 7):
        ts = sorted(set(rng.choice(w.T, 24, replace=False).tolist()) | {0, 31, 32, w.T - 1})
        ref = dense_oracle_rows(Q[0, h], K[0, h], V[0, h], cfg.scale, ts)
        err = np.abs(O[0, h, ts] - ref).max()
        assert err <= ATOL, "head %d: max |O - oracle| = %g" % (h, err)


def test_dense_equals_routing_with_full_budget(torch_dev):
    """With the budget covering every past key the routed path is dense
    attention: both kernels must agree on the same inputs.  The dense kernel
    forms P.V from bf16 heads and tails (three products), exact to within
    3 * 2^-18 * max|v| per output; the routed kernel is plain fp32."""
    import learned_tree_routed_amd as alhr
    torch, dev = torch_dev
    T = 64
    w = Workload("dense_vs_route", 22, 1, 4, T, 64, "clustered", fixed_budget=64)
    Q, K, V, _ = host_inputs(w)
    cfg = w.config()
    q, k, v = to_dev(torch, dev, Q, K, V)
    dense = alhr.alhr_dense_attend(cfg, q, k, v)
    routed = alhr.alhr_forward(cfg, q, k, v, None, fixed_budget=64)
    torch.cuda.synchronize()
    bound = 3 * 2.0 ** -18 * float(np.abs(V).max()) + 2e-6   # + fp32 rounding of both sums
    assert (dense - routed["O"]).abs().max().item() <= bound


def test_launches_split_by_query_range(torch_dev):
    """More queries than one launch covers (2^24, so that the work-item count
    of a dispatch stays 32-bit): 5 x 205 pairs of T = 16384 (16.8 M queries,
    d = 16, budget 8) run as two launches of the route and attention kernels.
    Every count is exact, and sampled queries of the pairs on both sides of the
    split equal the oracle."""
    import learned_tree_routed_amd as alhr
    from synth import device as sd
    from synth.workloads import pair_keys, pair_query_rows, pair_value_rows
    torch, dev = torch_dev
    B, H, T, d = 5, 205, 16384, 16
    assert B * H * T > 1 << 24
    w = Workload("split_launch", 9, B, H, T, d, "clustered", fixed_budget=8, max_budget=8)
    cfg = w.config()
    K = sd.keys_(torch.empty((B, H, T, d), dtype=torch.int8, device=dev), w.seed)
    Q = sd.queries_(torch.empty((B, H, T, d), dtype=torch.int8, device=dev), w.seed)
    V = sd.values_(torch.empty((B, H, T, d), dtype=torch.float32, device=dev), w.seed)
    say("alhr_forward B5 H205 T16384 d16 fixed 8 (two launches per kernel)")
    out = alhr.alhr_forward(cfg, Q, K, V, None, fixed_budget=8)
    torch.cuda.synchronize()
    want = torch.clamp(torch.arange(T, device=dev, dtype=torch.int32) + 1, max=8)
    assert torch.equal(out["count"], want.expand(B, H, T))
    # query index q = pair * T + (T - 1 - t) in the route kernel: the split at
    # 2^24 falls between pairs 1023 = (4, 203) and 1024 = (4, 204)
    ts = np.array([0, 1, 7, 8, 100, 5000, 12345, T - 2, T - 1])
    for pair in (1023, 1024):
        b, h = divmod(pair, H)
        Kp = pair_keys(w, b, h)
        Qp = pair_query_rows(w, b, h, np.arange(T))
        Vp = pair_value_rows(w, b, h, np.arange(T))
        ref = oracle.pair_forward(Qp, Kp, Vp, W=None, fixed_budget=8, window=cfg.window,
                                  keys_per_class=cfg.keys_per_class, max_budget=8,
                                  scale=cfg.scale, ts=ts)
        np.testing.assert_array_equal(out["idx"][b, h].cpu().numpy()[ts], ref["idx"])
        err = np.abs(out["O"][b, h].cpu().numpy()[ts] - ref["O"]).max()
        assert err <= ATOL, "pair %d: max |O - oracle| = %g" % (pair, err)
    # the attention kernel on its own over the same sets, also split
    O2 = alhr.alhr_sparse_attend(cfg, Q, K, V, out["idx"], out["count"])
    torch.cuda.synchronize()
    assert torch.equal(O2, out["O"])


def test_graph_replays_of_a_step_match_eager(torch_dev):
    """The bench's timed step (build + predict + route/attend captured in one
    HIP graph): every replay, with eager work on the same buffers in between,
    gives the eager outputs exactly, and those equal the oracle's on sampled
    queries."""
    import bench
    import learned_tree_routed_amd as alhr
    torch, dev = torch_dev
    w = WORKLOADS["t1k"]
    Q, K, V, W = host_inputs(w, B=2, H=4)
    w = Workload("t1k_graph", w.seed, 2, 4, w.T, w.d, w.kind)
    cfg = w.config()
    q, k, v, wt = to_dev(torch, dev, Q, K, V, W)
    rows = (w.B, w.H, w.T, w.d)
    nodes = torch.empty(rows, dtype=torch.int32, device=dev)
    budget = torch.empty((w.B, w.H, w.T), dtype=torch.int32, device=dev)
    idx = torch.empty((w.B, w.H, w.T, cfg.max_budget), dtype=torch.int32, device=dev)
    count = torch.empty((w.B, w.H, w.T), dtype=torch.int32, device=dev)
    O = torch.empty(rows, dtype=torch.float32, device=dev)
    ws = torch.empty(max(alhr.alhr_workspace_bytes(cfg), 256), dtype=torch.uint8, device=dev)
    outs = (nodes, budget, idx, count, O)
    for t in outs:   # the tail of the compact tree table is never written
        t.zero_()
    say("eager step, t1k B2 H4")
    bench.step_calls(alhr, cfg, q, k, v, wt, nodes, budget, ws, 0, idx, count, O)
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    say("capture step in a graph")
    graph = bench.capture_step(torch, lambda: bench.step_calls(alhr, cfg, q, k, v, wt, nodes, budget,
                                                               ws, 0, idx, count, O))
    for rep in range(3):
        for t in outs:
            t.zero_()
        # eager work on the same buffers between replays
        alhr.alhr_build_tree(cfg, k, nodes)
        torch.cuda.synchronize()
        say("graph replay", rep)
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, ref):
            assert torch.equal(a, b)
    got = {name: t.cpu().numpy() for name, t in
           (("nodes", nodes), ("budget", budget), ("idx", idx), ("count", count), ("O", O))}
    ts = np.array([0, 1, 2, 5, 100, 511, 1000, 1023])
    for (b, h) in ((0, 0), (1, 3)):
        check_pair(w, cfg, Q, K, V, W, got, b, h, ts=ts)


PREP_CASES = [
    # T, d, batch, heads: one shared pass (T2, T8), two (T1024 d64: 8 + 2 levels), three
    # build passes (T2^17 d64: 8 + 8 + 1 levels), T below one predictor chunk
    (2, 16, 1, 3), (8, 32, 2, 1), (128, 16, 1, 2), (1024, 64, 2, 2), (4096, 128, 1, 2),
    (2048, 256, 1, 1), (1 << 17, 64, 1, 1),
]


@pytest.mark.parametrize("T,d,B,H", PREP_CASES, ids=["T%d_d%d_B%d_H%d" % c for c in PREP_CASES])
def test_prepare_equals_build_and_predict(torch_dev, T, d, B, H):
    """alhr_prepare (tree and predictor sharing launches) writes exactly the
    tree and budgets of alhr_build_tree + alhr_predict_budget, and the budgets
    equal the oracle's on sampled pairs; with W NULL it builds the tree only."""
    import learned_tree_routed_amd as alhr
    torch, dev = torch_dev
    w = Workload("prep", 9, B, H, T, d, "clustered")
    Q, K, V, W = host_inputs(w)
    cfg = w.config()
    q, k, wt = to_dev(torch, dev, Q, K, W)
    say("alhr_prepare", "B%d H%d T%d d%d" % (B, H, T, d))
    nodes, bud = alhr.alhr_prepare(cfg, q, k, wt)
    nodes2 = alhr.alhr_build_tree(cfg, k)
    bud2 = alhr.alhr_predict_budget(cfg, q, k, wt)
    nodes3, none = alhr.alhr_prepare(cfg, None, k)
    torch.cuda.synchronize()
    assert none is None
    assert torch.equal(bud, bud2)
    # compare the stored rows (the tail of a compact table is never written)
    l16 = alhr.alhr_tree_int16_levels(cfg)
    a, b2, c = (x.cpu().numpy() for x in (nodes, nodes2, nodes3))
    for bb in range(B):
        for hh in range(H):
            ref_rows = decode_tree(b2[bb, hh], l16)[1:]
            np.testing.assert_array_equal(decode_tree(a[bb, hh], l16)[1:], ref_rows)
            np.testing.assert_array_equal(decode_tree(c[bb, hh], l16)[1:], ref_rows)
    ts = np.unique(np.r_[0, 1, T - 1, np.random.default_rng(T).integers(0, T, 16)])
    for (b, h) in ((0, 0), (B - 1, H - 1)):
        ref = oracle.pair_forward(Q[b, h], K[b, h], V[b, h], W=W, window=cfg.window,
                                  keys_per_class=cfg.keys_per_class, max_budget=cfg.max_budget,
                                  scale=cfg.scale, ts=ts)
        np.testing.assert_array_equal(bud[b, h].cpu().numpy()[ts], ref["budget"])
    check_nodes(a, K, 0, 0, cfg)
