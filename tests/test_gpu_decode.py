"""GPU parity of the decode path (append + decode step) and of the device
input generator.

The decode oracle replays the same appends on the CPU for a pair and routes
and attends the one query per step; tree rows, budgets, index sets and
counts must match bit for bit, outputs within 1e-4.  The full-size cache
(64 sequences x 16 heads, 2^17 positions, d = 128; 144 GiB of keys, values
and tree) is generated on the device and checked on sampled pairs.
"""
import sys

import numpy as np
import pytest

import oracle
import synth
from synth.workloads import WORKLOADS, Workload, host_inputs, pair_keys, pair_query_rows, pair_value_rows
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


def test_device_generator_matches_host(torch_dev):
    from synth import device as sd
    torch, dev = torch_dev
    w = WORKLOADS["t1k"]
    say("device generator vs host, t1k slice")
    Q, K, V, W = host_inputs(w, t0=100, nt=300, B=3, H=5)
    k = sd.keys_(torch.zeros((3, 5, 300, 64), dtype=torch.int8, device=dev), w.seed, 100)
    q = sd.queries_(torch.zeros((3, 5, 300, 64), dtype=torch.int8, device=dev), w.seed, 100)
    v = sd.values_(torch.zeros((3, 5, 300, 64), dtype=torch.float32, device=dev), w.seed, 100)
    wt = sd.weights_(torch.zeros((32, 128), dtype=torch.int8, device=dev), w.seed)
    u = sd.uniform_i8_(torch.zeros((3, 5, 300, 64), dtype=torch.int8, device=dev), 1,
                       synth.STREAM_UK, -4, 4, 100)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(k.cpu().numpy(), K)
    np.testing.assert_array_equal(q.cpu().numpy(), Q)
    np.testing.assert_array_equal(v.cpu().numpy(), V)
    np.testing.assert_array_equal(wt.cpu().numpy(), W)
    np.testing.assert_array_equal(u.cpu().numpy(),
                                  synth.uniform_i8(1, synth.STREAM_UK, -4, 4, 3, 5, 64, 100, 300))
    # strided rows (prefix of a larger cache), the rest untouched
    big = torch.zeros((2, 3, 64, 64), dtype=torch.int8, device=dev)
    sd.keys_(big, w.seed, 0, 40)
    torch.cuda.synchronize()
    b = big.cpu().numpy()
    np.testing.assert_array_equal(b[:, :, :40], synth.clustered_keys(w.seed, 2, 3, 64, 0, 40))
    assert not b[:, :, 40:].any()


def decode_oracle_pair(w, b, h, n0, steps, K_pair, q_rows, W, cfg):
    """Replays the decode steps of one pair on the CPU; returns per-step
    (budget, idx, count, O) and the final tree and prefix."""
    Kc = np.zeros_like(K_pair)
    Kc[:n0] = K_pair[:n0]
    V = np.zeros((w.T, w.d), np.float32)
    have = np.zeros(w.T, dtype=bool)          # value rows drawn so far
    nodes = oracle.build_tree(Kc)
    pre = Kc.astype(np.int64).sum(axis=0)
    res = []
    for s in range(steps):
        p = n0 + s
        v_new = pair_value_rows(w, b, h, [p])[0]
        oracle.append(p, K_pair[p], v_new, Kc, V, nodes, pre)
        have[p] = True
        q = q_rows[s]
        if W is not None:
            bud, _ = oracle.budget(q, pre, W, cfg.keys_per_class, cfg.max_budget)
        else:
            bud = w.fixed_budget
        idx, _, c, _ = oracle.route(p, bud, q, Kc, nodes, cfg.window, cfg.max_budget)
        need = idx[:c]
        missing = need[~have[need]]
        if len(missing):
            V[missing] = pair_value_rows(w, b, h, missing)
            have[missing] = True
        o = oracle.attend(need, q, Kc, V, cfg.scale)
        res.append((bud, idx, c, o))
    return res, nodes, pre


def run_decode(torch, dev, w, cfg, K_dev, V_dev, nodes, prefix, W_dev, n0, steps, pairs,
               q_src, k_src, v_src, fused=False):
    """fused: alhr_append_decode (one launch per step), else alhr_append then
    alhr_decode_step."""
    import learned_tree_routed_amd as alhr
    got = {pr: [] for pr in pairs}
    bsel = torch.tensor([p[0] for p in pairs], device=dev)
    hsel = torch.tensor([p[1] for p in pairs], device=dev)
    for s in range(steps):
        p = n0 + s
        k_new, v_new, q_new = k_src(p), v_src(p), q_src(p)
        bud = torch.empty((cfg.batch, cfg.heads), dtype=torch.int32, device=dev)
        if fused:
            idx, cnt, O = alhr.alhr_append_decode(cfg, p, k_new, v_new, q_new, K_dev, V_dev, nodes,
                                                  prefix, W_dev, fixed_budget=w.fixed_budget,
                                                  budget=bud)
        else:
            alhr.alhr_append(cfg, p, k_new, v_new, K_dev, V_dev, nodes, prefix)
            idx, cnt, O = alhr.alhr_decode_step(cfg, p, q_new, K_dev, V_dev, nodes, prefix, W_dev,
                                                fixed_budget=w.fixed_budget, budget=bud)
        sb, si, sc, so = (bud[bsel, hsel].cpu().numpy(), idx[bsel, hsel].cpu().numpy(),
                          cnt[bsel, hsel].cpu().numpy(), O[bsel, hsel].cpu().numpy())
        for k, pr in enumerate(pairs):
            got[pr].append((sb[k], si[k], sc[k], so[k]))
    torch.cuda.synchronize()
    return got


def compare(got, ref):
    assert len(got) == len(ref) > 0
    for s, ((gb, gi, gc, go), (rb, ri, rc, ro)) in enumerate(zip(got, ref)):
        assert gb == rb, "step %d: budget %d vs %d" % (s, gb, rb)
        assert gc == rc, "step %d: count %d vs %d" % (s, gc, rc)
        np.testing.assert_array_equal(gi, ri, err_msg="step %d" % s)
        err = np.abs(go - ro).max()
        assert err <= ATOL, "step %d: max |O - oracle| = %g" % (s, err)


@pytest.mark.parametrize("fused", [False, True], ids=["two_launches", "fused"])
@pytest.mark.parametrize("d,fixed", [(128, 0), (64, 0), (32, 20)])
def test_decode_small_every_step(torch_dev, d, fixed, fused):
    import learned_tree_routed_amd as alhr
    torch, dev = torch_dev
    T, n0, steps = 4096, 4096 - 48, 48
    w = Workload("decode_small", 7, 2, 3, T, d, "clustered", fixed_budget=fixed)
    cfg = w.config()
    Q, K, V, W = host_inputs(w)
    say("decode small: B2 H3 T%d d%d, %d steps" % (T, d, steps))
    Kd = torch.zeros((2, 3, T, d), dtype=torch.int8, device=dev)
    Vd = torch.zeros((2, 3, T, d), dtype=torch.float32, device=dev)
    Kd[:, :, :n0] = torch.from_numpy(K[:, :, :n0]).to(dev)
    Vd[:, :, :n0] = torch.from_numpy(V[:, :, :n0]).to(dev)
    nodes = alhr.alhr_build_tree(cfg, Kd)
    prefix = alhr.alhr_prefix_from_tree(cfg, n0, Kd, nodes)
    Wd = None if W is None else torch.from_numpy(W).to(dev)
    Kh, Vh, Qh = (torch.from_numpy(x).to(dev) for x in (K, V, Q))
    pairs = [(b, h) for b in range(2) for h in range(3)]
    got = run_decode(torch, dev, w, cfg, Kd, Vd, nodes, prefix, Wd, n0, steps, pairs,
                     lambda p: Qh[:, :, p].contiguous(), lambda p: Kh[:, :, p].contiguous(),
                     lambda p: Vh[:, :, p].contiguous(), fused=fused)
    l16 = alhr.alhr_tree_int16_levels(cfg)
    for (b, h) in pairs:
        ref, ref_nodes, ref_pre = decode_oracle_pair(w, b, h, n0, steps, K[b, h], Q[b, h, n0:], W, cfg)
        compare(got[(b, h)], ref)
        np.testing.assert_array_equal(decode_tree(nodes[b, h].cpu().numpy(), l16)[1:],
                                      ref_nodes[1:])
        np.testing.assert_array_equal(prefix[b, h].cpu().numpy(), ref_pre)
    # after the appends, the tree equals a fresh build of the full keys
    rebuilt = alhr.alhr_build_tree(cfg, Kh)
    torch.cuda.synchronize()
    for (b, h) in pairs:
        np.testing.assert_array_equal(decode_tree(rebuilt[b, h].cpu().numpy(), l16),
                                      decode_tree(nodes[b, h].cpu().numpy(), l16))
    # and every step's rows equal the prefill rows of the same positions on
    # the final cache: a query at position p reads only subtrees of [0, p]
    # and the key sum up to p, which later appends leave unchanged (the
    # decode bench's load counts rest on this)
    full = alhr.alhr_forward(cfg, Qh, Kh, Vh, Wd, fixed_budget=fixed)
    torch.cuda.synchronize()
    f_idx, f_cnt = full["idx"].cpu().numpy(), full["count"].cpu().numpy()
    for (b, h) in pairs:
        for s_, row in enumerate(got[(b, h)]):
            np.testing.assert_array_equal(row[1], f_idx[b, h, n0 + s_])
            assert int(row[2]) == int(f_cnt[b, h, n0 + s_])


@pytest.mark.parametrize("fused", [False, True], ids=["two_launches", "fused"])
def test_decode_full_cache_sampled_pairs(torch_dev, fused):
    """64 x 16 pairs, capacity 2^17, d = 128, 2^17 - 128 prefilled keys and
    128 appended tokens: every step compared on 8 sampled pairs.  The fused
    case is the launch configuration the decode bench times."""
    import learned_tree_routed_amd as alhr
    from synth import device as sd
    torch, dev = torch_dev
    w = WORKLOADS["decode"]
    cfg = w.config()
    B, H, T, d, n0, steps = w.B, w.H, w.T, w.d, w.n0, w.steps
    say("decode full cache: B%d H%d T%d d%d n0=%d steps=%d (144 GiB)" % (B, H, T, d, n0, steps))
    Kd = torch.zeros((B, H, T, d), dtype=torch.int8, device=dev)
    Vd = torch.zeros((B, H, T, d), dtype=torch.float32, device=dev)
    nodes = torch.empty((B, H, T, d), dtype=torch.int32, device=dev)
    sd.keys_(Kd, w.seed, 0, n0)
    sd.values_(Vd, w.seed, 0, n0)
    alhr.alhr_build_tree(cfg, Kd, nodes)
    prefix = alhr.alhr_prefix_from_tree(cfg, n0, Kd, nodes)
    Wd = sd.weights_(torch.empty((32, 2 * d), dtype=torch.int8, device=dev), w.seed)
    kbuf = torch.empty((B, H, 1, d), dtype=torch.int8, device=dev)
    qbuf = torch.empty((B, H, 1, d), dtype=torch.int8, device=dev)
    vbuf = torch.empty((B, H, 1, d), dtype=torch.float32, device=dev)
    rng = np.random.default_rng(w.seed)
    pairs = sorted({(int(rng.integers(0, B)), int(rng.integers(0, H))) for _ in range(8)})
    pairs = [(0, 0), (B - 1, H - 1)] + [p for p in pairs if p not in ((0, 0), (B - 1, H - 1))][:6]
    got = run_decode(torch, dev, w, cfg, Kd, Vd, nodes, prefix, Wd, n0, steps, pairs,
                     lambda p: sd.queries_(qbuf, w.seed, p, 1).view(B, H, d),
                     lambda p: sd.keys_(kbuf, w.seed, p, 1).view(B, H, d),
                     lambda p: sd.values_(vbuf, w.seed, p, 1).view(B, H, d), fused=fused)
    say("decode full cache: device steps done, oracle replay of %d pairs" % len(pairs))
    import time
    t_replay = time.time()
    W = synth.predictor_weights(w.seed, w.n_classes, d)
    l16 = alhr.alhr_tree_int16_levels(cfg)
    for (b, h) in pairs:
        K_pair = pair_keys(w, b, h)
        q_rows = pair_query_rows(w, b, h, np.arange(n0, n0 + steps))
        ref, ref_nodes, ref_pre = decode_oracle_pair(w, b, h, n0, steps, K_pair, q_rows, W, cfg)
        compare(got[(b, h)], ref)
        np.testing.assert_array_equal(prefix[b, h].cpu().numpy(), ref_pre)
        # the top 4095 rows (levels 6..17), int16 and int32 rows both
        top = decode_tree(nodes[b, h].cpu().numpy(), l16)[1:4096]
        np.testing.assert_array_equal(top, ref_nodes[1:4096])
    say("decode full cache: replayed %d pairs x %d steps in %.1f s" % (len(pairs), steps,
                                                                   time.time() - t_replay))
    del Kd, Vd, nodes
    torch.cuda.empty_cache()


@pytest.mark.parametrize("fused", [False, True], ids=["two_launches", "fused"])
@pytest.mark.parametrize("T,d,fixed", [(64, 32, 0), (128, 16, 5), (2, 16, 1), (256, 256, 0)])
def test_decode_from_empty_cache_every_step(torch_dev, T, d, fixed, fused):
    """Decoding from position 0 to T - 1: the first steps are served by the
    window alone (r = 0), the covers are tiny, and the last step fills the
    cache; every step, the tree and the prefix equal the oracle's replay."""
    import learned_tree_routed_amd as alhr
    torch, dev = torch_dev
    w = Workload("decode_empty", 8, 1, 2, T, d, "clustered", fixed_budget=fixed)
    cfg = w.config()
    Q, K, V, W = host_inputs(w)
    say("decode from empty: B1 H2 T%d d%d fixed %d" % (T, d, fixed))
    Kd = torch.zeros((1, 2, T, d), dtype=torch.int8, device=dev)
    Vd = torch.zeros((1, 2, T, d), dtype=torch.float32, device=dev)
    nodes = alhr.alhr_build_tree(cfg, Kd)
    prefix = alhr.alhr_prefix_from_tree(cfg, 0, Kd, nodes)
    Wd = None if W is None else torch.from_numpy(W).to(dev)
    Kh, Vh, Qh = (torch.from_numpy(x).to(dev) for x in (K, V, Q))
    pairs = [(0, 0), (0, 1)]
    got = run_decode(torch, dev, w, cfg, Kd, Vd, nodes, prefix, Wd, 0, T, pairs,
                     lambda p: Qh[:, :, p].contiguous(), lambda p: Kh[:, :, p].contiguous(),
                     lambda p: Vh[:, :, p].contiguous(), fused=fused)
    l16 = alhr.alhr_tree_int16_levels(cfg)
    for (b, h) in pairs:
        ref, ref_nodes, ref_pre = decode_oracle_pair(w, b, h, 0, T, K[b, h], Q[b, h], W, cfg)
        compare(got[(b, h)], ref)
        np.testing.assert_array_equal(decode_tree(nodes[b, h].cpu().numpy(), l16)[1:],
                                      ref_nodes[1:])
        np.testing.assert_array_equal(prefix[b, h].cpu().numpy(), ref_pre)


WINDOW_CASES = [
    # T, d, window, fixed budget (0 = predictor), max_budget
    (256, 64, 40, 16, 96),       # window wider than the budget: n = C, no cover
    (256, 32, 1, 0, 96),         # a window of one key (the own key)
    (256, 128, 7, 0, 96),        # an odd window
    (128, 64, 40, 0, 32),        # window wider than max_budget (the window is cut to it)
    (128, 16, 1 << 20, 0, 40),   # a window far past T
]


@pytest.mark.parametrize("fused", [False, True], ids=["two_launches", "fused"])
@pytest.mark.parametrize("T,d,window,fixed,mb", WINDOW_CASES,
                         ids=["T%d_d%d_w%d_f%d_mb%d" % c for c in WINDOW_CASES])
def test_decode_window_edges_every_step(torch_dev, T, d, window, fixed, mb, fused):
    """Decoding from an empty cache with windows other than 4: the decode
    kernel scores the window before the budget is known, for the widest n the
    query can have (at most window, max_budget and t + 1 keys), and places
    the last n of them; with a fixed budget and the fused append the own key's
    score comes from the new key row.  Every step equals the oracle's replay."""
    import learned_tree_routed_amd as alhr
    torch, dev = torch_dev
    w = Workload("decode_window", 9, 1, 2, T, d, "clustered", fixed_budget=fixed, window=window,
                 max_budget=mb)
    cfg = w.config()
    Q, K, V, W = host_inputs(w)
    say("decode window edges: B1 H2 T%d d%d window %d fixed %d max_budget %d"
        % (T, d, window, fixed, mb))
    Kd = torch.zeros((1, 2, T, d), dtype=torch.int8, device=dev)
    Vd = torch.zeros((1, 2, T, d), dtype=torch.float32, device=dev)
    nodes = alhr.alhr_build_tree(cfg, Kd)
    prefix = alhr.alhr_prefix_from_tree(cfg, 0, Kd, nodes)
    Wd = None if W is None else torch.from_numpy(W).to(dev)
    Kh, Vh, Qh = (torch.from_numpy(x).to(dev) for x in (K, V, Q))
    pairs = [(0, 0), (0, 1)]
    got = run_decode(torch, dev, w, cfg, Kd, Vd, nodes, prefix, Wd, 0, T, pairs,
                     lambda p: Qh[:, :, p].contiguous(), lambda p: Kh[:, :, p].contiguous(),
                     lambda p: Vh[:, :, p].contiguous(), fused=fused)
    l16 = alhr.alhr_tree_int16_levels(cfg)
    for (b, h) in pairs:
        ref, ref_nodes, ref_pre = decode_oracle_pair(w, b, h, 0, T, K[b, h], Q[b, h], W, cfg)
        compare(got[(b, h)], ref)
        np.testing.assert_array_equal(decode_tree(nodes[b, h].cpu().numpy(), l16)[1:],
                                      ref_nodes[1:])
        np.testing.assert_array_equal(prefix[b, h].cpu().numpy(), ref_pre)



def random_decode_config(i):
    rng = np.random.default_rng(7000 + i)
    d = int(rng.choice([16, 32, 64, 128, 256]))
    a = int(rng.choice([1, 4, 9, 31, 127]))
    T = 1 << int(rng.integers(1, 9))
    window = int(rng.integers(1, 10))
    max_budget = int(rng.integers(3, 129))
    if rng.random() < 0.4:
        mode = dict(fixed=int(rng.integers(1, max_budget + 1)), n_classes=32, kpc=3)
    else:
        mode = dict(fixed=0, n_classes=int(rng.integers(1, 33)), kpc=int(rng.integers(1, 5)))
    return rng, dict(B=int(rng.integers(1, 3)), H=int(rng.integers(1, 3)), T=T, d=d, a=a,
                     window=window, max_budget=max_budget, **mode)


@pytest.mark.parametrize("fused", [False, True], ids=["two_launches", "fused"])
@pytest.mark.parametrize("i", range(8))
def test_decode_random_configs_every_step(torch_dev, i, fused):
    """Seeded random small decode configurations (T = 2 .. 256, d = 16 .. 256,
    windows 1 .. 9, fixed or predicted budgets, |Q|, |K| up to 127), decoded
    from an empty cache through every position: every step's budget, index
    set, count and output, and the final tree and running sum, equal the
    oracle's replay."""
    import learned_tree_routed_amd as alhr
    torch, dev = torch_dev
    rng, c = random_decode_config(i)
    B, H, T, d, a = c["B"], c["H"], c["T"], c["d"], c["a"]
    w = Workload("decode_random%d" % i, 20 + i, B, H, T, d, "uniform", fixed_budget=c["fixed"],
                 window=c["window"], n_classes=c["n_classes"], keys_per_class=c["kpc"],
                 max_budget=c["max_budget"])
    cfg = alhr.Config(batch=B, heads=H, T=T, d=d, window=c["window"], n_classes=c["n_classes"],
                      keys_per_class=c["kpc"], max_budget=c["max_budget"], kmax=a, qmax=a, wmax=4)
    Q = rng.integers(-a, a + 1, size=(B, H, T, d)).astype(np.int8)
    K = rng.integers(-a, a + 1, size=(B, H, T, d)).astype(np.int8)
    V = synth.values(w.seed, B, H, d, 0, T)     # the rows the oracle replay draws
    W = None if c["fixed"] else rng.integers(-4, 5, size=(c["n_classes"], 2 * d)).astype(np.int8)
    say("decode random config", i, "fused" if fused else "two launches", c)
    Kd = torch.zeros((B, H, T, d), dtype=torch.int8, device=dev)
    Vd = torch.zeros((B, H, T, d), dtype=torch.float32, device=dev)
    nodes = alhr.alhr_build_tree(cfg, Kd)
    prefix = alhr.alhr_prefix_from_tree(cfg, 0, Kd, nodes)
    Wd = None if W is None else torch.from_numpy(W).to(dev)
    Kh, Vh, Qh = (torch.from_numpy(x).to(dev) for x in (K, V, Q))
    pairs = [(b, h) for b in range(B) for h in range(H)]
    got = run_decode(torch, dev, w, cfg, Kd, Vd, nodes, prefix, Wd, 0, T, pairs,
                     lambda p: Qh[:, :, p].contiguous(), lambda p: Kh[:, :, p].contiguous(),
                     lambda p: Vh[:, :, p].contiguous(), fused=fused)
    l16 = alhr.alhr_tree_int16_levels(cfg)
    for (b, h) in pairs:
        ref, ref_nodes, ref_pre = decode_oracle_pair(w, b, h, 0, T, K[b, h], Q[b, h], W, cfg)
        compare(got[(b, h)], ref)
        np.testing.assert_array_equal(decode_tree(nodes[b, h].cpu().numpy(), l16)[1:],
                                      ref_nodes[1:])
        np.testing.assert_array_equal(prefix[b, h].cpu().numpy(), ref_pre)



def test_decode_graph_replays_match_eager(torch_dev):
    """The decode loop as the benchmark runs it: fused append + decode launches
    captured in one HIP graph.  Each replay (from a rebuilt cache, with eager
    work between replays) gives exactly the eager loop's outputs, tree and
    running sum."""
    import learned_tree_routed_amd as alhr
    torch, dev = torch_dev
    T, d, steps = 1024, 128, 8
    n0 = T - steps
    w = Workload("decode_graph", 11, 2, 2, T, d, "clustered")
    cfg = w.config()
    Q, K, V, W = host_inputs(w)
    Kh, Vh, Qh = (torch.from_numpy(x).to(dev) for x in (K, V, Q))
    Wd = torch.from_numpy(W).to(dev)
    Kd = torch.zeros((2, 2, T, d), dtype=torch.int8, device=dev)
    Vd = torch.zeros((2, 2, T, d), dtype=torch.float32, device=dev)
    nodes = torch.empty((2, 2, T, d), dtype=torch.int32, device=dev)
    prefix = torch.empty((2, 2, d), dtype=torch.int32, device=dev)
    ks = [Kh[:, :, n0 + s].contiguous() for s in range(steps)]
    vs = [Vh[:, :, n0 + s].contiguous() for s in range(steps)]
    qs = [Qh[:, :, n0 + s].contiguous() for s in range(steps)]
    outs = [(torch.empty((2, 2), dtype=torch.int32, device=dev),
             torch.empty((2, 2, cfg.max_budget), dtype=torch.int32, device=dev),
             torch.empty((2, 2), dtype=torch.int32, device=dev),
             torch.empty((2, 2, d), dtype=torch.float32, device=dev)) for _ in range(steps)]

    def reset():
        Kd.zero_()
        Vd.zero_()
        Kd[:, :, :n0] = Kh[:, :, :n0]
        Vd[:, :, :n0] = Vh[:, :, :n0]
        alhr.alhr_build_tree(cfg, Kd, nodes)
        alhr.alhr_prefix_from_tree(cfg, n0, Kd, nodes, prefix)

    def loop():
        for s_ in range(steps):
            bud, idx, cnt, O = outs[s_]
            alhr.alhr_append_decode(cfg, n0 + s_, ks[s_], vs[s_], qs[s_], Kd, Vd, nodes, prefix,
                                    Wd, 0, bud, idx, cnt, O)

    say("decode graph: eager loop, B2 H2 T%d d%d, %d steps" % (T, d, steps))
    reset()
    loop()
    torch.cuda.synchronize()
    ref = [tuple(t.clone() for t in o) for o in outs]
    ref_nodes, ref_prefix = nodes.clone(), prefix.clone()
    reset()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        loop()
    torch.cuda.synchronize()
    for rep in range(3):
        for o in outs:
            for t in o:
                t.zero_()
        reset()
        torch.cuda.synchronize()
        say("decode graph replay", rep)
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, ref):
            for x, y in zip(a, b):
                assert torch.equal(x, y)
        assert torch.equal(nodes, ref_nodes) and torch.equal(prefix, ref_prefix)
