"""GPU parity of the query/key splitter (alhr_split_qk, through the C ABI)
against the CPU oracle on seeded inputs: Q and K bit-exact (integer work).

Small and ragged shapes are compared in full; the t16k-sized projection
(16384 tokens, 8 heads of d = 64 from d_model = 512, the shapes the bench
times) on sampled tokens, which the oracle projects row by row since tokens
are independent.  The chain test feeds the splitter's output to the tree
path and checks both stages against the oracle.
"""
import sys

import numpy as np
import pytest

import oracle
import synth
from synth.workloads import Workload

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    return torch, torch.device("cuda:0")


def run_split(torch, dev, s, X, W):
    import learned_tree_routed_amd as alhr
    x = torch.from_numpy(np.ascontiguousarray(X)).to(dev)
    w = torch.from_numpy(np.ascontiguousarray(W)).to(dev)
    say("alhr_split_qk", "B%d H%d T%d d%d d_model%d shift%d clamps %d/%d"
        % (s.batch, s.heads, s.T, s.d, s.d_model, s.shift, s.qclamp, s.kclamp))
    q, k = alhr.alhr_split_qk(s, x, w)
    torch.cuda.synchronize()
    return q.cpu().numpy(), k.cpu().numpy()


SMALL = [
    # batch, heads, T, d, d_model, shift, qclamp, kclamp, input range
    (2, 2, 64, 16, 48, 4, 9, 8, 8),          # N = 64 < tile, K tail (48 = 64 - 16)
    (1, 1, 5, 16, 16, 0, 127, 127, 8),       # 5 tokens, one K step, no rounding
    (3, 4, 100, 32, 256, 7, 20, 30, 8),      # ragged M = 300
    (1, 8, 256, 64, 512, 6, 9, 8, 8),        # the t16k head layout, short
    (1, 2, 64, 256, 1024, 9, 127, 127, 127), # d = 256, full int8 range
    (2, 3, 40, 128, 208, 3, 100, 90, 127),   # saturating clamps, odd K steps
    (1, 1, 3, 16, 16384, 12, 50, 60, 127),   # largest d_model
]


@pytest.mark.parametrize("case", SMALL, ids=["c%d" % i for i in range(len(SMALL))])
def test_split_small_every_output(torch_dev, case):
    import learned_tree_routed_amd as alhr
    torch, dev = torch_dev
    batch, heads, T, d, dm, shift, qc, kc, rng_hi = case
    X = synth.split_inputs(31, batch, dm, 0, T, -rng_hi - (rng_hi == 127), rng_hi)
    W = synth.split_weights(31, heads, d, dm, -rng_hi - (rng_hi == 127), rng_hi)
    s = alhr.SplitConfig(batch=batch, heads=heads, T=T, d=d, d_model=dm, shift=shift,
                         qclamp=qc, kclamp=kc)
    q, k = run_split(torch, dev, s, X, W)
    rq, rk = oracle.split_qk(X, W, heads, d, shift, qc, kc)
    np.testing.assert_array_equal(q, rq)
    np.testing.assert_array_equal(k, rk)
    assert np.abs(q.astype(int)).max() <= qc and np.abs(k.astype(int)).max() <= kc


def random_split_case(i):
    rng = np.random.default_rng(5000 + i)
    d = int(rng.choice([16, 32, 64, 128, 256]))
    return (int(rng.integers(1, 4)), int(rng.integers(1, 9)), int(rng.integers(1, 301)), d,
            16 * int(rng.integers(1, 129)), int(rng.integers(0, 13)), int(rng.integers(1, 128)),
            int(rng.integers(1, 128)), int(rng.choice([1, 8, 31, 127])))


@pytest.mark.parametrize("i", range(12))
def test_split_random_shapes_every_output(torch_dev, i):
    """Seeded random shapes (1 .. 3 sequences of 1 .. 300 tokens, 1 .. 8 heads,
    d = 16 .. 256, d_model a multiple of 16 up to 2048, shifts 0 .. 12, clamps
    1 .. 127, inputs up to the full int8 range): every output bit-exact."""
    import learned_tree_routed_amd as alhr
    torch, dev = torch_dev
    batch, heads, T, d, dm, shift, qc, kc, hi = random_split_case(i)
    lo = -hi - (hi == 127)
    X = synth.split_inputs(40 + i, batch, dm, 0, T, lo, hi)
    W = synth.split_weights(40 + i, heads, d, dm, lo, hi)
    s = alhr.SplitConfig(batch=batch, heads=heads, T=T, d=d, d_model=dm, shift=shift,
                         qclamp=qc, kclamp=kc)
    q, k = run_split(torch, dev, s, X, W)
    rq, rk = oracle.split_qk(X, W, heads, d, shift, qc, kc)
    np.testing.assert_array_equal(q, rq)
    np.testing.assert_array_equal(k, rk)


def test_split_full_size_sampled_tokens(torch_dev):
    """16384 tokens x d_model 512 -> 8 heads x d 64 (the bench's shapes):
    512 sampled tokens against the oracle, plus whole-output invariants."""
    import learned_tree_routed_amd as alhr
    torch, dev = torch_dev
    T, heads, d, dm = 16384, 8, 64, 512
    X = synth.split_inputs(5, 1, dm, 0, T)
    W = synth.split_weights(5, heads, d, dm)
    s = alhr.SplitConfig(batch=1, heads=heads, T=T, d=d, d_model=dm, shift=6, qclamp=9, kclamp=8)
    q, k = run_split(torch, dev, s, X, W)
    ts = np.unique(np.concatenate([np.random.default_rng(2).choice(T, 508, replace=False),
                                   [0, 1, T - 2, T - 1]]))
    rq, rk = oracle.split_qk(X[:, ts], W, heads, d, 6, 9, 8)
    np.testing.assert_array_equal(q[:, :, ts], rq)
    np.testing.assert_array_equal(k[:, :, ts], rk)
    assert np.abs(q.astype(int)).max() <= 9 and np.abs(k.astype(int)).max() <= 8
    # the clamps bind for some outputs but not for most
    sat = np.mean(np.abs(k.astype(int)) == 8)
    assert 0.0 < sat < 0.5


def test_split_repeat_is_bit_identical(torch_dev):
    import learned_tree_routed_amd as alhr
    torch, dev = torch_dev
    X = synth.split_inputs(6, 2, 256, 0, 300)
    W = synth.split_weights(6, 4, 32, 256)
    s = alhr.SplitConfig(batch=2, heads=4, T=300, d=32, d_model=256, shift=5)
    first = run_split(torch, dev, s, X, W)
    for _ in range(3):
        again = run_split(torch, dev, s, X, W)
        np.testing.assert_array_equal(first[0], again[0])
        np.testing.assert_array_equal(first[1], again[1])


def test_split_then_route_chain(torch_dev):
    """X -> splitter -> tree path: the GPU splitter's Q/K equal the oracle's,
    and the forward pass on them equals the oracle's forward on the oracle's
    Q/K for every query."""
    import learned_tree_routed_amd as alhr
    torch, dev = torch_dev
    B, H, T, d, dm = 1, 2, 512, 32, 128
    X = synth.split_inputs(7, B, dm, 0, T)
    Wsplit = synth.split_weights(7, H, d, dm)
    s = alhr.SplitConfig(batch=B, heads=H, T=T, d=d, d_model=dm, shift=5, qclamp=9, kclamp=8)
    q, k = run_split(torch, dev, s, X, Wsplit)
    rq, rk = oracle.split_qk(X, Wsplit, H, d, 5, 9, 8)
    np.testing.assert_array_equal(q, rq)
    np.testing.assert_array_equal(k, rk)
    V = synth.values(7, B, H, d, 0, T)
    Wp = synth.predictor_weights(7, 32, d)
    w = Workload("chain", 7, B, H, T, d, "uniform")
    cfg = w.config(kmax=8, qmax=9)
    qd, kd, vd, wd = (torch.from_numpy(np.ascontiguousarray(a)).to(dev) for a in (q, k, V, Wp))
    say("alhr_forward on splitter output", "B%d H%d T%d d%d" % (B, H, T, d))
    out = alhr.alhr_forward(cfg, qd, kd, vd, wd)
    torch.cuda.synchronize()
    for h in range(H):
        ref = oracle.pair_forward(rq[0, h], rk[0, h], V[0, h], W=Wp, window=cfg.window,
                                  keys_per_class=cfg.keys_per_class, max_budget=cfg.max_budget,
                                  scale=cfg.scale)
        np.testing.assert_array_equal(out["budget"][0, h].cpu().numpy(), ref["budget"])
        np.testing.assert_array_equal(out["count"][0, h].cpu().numpy(), ref["count"])
        np.testing.assert_array_equal(out["idx"][0, h].cpu().numpy(), ref["idx"])
        np.testing.assert_allclose(out["O"][0, h].cpu().numpy(), ref["O"], rtol=0, atol=1e-4)


def test_split_invalid_arguments_rejected_on_device(torch_dev):
    import learned_tree_routed_amd as alhr
    torch, dev = torch_dev
    s = alhr.SplitConfig(batch=1, heads=1, T=8, d=16, d_model=24, shift=2)
    x = torch.zeros((1, 8, 24), dtype=torch.int8, device=dev)
    w = torch.zeros((32, 24), dtype=torch.int8, device=dev)
    with pytest.raises(alhr.AlhrError) as e:
        alhr.alhr_split_qk(s, x, w)
    assert e.value.status == -1 and "multiple of 16" in e.value.detail
