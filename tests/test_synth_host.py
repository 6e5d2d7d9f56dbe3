"""Host generator checks (no GPU): value ranges and distributions of the
workload recipe, and that the single-pair helpers equal the batched draws."""
import numpy as np

import synth
from synth.workloads import WORKLOADS, host_inputs, pair_keys, pair_query_rows, pair_value_rows


def test_mix64_matches_published_splitmix64_outputs():
    # SplitMix64 seeded with 0 yields these first outputs (state advanced by
    # the golden-ratio increment each call); mix64(k * increment) reproduces them.
    inc = 0x9E3779B97F4A7C15
    expect = [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]
    got = [int(synth.mix64(np.uint64((k * inc) % (1 << 64)))) for k in range(3)]
    assert got == expect


def test_ranges_and_shapes():
    w = WORKLOADS["t1k"]
    Q, K, V, W = host_inputs(w, nt=256, B=2, H=3)
    assert Q.shape == K.shape == V.shape == (2, 3, 256, 64)
    assert K.min() >= -8 and K.max() <= 8 and Q.min() >= -9 and Q.max() <= 9
    assert W.shape == (32, 128) and W.min() >= -4 and W.max() <= 4
    assert abs(float(V.mean())) < 0.02 and abs(float(V.std()) - 1.0) < 0.02
    # V values are exact multiples of 2^-17
    assert np.all((V * 2 ** 17) == np.round(V * 2 ** 17))


def test_queries_copy_an_earlier_key():
    w = WORKLOADS["t1k"]
    Q, K, _, _ = host_inputs(w, nt=512, B=1, H=1)
    src = synth.query_sources(w.seed, 1, 1, 0, 512)[0, 0]
    assert src[0] == 0 and np.all(src[1:] < np.arange(1, 512))
    diff = Q[0, 0].astype(int) - K[0, 0][src].astype(int)
    assert np.abs(diff).max() <= 1


def test_single_pair_helpers_equal_batched_draws():
    w = WORKLOADS["t1k"]
    Q, K, V, _ = host_inputs(w, nt=300)
    for b, h in ((0, 0), (3, 5), (7, 7)):
        np.testing.assert_array_equal(pair_keys(w, b, h, 0, 300), K[b, h])
        rows = np.array([0, 1, 77, 299])
        np.testing.assert_array_equal(pair_query_rows(w, b, h, rows), Q[b, h, rows])
        np.testing.assert_array_equal(pair_value_rows(w, b, h, rows), V[b, h, rows])


def test_split_generators_are_slices_of_one_stream():
    """Splitter inputs and weights are pure functions of their counters:
    any slice regenerates identically, and distinct seeds differ."""
    import numpy as np
    import synth
    X = synth.split_inputs(4, 2, 48, 0, 40)
    np.testing.assert_array_equal(synth.split_inputs(4, 2, 48, 10, 20), X[:, 10:30])
    assert X.min() >= -8 and X.max() <= 8 and X.dtype == np.int8
    Wsp = synth.split_weights(4, 3, 16, 48)
    assert Wsp.shape == (96, 48) and Wsp.min() >= -4 and Wsp.max() <= 4
    assert not np.array_equal(Wsp, synth.split_weights(5, 3, 16, 48))
    # both values of each extreme occur in a large draw
    big = synth.split_inputs(4, 1, 1024, 0, 64, lo=-128, hi=127)
    assert big.min() == -128 and big.max() == 127
