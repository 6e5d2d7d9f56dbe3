"""The host reader of the GPU tree table against an encoder written from the
nodes layout described in include/alhr.h (int32 rows with block-interleaved
16-byte slots above level l16, dense int16 rows for levels 1..l16)."""
import numpy as np
import pytest

from tree_layout import decode_tree, wide_slot


def encode_tree(nodes, l16):
    """int32 [T, d] table holding int64 [T, d] heap-order node values."""
    T, d = nodes.shape
    m = d // 16
    b = T >> l16
    table = np.zeros(T * d, dtype=np.int32)
    for r in range(1, b):
        for g in range(d // 4):
            p = (2 * ((g // 2) // m) + g % 2) * m + (g // 2) % m
            table[r * d + 4 * p: r * d + 4 * p + 4] = nodes[r, 4 * g: 4 * g + 4]
    as16 = table.view(np.int16)
    for r in range(b, T):
        base = 2 * d * b + d * (r - b)          # int16 units: byte 4db + 2d(r - b)
        as16[base: base + d] = nodes[r]
    return table.reshape(T, d)


@pytest.mark.parametrize("d", [16, 32, 64, 128, 256])
def test_wide_slot_is_a_permutation(d):
    perm = [wide_slot(g, d) for g in range(d // 4)]
    assert sorted(perm) == list(range(d // 4))
    if d == 16:
        assert perm == [0, 1, 2, 3]


@pytest.mark.parametrize("T,d,l16", [(64, 16, 0), (64, 32, 3), (128, 64, 7), (256, 128, 5),
                                     (32, 256, 2)])
def test_decode_inverts_the_documented_layout(T, d, l16):
    rng = np.random.default_rng(T * 1000 + d + l16)
    L = T.bit_length() - 1
    nodes = np.zeros((T, d), dtype=np.int64)
    for r in range(1, T):
        level = L - (r.bit_length() - 1)
        lim = 32767 if level <= l16 else 2 ** 30
        nodes[r] = rng.integers(-lim, lim + 1, size=d)
    got = decode_tree(encode_tree(nodes, l16), l16)
    np.testing.assert_array_equal(got, nodes)
