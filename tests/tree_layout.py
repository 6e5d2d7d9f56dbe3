"""Reading the GPU tree table (the nodes layout in include/alhr.h): heap
rows of levels l > l16 are d int32 at their own row, their 16-byte slots in
block-interleaved order; rows of levels 1..l16 are d int16 in natural column
order, packed densely after the int32 rows."""
import numpy as np


def wide_slot(g, d):
    """Stored 16-byte slot of natural slot g (columns 4g .. 4g+3) in an
    int32 row."""
    lpr = d // 16
    c, h = g >> 1, g & 1
    return (2 * (c // lpr) + h) * lpr + c % lpr


def decode_tree(nodes, l16):
    """int64 [T, d] node values (heap order, natural columns) from one pair's
    int32 [T, d] table; row 0 = 0."""
    nodes = np.ascontiguousarray(nodes, dtype=np.int32)
    T, d = nodes.shape
    L = T.bit_length() - 1
    l16 = min(l16, L)
    b16 = T >> l16
    perm = [wide_slot(g, d) for g in range(d // 4)]
    out = np.empty((T, d), dtype=np.int64)
    out[:b16] = nodes[:b16].reshape(b16, d // 4, 4)[:, perm, :].reshape(b16, d)
    if l16 >= 1:
        packed = nodes.reshape(-1).view(np.int16)[b16 * 2 * d:]
        out[b16:] = packed[:(T - b16) * d].reshape(T - b16, d)
    out[0] = 0
    return out
