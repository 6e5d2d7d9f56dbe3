"""Seeded synthetic inputs for the ALHR tree-attention path (host side).

This module holds no step of the method: it only draws the integer keys and
queries, the fp32 values and the int8 predictor weights that both the CPU
oracle and the GPU path consume.  The same counter-based generator is
implemented on the device in ``synth_device.hip``; every value is a pure
function of (seed, stream, b, h, t, i), so any slice can be regenerated on
either side and the two agree bit for bit (integer arithmetic throughout, and
values are exact multiples of 2^-17 well inside fp32's 24-bit mantissa).

Generator: the SplitMix64 output function (Steele, Lea & Flood, "Fast
splittable pseudorandom number generators", OOPSLA 2014) applied to a packed
64-bit counter

    key = seed<<56 | stream<<52 | b<<44 | h<<36 | t<<16 | i

with seed < 256, stream < 16, b < 256, h < 256, t < 2^20, i < 2^16.
A uniform integer in [lo, hi] is lo + (((x >> 32) * (hi - lo + 1)) >> 32).

Workload shape (stands in for the multi-query associative-recall runs of the
ALHR README, "Results and Variables"): keys are one of 64 per-(b, h) cluster
centres in [-6, 6] plus noise in [-2, 2]; query t copies a random earlier key
src(t) in [0, t-1] plus noise in [-1, 1]; values are an Irwin-Hall sum of
twelve 16-bit uniforms, centred and scaled to mean 0 and variance ~1; the
predictor weights are uniform in [-4, 4].  The tiny configuration instead
draws Q and K uniformly in [-4, 4].

Streams: 0 centres, 1 cluster id, 2 key noise, 3 query source, 4 query noise,
5 values, 6 predictor weights, 7 uniform queries, 8 uniform keys, 10 the
query/key splitter's input rows (b, t, feature i), 11 the splitter's weights
(t := output feature o, i := input feature).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "mix64", "pack_key", "uniform_int",
    "clustered_keys", "copied_queries", "values", "predictor_weights",
    "uniform_i8", "query_sources", "split_inputs", "split_weights", "STREAM_X", "STREAM_WS",
    "STREAM_CENTRE", "STREAM_CLUSTER", "STREAM_KNOISE", "STREAM_SRC",
    "STREAM_QNOISE", "STREAM_V", "STREAM_W", "STREAM_UQ", "STREAM_UK",
    "N_CENTRES",
]

STREAM_CENTRE, STREAM_CLUSTER, STREAM_KNOISE = 0, 1, 2
STREAM_SRC, STREAM_QNOISE, STREAM_V, STREAM_W = 3, 4, 5, 6
STREAM_UQ, STREAM_UK = 7, 8
STREAM_X, STREAM_WS = 10, 11
N_CENTRES = 64

_U64 = np.uint64
_GOLDEN = _U64(0x9E3779B97F4A7C15)
_M1 = _U64(0xBF58476D1CE4E5B9)
_M2 = _U64(0x94D049BB133111EB)


def mix64(x):
    """SplitMix64 output for state ``x`` (uint64 array or scalar), wrapping."""
    x = np.asarray(x, dtype=_U64)
    with np.errstate(over="ignore"):
        z = x + _GOLDEN
        z = (z ^ (z >> _U64(30))) * _M1
        z = (z ^ (z >> _U64(27))) * _M2
    return z ^ (z >> _U64(31))


def pack_key(seed, stream, b, h, t, i):
    """Packed counter; every argument broadcasts (ints or integer arrays)."""
    def u(v):
        return np.asarray(v).astype(_U64)
    return ((u(seed) << _U64(56)) | (u(stream) << _U64(52)) | (u(b) << _U64(44))
            | (u(h) << _U64(36)) | (u(t) << _U64(16)) | u(i))


def uniform_int(x, lo, hi):
    """Map 64-bit draws to integers in [lo, hi] (int64 result)."""
    span = _U64(hi - lo + 1)
    with np.errstate(over="ignore"):
        v = ((np.asarray(x, dtype=_U64) >> _U64(32)) * span) >> _U64(32)
    return v.astype(np.int64) + lo


def _grid(B, H, t0, nt, d):
    b = np.arange(B, dtype=np.int64)[:, None, None, None]
    h = np.arange(H, dtype=np.int64)[None, :, None, None]
    t = (t0 + np.arange(nt, dtype=np.int64))[None, None, :, None]
    i = np.arange(d, dtype=np.int64)[None, None, None, :]
    return b, h, t, i


def _check(B, H, t0, nt, d):
    assert 0 < B <= 256 and 0 < H <= 256 and 0 < d <= 256
    assert t0 >= 0 and nt >= 0 and t0 + nt <= (1 << 20)


def _key_rows(seed, B, H, t, d):
    """Clustered key rows for positions ``t`` (int64 array broadcastable to
    [B, H, n, 1]); returns int64 [B, H, n, d]."""
    b = np.arange(B, dtype=np.int64)[:, None, None, None]
    h = np.arange(H, dtype=np.int64)[None, :, None, None]
    i = np.arange(d, dtype=np.int64)[None, None, None, :]
    cl = uniform_int(mix64(pack_key(seed, STREAM_CLUSTER, b, h, t, 0)), 0, N_CENTRES - 1)
    centre = uniform_int(mix64(pack_key(seed, STREAM_CENTRE, b, h, cl, i)), -6, 6)
    noise = uniform_int(mix64(pack_key(seed, STREAM_KNOISE, b, h, t, i)), -2, 2)
    return centre + noise


def clustered_keys(seed, B, H, d, t0, nt):
    """K rows t0..t0+nt-1 as int8 [B, H, nt, d], values in [-8, 8]."""
    _check(B, H, t0, nt, d)
    t = (t0 + np.arange(nt, dtype=np.int64))[None, None, :, None]
    return _key_rows(seed, B, H, t, d).astype(np.int8)


def query_sources(seed, B, H, t0, nt):
    """src(t) for t in [t0, t0+nt): uniform in [0, t-1], and 0 at t = 0."""
    b = np.arange(B, dtype=np.int64)[:, None, None]
    h = np.arange(H, dtype=np.int64)[None, :, None]
    t = (t0 + np.arange(nt, dtype=np.int64))[None, None, :]
    x = mix64(pack_key(seed, STREAM_SRC, b, h, t, 0))
    # uniform in [0, t-1]: ((x>>32) * t) >> 32, which is 0 when t == 0
    with np.errstate(over="ignore"):
        s = ((x >> _U64(32)) * t.astype(_U64)) >> _U64(32)
    return np.broadcast_to(s.astype(np.int64), (B, H, nt)).copy()


def copied_queries(seed, B, H, d, t0, nt):
    """Q rows: a noisy copy of the key at src(t); int8 [B, H, nt, d] in [-9, 9]."""
    _check(B, H, t0, nt, d)
    src = query_sources(seed, B, H, t0, nt)[..., None]
    krow = _key_rows(seed, B, H, src, d)
    b, h, t, i = _grid(B, H, t0, nt, d)
    noise = uniform_int(mix64(pack_key(seed, STREAM_QNOISE, b, h, t, i)), -1, 1)
    return (krow + noise).astype(np.int8)


def values(seed, B, H, d, t0, nt):
    """V rows as fp32 [B, H, nt, d]: (2*sum of 12 16-bit uniforms - 786420) * 2^-17."""
    _check(B, H, t0, nt, d)
    b, h, t, i = _grid(B, H, t0, nt, d)
    acc = np.zeros((B, H, nt, d), dtype=np.int64)
    for k in range(3):
        x = mix64(pack_key(seed, STREAM_V, b, h, t, 4 * i + k))
        for m in range(4):
            acc += ((x >> _U64(16 * m)) & _U64(0xFFFF)).astype(np.int64)
    centred = 2 * acc - 12 * 65535
    return (centred.astype(np.float32) * np.float32(2.0 ** -17)).astype(np.float32)


def predictor_weights(seed, n_classes, d):
    """Predictor weights as int8 [n_classes, 2d] in [-4, 4]."""
    c = np.arange(n_classes, dtype=np.int64)[:, None]
    i = np.arange(2 * d, dtype=np.int64)[None, :]
    return uniform_int(mix64(pack_key(seed, STREAM_W, 0, 0, c, i)), -4, 4).astype(np.int8)


def uniform_i8(seed, stream, lo, hi, B, H, d, t0, nt):
    """Uniform int8 rows in [lo, hi] from ``stream``; [B, H, nt, d]."""
    _check(B, H, t0, nt, d)
    b, h, t, i = _grid(B, H, t0, nt, d)
    return uniform_int(mix64(pack_key(seed, stream, b, h, t, i)), lo, hi).astype(np.int8)


def split_inputs(seed, batch, d_model, t0, nt, lo=-8, hi=8):
    """Splitter input rows, int8 [batch, nt, d_model] uniform in [lo, hi]
    (positions t0 .. t0 + nt - 1)."""
    assert 0 <= t0 and t0 + nt <= (1 << 20) and d_model <= (1 << 16) and batch <= 256
    b = np.arange(batch, dtype=np.int64)[:, None, None]
    t = np.arange(t0, t0 + nt, dtype=np.int64)[None, :, None]
    i = np.arange(d_model, dtype=np.int64)[None, None, :]
    return uniform_int(mix64(pack_key(seed, STREAM_X, b, 0, t, i)), lo, hi).astype(np.int8)


def split_weights(seed, heads, d, d_model, lo=-4, hi=4):
    """Splitter weights, int8 [2 * heads * d, d_model] uniform in [lo, hi]
    (rows: query features of every head, then key features)."""
    n = 2 * heads * d
    assert n <= (1 << 20) and d_model <= (1 << 16)
    o = np.arange(n, dtype=np.int64)[:, None]
    i = np.arange(d_model, dtype=np.int64)[None, :]
    return uniform_int(mix64(pack_key(seed, STREAM_WS, 0, 0, o, i)), lo, hi).astype(np.int8)
