"""The five synthetic workloads of the ALHR path (shapes, seeds and input
recipes), and host-side makers for their inputs.  Input generation only: no
step of the method is computed here.

    tiny     B1  H1  T256    d32   uniform Q, K in [-4, 4]; fixed budget 16
    t1k      B8  H8  T1024   d64   clustered keys, copied queries, predictor
    t4k      B4  H8  T4096   d64   same generator
    t16k     B1  H8  T16384  d64   same generator (the headline roofline case)
    decode   64 sequences x 16 heads, capacity 2^17, d128; prefilled with
             2^17 - 128 keys, then 128 appended tokens, one query per head
             and step

All use window 4, 32 budget classes of 3 keys (at most 96 keys), and seeds
1..5 in that order.
"""
from __future__ import annotations

import dataclasses

import numpy as np

from . import (STREAM_UK, STREAM_UQ, clustered_keys, copied_queries, predictor_weights,
               uniform_i8, values)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    B: int
    H: int
    T: int
    d: int
    kind: str                  # "uniform" or "clustered"
    fixed_budget: int = 0      # > 0: no predictor
    window: int = 4
    n_classes: int = 32
    keys_per_class: int = 3
    max_budget: int = 96
    n0: int = 0                # decode: prefilled positions
    steps: int = 0             # decode: appended tokens

    @property
    def kmax(self):
        return 4 if self.kind == "uniform" else 8

    @property
    def qmax(self):
        return 4 if self.kind == "uniform" else 9

    @property
    def wmax(self):
        return 4

    @property
    def queries(self):
        return self.B * self.H * (self.steps if self.steps else self.T)

    def config(self, **over):
        import learned_tree_routed_amd as alhr
        kw = dict(batch=self.B, heads=self.H, T=self.T, d=self.d, window=self.window,
                  n_classes=self.n_classes, keys_per_class=self.keys_per_class,
                  max_budget=self.max_budget, kmax=self.kmax, qmax=self.qmax, wmax=self.wmax)
        kw.update(over)
        return alhr.Config(**kw)


WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 1, 256, 32, "uniform", fixed_budget=16),
    "t1k": Workload("t1k", 2, 8, 8, 1024, 64, "clustered"),
    "t4k": Workload("t4k", 3, 4, 8, 4096, 64, "clustered"),
    "t16k": Workload("t16k", 4, 1, 8, 16384, 64, "clustered"),
    "decode": Workload("decode", 5, 64, 16, 1 << 17, 128, "clustered",
                       n0=(1 << 17) - 128, steps=128),
}


def host_inputs(w: Workload, t0=0, nt=None, B=None, H=None):
    """(Q, K, V, W) as numpy arrays [B, H, nt, d] (W: [n_classes, 2d] or None)."""
    nt = w.T if nt is None else nt
    B = w.B if B is None else B
    H = w.H if H is None else H
    if w.kind == "uniform":
        Q = uniform_i8(w.seed, STREAM_UQ, -4, 4, B, H, w.d, t0, nt)
        K = uniform_i8(w.seed, STREAM_UK, -4, 4, B, H, w.d, t0, nt)
    else:
        Q = copied_queries(w.seed, B, H, w.d, t0, nt)
        K = clustered_keys(w.seed, B, H, w.d, t0, nt)
    V = values(w.seed, B, H, w.d, t0, nt)
    W = None if w.fixed_budget else predictor_weights(w.seed, w.n_classes, w.d)
    return Q, K, V, W


def pair_keys(w: Workload, b: int, h: int, t0=0, nt=None):
    """Clustered key rows t0..t0+nt-1 of the single pair (b, h): int8 [nt, d].
    The generator is a pure function of (b, h, t, i), so one pair is drawn
    without the others."""
    from . import N_CENTRES, STREAM_CENTRE, STREAM_CLUSTER, STREAM_KNOISE, mix64, pack_key, uniform_int
    if w.kind != "clustered":
        raise ValueError("pair_keys draws the clustered generator")
    nt = w.T if nt is None else nt
    t = (t0 + np.arange(nt, dtype=np.int64))[:, None]
    i = np.arange(w.d, dtype=np.int64)[None, :]
    cl = uniform_int(mix64(pack_key(w.seed, STREAM_CLUSTER, b, h, t, 0)), 0, N_CENTRES - 1)
    centre = uniform_int(mix64(pack_key(w.seed, STREAM_CENTRE, b, h, cl, i)), -6, 6)
    noise = uniform_int(mix64(pack_key(w.seed, STREAM_KNOISE, b, h, t, i)), -2, 2)
    return (centre + noise).astype(np.int8)


def pair_value_rows(w: Workload, b: int, h: int, rows):
    """Value rows at arbitrary positions ``rows`` of pair (b, h): fp32 [len(rows), d]."""
    from . import STREAM_V, mix64, pack_key
    rows = np.asarray(rows, dtype=np.int64)[:, None]
    i = np.arange(w.d, dtype=np.int64)[None, :]
    acc = np.zeros((rows.shape[0], w.d), dtype=np.int64)
    for k in range(3):
        x = mix64(pack_key(w.seed, STREAM_V, b, h, rows, 4 * i + k))
        for m in range(4):
            acc += ((x >> np.uint64(16 * m)) & np.uint64(0xFFFF)).astype(np.int64)
    return ((2 * acc - 12 * 65535).astype(np.float32) * np.float32(2.0 ** -17)).astype(np.float32)


def pair_query_rows(w: Workload, b: int, h: int, rows):
    """Copied-query rows at positions ``rows`` of pair (b, h): [len(rows), d]."""
    from . import (N_CENTRES, STREAM_CENTRE, STREAM_CLUSTER, STREAM_KNOISE, STREAM_QNOISE,
                   STREAM_SRC, mix64, pack_key, uniform_int)
    rows = np.asarray(rows, dtype=np.int64)[:, None]
    i = np.arange(w.d, dtype=np.int64)[None, :]
    x = mix64(pack_key(w.seed, STREAM_SRC, b, h, rows, 0))
    src = (((x >> np.uint64(32)) * rows.astype(np.uint64)) >> np.uint64(32)).astype(np.int64)
    cl = uniform_int(mix64(pack_key(w.seed, STREAM_CLUSTER, b, h, src, 0)), 0, N_CENTRES - 1)
    centre = uniform_int(mix64(pack_key(w.seed, STREAM_CENTRE, b, h, cl, i)), -6, 6)
    noise = uniform_int(mix64(pack_key(w.seed, STREAM_KNOISE, b, h, src, i)), -2, 2)
    qn = uniform_int(mix64(pack_key(w.seed, STREAM_QNOISE, b, h, rows, i)), -1, 1)
    return (centre + noise + qn).astype(np.int8)
