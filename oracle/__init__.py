"""ctypes wrapper around the ALHR CPU oracle (``alhr_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke``
and by the CPU-baseline leg of ``bench.py``; never by the GPU library or its
Python binding.  The oracle is plain single-threaded C (gcc), exact int64 for
every integer step; attention logits are fp32 products of the exact score and
the fp32 scale, the softmax and weighted sum fp64.

Each function works on one (batch, head) pair with host numpy arrays:
    build_tree(K)            -> int64 [T, d] heap table (row 0 unused)
    prefix(K)                -> int64 [T, d] inclusive prefix sums
    budget(q, s, W, ...)     -> (budget, logits[n_classes])
    route(t, budget, q, K, nodes, window, cap) -> (idx[cap], scores[cap], count, stats)
    attend(idx[:C], q, K, V, scale)            -> fp32 [d]
    pair_forward(...)        -> dict of per-query outputs
    pair_budgets(Q, K, W)    -> int32 [T] predicted budgets
    append(p, k, v, K, V, nodes, prefix)       (in place)

ALHR_ORACLE_LIB, when set, names another build of the same source to load
(the sanitizer build of ``build_sanitized``).
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "alhr_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_lib = None


class RouteStats(C.Structure):
    _fields_ = [
        ("cover_internal", C.c_int64),
        ("cover_leaf", C.c_int64),
        ("child_internal", C.c_int64),
        ("child_leaf", C.c_int64),
        ("rounds", C.c_int64),
        ("neighbours", C.c_int64),
        ("count", C.c_int64),
        ("cover_by_level", C.c_int64 * 24),
        ("child_by_level", C.c_int64 * 24),
    ]

    def as_dict(self):
        out = {}
        for f, _ in self._fields_:
            v = getattr(self, f)
            out[f] = [int(x) for x in v] if f.endswith("_by_level") else int(v)
        return out


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, single-threaded)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-shared",
                               "-fPIC", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def build_sanitized(out_path: str) -> str:
    """The same source built with AddressSanitizer and UndefinedBehaviorSanitizer
    (any finding aborts), for running the pin tests under the sanitizers: load
    it through ALHR_ORACLE_LIB with the ASan runtime preloaded."""
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                           "-fno-omit-frame-pointer", "-o", out_path, _SRC, "-lm"])
    return out_path


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = os.environ.get("ALHR_ORACLE_LIB")
    if not path:
        path = _LIB
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
    lib = C.CDLL(path)
    P = C.c_void_p
    i32, i64, dbl = C.c_int32, C.c_int64, C.c_double
    lib.alhr_ref_build_tree.argtypes = [i32, i32, P, P]
    lib.alhr_ref_build_tree.restype = C.c_int
    lib.alhr_ref_prefix.argtypes = [i32, i32, P, P]
    lib.alhr_ref_prefix.restype = C.c_int
    lib.alhr_ref_budget.argtypes = [i32, P, P, P, i32, i32, i32, P]
    lib.alhr_ref_budget.restype = i32
    lib.alhr_ref_route.argtypes = [i32, i32, i32, i32, i32, P, P, P, i32, P, P, P]
    lib.alhr_ref_route.restype = i32
    lib.alhr_ref_attend.argtypes = [i32, i32, P, P, P, P, dbl, P]
    lib.alhr_ref_attend.restype = C.c_int
    lib.alhr_ref_pair_forward.argtypes = [i32, i32, i32, i32, i32, i32, dbl, P, P, P, P, i32,
                                          P, i32, P, P, P, i32, P, P, P, P]
    lib.alhr_ref_pair_forward.restype = C.c_int
    lib.alhr_ref_pair_budgets.argtypes = [i32, i32, P, P, P, i32, i32, i32, P, P]
    lib.alhr_ref_pair_budgets.restype = C.c_int
    lib.alhr_ref_append.argtypes = [i32, i32, i32, P, P, P, P, P, P]
    lib.alhr_ref_append.restype = C.c_int
    lib.alhr_ref_requant.argtypes = [i64, i32, i32]
    lib.alhr_ref_requant.restype = i64
    lib.alhr_ref_split_qk.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, P, P, P, P]
    lib.alhr_ref_split_qk.restype = C.c_int
    _lib = lib
    return lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def build_tree(K):
    K = _c(K, np.int8)
    T, d = K.shape
    nodes = np.zeros((T, d), dtype=np.int64)
    rc = _load().alhr_ref_build_tree(T, d, _p(K), _p(nodes))
    if rc:
        raise ValueError("alhr_ref_build_tree failed: %d" % rc)
    return nodes


def prefix(K):
    K = _c(K, np.int8)
    T, d = K.shape
    S = np.zeros((T, d), dtype=np.int64)
    rc = _load().alhr_ref_prefix(T, d, _p(K), _p(S))
    if rc:
        raise ValueError("alhr_ref_prefix failed: %d" % rc)
    return S


def budget(q, s, W, keys_per_class=3, max_budget=96):
    q = _c(q, np.int8)
    s = _c(s, np.int64)
    W = _c(W, np.int8)
    n_classes, two_d = W.shape
    d = q.shape[0]
    assert two_d == 2 * d and s.shape == (d,)
    logits = np.zeros(n_classes, dtype=np.int64)
    b = _load().alhr_ref_budget(d, _p(q), _p(s), _p(W), n_classes, keys_per_class,
                                max_budget, _p(logits))
    if b < 1:
        raise ValueError("alhr_ref_budget failed: %d" % b)
    return int(b), logits


def route(t, budget_t, q, K, nodes, window=4, cap=96):
    q = _c(q, np.int8)
    K = _c(K, np.int8)
    nodes = _c(nodes, np.int64)
    T, d = K.shape
    idx = np.full(cap, -7, dtype=np.int32)
    scores = np.zeros(cap, dtype=np.int64)
    st = RouteStats()
    c = _load().alhr_ref_route(T, d, window, int(t), int(budget_t), _p(q), _p(K), _p(nodes),
                               cap, _p(idx), _p(scores), C.byref(st))
    if c < 1:
        raise ValueError("alhr_ref_route failed: %d" % c)
    return idx, scores, int(c), st.as_dict()


def attend(idx, q, K, V, scale):
    idx = _c(idx, np.int32)
    q = _c(q, np.int8)
    K = _c(K, np.int8)
    V = _c(V, np.float32)
    d = q.shape[0]
    out = np.zeros(d, dtype=np.float32)
    rc = _load().alhr_ref_attend(d, idx.shape[0], _p(idx), _p(q), _p(K), _p(V), float(scale),
                                 _p(out))
    if rc:
        raise ValueError("alhr_ref_attend failed: %d" % rc)
    return out


def pair_forward(Q, K, V, W=None, fixed_budget=16, window=4, n_classes=32,
                 keys_per_class=3, max_budget=96, scale=None, ts=None, cap=None,
                 with_stats=False):
    """All stages for one (batch, head) pair; ``ts`` selects the queries."""
    Q = _c(Q, np.int8)
    K = _c(K, np.int8)
    V = _c(V, np.float32)
    T, d = K.shape
    if scale is None:
        scale = float(np.float32(1.0 / np.sqrt(d)))
    if W is not None:
        W = _c(W, np.int8)
        n_classes = W.shape[0]
    if ts is None:
        tsa = None
        nt = T
    else:
        tsa = _c(ts, np.int32)
        nt = tsa.shape[0]
    cap = cap or max_budget
    nodes = np.zeros((T, d), dtype=np.int64)
    S = np.zeros((T, d), dtype=np.int64)
    bud = np.zeros(nt, dtype=np.int32)
    idx = np.zeros((nt, cap), dtype=np.int32)
    cnt = np.zeros(nt, dtype=np.int32)
    O = np.zeros((nt, d), dtype=np.float32)
    stats = (RouteStats * nt)() if with_stats else None
    rc = _load().alhr_ref_pair_forward(T, d, window, n_classes, keys_per_class, max_budget,
                                       float(scale), _p(Q), _p(K), _p(V), _p(W), int(fixed_budget),
                                       _p(tsa), nt, _p(nodes), _p(S), _p(bud), cap, _p(idx),
                                       _p(cnt), _p(O), stats)
    if rc:
        raise ValueError("alhr_ref_pair_forward failed: %d" % rc)
    out = {"nodes": nodes, "budget": bud, "idx": idx, "count": cnt, "O": O}
    if W is not None:
        out["S"] = S
    if with_stats:
        out["stats"] = [s.as_dict() for s in stats]
    return out


def pair_budgets(Q, K, W, keys_per_class=3, max_budget=96):
    """Predicted budget of every query of one pair."""
    Q = _c(Q, np.int8)
    K = _c(K, np.int8)
    W = _c(W, np.int8)
    T, d = K.shape
    S = np.zeros((T, d), dtype=np.int64)
    out = np.zeros(T, dtype=np.int32)
    rc = _load().alhr_ref_pair_budgets(T, d, _p(Q), _p(K), _p(W), W.shape[0], keys_per_class,
                                       max_budget, _p(S), _p(out))
    if rc:
        raise ValueError("alhr_ref_pair_budgets failed: %d" % rc)
    return out


def append(p, k_new, v_new, K, V, nodes, prefix_row):
    """Decode append at position p, in place on K, V, nodes, prefix_row."""
    for a, dt in ((K, np.int8), (V, np.float32), (nodes, np.int64), (prefix_row, np.int64)):
        assert a is None or (a.dtype == dt and a.flags.c_contiguous)
    k_new = _c(k_new, np.int8)
    v_new = None if v_new is None else _c(v_new, np.float32)
    T, d = K.shape
    rc = _load().alhr_ref_append(T, d, int(p), _p(k_new), _p(v_new), _p(K), _p(V), _p(nodes),
                                 _p(prefix_row))
    if rc:
        raise ValueError("alhr_ref_append failed: %d" % rc)


def requant(acc, shift, clamp):
    """The splitter's requantisation of one int64 accumulator."""
    return int(_load().alhr_ref_requant(int(acc), int(shift), int(clamp)))


def split_qk(X, W, heads, d, shift, qclamp, kclamp):
    """Query/key splitter: X int8 [batch, T, d_model], W int8
    [2*heads*d, d_model] -> (Q, K) int8 [batch, heads, T, d]."""
    X = _c(X, np.int8)
    W = _c(W, np.int8)
    batch, T, d_model = X.shape
    assert W.shape == (2 * heads * d, d_model)
    Q = np.zeros((batch, heads, T, d), dtype=np.int8)
    K = np.zeros((batch, heads, T, d), dtype=np.int8)
    rc = _load().alhr_ref_split_qk(batch, heads, T, d, d_model, shift, qclamp, kclamp,
                                   _p(X), _p(W), _p(Q), _p(K))
    if rc:
        raise ValueError("alhr_ref_split_qk failed: %d" % rc)
    return Q, K
