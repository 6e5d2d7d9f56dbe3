"""Python binding of libalhr, the MI355X (gfx950) ALHR tree-attention path.

Argument marshalling only: every function checks tensor dtypes, shapes and
devices, allocates outputs the caller did not pass, and calls the C function
of the same name in ``libalhr.so`` (declared in include/alhr.h) on the
current torch stream.  Every step of the path runs in the HIP kernels of that
library; there is no Python or CPU fallback, and a missing library raises.

    from learned_tree_routed_amd import Config, alhr_forward
    cfg = Config(batch=1, heads=8, T=16384, d=64)
    out = alhr_forward(cfg, Q, K, V, W)        # dict of device tensors
"""
from __future__ import annotations

import ctypes as C
import dataclasses
import os

import numpy as np

__all__ = [
    "Config", "AlhrError", "lib_path", "load",
    "alhr_workspace_bytes", "alhr_build_tree", "alhr_predict_budget", "alhr_route",
    "alhr_route_stats", "alhr_sparse_attend", "alhr_route_attend", "alhr_forward",
    "alhr_prefix_from_tree", "alhr_append", "alhr_decode_step", "alhr_dense_attend",
    "alhr_status_string", "alhr_last_error", "alhr_version", "alhr_tree_int16_levels",
    "alhr_split_qk", "alhr_append_decode", "alhr_prepare", "alhr_forward_noalloc", "SplitConfig",
    "EXPORTED", "load_geometry_variant",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libalhr.so")

# every function include/alhr.h declares
EXPORTED = (
    "alhr_workspace_bytes", "alhr_build_tree", "alhr_predict_budget", "alhr_route",
    "alhr_route_stats", "alhr_sparse_attend", "alhr_route_attend", "alhr_forward",
    "alhr_prefix_from_tree", "alhr_append", "alhr_decode_step", "alhr_dense_attend",
    "alhr_status_string", "alhr_last_error", "alhr_version", "alhr_tree_int16_levels",
    "alhr_split_qk", "alhr_append_decode", "alhr_prepare", "alhr_forward_noalloc",
)

STATUS = {0: "ALHR_OK", -1: "ALHR_ERR_ARG", -2: "ALHR_ERR_OVERFLOW", -3: "ALHR_ERR_DEVICE",
          -4: "ALHR_ERR_UNSUPPORTED", -5: "ALHR_ERR_WORKSPACE"}


class AlhrError(RuntimeError):
    def __init__(self, fn, status, detail):
        self.status = status
        self.detail = detail
        super().__init__("%s -> %s (%d): %s" % (fn, STATUS.get(status, "?"), status, detail))


class CConfig(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("batch", "heads", "T", "d", "window", "n_classes",
                                         "keys_per_class", "max_budget", "kmax", "qmax", "wmax")]
    _fields_ += [("scale", C.c_float)]


@dataclasses.dataclass
class Config:
    """Mirror of ``alhr_config``; defaults follow the ALHR README's caps (32
    budget classes of 3 keys, at most 96 keys) and a window of 4 keys."""
    batch: int
    heads: int
    T: int
    d: int
    window: int = 4
    n_classes: int = 32
    keys_per_class: int = 3
    max_budget: int = 96
    kmax: int = 8
    qmax: int = 9
    wmax: int = 4
    scale: float | None = None

    def __post_init__(self):
        if self.scale is None:
            self.scale = float(np.float32(1.0) / np.sqrt(np.float32(self.d)))

    @property
    def pairs(self):
        return self.batch * self.heads

    def c(self):
        cc = CConfig()
        for f in CConfig._fields_:
            setattr(cc, f[0], getattr(self, f[0]))
        return cc


class CSplitConfig(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("batch", "heads", "T", "d", "d_model", "shift",
                                         "qclamp", "kclamp")]


@dataclasses.dataclass
class SplitConfig:
    """Mirror of ``alhr_split_config``: the query/key splitter's shapes and
    its requantisation (round-half-up right shift, then symmetric clamps that
    become the tree path's qmax / kmax)."""
    batch: int
    heads: int
    T: int
    d: int
    d_model: int
    shift: int
    qclamp: int = 9
    kclamp: int = 8

    def c(self):
        cc = CSplitConfig()
        for f in CSplitConfig._fields_:
            setattr(cc, f[0], getattr(self, f[0]))
        return cc


_lib = None


def lib_path():
    return _LIB_PATH


def _bind(lib):
    """Give every exported function of a loaded libalhr its C signature."""
    P, i32, sz = C.c_void_p, C.c_int32, C.c_size_t
    cfgp = C.POINTER(CConfig)
    sigs = {
        "alhr_workspace_bytes": ([cfgp], sz),
        "alhr_build_tree": ([cfgp, P, P, P], C.c_int),
        "alhr_predict_budget": ([cfgp, P, P, P, P, P, sz, P], C.c_int),
        "alhr_prepare": ([cfgp, P, P, P, P, P, P, sz, P], C.c_int),
        "alhr_route": ([cfgp, P, P, P, P, i32, P, P, P, P], C.c_int),
        "alhr_route_stats": ([cfgp, P, P, P, P, i32, P, P, P, P], C.c_int),
        "alhr_sparse_attend": ([cfgp, P, P, P, P, P, P, P], C.c_int),
        "alhr_route_attend": ([cfgp, P, P, P, P, P, i32, P, P, P, P], C.c_int),
        "alhr_forward": ([cfgp, P, P, P, P, i32, P, P, P, P, P, P, sz, P], C.c_int),
        "alhr_forward_noalloc": ([cfgp, P, P, P, P, i32, P, P, P, P, P, P], C.c_int),
        "alhr_prefix_from_tree": ([cfgp, i32, P, P, P, P], C.c_int),
        "alhr_append": ([cfgp, i32, P, P, P, P, P, P, P], C.c_int),
        "alhr_decode_step": ([cfgp, i32, P, P, P, P, P, P, i32, P, P, P, P, P], C.c_int),
        "alhr_append_decode": ([cfgp, i32, P, P, P, P, P, P, P, P, i32, P, P, P, P, P], C.c_int),
        "alhr_dense_attend": ([cfgp, P, P, P, P, P], C.c_int),
        "alhr_status_string": ([C.c_int], C.c_char_p),
        "alhr_last_error": ([], C.c_char_p),
        "alhr_version": ([], i32),
        "alhr_tree_int16_levels": ([cfgp], i32),
        "alhr_split_qk": ([C.POINTER(CSplitConfig), P, P, P, P, P], C.c_int),
    }
    for name, (args, res) in sigs.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    return lib


def load():
    """Load libalhr.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError("libalhr.so is not built at %s: run `python -m "
                           "learned_tree_routed_amd.build` (no fallback path exists)" % _LIB_PATH)
    _lib = _bind(C.CDLL(_LIB_PATH))
    return _lib


def load_geometry_variant(waves):
    """A copy of libalhr.so built with ``waves`` (2 or 8) queries per prefill
    routing workgroup, bound like load()'s; for checking that results do not
    depend on the launch geometry.  Raises if it has not been built."""
    from .build import GEOMETRY_VARIANTS
    path = GEOMETRY_VARIANTS[waves]
    if not os.path.exists(path):
        raise RuntimeError("%s is not built: run `python -m learned_tree_routed_amd.build`" % path)
    return _bind(C.CDLL(path))


# ----------------------------------------------------------------- helpers --
def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def _check(name, t, dtype, shape, device=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


def _out(t, name, dtype, shape, device):
    torch = _torch()
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    return _check(name, t, dtype, shape, device)


def _call(name, *args):
    lib = load()
    st = getattr(lib, name)(*args)
    if st != 0:
        raise AlhrError(name, st, lib.alhr_last_error().decode())


def _shapes(cfg):
    B, H, T, d = cfg.batch, cfg.heads, cfg.T, cfg.d
    return (B, H, T, d), (B, H, T), (B, H, T, cfg.max_budget)


# ------------------------------------------------------------ entry points --
def alhr_workspace_bytes(cfg: Config) -> int:
    return int(load().alhr_workspace_bytes(C.byref(cfg.c())))


def alhr_tree_int16_levels(cfg: Config) -> int:
    """Tree levels 1..l16 are stored as int16 rows (the nodes layout in
    include/alhr.h); -1 for an invalid configuration."""
    return int(load().alhr_tree_int16_levels(C.byref(cfg.c())))


def alhr_status_string(status: int) -> str:
    return load().alhr_status_string(int(status)).decode()


def alhr_last_error() -> str:
    return load().alhr_last_error().decode()


def alhr_version() -> int:
    return int(load().alhr_version())


def alhr_build_tree(cfg, K, nodes=None, stream=None):
    torch = _torch()
    rows, _, _ = _shapes(cfg)
    _check("K", K, torch.int8, rows)
    nodes = _out(nodes, "nodes", torch.int32, rows, K.device)
    _call("alhr_build_tree", C.byref(cfg.c()), _ptr(K), _ptr(nodes), _stream(stream))
    return nodes


def _workspace(cfg, ws, device):
    torch = _torch()
    need = alhr_workspace_bytes(cfg)
    if ws is None:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
    return ws, ws.numel() * ws.element_size()


def alhr_predict_budget(cfg, Q, K, W, budget=None, ws=None, stream=None):
    torch = _torch()
    rows, per_q, _ = _shapes(cfg)
    _check("Q", Q, torch.int8, rows)
    _check("K", K, torch.int8, rows, Q.device)
    _check("W", W, torch.int8, (cfg.n_classes, 2 * cfg.d), Q.device)
    budget = _out(budget, "budget", torch.int32, per_q, Q.device)
    ws, nbytes = _workspace(cfg, ws, Q.device)
    _call("alhr_predict_budget", C.byref(cfg.c()), _ptr(Q), _ptr(K), _ptr(W), _ptr(budget),
          _ptr(ws), nbytes, _stream(stream))
    return budget


def alhr_prepare(cfg, Q, K, W=None, nodes=None, budget=None, ws=None, stream=None):
    """Tree and (W given) budgets in shared launches; returns (nodes, budget)."""
    torch = _torch()
    rows, per_q, _ = _shapes(cfg)
    _check("K", K, torch.int8, rows)
    nodes = _out(nodes, "nodes", torch.int32, rows, K.device)
    nbytes = 0
    if W is not None:
        _check("Q", Q, torch.int8, rows, K.device)
        _check("W", W, torch.int8, (cfg.n_classes, 2 * cfg.d), K.device)
        budget = _out(budget, "budget", torch.int32, per_q, K.device)
        ws, nbytes = _workspace(cfg, ws, K.device)
    _call("alhr_prepare", C.byref(cfg.c()), _ptr(Q), _ptr(K), _ptr(W), _ptr(nodes),
          _ptr(budget if W is not None else None), _ptr(ws if W is not None else None), nbytes,
          _stream(stream))
    return nodes, (budget if W is not None else None)


def _route_args(cfg, Q, K, nodes, budget, idx, count):
    torch = _torch()
    rows, per_q, idx_shape = _shapes(cfg)
    _check("Q", Q, torch.int8, rows)
    _check("K", K, torch.int8, rows, Q.device)
    _check("nodes", nodes, torch.int32, rows, Q.device)
    if budget is not None:
        _check("budget", budget, torch.int32, per_q, Q.device)
    idx = _out(idx, "idx", torch.int32, idx_shape, Q.device)
    count = _out(count, "count", torch.int32, per_q, Q.device)
    return idx, count


def alhr_route(cfg, Q, K, nodes, budget=None, fixed_budget=0, idx=None, count=None,
               score=None, with_score=False, stream=None):
    """Routing only.  Returns (idx, count), or (idx, count, score) when a score
    tensor is passed or with_score is set (q . K[j] of the selected keys, 0 in
    the padding)."""
    torch = _torch()
    idx, count = _route_args(cfg, Q, K, nodes, budget, idx, count)
    if score is not None or with_score:
        score = _out(score, "score", torch.int32, _shapes(cfg)[2], Q.device)
    _call("alhr_route", C.byref(cfg.c()), _ptr(Q), _ptr(K), _ptr(nodes), _ptr(budget),
          int(fixed_budget), _ptr(idx), _ptr(count), _ptr(score), _stream(stream))
    return (idx, count) if score is None else (idx, count, score)


def alhr_route_stats(cfg, Q, K, nodes, budget=None, fixed_budget=0, idx=None, count=None,
                     stats=None, stream=None):
    torch = _torch()
    idx, count = _route_args(cfg, Q, K, nodes, budget, idx, count)
    stats = _out(stats, "stats", torch.int32, (cfg.batch, cfg.heads, cfg.T, 4), Q.device)
    _call("alhr_route_stats", C.byref(cfg.c()), _ptr(Q), _ptr(K), _ptr(nodes), _ptr(budget),
          int(fixed_budget), _ptr(idx), _ptr(count), _ptr(stats), _stream(stream))
    return idx, count, stats


def alhr_sparse_attend(cfg, Q, K, V, idx, count, O=None, stream=None):
    torch = _torch()
    rows, per_q, idx_shape = _shapes(cfg)
    _check("Q", Q, torch.int8, rows)
    _check("K", K, torch.int8, rows, Q.device)
    _check("V", V, torch.float32, rows, Q.device)
    _check("idx", idx, torch.int32, idx_shape, Q.device)
    _check("count", count, torch.int32, per_q, Q.device)
    O = _out(O, "O", torch.float32, rows, Q.device)
    _call("alhr_sparse_attend", C.byref(cfg.c()), _ptr(Q), _ptr(K), _ptr(V), _ptr(idx),
          _ptr(count), _ptr(O), _stream(stream))
    return O


def alhr_route_attend(cfg, Q, K, V, nodes, budget=None, fixed_budget=0, idx=None, count=None,
                      O=None, stream=None):
    torch = _torch()
    rows, _, _ = _shapes(cfg)
    idx, count = _route_args(cfg, Q, K, nodes, budget, idx, count)
    _check("V", V, torch.float32, rows, Q.device)
    O = _out(O, "O", torch.float32, rows, Q.device)
    _call("alhr_route_attend", C.byref(cfg.c()), _ptr(Q), _ptr(K), _ptr(V), _ptr(nodes),
          _ptr(budget), int(fixed_budget), _ptr(idx), _ptr(count), _ptr(O), _stream(stream))
    return idx, count, O


def alhr_forward(cfg, Q, K, V, W=None, fixed_budget=0, nodes=None, budget=None, idx=None,
                 count=None, O=None, ws=None, stream=None):
    """Build + predict (W given) + route + attend.  Returns a dict of tensors."""
    torch = _torch()
    rows, per_q, idx_shape = _shapes(cfg)
    _check("Q", Q, torch.int8, rows)
    _check("K", K, torch.int8, rows, Q.device)
    _check("V", V, torch.float32, rows, Q.device)
    nodes = _out(nodes, "nodes", torch.int32, rows, Q.device)
    idx = _out(idx, "idx", torch.int32, idx_shape, Q.device)
    count = _out(count, "count", torch.int32, per_q, Q.device)
    O = _out(O, "O", torch.float32, rows, Q.device)
    if W is not None:
        _check("W", W, torch.int8, (cfg.n_classes, 2 * cfg.d), Q.device)
        budget = _out(budget, "budget", torch.int32, per_q, Q.device)
        ws, nbytes = _workspace(cfg, ws, Q.device)
    else:
        ws, nbytes = None, 0
    _call("alhr_forward", C.byref(cfg.c()), _ptr(Q), _ptr(K), _ptr(V), _ptr(W),
          int(fixed_budget), _ptr(nodes), _ptr(budget), _ptr(idx), _ptr(count), _ptr(O),
          _ptr(ws), nbytes, _stream(stream))
    return {"nodes": nodes, "budget": budget, "idx": idx, "count": count, "O": O}


def alhr_forward_noalloc(cfg, Q, K, V, W=None, fixed_budget=0, nodes=None, budget=None, idx=None,
                         count=None, O=None, stream=None):
    """alhr_forward with the library's own scratch array instead of a workspace
    (for callers that cannot allocate: pass every output to allocate nothing
    here either).  Returns a dict of tensors."""
    torch = _torch()
    rows, per_q, idx_shape = _shapes(cfg)
    _check("Q", Q, torch.int8, rows)
    _check("K", K, torch.int8, rows, Q.device)
    _check("V", V, torch.float32, rows, Q.device)
    nodes = _out(nodes, "nodes", torch.int32, rows, Q.device)
    idx = _out(idx, "idx", torch.int32, idx_shape, Q.device)
    count = _out(count, "count", torch.int32, per_q, Q.device)
    O = _out(O, "O", torch.float32, rows, Q.device)
    if W is not None:
        _check("W", W, torch.int8, (cfg.n_classes, 2 * cfg.d), Q.device)
        budget = _out(budget, "budget", torch.int32, per_q, Q.device)
    _call("alhr_forward_noalloc", C.byref(cfg.c()), _ptr(Q), _ptr(K), _ptr(V), _ptr(W),
          int(fixed_budget), _ptr(nodes), _ptr(budget), _ptr(idx), _ptr(count), _ptr(O),
          _stream(stream))
    return {"nodes": nodes, "budget": budget, "idx": idx, "count": count, "O": O}


def alhr_prefix_from_tree(cfg, n, K, nodes, prefix=None, stream=None):
    torch = _torch()
    rows, _, _ = _shapes(cfg)
    _check("K", K, torch.int8, rows)
    _check("nodes", nodes, torch.int32, rows, K.device)
    prefix = _out(prefix, "prefix", torch.int32, (cfg.batch, cfg.heads, cfg.d), K.device)
    _call("alhr_prefix_from_tree", C.byref(cfg.c()), int(n), _ptr(K), _ptr(nodes), _ptr(prefix),
          _stream(stream))
    return prefix


def alhr_append(cfg, pos, k_new, v_new, K, V, nodes, prefix, stream=None):
    torch = _torch()
    rows, _, _ = _shapes(cfg)
    one = (cfg.batch, cfg.heads, cfg.d)
    _check("K", K, torch.int8, rows)
    dev = K.device
    _check("k_new", k_new, torch.int8, one, dev)
    _check("v_new", v_new, torch.float32, one, dev)
    _check("V", V, torch.float32, rows, dev)
    _check("nodes", nodes, torch.int32, rows, dev)
    _check("prefix", prefix, torch.int32, one, dev)
    _call("alhr_append", C.byref(cfg.c()), int(pos), _ptr(k_new), _ptr(v_new), _ptr(K), _ptr(V),
          _ptr(nodes), _ptr(prefix), _stream(stream))


def alhr_decode_step(cfg, pos, q_new, K, V, nodes, prefix, W=None, fixed_budget=0, budget=None,
                     idx=None, count=None, O=None, stream=None):
    torch = _torch()
    rows, _, _ = _shapes(cfg)
    one = (cfg.batch, cfg.heads, cfg.d)
    _check("q_new", q_new, torch.int8, one)
    dev = q_new.device
    _check("K", K, torch.int8, rows, dev)
    _check("V", V, torch.float32, rows, dev)
    _check("nodes", nodes, torch.int32, rows, dev)
    if prefix is not None:
        _check("prefix", prefix, torch.int32, one, dev)
    if W is not None:
        _check("W", W, torch.int8, (cfg.n_classes, 2 * cfg.d), dev)
    per_pair = (cfg.batch, cfg.heads)
    if budget is not None:
        _check("budget", budget, torch.int32, per_pair, dev)
    idx = _out(idx, "idx", torch.int32, (cfg.batch, cfg.heads, cfg.max_budget), dev)
    count = _out(count, "count", torch.int32, per_pair, dev)
    O = _out(O, "O", torch.float32, one, dev)
    _call("alhr_decode_step", C.byref(cfg.c()), int(pos), _ptr(q_new), _ptr(K), _ptr(V),
          _ptr(nodes), _ptr(prefix), _ptr(W), int(fixed_budget), _ptr(budget), _ptr(idx),
          _ptr(count), _ptr(O), _stream(stream))
    return idx, count, O


def alhr_append_decode(cfg, pos, k_new, v_new, q_new, K, V, nodes, prefix, W=None,
                       fixed_budget=0, budget=None, idx=None, count=None, O=None, stream=None):
    """alhr_append(pos, k_new, v_new) and alhr_decode_step(pos, q_new) in one launch."""
    torch = _torch()
    rows, _, _ = _shapes(cfg)
    one = (cfg.batch, cfg.heads, cfg.d)
    _check("q_new", q_new, torch.int8, one)
    dev = q_new.device
    _check("k_new", k_new, torch.int8, one, dev)
    _check("v_new", v_new, torch.float32, one, dev)
    _check("K", K, torch.int8, rows, dev)
    _check("V", V, torch.float32, rows, dev)
    _check("nodes", nodes, torch.int32, rows, dev)
    _check("prefix", prefix, torch.int32, one, dev)
    if W is not None:
        _check("W", W, torch.int8, (cfg.n_classes, 2 * cfg.d), dev)
    per_pair = (cfg.batch, cfg.heads)
    if budget is not None:
        _check("budget", budget, torch.int32, per_pair, dev)
    idx = _out(idx, "idx", torch.int32, (cfg.batch, cfg.heads, cfg.max_budget), dev)
    count = _out(count, "count", torch.int32, per_pair, dev)
    O = _out(O, "O", torch.float32, one, dev)
    _call("alhr_append_decode", C.byref(cfg.c()), int(pos), _ptr(k_new), _ptr(v_new),
          _ptr(q_new), _ptr(K), _ptr(V), _ptr(nodes), _ptr(prefix), _ptr(W), int(fixed_budget),
          _ptr(budget), _ptr(idx), _ptr(count), _ptr(O), _stream(stream))
    return idx, count, O


def alhr_split_qk(scfg, X, W, Q=None, K=None, stream=None):
    """Query/key splitter: X int8 [batch, T, d_model] and W int8
    [2 * heads * d, d_model] -> (Q, K) int8 [batch, heads, T, d]."""
    torch = _torch()
    _check("X", X, torch.int8, (scfg.batch, scfg.T, scfg.d_model))
    _check("W", W, torch.int8, (2 * scfg.heads * scfg.d, scfg.d_model), X.device)
    rows = (scfg.batch, scfg.heads, scfg.T, scfg.d)
    Q = _out(Q, "Q", torch.int8, rows, X.device)
    K = _out(K, "K", torch.int8, rows, X.device)
    _call("alhr_split_qk", C.byref(scfg.c()), _ptr(X), _ptr(W), _ptr(Q), _ptr(K), _stream(stream))
    return Q, K


def alhr_dense_attend(cfg, Q, K, V, O=None, stream=None):
    """Dense causal softmax attention over every past key (the baseline)."""
    torch = _torch()
    rows, _, _ = _shapes(cfg)
    _check("Q", Q, torch.int8, rows)
    _check("K", K, torch.int8, rows, Q.device)
    _check("V", V, torch.float32, rows, Q.device)
    O = _out(O, "O", torch.float32, rows, Q.device)
    _call("alhr_dense_attend", C.byref(cfg.c()), _ptr(Q), _ptr(K), _ptr(V), _ptr(O),
          _stream(stream))
    return O
