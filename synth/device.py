"""ctypes wrapper of libalhr_synth.so: the device twin of this package's
host generator (same counters, bit-identical values), for inputs too large
to build on the host.  Fills caller-owned torch device tensors in place."""
from __future__ import annotations

import ctypes as C
import os

_LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libalhr_synth.so")
_lib = None


def load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            raise RuntimeError("libalhr_synth.so is not built: run `python -m "
                               "learned_tree_routed_amd.build`")
        lib = C.CDLL(_LIB)
        i, P, i64 = C.c_int, C.c_void_p, C.c_int64
        for name in ("alhr_synth_keys", "alhr_synth_queries", "alhr_synth_values"):
            getattr(lib, name).argtypes = [i, i, i, i, i, i, i64, P, P]
            getattr(lib, name).restype = i
        lib.alhr_synth_uniform_i8.argtypes = [i, i, i, i, i, i, i, i, i, i64, P, P]
        lib.alhr_synth_uniform_i8.restype = i
        lib.alhr_synth_weights.argtypes = [i, i, i, P, P]
        lib.alhr_synth_weights.restype = i
        _lib = lib
    return _lib


def _stream():
    import torch
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _rows(out, B, H, d, nt, dtype):
    import torch
    assert out.is_cuda and out.is_contiguous() and out.dtype == dtype
    assert out.dim() == 4 and out.shape[0] == B and out.shape[1] == H and out.shape[3] == d
    assert out.shape[2] >= nt
    return out.shape[2]


def _ok(rc, name):
    if rc != 0:
        raise RuntimeError("%s failed (%d)" % (name, rc))


def keys_(out, seed, t0=0, nt=None):
    """Clustered keys for positions t0 .. t0+nt-1 into out[:, :, 0:nt]."""
    import torch
    B, H, R, d = out.shape
    nt = R if nt is None else nt
    _rows(out, B, H, d, nt, torch.int8)
    _ok(load().alhr_synth_keys(seed, B, H, d, t0, nt, R, C.c_void_p(out.data_ptr()), _stream()),
        "alhr_synth_keys")
    return out


def queries_(out, seed, t0=0, nt=None):
    import torch
    B, H, R, d = out.shape
    nt = R if nt is None else nt
    _rows(out, B, H, d, nt, torch.int8)
    _ok(load().alhr_synth_queries(seed, B, H, d, t0, nt, R, C.c_void_p(out.data_ptr()),
                                  _stream()), "alhr_synth_queries")
    return out


def values_(out, seed, t0=0, nt=None):
    import torch
    B, H, R, d = out.shape
    nt = R if nt is None else nt
    _rows(out, B, H, d, nt, torch.float32)
    _ok(load().alhr_synth_values(seed, B, H, d, t0, nt, R, C.c_void_p(out.data_ptr()),
                                 _stream()), "alhr_synth_values")
    return out


def uniform_i8_(out, seed, stream_id, lo, hi, t0=0, nt=None):
    import torch
    B, H, R, d = out.shape
    nt = R if nt is None else nt
    _rows(out, B, H, d, nt, torch.int8)
    _ok(load().alhr_synth_uniform_i8(seed, stream_id, lo, hi, B, H, d, t0, nt, R,
                                     C.c_void_p(out.data_ptr()), _stream()),
        "alhr_synth_uniform_i8")
    return out


def weights_(out, seed):
    import torch
    nc, two_d = out.shape
    assert out.is_cuda and out.is_contiguous() and out.dtype == torch.int8
    _ok(load().alhr_synth_weights(seed, nc, two_d // 2, C.c_void_p(out.data_ptr()), _stream()),
        "alhr_synth_weights")
    return out
