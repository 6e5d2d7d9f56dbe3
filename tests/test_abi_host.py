"""Host-side checks of libalhr that need no GPU: the library loads, exports
every function include/alhr.h declares, and rejects each bad argument with
its status code before any HIP call.

The calls below pass placeholder (never dereferenced) device addresses.  Each
call is built to fail host validation; because a call that passed validation
would launch kernels on those addresses, this module is skipped wherever a
GPU is visible (the same checks run with real tensors in the GPU suite).
"""
import ctypes as C
import os
import re
import subprocess

import pytest

import learned_tree_routed_amd as alhr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "alhr.h")


def _gpu_visible():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(alhr_[a-z0-9_]+)\s*\(", text)))


def test_header_declarations_match_binding():
    names = declared_functions()
    assert len(names) >= 14
    assert sorted(alhr.EXPORTED) == names


def test_library_exports_every_declared_symbol():
    lib = alhr.load()
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", alhr.lib_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r" T (alhr_\w+)", out))
    assert set(declared_functions()) <= exported


@pytest.mark.parametrize("waves", [2, 8])
def test_geometry_variants_export_the_same_symbols(waves):
    """The launch-geometry copies of the library (route kernels at 2 or 8
    queries per workgroup) load and export every declared function."""
    from learned_tree_routed_amd.build import GEOMETRY_VARIANTS
    lib = alhr.load_geometry_variant(waves)
    out = subprocess.run(["nm", "-D", "--defined-only", GEOMETRY_VARIANTS[waves]],
                         capture_output=True, text=True, check=True).stdout
    assert set(declared_functions()) <= set(re.findall(r" T (alhr_\w+)", out))
    assert lib.alhr_version() == alhr.load().alhr_version()


def test_status_strings_and_version():
    assert alhr.alhr_version() >= 100
    for code, name in alhr.STATUS.items():
        assert alhr.alhr_status_string(code).startswith(name)


pytestmark_cpu = pytest.mark.skipif(_gpu_visible(), reason="placeholder pointers: CPU host only")

P0 = C.c_void_p(0x10000)       # aligned placeholder address, never dereferenced
P_ODD = C.c_void_p(0x10004)    # not 16-byte aligned
NULL = None


def cfg(**kw):
    c = alhr.Config(batch=1, heads=8, T=16384, d=64)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def status(fn, *args):
    lib = alhr.load()
    return getattr(lib, fn)(*args), lib.alhr_last_error().decode()


def route_call(c, **over):
    a = dict(Q=P0, K=P0, nodes=P0, budget=NULL, fixed=16, idx=P0, count=P0, score=NULL)
    a.update(over)
    return status("alhr_route", C.byref(c.c()), a["Q"], a["K"], a["nodes"], a["budget"],
                  a["fixed"], a["idx"], a["count"], a["score"], NULL)


@pytestmark_cpu
@pytest.mark.parametrize("field,value,code,frag", [
    ("T", 1000, -1, "power of two"),
    ("T", 1, -1, "power of two"),
    ("T", 1 << 21, -1, "power of two"),
    ("d", 48, -4, "not built"),
    ("d", 40, -1, "multiple of 16"),
    ("batch", 0, -1, "batch"),
    ("heads", 70000, -1, "exceeds 65536"),
    ("window", 0, -1, "window"),
    ("n_classes", 33, -1, "n_classes"),
    ("keys_per_class", 0, -1, "keys_per_class"),
    ("max_budget", 129, -1, "max_budget"),
    ("max_budget", 0, -1, "max_budget"),
    ("kmax", 128, -1, "kmax"),
    ("scale", float("nan"), -1, "scale"),
])
def test_config_rejected_before_launch(field, value, code, frag):
    st, msg = route_call(cfg(**{field: value}))
    assert st == code, msg
    assert frag in msg


@pytestmark_cpu
def test_overflow_bounds():
    # (node sums cannot reach 2^31 inside the accepted ranges: 127 * 2^20 < 2^31)
    # scores: qmax * kmax * d * T/2 >= 2^31
    st, msg = route_call(cfg(qmax=127, kmax=127))
    assert st == -2 and "scores" in msg
    # predictor logits: wmax * d * (qmax + kmax * T) >= 2^31
    st, msg = route_call(cfg(T=1 << 20, kmax=8, qmax=0, wmax=127, d=256))
    assert st == -2 and "logits" in msg
    # the decode cache shape stays inside every bound
    c5 = alhr.Config(batch=64, heads=16, T=1 << 17, d=128)
    assert alhr.alhr_workspace_bytes(c5) > 0


@pytestmark_cpu
@pytest.mark.parametrize("arg", ["Q", "K", "nodes", "idx", "count"])
def test_null_and_misaligned_pointers(arg):
    st, msg = route_call(cfg(), **{arg: NULL})
    assert st == -1 and ("'%s' is NULL" % arg) in msg
    st, msg = route_call(cfg(), **{arg: P_ODD})
    assert st == -1 and "aligned" in msg


@pytestmark_cpu
def test_fixed_budget_range():
    for fb in (0, 97, -3):
        st, msg = route_call(cfg(), fixed=fb)
        assert st == -1 and "fixed_budget" in msg


@pytestmark_cpu
def test_workspace_checks():
    c = cfg()
    need = alhr.alhr_workspace_bytes(c)
    assert need > 0 and need % 256 == 0
    lib = alhr.load()
    st = lib.alhr_predict_budget(C.byref(c.c()), P0, P0, P0, P0, P0, need - 256, NULL)
    assert st == -5 and "workspace" in lib.alhr_last_error().decode()
    st = lib.alhr_predict_budget(C.byref(c.c()), P0, P0, P0, P0, NULL, need, NULL)
    assert st == -5
    st = lib.alhr_forward(C.byref(c.c()), P0, P0, P0, P0, 0, P0, P0, P0, P0, P0, P0, 0, NULL)
    assert st == -5
    # W given but no budget output
    st = lib.alhr_forward(C.byref(c.c()), P0, P0, P0, P0, 0, P0, NULL, P0, P0, P0, P0, need,
                          NULL)
    assert st == -1
    assert alhr.alhr_workspace_bytes(cfg(T=3)) == 0


@pytestmark_cpu
def test_route_score_output_checks():
    """alhr_route takes an optional score output, which must be aligned when
    given; alhr_forward without W needs no workspace."""
    c = cfg()
    st, msg = route_call(c, score=P_ODD)
    assert st == -1 and "'score'" in msg
    # valid with or without a score output: reaches the device
    assert route_call(c, score=P0)[0] == -3
    assert route_call(c)[0] == -3
    lib = alhr.load()
    cc = C.byref(c.c())
    assert lib.alhr_forward(cc, P0, P0, P0, NULL, 16, P0, NULL, P0, P0, P0, NULL, 0, NULL) == -3


@pytestmark_cpu
def test_prepare_argument_checks():
    c = cfg()
    lib = alhr.load()
    cc = C.byref(c.c())
    need = alhr.alhr_workspace_bytes(c)
    prep = lib.alhr_prepare
    # K and nodes always; Q, budget and a large enough workspace when W is given
    assert prep(cc, P0, NULL, P0, P0, P0, P0, need, NULL) == -1
    assert prep(cc, P0, P0, P0, NULL, P0, P0, need, NULL) == -1
    assert prep(cc, NULL, P0, P0, P0, P0, P0, need, NULL) == -1
    assert prep(cc, P0, P0, P0, P0, NULL, P0, need, NULL) == -1
    assert prep(cc, P0, P0, P_ODD, P0, P0, P0, need, NULL) == -1
    assert prep(cc, P0, P0, P0, P0, P0, P0, need - 256, NULL) == -5
    assert prep(cc, P0, P0, P0, P0, P0, NULL, need, NULL) == -5
    c.T = 1000
    assert prep(C.byref(c.c()), P0, P0, P0, P0, P0, P0, need, NULL) == -1
    # a valid call reaches the device (W NULL: the tree only, Q and ws unused)
    assert prep(cc, NULL, P0, NULL, P0, NULL, NULL, 0, NULL) == -3


@pytestmark_cpu
def test_decode_and_append_argument_checks():
    c = alhr.Config(batch=2, heads=2, T=1024, d=128)
    lib = alhr.load()
    cc = C.byref(c.c())
    assert lib.alhr_append(cc, 1024, P0, P0, P0, P0, P0, P0, NULL) == -1
    assert lib.alhr_append(cc, -1, P0, P0, P0, P0, P0, P0, NULL) == -1
    assert lib.alhr_append(cc, 5, P0, P0, P0, P0, P0, NULL, NULL) == -1
    assert lib.alhr_decode_step(cc, 1024, P0, P0, P0, P0, P0, NULL, 16, NULL, P0, P0, P0,
                                NULL) == -1
    assert lib.alhr_decode_step(cc, 5, P0, P0, P0, P0, P0, NULL, 0, NULL, P0, P0, P0, NULL) == -1
    # W given, prefix missing
    assert lib.alhr_decode_step(cc, 5, P0, P0, P0, P0, NULL, P0, 0, NULL, P0, P0, P0, NULL) == -1
    # fused append + decode: the union of both entry points' checks
    ad = lib.alhr_append_decode
    assert ad(cc, 1024, P0, P0, P0, P0, P0, P0, P0, NULL, 16, NULL, P0, P0, P0, NULL) == -1
    assert ad(cc, 5, NULL, P0, P0, P0, P0, P0, P0, NULL, 16, NULL, P0, P0, P0, NULL) == -1
    assert ad(cc, 5, P0, NULL, P0, P0, P0, P0, P0, NULL, 16, NULL, P0, P0, P0, NULL) == -1
    # prefix is required even with a fixed budget
    assert ad(cc, 5, P0, P0, P0, P0, P0, P0, NULL, NULL, 16, NULL, P0, P0, P0, NULL) == -1
    assert ad(cc, 5, P0, P0, P0, P0, P0, P0, P0, NULL, 0, NULL, P0, P0, P0, NULL) == -1
    assert ad(cc, 5, P0, P0, P0, P0, P0, P0, P0, NULL, 97, NULL, P0, P0, P0, NULL) == -1
    # a valid call reaches the device and fails there without a GPU
    assert ad(cc, 5, P0, P0, P0, P0, P0, P0, P0, NULL, 16, NULL, P0, P0, P0, NULL) == -3
    assert lib.alhr_prefix_from_tree(cc, 1025, P0, P0, P0, NULL) == -1
    assert lib.alhr_sparse_attend(cc, P0, P0, NULL, P0, P0, P0, NULL) == -1
    assert lib.alhr_build_tree(None, P0, P0, NULL) == -1


@pytestmark_cpu
def test_valid_call_without_a_gpu_fails_loudly():
    """A call that passes validation on a host with no GPU must report a
    device error rather than fall back to anything."""
    st, msg = route_call(cfg())
    assert st == -3, msg


@pytestmark_cpu
def test_python_binding_requires_device_tensors():
    import torch
    c = alhr.Config(batch=1, heads=1, T=8, d=16)
    K = torch.zeros((1, 1, 8, 16), dtype=torch.int8)
    with pytest.raises(ValueError, match="device tensor"):
        alhr.alhr_build_tree(c, K)
    with pytest.raises(TypeError):
        alhr.alhr_build_tree(c, K.float())


def test_int16_tree_levels_follow_the_key_bound():
    """Levels whose sums fit int16 (kmax * 2^l <= 32767) are stored compactly."""
    c = alhr.Config(batch=1, heads=1, T=1 << 14, d=64, kmax=8)
    assert alhr.alhr_tree_int16_levels(c) == 11          # 8 * 2^11 = 16384, 8 * 2^12 = 32768
    c.T = 1 << 10
    assert alhr.alhr_tree_int16_levels(c) == 10          # every level of a 2^10 tree
    c = alhr.Config(batch=1, heads=1, T=1 << 12, d=16, kmax=127, qmax=1, wmax=1)
    assert alhr.alhr_tree_int16_levels(c) == 8           # 127 * 2^8 = 32512
    c = alhr.Config(batch=1, heads=1, T=1 << 12, d=16, kmax=0)
    assert alhr.alhr_tree_int16_levels(c) == 12
    c.T = 1000
    assert alhr.alhr_tree_int16_levels(c) == -1


def split_call(**over):
    c = alhr.SplitConfig(batch=1, heads=8, T=16384, d=64, d_model=512, shift=6)
    ptrs = dict(X=P0, W=P0, Q=P0, K=P0)
    for k, v in over.items():
        if k in ptrs:
            ptrs[k] = v
        else:
            setattr(c, k, v)
    return status("alhr_split_qk", C.byref(c.c()), ptrs["X"], ptrs["W"], ptrs["Q"], ptrs["K"], NULL)


@pytestmark_cpu
@pytest.mark.parametrize("over,code,frag", [
    ({"batch": 0}, -1, "batch"),
    ({"heads": 0}, -1, "heads"),
    ({"T": 0}, -1, "T = 0"),
    ({"T": (1 << 20) + 1}, -1, "outside"),
    ({"d": 48}, -4, "not built"),
    ({"d_model": 8}, -1, "d_model"),
    ({"d_model": 520}, -1, "multiple of 16"),
    ({"d_model": 16400}, -1, "d_model"),
    ({"shift": -1}, -1, "shift"),
    ({"shift": 31}, -1, "shift"),
    ({"qclamp": 0}, -1, "qclamp"),
    ({"kclamp": 128}, -1, "kclamp"),
    ({"batch": 64, "T": 1 << 20, "d_model": 64}, -1, "2^31"),
    ({"X": NULL}, -1, "'X'"),
    ({"K": P_ODD}, -1, "aligned"),
])
def test_split_config_rejected_before_launch(over, code, frag):
    st, msg = split_call(**over)
    assert st == code, msg
    assert frag in msg, msg


def test_split_binding_checks_shapes_before_the_library():
    torch = pytest.importorskip("torch")
    s = alhr.SplitConfig(batch=1, heads=2, T=16, d=16, d_model=32, shift=3)
    with pytest.raises(ValueError):
        alhr.alhr_split_qk(s, torch.zeros((1, 16, 48), dtype=torch.int8),
                           torch.zeros((64, 32), dtype=torch.int8))
    with pytest.raises(TypeError):
        alhr.alhr_split_qk(s, torch.zeros((1, 16, 32), dtype=torch.float32),
                           torch.zeros((64, 32), dtype=torch.int8))


@pytestmark_cpu
def test_dense_rejects_more_queries_than_one_launch_holds():
    c = alhr.Config(batch=65536, heads=1, T=1 << 15, d=32, kmax=1, qmax=1, wmax=1)
    st, msg = status("alhr_dense_attend", C.byref(c.c()), P0, P0, P0, P0, NULL)
    assert st == -4 and "2^31" in msg, msg
