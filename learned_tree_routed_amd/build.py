"""Build the gfx950 shared libraries in-tree with hipcc.

    python -m learned_tree_routed_amd.build

builds ``learned_tree_routed_amd/libalhr.so`` (the C ABI of include/alhr.h)
and ``synth/libalhr_synth.so`` (the device-side input generator).  Every HIP
source is compiled for gfx950 only, with packed-FP32 instruction selection
turned off.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libalhr.so")
SYNTH_DIR = os.path.join(ROOT, "synth")
SYNTH_LIB = os.path.join(SYNTH_DIR, "libalhr_synth.so")
BUILD_DIR = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"),
]

SOURCES = ["api.hip", "build.hip", "predict.hip", "prep.hip", "route.hip", "decode.hip",
           "dense.hip", "split.hip"]

# Per-source extra flags.  dense.hip: matrix-core accumulators and results in
# ordinary vector registers, so the softmax and rescaling between the
# products do not copy them out of and back into the accumulation registers
# on every key block.
# route.hip: the instruction scheduler's max-ILP strategy (about 1% faster for
# the fused route + attend and the decode kernels, same register counts).
EXTRA = {"dense.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "route.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"]}


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; harmless
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError("command failed (%d): %s\n%s" % (p.returncode, " ".join(cmd), out))
    return out


def _compile(src, obj):
    return _run([HIPCC] + FLAGS + EXTRA.get(os.path.basename(src), []) + ["-c", src, "-o", obj])


def _link(objs, out):
    tmp = out + ".tmp%d" % os.getpid()
    _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs)
    os.replace(tmp, out)


# Copies of libalhr.so whose prefill routing kernels run 2 or 8 queries per
# workgroup instead of 4 (route.hip built with ALHR_ROUTE_WAVES_PER_BLOCK).
# Only the launch-geometry test loads them: the same queries at other block
# and wave positions must give identical results.
GEOMETRY_VARIANTS = {2: os.path.join(PKG, "libalhr_wpb2.so"),
                     8: os.path.join(PKG, "libalhr_wpb8.so")}


def _objects():
    return [os.path.join(BUILD_DIR, s.replace(".hip", ".o")) for s in SOURCES]


def _variant_object(waves):
    return os.path.join(BUILD_DIR, "route_wpb%d.o" % waves)


def _compile_variant(waves):
    return _run([HIPCC] + FLAGS + EXTRA["route.hip"] +
                ["-DALHR_ROUTE_WAVES_PER_BLOCK=%d" % waves, "-c",
                 os.path.join(CSRC, "route.hip"), "-o", _variant_object(waves)])


def _link_variant(waves):
    objs = [_variant_object(waves) if s == "route.hip" else o for s, o in zip(SOURCES, _objects())]
    _link(objs, GEOMETRY_VARIANTS[waves])
    return GEOMETRY_VARIANTS[waves]


def build_alhr(jobs=8, variants=False):
    """libalhr.so; with ``variants`` also the launch-geometry copies."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        futs = [ex.submit(_compile, os.path.join(CSRC, s), o) for s, o in zip(SOURCES, _objects())]
        if variants:
            futs += [ex.submit(_compile_variant, w) for w in GEOMETRY_VARIANTS]
        for f in futs:
            f.result()
    _link(_objects(), LIB)
    if variants:
        return [LIB] + [_link_variant(w) for w in GEOMETRY_VARIANTS]
    return [LIB]


def build_synth():
    os.makedirs(BUILD_DIR, exist_ok=True)
    obj = os.path.join(BUILD_DIR, "synth_device.o")
    _compile(os.path.join(SYNTH_DIR, "synth_device.hip"), obj)
    _link([obj], SYNTH_LIB)
    return SYNTH_LIB


def build_all(jobs=8):
    with cf.ThreadPoolExecutor(max_workers=2) as ex:
        a = ex.submit(build_alhr, jobs, True)
        b = ex.submit(build_synth)
        return tuple(a.result()) + (b.result(),)


if __name__ == "__main__":
    for p in build_all():
        print("built", p)
    sys.exit(0)
