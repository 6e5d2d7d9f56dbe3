"""Host-side checks of bench.py's own logic (no GPU): the one-GPU guard, the
algorithmic byte model, the counter-file reader and the oracle baseline.
"""
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
from synth.workloads import WORKLOADS, host_inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr and p.stdout == ""


def test_byte_model_by_hand():
    """One query of d = 64 with window 4: 3 int32 rows, 10 int16 rows, 5 key
    rows loaded, 20 keys selected, budget read."""
    class Cfg:
        d, window, max_budget = 64, 4, 96
    stats = np.array([[3, 10, 5, 20]], dtype=np.int32)
    d = 64
    want = (d + 4 * d + 3 * 4 * d + 10 * 2 * d + 5 * d + 20 * 4 * d + 4 * d
            + 4 * 96 + 4 + 4)
    assert int(bench.bytes_per_query(stats, Cfg())[0]) == want
    assert int(bench.bytes_per_query(stats, Cfg(), budget_read=False)[0]) == want - 4
    # fewer selected keys than the window: only C neighbours are read
    stats = np.array([[0, 0, 0, 2]], dtype=np.int32)
    assert int(bench.bytes_per_query(stats, Cfg())[0]) == (
        d + 2 * d + 2 * 4 * d + 4 * d + 4 * 96 + 4 + 4)


def test_counter_file_is_read_only_for_the_matching_source(tmp_path, monkeypatch):
    f = tmp_path / "counters.txt"
    sha = bench.route_source_sha()
    body = ("# comment: 1\nroute_source_sha: %s\nfetch_kib_per_dispatch: 10.0\n"
            "write_kib_per_dispatch: 4.0\ncopy_fetch_factor: 2.0\ncopy_write_factor: 1.0\n")
    f.write_text(body % sha)
    monkeypatch.setattr(bench, "PROFILE_COUNTERS", str(f))
    assert bench.read_traffic() == (2.0 * 10.0 + 4.0) * 1024
    f.write_text(body % ("0" * 16))
    assert bench.read_traffic() is None
    f.write_text("route_source_sha: %s\nfetch_kib_per_dispatch: x\n" % sha)
    assert bench.read_traffic() is None
    monkeypatch.setattr(bench, "PROFILE_COUNTERS", str(tmp_path / "absent.txt"))
    assert bench.read_traffic() is None


def test_committed_counter_file_parses():
    """The committed summary carries every key the reader needs (whether its
    hash matches the current source is the bench's business)."""
    kv = {}
    for line in open(bench.PROFILE_COUNTERS):
        line = line.split("#")[0].strip()
        if ":" in line:
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    for k in ("route_source_sha", "fetch_kib_per_dispatch", "write_kib_per_dispatch",
              "copy_fetch_factor", "copy_write_factor"):
        assert k in kv, k
    assert len(kv["route_source_sha"]) == 16
    assert float(kv["fetch_kib_per_dispatch"]) > 0 and float(kv["write_kib_per_dispatch"]) > 0


@pytest.mark.parametrize("threads", [1, 2])
def test_oracle_baseline_counts_the_sample(threads):
    w = WORKLOADS["tiny"]
    Q, K, V, W = host_inputs(w)
    out = bench.cpu_baseline(w, Q, K, V, W, 8, threads)
    assert out["kind"] == "oracle" and out["unit"] == "queries/s"
    assert out["cores"] == min(threads, w.B * w.H)
    assert "(%d queries)" % (w.B * w.H * len(range(0, w.T, 8))) in out["sample"]
    assert out["value"] > 0


def test_host_cores_is_bounded():
    assert 1 <= bench.host_cores() <= 16


def test_dense_roofline_by_hand():
    """Two pairs of T = 4, d = 32: 2 * 10 (query, past key) pairs, three bf16
    products of 2d flops each; 1 ms."""
    class W:
        B, H, T, d = 1, 2, 4, 32
    out = bench.dense_summary(W(), 1.0, 0.5)
    flops = 3 * 2 * 32 * 2 * 10
    assert out["roofline"]["achieved"] == pytest.approx(flops / 1e-3 / 1e12)
    assert out["roofline"]["frac"] == pytest.approx(out["roofline"]["achieved"] / 2500.0)
    assert out["routed_step_speedup"] == 2.0
    assert "precision" not in out
    # 3 * 2^-18 * max|V|: 1.14e-5 at |V| = 1, beyond the 1e-4 bar above |V| = 8.74
    prec = bench.dense_summary(W(), 1.0, 0.5, max_abs_v=1.0)["precision"]
    assert prec["pv_abs_error_bound"] == pytest.approx(3 * 2.0 ** -18)
    assert prec["within_parity_atol"] and prec["max_abs_v_for_atol"] == pytest.approx(8.738, rel=1e-3)
    assert not bench.dense_summary(W(), 1.0, 0.5, max_abs_v=9.0)["precision"]["within_parity_atol"]


def test_issue_file_is_read_only_for_the_matching_source(tmp_path, monkeypatch):
    f = tmp_path / "sq.txt"
    body = ("# kernel source: route_source_sha %s\n#\n#   SQ_INSTS_VALU   2000   2100\n"
            "#   SQ_INSTS_SALU   1000   1900\n")
    f.write_text(body % bench.route_source_sha())
    monkeypatch.setattr(bench, "PROFILE_SQ", str(f))
    out = bench.read_issue(1.0, 1024)
    # 1 ms at 2.4 GHz on 1024 SIMDs, 4 cycles per wave64 instruction
    cap = 1e-3 * 2.4e9 * 1024 / 4
    assert out["valu_per_query"] == 2000 and out["salu_per_query"] == 1000
    assert out["valu_issue_frac"] == pytest.approx(2000 * 1024 / cap)
    f.write_text(body % ("0" * 16))
    assert bench.read_issue(1.0, 1024) is None


def test_committed_sq_file_parses():
    txt = open(bench.PROFILE_SQ).read()
    assert "route_source_sha" in txt and "SQ_INSTS_VALU" in txt and "SQ_INSTS_SALU" in txt


def test_route_roofline_by_hand():
    """2000 VALU instructions per query, 131072 queries in 0.5 ms: 524.3 G/s
    against 1024 SIMDs x 2.4 GHz / 4 = 614.4 G/s; 400 MB past L2 in 0.5 ms is
    800 GB/s of 8000."""
    issue = {"valu_per_query": 2000.0, "salu_per_query": 1500.0}
    out = bench.route_roofline(0.5, 131072, 8e9, issue, 4e8)
    assert out["bound"] == "alu" and out["peak"] == pytest.approx(614.4)
    assert out["achieved"] == pytest.approx(2000 * 131072 / 0.5e-3 / 1e9)
    assert out["frac"] == pytest.approx(out["achieved"] / 614.4)
    assert 0 < out["frac"] <= 1
    assert out["hbm"]["achieved"] == pytest.approx(800.0) and out["hbm"]["frac"] == pytest.approx(0.1)
    assert out["bytes_touched"]["GBps"] == pytest.approx(16000.0)
    none = bench.route_roofline(0.5, 131072, 8e9, None, None)
    assert none["achieved"] is None and none["frac"] is None and "hbm" not in none


def test_single_core_baseline_is_pinned_and_restored():
    before = os.sched_getaffinity(0)
    with bench.pinned_to_one_core() as cpu:
        assert os.sched_getaffinity(0) == {cpu}
    assert os.sched_getaffinity(0) == before
    w = WORKLOADS["tiny"]
    Q, K, V, W = host_inputs(w)
    out = bench.cpu_baseline(w, Q, K, V, W, 16, 1)
    assert "pinned to CPU" in out["sample"]
    assert out["process_cpus"] == len(before) and out["host_cpus"] >= 1


def test_committed_counter_summaries_match_the_source():
    """The committed counter summaries were taken on the current route and
    decode kernel source (else the bench reports their figures as null)."""
    assert bench.read_traffic() is not None
    assert bench.read_traffic(path=bench.PROFILE_DECODE_COUNTERS) is not None
    assert bench.read_issue(0.5, 131072) is not None


def test_timing_events_fall_back_to_torch_events():
    """Without a HIP device (or when the runtime refuses the fence-free flag)
    the bench times with torch's events and says so."""
    import types

    class FakeEvent:
        def __init__(self, enable_timing):
            assert enable_timing

        def record(self):
            pass

        def elapsed_time(self, other):
            return 1.25

    def no_stream():
        raise RuntimeError("no device")

    fake = types.SimpleNamespace(cuda=types.SimpleNamespace(Event=FakeEvent,
                                                            current_stream=no_stream))
    ev = bench.timing_events(fake, 2)
    ev.record(0)
    ev.record(1)
    assert isinstance(ev, bench.TorchEvents) and ev.kind == "torch default events"
    assert ev.ms(0, 1) == 1.25
    ev.close()
