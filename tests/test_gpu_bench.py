"""The benchmark's timing events on the GPU: HIP events created without the
system-scope fence, recorded on torch's current stream, time the same work
as torch's own events."""
import pytest

pytestmark = pytest.mark.gpu


def test_fence_free_events_time_like_torch_events():
    import torch

    import bench
    dev = torch.device("cuda:0")
    a = torch.randn(2048, 2048, device=dev) / 2048 ** 0.5   # keeps the products bounded
    b = a @ a
    torch.cuda.synchronize()
    ev = bench.TimingEvents(torch, 4)
    assert ev.kind.startswith("HIP events")
    try:
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        ev.record(0)
        for _ in range(20):
            b = a @ b
        ev.record(1)
        t1.record()
        ev.record(2)
        ev.record(3)
        torch.cuda.synchronize()
        ms, ref = ev.ms(0, 1), t0.elapsed_time(t1)
        print("fence-free %.4f ms, torch events %.4f ms" % (ms, ref), flush=True)
        assert 0.0 < ms <= ref * 1.02 + 0.01
        assert ms >= 0.9 * ref - 0.05
        assert 0.0 <= ev.ms(2, 3) < 0.05
        assert ev.ms(0, 3) >= ms
    finally:
        ev.close()
    assert torch.isfinite(b).all()
