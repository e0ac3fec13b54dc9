"""The benchmark's timing events: HIP events without the system-scope fence,
recorded on torch's current stream through the HIP runtime torch has loaded.
They must time a known stretch of work like torch's own events do."""
import pytest
import torch

pytestmark = pytest.mark.gpu


def test_timing_events_match_torch_events(lib):
    import bench

    x = torch.randn((4096, 4096), device="cuda", dtype=torch.float32)
    y = x @ x  # warm up the library call and the allocator
    torch.cuda.synchronize()
    ours = [bench.TimingEvent(), bench.TimingEvent()]
    theirs = [torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
    times = []
    for rep in range(3):
        ours[0].record()
        theirs[0].record()
        for _ in range(20):
            y = x @ x
        theirs[1].record()
        ours[1].record()
        torch.cuda.synchronize()
        a = ours[0].elapsed_time(ours[1])
        b = theirs[0].elapsed_time(theirs[1])
        print(f"[gpu-case] timing events rep {rep}: {a:.3f} ms against torch events {b:.3f} ms", flush=True)
        times.append((a, b))
    assert torch.isfinite(y).all()
    for a, b in times:
        # the same 20 products; the outer pair of our events encloses torch's pair
        assert a > 0.0 and b > 0.0
        assert 0.9 * b <= a <= 1.5 * b + 0.05
