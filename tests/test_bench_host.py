"""Host logic of bench.py that needs no GPU: how a batch is split into calls, and which
workloads run as several calls."""
import bench
from synth import workloads


def test_call_sizes_cover_the_batch_once():
    for B in (1, 2, 7, 8, 16, 32, 33, 64, 256):
        for S in range(1, min(B, 5) + 1):
            sizes, starts = bench.call_sizes(B, S)
            assert len(sizes) == S and sum(sizes) == B
            assert max(sizes) - min(sizes) <= 1 and min(sizes) >= 1
            assert starts[0] == 0
            assert all(starts[p + 1] == starts[p] + sizes[p] for p in range(S - 1))


def test_default_calls_per_step():
    assert bench.default_streams(workloads.get("headline")) == 2
    assert bench.default_streams(workloads.get("headline_fp32")) == 2
    assert bench.default_streams(workloads.get("stress")) == 2
    assert bench.default_streams(workloads.get("b8")) == 1
    assert bench.default_streams(workloads.get("smart")) == 1
    assert bench.default_streams(workloads.get("tiny")) == 1
