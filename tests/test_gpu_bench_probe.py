"""The benchmark's streaming-read probe (bench_probe.hip, a measurement helper
outside the layer's library) runs on odd sizes and leaves its sink alone when
the data's checksum is not its trigger value (all-zero data)."""
import os
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

pytestmark = pytest.mark.gpu


def test_stream_read_probe_runs():
    for n in (4, 1000, (1 << 20) + 4):
        print(f"[probe] {n} floats", file=sys.stderr, flush=True)
        src = torch.zeros(n, dtype=torch.float32, device="cuda")
        sink = torch.full((64,), 7, dtype=torch.int32, device="cuda")
        bench.stream_read(src, sink)
        torch.cuda.synchronize()
        assert torch.all(sink == 7)
