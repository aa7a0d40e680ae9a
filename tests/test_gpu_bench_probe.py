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


def test_probe_same_bytes_reads_the_asked_byte_count():
    # rounded up to 16 bytes; below 512 MiB it cycles over fresh regions of 1 GiB
    print("[probe] same-bytes probe, 1 MiB + 5 bytes", file=sys.stderr, flush=True)
    r = bench.probe_same_bytes((1 << 20) + 5, torch.device("cuda:0"), launches=3)
    assert r["bytes"] == (1 << 20) + 16
    assert r["us"] > 0 and r["gbs"] > 0
