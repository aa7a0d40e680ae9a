"""The benchmark's host-side logic, on the CPU: the HBM traffic summary built
from two rocprofv3 --pmc CSVs (each counter scaled by what it reads for a
plain copy of known size), the record line it writes and reads back (refused
once the grouped-GEMM sources differ from the ones it was taken on), the
gate/up / down split of the GEMM kernel names, and the refusal of more than
one GPU."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

GATEUP = "_ZN3moe13k_expert_gemmIDF16_Lb1ELb1ELb1EEEvNS_8GemmArgsEPKiPKNS_8WorkItemE"
DOWN = "_ZN3moe13k_expert_gemmIDF16_Lb0ELb0ELb1EEEvNS_8GemmArgsEPKiPKNS_8WorkItemE"
COMBINE = "moe::k_combine(HIP_vector_type<float, 4u> const*, long, int, int const*, int, int, " \
          "HIP_vector_type<float, 4u>*)"


def write_csv(path, counter, rows):
    """rows: (kernel, dispatch, [values of the counter's instances])"""
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for kernel, disp, vals in rows:
            for v in vals:
                w.writerow({"Dispatch_Id": disp, "Kernel_Name": kernel, "Counter_Name": counter,
                            "Counter_Value": v})
            # another counter in the same file is ignored
            w.writerow({"Dispatch_Id": disp, "Kernel_Name": kernel, "Counter_Name": "GRBM_COUNT",
                        "Counter_Value": 1e9})


def test_kernel_names_split_into_gateup_and_down():
    assert bench.gemm_is_gateup(GATEUP)
    assert not bench.gemm_is_gateup(DOWN)
    assert bench.gemm_is_gateup("_ZN3moe13k_expert_gemmIDF16bLb1ELb0ELb0EEEvNS_8GemmArgsE")
    assert not bench.gemm_is_gateup("_ZN3moe13k_expert_gemmIfLb0ELb0ELb0EEEvNS_8GemmArgsE")
    assert bench.gemm_is_gateup("void moe::k_expert_gemm<_Float16, true, true, true>(...)")
    assert not bench.gemm_is_gateup("void moe::k_expert_gemm<__bf16, false, false, true>(...)")
    assert not bench.gemm_is_gateup(COMBINE)


def test_traffic_summary_scales_by_the_copy_and_round_trips(tmp_path, monkeypatch):
    mib = 1024
    kib = mib * 1024
    # the copy reads 2 x its size by FETCH_SIZE (say) and 0.8 x by WRITE_SIZE; a small copy
    # of the same kernel (not the calibration one) is ignored
    fetch_rows = [(bench.COPY_KERNEL, 1, [kib * 1.5, kib * 0.5]), (bench.COPY_KERNEL, 2, [10.0]),
                  (GATEUP, 3, [1000.0, 3000.0]), (GATEUP, 7, [2000.0, 2000.0]),
                  (DOWN, 4, [500.0]), (COMBINE, 5, [800.0])]
    write_rows = [(bench.COPY_KERNEL, 1, [kib * 0.8]), (bench.COPY_KERNEL, 2, [4.0]),
                  (GATEUP, 3, [100.0]), (GATEUP, 7, [300.0]), (DOWN, 4, [640.0]),
                  (COMBINE, 5, [160.0])]
    fc, wc = tmp_path / "fetch.csv", tmp_path / "write.csv"
    write_csv(fc, "FETCH_SIZE", fetch_rows)
    write_csv(wc, "WRITE_SIZE", write_rows)
    out = tmp_path / "traffic.md"
    rec = bench.pmc_summary(str(fc), str(wc), str(out), "rocprofv3 --pmc ...")

    # the calibration size is taken from WRITE_SIZE rounded to whole MiB: 0.8 x 1024 MiB
    assert rec["copy_mib"] == round(0.8 * mib)
    copy_kib = rec["copy_mib"] * 1024
    kf, kw = copy_kib / (2 * kib), copy_kib / (0.8 * kib)
    assert rec["fetch_scale"] == pytest.approx(kf)
    assert rec["write_scale"] == pytest.approx(kw)
    gu = rec["kernels"]["k_expert_gemm/gateup"]
    assert gu["dispatches"] == 2
    # per dispatch: instances summed, then the dispatches averaged, KiB -> bytes
    assert gu["read_bytes"] == pytest.approx(kf * 4000.0 * 1024)
    assert gu["write_bytes"] == pytest.approx(kw * 200.0 * 1024)
    dn = rec["kernels"]["k_expert_gemm/down"]
    assert dn["read_bytes"] == pytest.approx(kf * 500.0 * 1024)
    assert dn["write_bytes"] == pytest.approx(kw * 640.0 * 1024)
    assert rec["kernels"]["k_combine"]["read_bytes"] == pytest.approx(kf * 800.0 * 1024)
    assert bench.COPY_KERNEL not in rec["kernels"]
    assert rec["source_hash"] == bench.gemm_source_hash()

    # the record line reads back as read + write bytes of one launch
    text = out.read_text()
    line = [ln for ln in text.splitlines() if ln.startswith("traffic-record: ")]
    assert len(line) == 1 and json.loads(line[0][len("traffic-record: "):]) == rec
    monkeypatch.setattr(bench, "TRAFFIC_RECORD", str(out))
    assert bench.recorded_traffic("k_expert_gemm/gateup") == pytest.approx(
        gu["read_bytes"] + gu["write_bytes"])
    assert bench.recorded_traffic("no_such_kernel") is None

    # taken on other grouped-GEMM sources: no figure
    stale = tmp_path / "stale.md"
    rec2 = dict(rec, source_hash="0" * 16)
    stale.write_text("traffic-record: " + json.dumps(rec2) + "\n")
    monkeypatch.setattr(bench, "TRAFFIC_RECORD", str(stale))
    assert bench.recorded_traffic("k_expert_gemm/gateup") is None
    monkeypatch.setattr(bench, "TRAFFIC_RECORD", str(tmp_path / "missing.md"))
    assert bench.recorded_traffic("k_expert_gemm/gateup") is None


def test_committed_traffic_record_is_current():
    """the summary under profiles/ was taken on the grouped-GEMM sources in the tree"""
    assert bench.recorded_traffic("k_expert_gemm/gateup") is not None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in (r.stdout + r.stderr)
    assert r.stdout.strip() == ""  # no bench line


def test_read_probe_is_outside_the_layer_library_and_rejects_bad_arguments():
    """the benchmark's read probe lives in its own library beside bench.py: the
    layer's library exports no probe, and the probe refuses bad arguments before
    any HIP call (status 1)"""
    import ctypes

    from mixture_experts_routed_amd import abi

    assert not hasattr(abi.lib(), "moe_stream_read")
    assert "stream_read" not in open(os.path.join(ROOT, "include", "moe_routed.h")).read()
    L = bench.probe_lib()
    A = 1 << 20  # a made-up, never dereferenced address
    assert L.bench_stream_read(A + 8, 1 << 20, A, 16, None) == 1  # src not 16-byte aligned
    assert L.bench_stream_read(A, 8, A, 16, None) == 1            # fewer than 16 bytes
    assert L.bench_stream_read(A, 1 << 20, A, 0, None) == 1       # no sink
    assert L.bench_stream_read(None, 1 << 20, A, 16, None) == 1
    assert L.bench_stream_read(A, 1 << 20, A + 2, 16, None) == 1  # sink not 4-byte aligned
    del ctypes


def test_kernel_short_names_keep_the_weight_layout_and_variant_apart():
    rowmajor = GATEUP.replace("Lb1ELb1ELb1E", "Lb1ELb1ELb0E")
    assert bench.kernel_short_name(GATEUP) == "k_expert_gemm/gateup"
    assert bench.kernel_short_name(rowmajor) == "k_expert_gemm/gateup_rowmajor"
    assert bench.kernel_short_name(DOWN) == "k_expert_gemm/down"
    assert bench.kernel_short_name("void moe::k_combine<true>(void const*, signed char const*, "
                                   "long, int, int const*, int, int, "
                                   "HIP_vector_type<float, 4u>*)") == "k_combine<true>"
    assert bench.kernel_short_name(COMBINE) == "k_combine"
