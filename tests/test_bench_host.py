"""Host logic of bench.py (no GPU): the one-GPU guard, the HBM traffic
figures derived from rocprofv3 counter CSVs, and their source-hash gating."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr
    assert p.stdout == ""


def _counter_csv(path, counter, rows):
    fields = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for i, (name, kib) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": counter,
                        "Counter_Value": kib})


def test_write_traffic_scales_by_the_copy_probe(tmp_path, monkeypatch):
    """FETCH_SIZE counts 128-byte reads as 64 bytes on this chip: the probe
    copy of exactly 1 GiB reads back half of it, so every read figure is
    doubled; WRITE_SIZE of the probe is exact, so writes are unscaled."""
    gib_kib = bench.COPY_BYTES / 1024
    copy = "__amd_rocclr_copyBuffer.kd"
    kern = "void up::(anonymous namespace)::up_compact_copy_kernel<16, false>(up::CompactArgs)"
    scan = "up::(anonymous namespace)::up_compact_scan_kernel(up::CompactArgs)"
    other = "void at::native::vectorized_elementwise_kernel<4, copy_kernel>"  # not the probe
    fetch = tmp_path / "fetch.csv"
    write = tmp_path / "write.csv"
    _counter_csv(fetch, "FETCH_SIZE", [(copy, gib_kib / 2), (copy, 10.0), (other, 5.0),
                                       (kern, 1000.0), (kern, 3000.0), (scan, 4.0)])
    _counter_csv(write, "WRITE_SIZE", [(copy, gib_kib), (kern, 2000.0), (kern, 2000.0),
                                       (scan, 8.0)])
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    bench.write_traffic(str(fetch), str(write), "llama8b_L131072")
    rec = json.loads(out.read_text())
    c = rec["up_compact_copy_kernel"]
    assert c["fetch_scale"] == pytest.approx(2.0)
    assert c["write_scale"] == pytest.approx(1.0)
    assert c["fetch_bytes_per_launch"] == pytest.approx(2000.0 * 1024 * 2.0)  # mean of two dispatches
    assert c["write_bytes_per_launch"] == pytest.approx(2000.0 * 1024)
    assert c["bytes_per_launch"] == pytest.approx(2000.0 * 1024 * 3.0)
    assert c["source_sha"] == bench.source_sha("up_compact.hip")
    s = rec["up_compact_scan_kernel"]
    assert s["bytes_per_launch"] == pytest.approx((4.0 * 2.0 + 8.0) * 1024)
    assert "up_revive_copy_kernel" not in rec  # no dispatch of it in the CSVs
    # the stored figure is used only while the kernel's source is unchanged
    assert bench.load_traffic("up_compact_copy_kernel", "up_compact.hip", "llama8b_L131072") \
        == c["bytes_per_launch"]
    # ... and on the workload the counters were taken on
    assert bench.load_traffic("up_compact_copy_kernel", "up_compact.hip", "llama8b_L32768") is None
    rec["up_compact_copy_kernel"]["source_sha"] = "0" * 16
    out.write_text(json.dumps(rec))
    assert bench.load_traffic("up_compact_copy_kernel", "up_compact.hip", "llama8b_L131072") is None
    assert bench.load_traffic("no_such_kernel", "up_compact.hip", "llama8b_L131072") is None

