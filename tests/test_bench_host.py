"""Host logic of bench.py (no GPU): the HBM-traffic summary from counter collections."""
import csv
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

STEP = "void qmm::step::gemv_step_single_inline_kernel<true>(qmm::step::InlineLaunch, long, long)"
GU = "void qmm::b4::gemv_u4_s1_kernel<32, 5, 2, false, 1, 1>(qmm::GemvArgs, long, long)"
QKV = "void qmm::b4::gemv_u4_s1_kernel<32, 5, 1, false, 1, 1>(qmm::GemvArgs, long, long)"
COPY = "__amd_rocclr_copyBuffer"


def _csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, ["Kernel_Name", "Counter_Value"])
        w.writeheader()
        for name, v in rows:
            w.writerow({"Kernel_Name": name, "Counter_Value": v})


def test_traffic_summary_calibrates_on_the_ten_device_copies(tmp_path):
    # ten 2 GiB copies read as 1 GiB by FETCH_SIZE and 2 GiB by WRITE_SIZE, plus small plan uploads
    # through the same copy kernel, which must not enter the calibration
    fetch = [(COPY, 1048576.0)] * 10 + [(COPY, 4.0)] * 30 + [(STEP, 49000.0), (STEP, 49200.0), (GU, 39000.0),
                                                             (QKV, 10100.0)]
    write = [(COPY, 2097152.0)] * 10 + [(COPY, 8.0)] * 30 + [(STEP, 54.0), (STEP, 54.0), (GU, 37.0), (QKV, 24.0)]
    f, w, out = tmp_path / "f.csv", tmp_path / "w.csv", tmp_path / "summary.md"
    _csv(f, fetch)
    _csv(w, write)
    text = bench.summarize_counters(str(f), str(w), str(out))
    assert "factors fetch 2.0000, write 1.0000" in text
    want = round((49100.0 * 2 + 54.0) * 1024)
    assert bench.counted_traffic("step", str(out)) == want
    assert bench.counted_traffic("gate_up", str(out)) == round((39000.0 * 2 + 37.0) * 1024)
    # a summary whose source hash differs from the kernel sources gives no traffic
    stale = out.read_text().replace(bench._source_hash(), "0" * 16)
    (tmp_path / "stale.md").write_text(stale)
    assert bench.counted_traffic("step", str(tmp_path / "stale.md")) is None


def test_traffic_summary_refuses_a_run_without_the_device_copies(tmp_path):
    f, w = tmp_path / "f.csv", tmp_path / "w.csv"
    _csv(f, [(COPY, 4.0)] * 12 + [(STEP, 49000.0), (GU, 1.0), (QKV, 1.0)])
    _csv(w, [(COPY, 8.0)] * 12 + [(STEP, 54.0), (GU, 1.0), (QKV, 1.0)])
    with pytest.raises(SystemExit):
        bench.summarize_counters(str(f), str(w), str(tmp_path / "out.md"))
