"""Host-side checks of bench.py's rocprofv3 summary helpers on synthetic counter files (no GPU):
the traffic summary scales each counter by its calibration kernel, tells the 1 GiB calibration
probe from a smaller probe run inside a leg, splits the GEMV's dispatches into its three batch
sizes and reports the M = 1 figure, and the figure is withheld once the measured sources change."""
import csv
import os

import pytest

import bench

MIB = 64
KNOWN = MIB * (1 << 20)
NEG = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda(at::TensorIteratorBase&)>"


def _write(d, counter, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for i, (name, value_bytes) in enumerate(rows):
            w.writerow([i + 1, name, counter, value_bytes / 1024.0])  # the CSV holds KiB


def _gemv_rows(fetch_factor, per_m):
    rows = [(NEG, fetch_factor * KNOWN), ("dapf8::read_probe_kernel(...)", fetch_factor * KNOWN)]
    for m_bytes in per_m:  # three batch sizes in order, two calls each
        rows += [("void dapf8::w4_gemv_kernel<true, 7, 2>(...)", fetch_factor * m_bytes)] * 2
    rows += [("dapf8::read_probe_kernel(...)", fetch_factor * 0.1 * KNOWN)] * 3  # the leg's own, smaller probe
    return rows


def test_gemv_traffic_is_the_m1_call_scaled_by_calibration(tmp_path, monkeypatch):
    fetch = [100e6, 110e6, 130e6]
    _write(str(tmp_path / "f"), "FETCH_SIZE", _gemv_rows(0.5, fetch))
    write_rows = [(NEG, 1.0 * KNOWN)] + [("void dapf8::w4_gemv_kernel<true, 7, 2>(...)", 1e5)] * 6
    _write(str(tmp_path / "w"), "WRITE_SIZE", write_rows)
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    out = str(tmp_path / bench.TRAFFIC_FILES["w4gemv"])
    bench.summarize_traffic(str(tmp_path / "f"), str(tmp_path / "w"), "cmd f", "cmd w", out, MIB, "test")
    text = open(out).read()
    assert "| w4gemv | M1 | 2 |" in text and "| w4gemv | M16 | 2 |" in text
    # fetch scaled by the probe's 0.5, write by the elementwise kernel's 1.0; the small probe ignored
    assert bench.measured_traffic("w4gemv", "w4gemv") == int(round(fetch[0] + 1e5))


def test_traffic_withheld_when_sources_change(tmp_path, monkeypatch):
    _write(str(tmp_path / "f"), "FETCH_SIZE", [(NEG, KNOWN), ("dapf8::transcode_kernel<true>(...)", 3e6)])
    _write(str(tmp_path / "w"), "WRITE_SIZE", [(NEG, KNOWN), ("dapf8::transcode_kernel<true>(...)", 2e6)])
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    out = str(tmp_path / bench.TRAFFIC_FILES["transcode"])
    bench.summarize_traffic(str(tmp_path / "f"), str(tmp_path / "w"), "cmd f", "cmd w", out, MIB, "test")
    assert bench.measured_traffic("transcode", "transcode") == 5_000_000  # no probe ran: elementwise 1.0 both
    monkeypatch.setattr(bench, "kernel_source_hash", lambda workload=None: "changed")
    assert bench.measured_traffic("transcode", "transcode") is None


def test_gemv_dispatches_must_split_into_three_batches(tmp_path):
    rows = [(NEG, KNOWN)] + [("void dapf8::w4_gemv_kernel<true, 7, 2>(...)", 1e6)] * 5
    _write(str(tmp_path / "f"), "FETCH_SIZE", rows)
    _write(str(tmp_path / "w"), "WRITE_SIZE", rows)
    with pytest.raises(SystemExit):
        bench.summarize_traffic(str(tmp_path / "f"), str(tmp_path / "w"), "f", "w",
                                str(tmp_path / bench.TRAFFIC_FILES["w4gemv"]), MIB, "test")
