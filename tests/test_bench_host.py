"""Host logic of bench.py, on the CPU (no GPU is touched):

* `--gpus N` with N > 1 exits with status 2 and says that one GPU is measured;
* the counter summary turns FETCH_SIZE / WRITE_SIZE readings (KiB per
  dispatch) into HBM bytes per decode launch, each scaled by what the same
  counter reads for a copy of known size: checked on synthetic counter files
  against the arithmetic done by hand;
* a counter summary is refused without the command that made its runs;
* a traffic record is used only while the decode kernel's code is the code
  it was taken on (comment edits do not void it, code edits do).
"""

import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_counter_summary_needs_its_command(tmp_path):
    # a traffic record names the counter runs it summarises: without the
    # command the summary is refused and nothing is written
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--pmc-summary", str(tmp_path / "f"),
                        str(tmp_path / "w"), "--config", "tiny"], capture_output=True, text=True, timeout=120,
                       cwd=ROOT)
    assert r.returncode != 0
    assert "--pmc-command" in r.stderr


def _write_counters(path, counter, rows):
    """rows: (dispatch id, kernel name, [values over dimensions])."""
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "p_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for d, name, vals in rows:
            for v in vals:
                w.writerow([d, name, counter, v])


DEC = "void (anonymous namespace)::decode_kernel<64, 128, 6, false>(unsigned short*, ...)"
DEC8 = "void (anonymous namespace)::decode_kernel<64, 128, 6, true>(unsigned short*, ...)"
CPY = "__amd_rocclr_copyBuffer"


def test_pmc_summary_arithmetic(tmp_path):
    copy_bytes = 64 << 20
    fetch, write = str(tmp_path / "fetch"), str(tmp_path / "write")
    # decode dispatches: fetch readings split over two dimensions; the median
    # of (1000, 1100, 1200) KiB is 1100. The copy reads copy_bytes as 2 x 16 MiB
    # (a counter that sees half the traffic: scale 2); small copies are ignored.
    rows_f = [(1, DEC, [400, 600]), (2, DEC, [500, 600]), (3, DEC, [700, 500]), (4, DEC8, [9e9])]
    rows_w = [(1, DEC, [100]), (2, DEC, [300]), (3, DEC, [200]), (4, DEC8, [9e9])]
    for i in range(bench.COPY_REPS):
        rows_f.append((10 + i, CPY, [16384, 16384]))
        rows_w.append((10 + i, CPY, [65536]))
    rows_f.append((99, CPY, [1]))
    rows_w.append((99, CPY, [1]))
    _write_counters(fetch, "FETCH_SIZE", rows_f)
    _write_counters(write, "WRITE_SIZE", rows_w)
    text = bench.pmc_summary(fetch, write, "tiny", copy_bytes, "synthetic")
    fields = dict(line.split(": ", 1) for line in text.splitlines() if not line.startswith("#"))
    assert float(fields["fetch_scale"]) == pytest.approx(2.0)
    assert float(fields["write_scale"]) == pytest.approx(1.0)
    assert fields["decode_fetch_kib_per_dispatch_median"].startswith("1100.0")
    assert fields["decode_write_kib_per_dispatch_median"].startswith("200.0")
    assert int(fields["traffic_bytes_per_launch"]) == 1100 * 1024 * 2 + 200 * 1024
    assert fields["kernel_source_sha256_16"] == bench.kernel_source_hash()


def test_traffic_record_follows_the_kernel_code(tmp_path, monkeypatch):
    src = tmp_path / "kernel.h"
    src.write_text("// a comment\nint f() { return 1; }\n")
    monkeypatch.setattr(bench, "KERNEL_SRCS", [str(src)])
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    h = bench.kernel_source_hash()
    with open(bench.traffic_file("tiny"), "w") as f:
        f.write(f"workload: tiny\nkernel_source_sha256_16: {h}\ntraffic_bytes_per_launch: 12345\n")
    assert bench.read_traffic("tiny") == 12345
    src.write_text("// another comment\n\nint f() { return 1; }   \n")  # comments and blank space only
    assert bench.read_traffic("tiny") == 12345
    src.write_text("// a comment\nint f() { return 2; }\n")  # a code change voids the record
    assert bench.read_traffic("tiny") is None
    assert bench.read_traffic("mixed") is None  # no record at all
