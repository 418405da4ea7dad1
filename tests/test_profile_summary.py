"""The HBM-traffic arithmetic behind the benchmark's `traffic` figures (CPU only).

profile_summary.py turns two rocprofv3 --pmc databases (FETCH_SIZE, WRITE_SIZE) into bytes per
launch by scaling each counter with its reading for a streaming copy of known size; bench.py
reports the figure only while the kernel source still hashes to the recorded value.  Both are
checked here on a small synthetic counter database with known answers.
"""

import argparse
import glob
import json
import os
import sqlite3

import bench
import profile_summary as ps

KIB = 1024.0
CALIB_MIB = 64


def _db(path, counter, rows):
    """rows: (kernel name, dispatch id, value, duration ns); each dispatch's value is split over
    two rows, as the per-XCD rows of a real run are."""
    db = sqlite3.connect(path)
    db.execute("create table counters_collection (kernel_name text, dispatch_id int, counter_name text, "
               "value real, duration int)")
    for k, d, v, du in rows:
        db.execute("insert into counters_collection values (?, ?, ?, ?, ?)", (k, d, counter, 0.25 * v, du))
        db.execute("insert into counters_collection values (?, ?, ?, ?, ?)", (k, d, counter, 0.75 * v, du))
        db.execute("insert into counters_collection values (?, ?, ?, ?, ?)", (k, d, "OTHER", 1e9, du))
    db.commit()
    db.close()


def test_traffic_scaling(tmp_path):
    neg = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda(...)>"
    main = "void ccq::gla_main_kernel<128, __bf16>(ccq::FwdArgs)"
    calib_kib = CALIB_MIB * 1024.0
    # the fetch counter reads half of the streamed bytes, the write counter all of them; a small
    # launch of the same torch kernel must not enter the calibration
    _db(tmp_path / "f.db", "FETCH_SIZE", [(neg, 1, calib_kib / 2, 1000), (neg, 2, 10.0, 10),
                                          (main, 3, 1000.0, 5000), (main, 4, 1200.0, 7000)])
    _db(tmp_path / "w.db", "WRITE_SIZE", [(neg, 1, calib_kib, 1000), (main, 3, 300.0, 5000),
                                          (main, 4, 500.0, 5000)])
    src = tmp_path / "k.hip"
    src.write_text("kernel source\n")
    a = argparse.Namespace(fetch=str(tmp_path / "f.db"), write=str(tmp_path / "w.db"), kernel="gla_main_kernel",
                           calib_mib=CALIB_MIB, source=str(src), workload="w", fetch_command="f",
                           write_command="w")
    rec = ps.traffic_summary(a)
    assert rec["calibration"]["fetch_scale"] == 2.0
    assert rec["calibration"]["write_scale"] == 1.0
    assert rec["fetch_kib_per_dispatch"] == 1100.0
    assert rec["write_kib_per_dispatch"] == 400.0
    assert rec["hbm_read_bytes_per_launch"] == round(1100.0 * KIB * 2.0)
    assert rec["hbm_write_bytes_per_launch"] == round(400.0 * KIB)
    assert rec["hbm_bytes_per_launch"] == round(1100.0 * KIB * 2.0 + 400.0 * KIB)
    assert rec["avg_duration_us_under_counters"]["fetch_run"] == 6.0
    assert rec["source_sha256"] == bench.file_sha(str(src))


def test_committed_records_are_read_only_for_their_source_hash():
    names = sorted(glob.glob(os.path.join(bench.ROOT, "profiles", "traffic_*.json")))
    assert names
    for path in names:
        with open(path) as f:
            rec = json.load(f)
        name = os.path.basename(path)
        assert bench.measured_traffic(name, rec["source_sha256"]) == rec["hbm_bytes_per_launch"]
        assert bench.measured_traffic(name, "0" * 64) is None
        # every record names the kernel source it was taken on and both counter commands
        assert os.path.exists(os.path.join(bench.ROOT, rec["source"]))
        assert "FETCH_SIZE" in rec["commands"]["fetch"] and "WRITE_SIZE" in rec["commands"]["write"]
    assert bench.measured_traffic("traffic_no-such-workload.json", "0" * 64) is None
