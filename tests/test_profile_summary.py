"""The HBM-traffic arithmetic behind the benchmark's `traffic` figures (CPU only).

profile_summary.py turns two rocprofv3 --pmc databases (FETCH_SIZE, WRITE_SIZE) into bytes per
launch by scaling each counter with its reading for a streaming copy of known size; bench.py
reports the figure only while the library (every source, header and compile flag) still hashes
to the recorded value.  Both are
checked here on a small synthetic counter database with known answers.
"""

import argparse
import glob
import json
import os
import sqlite3

import bench
import profile_summary as ps
from curvature_conditioned_query_amd import build

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
    assert rec["library_sha256"] == build.library_sha256()


def test_mfma_busy_fraction(tmp_path):
    """SQ_VALU_MFMA_BUSY_CYCLES (summed over SIMDs) over 1024 SIMDs x duration x 2.4 GHz."""
    main = "void ccq::gdn_main_kernel<128, __bf16>(ccq::FwdArgs)"
    busy = 0.25 * 1024 * 100e-6 * 2.4e9  # a quarter of the SIMD cycles of a 100 us dispatch
    _db(tmp_path / "m.db", "SQ_VALU_MFMA_BUSY_CYCLES", [(main, 1, busy, 100_000), (main, 2, busy, 100_000)])
    a = argparse.Namespace(db=str(tmp_path / "m.db"), kernel="gdn_main_kernel", workload="w", command="c")
    rec = ps.mfma_summary(a)
    assert rec["mfma_busy_frac"] == 0.25
    assert rec["dispatches"] == 2
    assert rec["library_sha256"] == build.library_sha256()


def test_library_hash_covers_sources_headers_and_flags(tmp_path, monkeypatch):
    """Any change to a source, a header or a compile flag changes the hash the records are read by."""
    base = build.library_sha256()
    monkeypatch.setitem(build.EXTRA, "ccq_api.cpp", ["-DCCQ_SOME_FLAG"])
    assert build.library_sha256() != base
    monkeypatch.delitem(build.EXTRA, "ccq_api.cpp")
    assert build.library_sha256() == base
    csrc = tmp_path / "csrc"
    inc = tmp_path / "include"
    csrc.mkdir()
    inc.mkdir()
    (csrc / "a.hpp").write_text("int a;\n")
    (inc / "ccq.h").write_text("int b;\n")
    monkeypatch.setattr(build, "CSRC", str(csrc))
    monkeypatch.setattr(build, "INCLUDE", str(inc))
    h1 = build.library_sha256()
    (csrc / "a.hpp").write_text("int a2;\n")
    h2 = build.library_sha256()
    (inc / "ccq.h").write_text("int b2;\n")
    h3 = build.library_sha256()
    assert len({h1, h2, h3}) == 3


def test_library_hash_does_not_depend_on_where_the_tree_is(tmp_path, monkeypatch):
    """The same sources and flags give the same hash in another checkout directory (records are
    taken on one machine and read on another)."""
    import shutil
    base = build.library_sha256()
    root2 = tmp_path / "elsewhere"
    csrc2 = root2 / os.path.relpath(build.CSRC, build.ROOT)
    inc2 = root2 / os.path.relpath(build.INCLUDE, build.ROOT)
    shutil.copytree(build.CSRC, csrc2)
    shutil.copytree(build.INCLUDE, inc2)
    common2 = [f.replace(build.ROOT, str(root2)) for f in build.COMMON]
    assert common2 != build.COMMON  # the flags do name the directories
    monkeypatch.setattr(build, "ROOT", str(root2))
    monkeypatch.setattr(build, "CSRC", str(csrc2))
    monkeypatch.setattr(build, "INCLUDE", str(inc2))
    monkeypatch.setattr(build, "COMMON", common2)
    assert build.library_sha256() == base


def test_committed_records_are_read_only_for_the_library_they_were_taken_on():
    names = sorted(glob.glob(os.path.join(bench.ROOT, "profiles", "traffic_*.json")))
    for path in names:
        with open(path) as f:
            rec = json.load(f)
        name = os.path.basename(path)
        assert bench.measured_traffic(name, rec["library_sha256"]) == rec["hbm_bytes_per_launch"]
        assert bench.measured_traffic(name, "0" * 64) is None
        # every record names the kernel source it was taken on and both counter commands
        assert os.path.exists(os.path.join(bench.ROOT, rec["source"]))
        assert "FETCH_SIZE" in rec["commands"]["fetch"] and "WRITE_SIZE" in rec["commands"]["write"]
    for path in sorted(glob.glob(os.path.join(bench.ROOT, "profiles", "mfma_*.json"))):
        with open(path) as f:
            rec = json.load(f)
        name = os.path.basename(path)
        assert bench.measured_mfma(name, rec["library_sha256"]) == rec["mfma_busy_frac"]
        assert bench.measured_mfma(name, "0" * 64) is None
        assert "SQ_VALU_MFMA_BUSY_CYCLES" in rec["command"]
    assert bench.measured_traffic("traffic_no-such-workload.json", "0" * 64) is None
