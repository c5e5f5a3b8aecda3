"""Host-side checks of bench.py's counter summary (no GPU): the HBM traffic
of the encoder is its FETCH_SIZE and WRITE_SIZE scaled by what the same
counters read for a device copy of known size."""
import os
import sqlite3
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

COPY = "__amd_rocclr_copyBuffer"
ENC = "lynx::(anonymous namespace)::encode_kv_kernel(unsigned short const*, ...)"


def _db(path, counter, rows):
    os.makedirs(path, exist_ok=True)
    con = sqlite3.connect(os.path.join(path, "p_results.db"))
    con.execute("create table counters_collection (kernel_name text, counter_name text, value real)")
    con.executemany("insert into counters_collection values (?, ?, ?)",
                    [(name, counter, val) for name, val in rows])
    con.commit()
    con.close()


def _runs(tmp_path, extra_copies=()):
    probe_kib = bench.COPY_PROBE_BYTES / 1024.0
    f, w = str(tmp_path / "fetch"), str(tmp_path / "write")
    # the probe copy reads 1/2 and writes 1/1 of its bytes in counter units
    _db(f, "FETCH_SIZE", [(COPY, probe_kib / 2)] + [(COPY, c / 2) for c in extra_copies] +
        [(ENC, 100.0), (ENC, 100.0)])
    _db(w, "WRITE_SIZE", [(COPY, probe_kib)] + [(COPY, c) for c in extra_copies] +
        [(ENC, 200.0), (ENC, 200.0)])
    return f + "," + w


def test_traffic_scales_the_counters_by_the_copy_probe(tmp_path):
    out = str(tmp_path / "summary.txt")
    bench.summarize("pmc", _runs(tmp_path), out, "test")
    kv = dict(line.split(":", 1) for line in open(out) if ":" in line)
    assert float(kv["fetch_scale"]) == pytest.approx(2.0)
    assert float(kv["write_scale"]) == pytest.approx(1.0)
    # (100 KiB x 2 + 200 KiB x 1) per dispatch
    assert float(kv["traffic_bytes_per_launch"]) == pytest.approx(400.0 * 1024)


def test_other_large_copies_are_not_taken_for_the_probe(tmp_path):
    # six copies of 1 GiB beside the probe would scale the counters 25x down
    # (copies of up to 64 MiB, like pool uploads, are not taken for the probe)
    with pytest.raises(SystemExit):
        bench.summarize("pmc", _runs(tmp_path, extra_copies=[1 << 20] * 6),
                        str(tmp_path / "summary.txt"), "test")


def test_pool_sized_copies_are_not_taken_for_the_probe(tmp_path):
    out = str(tmp_path / "summary.txt")
    bench.summarize("pmc", _runs(tmp_path, extra_copies=[32 << 10] * 300), out, "test")
    kv = dict(line.split(":", 1) for line in open(out) if ":" in line)
    assert float(kv["fetch_scale"]) == pytest.approx(2.0)
    assert float(kv["write_scale"]) == pytest.approx(1.0)
