"""Host checks of the rocprof database reader used for the committed profile
summaries, on a small SQLite database with the two views it reads (kernel
dispatches with durations; counter values per dispatch and instance)."""

import sqlite3

import pytest

from rope_frequency_pair_amd import rocprof_summary as rs


@pytest.fixture()
def db(tmp_path):
    path = str(tmp_path / "run_results.db")
    con = sqlite3.connect(path)
    con.execute("create table kernels (name text, duration integer, grid_x integer, grid_y integer, "
                "grid_z integer, workgroup_x integer, start integer)")
    con.execute("create table counters_collection (kernel_name text, dispatch_id integer, "
                "counter_name text, value real)")
    rows = [("copyBuffer", 500, 1024, 1, 1, 256, 0),
            ("k<1>", 100, 64, 1, 1, 64, 1), ("k<1>", 300, 64, 1, 1, 64, 2),
            ("k<1>", 200, 128, 1, 1, 64, 3), ("other", 7, 1, 1, 1, 1, 4)]
    con.executemany("insert into kernels values (?, ?, ?, ?, ?, ?, ?)", rows)
    # FETCH_SIZE in two instances per dispatch (summed), WRITE_SIZE in one
    cc = [("copyBuffer", 1, "FETCH_SIZE", 256.0), ("copyBuffer", 1, "FETCH_SIZE", 256.0),
          ("copyBuffer", 1, "WRITE_SIZE", 1024.0),
          ("k<1>", 2, "FETCH_SIZE", 10.0), ("k<1>", 2, "FETCH_SIZE", 30.0), ("k<1>", 2, "WRITE_SIZE", 8.0),
          ("k<1>", 3, "FETCH_SIZE", 20.0), ("k<1>", 3, "FETCH_SIZE", 20.0), ("k<1>", 3, "WRITE_SIZE", 4.0)]
    con.executemany("insert into counters_collection values (?, ?, ?, ?)", cc)
    con.commit()
    con.close()
    return path


def test_stats_and_dispatch_groups(db):
    st = {r["name"]: r for r in rs.kernel_stats(db)}
    assert st["k<1>"]["calls"] == 3 and st["k<1>"]["total_ns"] == 600
    groups = rs.dispatch_groups(db, kernel="k<")
    assert [(g["grid"], g["calls"], g["avg_ns"]) for g in groups] == [((64, 1, 1), 2, 200), ((128, 1, 1), 1, 200)]
    g = rs.dispatch_groups(db, kernel="k<", skip=1, first=1)
    assert [(x["grid"], x["calls"], x["avg_ns"]) for x in g] == [((64, 1, 1), 1, 300)]


def test_counters_sum_instances(db):
    c = rs.counters(db)
    assert sorted(c["k<1>"]["FETCH_SIZE"]) == [40.0, 40.0]
    assert sorted(c["k<1>"]["WRITE_SIZE"]) == [4.0, 8.0]


def test_sequence_scales_by_the_calibration_copy(db):
    rows, scale = rs.sequence(db, "k<", "FETCH_SIZE", copy_bytes=1024)
    assert scale == 1024 / 512
    assert [(r["dispatch"], r["value"], r["bytes"]) for r in rows] == [(2, 40.0, 80.0), (3, 40.0, 80.0)]
    rows, scale = rs.sequence(db, "k<", "duration")
    assert scale is None and [r["value"] for r in rows] == [100.0, 300.0, 200.0]


def test_traffic(db):
    t = rs.traffic(db, db, "k<1>", 1024)
    assert t["fetch_scale"] == 2.0 and t["write_scale"] == 1.0
    assert t["fetch_bytes"] == 80.0 and t["write_bytes"] == 6.0
