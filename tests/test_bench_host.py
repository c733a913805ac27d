"""Host-side logic of bench.py (no GPU): the committed-counter lookups and the
roofline of the culled searches."""
import hashlib
import json
import os

import pytest

import bench


def _profiles(tmp_path, src_text=b"kernel v1"):
    (tmp_path / "profiles").mkdir()
    (tmp_path / "k.hip").write_bytes(src_text)
    digest = hashlib.sha256(b"kernel v1").hexdigest()
    (tmp_path / "profiles" / "traffic.json").write_text(json.dumps(
        {"knn": {"sources": ["k.hip"], "sha256": digest, "bytes": 4.0e7}}))
    (tmp_path / "profiles" / "work.json").write_text(json.dumps(
        {"knn": {"sources": ["k.hip"], "sha256": digest, "f32_lane_ops": 8.0e9,
                 "profile": "profiles/x.md"}}))


def test_counters_found_for_matching_sources(tmp_path, monkeypatch):
    _profiles(tmp_path)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("knn") == 4.0e7
    assert bench.measured_work("knn")["f32_lane_ops"] == 8.0e9
    assert bench.measured_traffic("bq") is None
    assert bench.measured_work("bq") is None


def test_counters_dropped_once_the_source_changes(tmp_path, monkeypatch):
    _profiles(tmp_path, src_text=b"kernel v2")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("knn") is None
    assert bench.measured_work("knn") is None


def test_culled_roofline_takes_the_nearer_bound(tmp_path, monkeypatch):
    _profiles(tmp_path)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    t = 1e-3  # 1 ms per launch
    roof = bench.culled_roofline("knn", t, {"bound": "hbm", "frac": 0.0})
    # 8e9 lane ops = 1e9 pair-equivalents of 8, each 9 ops: 9 T ops/s
    alu = 9e9 / t / 1e12
    assert roof["bound"] == "alu"
    assert roof["achieved"] == pytest.approx(alu)
    assert roof["frac"] == pytest.approx(alu / bench.ALU_PEAK_TOPS)
    assert roof["traffic"] == 4.0e7
    other = roof["other"]
    assert other["bound"] == "hbm"
    assert other["achieved"] == pytest.approx(4.0e7 / t / 1e9)
    assert other["frac"] < roof["frac"]


def test_culled_roofline_falls_back_without_counters(tmp_path, monkeypatch):
    _profiles(tmp_path, src_text=b"kernel v2")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    fallback = {"bound": "hbm", "achieved": 1.0, "peak": 8000.0, "frac": 1.0 / 8000.0}
    roof = bench.culled_roofline("knn", 1e-3, fallback)
    assert roof["bound"] == "hbm" and roof["achieved"] == 1.0
    assert "no counters" in roof["model"]


def test_committed_counter_files_are_well_formed():
    for name, keys in (("traffic.json", ("bytes",)), ("work.json", ("f32_lane_ops",))):
        path = os.path.join(bench.ROOT, "profiles", name)
        with open(path) as f:
            data = json.load(f)
        assert data, name
        for op, entry in data.items():
            assert set(("sources", "sha256", "profile") + keys) <= set(entry), (name, op)
            for src in entry["sources"]:
                assert os.path.exists(os.path.join(bench.ROOT, src)), src
            assert os.path.exists(os.path.join(bench.ROOT, entry["profile"])), entry["profile"]
