"""Host-side checks of bench.py's contract (CPU only): the one-GPU guard and the rule that the
HBM traffic figure is used only when it was measured on the current kernel source."""
import hashlib
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]


def test_traffic_only_for_the_measured_source(tmp_path, monkeypatch):
    src_dir = tmp_path / "gaussian_splatting_tile_gs_amd" / "csrc"
    src_dir.mkdir(parents=True)
    (tmp_path / "profiles").mkdir()
    src = src_dir / "raster.hip"
    src.write_text("// kernel source\n")
    sha = hashlib.sha256(src.read_bytes()).hexdigest()
    rec = {"source": "raster.hip", "bytes_per_launch": 123.0, "sha256": sha, "workload": "distill_30k"}
    (tmp_path / "profiles" / "traffic.json").write_text(json.dumps({"rbwd": rec}))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.traffic_for("rbwd", "distill_30k") == 123.0
    assert bench.traffic_for("rbwd", "mid_150k_sh3") is None  # another workload
    assert bench.traffic_for("blend", "distill_30k") is None  # not measured
    src.write_text("// kernel source, changed\n")
    assert bench.traffic_for("rbwd", "distill_30k") is None  # measured on an older source


def test_committed_traffic_records_name_their_source():
    path = os.path.join(ROOT, "profiles", "traffic.json")
    recs = json.load(open(path))
    assert {"blend", "rbwd"} <= set(recs)
    for r in recs.values():
        assert r["source"] == "raster.hip" and len(r["sha256"]) == 64 and r["bytes_per_launch"] > 0
