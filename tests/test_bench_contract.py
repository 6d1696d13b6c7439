"""bench.py's command-line contract that needs no GPU: more than one GPU is refused with a
message (the path runs on one GPU), and the HBM traffic record is only used for the kernel
sources it was measured on."""

from __future__ import annotations

import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"]


def test_traffic_record_matches_sources_only(tmp_path, monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    rec_path = os.path.join(bench.PROFILES, "pmc_dual_sustained.json")
    if not os.path.exists(rec_path):
        return
    with open(rec_path) as f:
        rec = json.load(f)
    got = bench.load_traffic("dual", "sustained")
    assert got in (None, rec["hbm_bytes_per_launch"])
    # a record naming other sources (or a changed hash) is never used
    bad = dict(rec, sources_sha256="0" * 64)
    (tmp_path / "pmc_dual_sustained.json").write_text(json.dumps(bad))
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.load_traffic("dual", "sustained") is None
