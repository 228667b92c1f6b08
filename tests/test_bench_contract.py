"""bench.py's contract pieces that need no GPU: it refuses more than one
GPU; the measured HBM traffic it reports comes from the committed counter
record only while that record was taken on the current kernel source, and
the record's figures agree with each other (scaled counters, calibration,
algorithmic bytes of the extreme mix)."""

import hashlib
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2, r.stderr
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "error" in line and line["n_gpus"] == 2


def test_traffic_record_is_consistent():
    rec = json.load(open(os.path.join(ROOT, "profiles", "hda_decode_extreme_traffic.json")))
    # raw counters (KiB per launch) times the copy calibration give the bytes
    assert rec["fetch_bytes_per_launch"] == pytest.approx(
        rec["fetch_kib_per_launch_raw"] * 1024 * rec["fetch_scale"], rel=1e-4)
    assert rec["write_bytes_per_launch"] == pytest.approx(
        rec["write_kib_per_launch_raw"] * 1024 * rec["write_scale"], rel=1e-4)
    assert rec["bytes_per_launch"] == rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"]
    # the calibration copy reads and writes 1 GiB: FETCH_SIZE reports half
    # the bytes read on gfx950, WRITE_SIZE all of them
    assert rec["fetch_scale"] == pytest.approx(2.0, rel=1e-3)
    assert rec["write_scale"] == pytest.approx(1.0, rel=1e-3)
    # every K/V byte once: the fetched bytes match the algorithmic bytes of
    # the extreme mix -- 1 x 131072 + 31 x 4096 tokens x 8 kv heads x 128
    # dims x 2 bytes x (K, V); q (bf16) and the output (fp32) of 32 x 64
    # heads x 128; the 2048 + 31 x 64 block-table entries in use; 32 lengths;
    # the 357-int plan
    kv = (131072 + 31 * 4096) * 8 * 128 * 2 * 2
    algo = kv + 32 * 64 * 128 * (2 + 4) + (2048 + 31 * 64) * 4 + 32 * 4 + 357 * 4
    assert rec["algorithmic_bytes_per_launch"] == algo
    assert rec["fetch_bytes_per_launch"] / rec["algorithmic_bytes_per_launch"] == pytest.approx(1.0, abs=0.01)
    assert all("rocprofv3 --pmc" in c and "bench.py" in c for c in rec["commands"])


def test_traffic_reported_only_for_the_source_it_was_taken_on(tmp_path, monkeypatch):
    rec = json.load(open(os.path.join(ROOT, "profiles", "hda_decode_extreme_traffic.json")))
    src = tmp_path / "kernel.hip"
    src.write_bytes(b"// a kernel source\n")
    prof = tmp_path / "profiles"
    prof.mkdir()
    good = dict(rec, kernel_source_sha256=hashlib.sha256(src.read_bytes()).hexdigest())
    (prof / "hda_decode_extreme_traffic.json").write_text(json.dumps(good))
    monkeypatch.setattr(bench, "KERNEL_SRC", str(src))
    monkeypatch.setattr(bench, "PROFILES", str(prof))
    assert bench.traffic_from_profiles("extreme") == rec["bytes_per_launch"]
    src.write_bytes(b"// the kernel source, changed\n")
    assert bench.traffic_from_profiles("extreme") is None
    assert bench.traffic_from_profiles("uniform") is None          # no record for that mix
