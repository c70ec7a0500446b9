"""Host-side logic of bench.py (no GPU): the one-GPU guard, the algorithmic byte count of a scan
launch, and the rule that a committed counter record is used only while its kernel's sources are
unchanged."""
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
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""  # no JSON line for a configuration that was not measured


def test_scan_bytes_counts_keys_queries_and_block_maxima():
    # 68 B per key, 32 x 68 B of query codes and scales + 32 x 4 B of weights per query, 4 B per
    # block maximum (ceil(n / 8) blocks per query)
    n_vis = [1 << 20] * 8
    assert bench.scan_bytes(n_vis, 8) == 8 * (1 << 20) * 68 + 8 * (32 * 68 + 128) + 8 * (1 << 17) * 4
    assert bench.scan_bytes([9, 0], 2) == 9 * 68 + 2 * (32 * 68 + 128) + 2 * 4
    # the bench's default workload: the figure its roofline divides by
    assert bench.scan_bytes(n_vis, 8) == 574638080


def _record(tmp_path, sources, digest, traffic=123456789):
    rec = {"source_files": sources, "source_sha256": digest, "traffic_bytes_per_launch": traffic}
    (tmp_path / "profiles").mkdir(exist_ok=True)
    (tmp_path / "profiles" / "r.json").write_text(json.dumps(rec))


def test_traffic_record_needs_unchanged_sources(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_bytes(b"kernel source v1\n")
    digest = hashlib.sha256(b"kernel source v1\n").hexdigest()
    _record(tmp_path, ["k.hip"], digest)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("r") == 123456789
    src.write_bytes(b"kernel source v2\n")  # the kernel changed since the counters were taken
    assert bench.measured_traffic("r") is None
    assert bench.measured_traffic("missing") is None


@pytest.mark.parametrize("name", ["score_full_fullscan_1m_traffic", "score_multi_prefill_128k_traffic",
                                  "score_gather_reindex_1m_traffic"])
def test_committed_traffic_records_are_current(name):
    # every committed record matches the sources in the tree (otherwise the bench line would
    # report traffic null): re-take the counters after a kernel change
    rec = json.load(open(os.path.join(ROOT, "profiles", name + ".json")))
    h = hashlib.sha256()
    for f in rec["source_files"]:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    assert h.hexdigest() == rec["source_sha256"], f"{name}: sources changed since the counters were taken"
    assert bench.measured_traffic(name) == rec["traffic_bytes_per_launch"]
    # never below the bytes the kernel must move
    assert rec["traffic_bytes_per_launch"] >= 0.99 * rec["algorithmic_bytes_per_launch"]


def test_cpu_baseline_reports_cores_model_and_median():
    import synth

    wl = synth.decode_workload("cpu", 9, [20000, 17001], layers=1)
    r = bench.cpu_baseline(wl, target_s=0.5, runs=3)
    assert r["kind"] == "oracle" and r["unit"] == "entries/s" and r["value"] > 0
    assert r["cores"] == bench.host_threads() and r["nproc"] == os.cpu_count()
    assert isinstance(r["cpu_model"], str) and r["cpu_model"]
    assert "median of 3 runs" in r["sample"]
    # the step's entries: every visible key of the Full layer plus the pooled keys of the Reindex layer
    assert r["entries_per_run"] == 20000 + 17001 + min(20000, 16384) + min(17001, 16384)
