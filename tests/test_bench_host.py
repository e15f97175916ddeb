"""Host logic of bench.py that runs without a GPU: the refusal of more than one GPU and the rule
that counter-measured traffic is reported only for the kernel sources and workload it was taken on."""

import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr or "--gpus 1" in r.stderr
    assert r.stdout.strip() == ""


def _record(tmp_path, **kw):
    rec = {"kernel": "vocabulary kernels", "workload": "c3", "hbm_bytes_per_launch": 123456789,
           "kernel_source_sha256": bench.kernel_source_sha256()}
    rec.update(kw)
    p = tmp_path / "pmc.json"
    p.write_text(json.dumps(rec))
    return str(p)


def test_traffic_only_for_matching_sources_and_workload(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PMC_FILE", _record(tmp_path))
    assert bench.measured_traffic("c3") == 123456789
    assert bench.measured_traffic("c2") is None
    assert bench.measured_traffic("c5") is None
    monkeypatch.setattr(bench, "PMC_FILE", _record(tmp_path, kernel_source_sha256="0" * 64))
    assert bench.measured_traffic("c3") is None
    monkeypatch.setattr(bench, "PMC_FILE", str(tmp_path / "missing.json"))
    assert bench.measured_traffic("c3") is None


def test_committed_record_names_its_workload():
    rec = json.load(open(os.path.join(ROOT, "profiles", "pmc_vocab_worker_batched_verify.json")))
    assert rec["workload"] == "c3"
    assert rec["hbm_bytes_per_launch"] > 0
    assert len(rec["kernel_source_sha256"]) == 64
