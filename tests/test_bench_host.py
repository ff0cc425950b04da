"""Host logic of bench.py that runs without a GPU: the one-GPU refusal and the gating of the
committed HBM-traffic figure on the decode kernel's source hash and launch configuration."""
import importlib.util
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_source_hash_covers_the_decode_kernel_sources():
    b = _bench()
    assert len(b.kernel_source_sha()) == 16
    assert b.kernel_source_sha() == b.kernel_source_sha()
    for rel in b.KERNEL_SOURCES:
        assert os.path.isfile(os.path.join(ROOT, rel)), rel
    names = {os.path.basename(p) for p in b.KERNEL_SOURCES}
    assert {"decode_mfma.hip", "schedule.h", "device_common.h", "mfma_common.h"} <= names


def test_traffic_is_reported_only_for_the_measured_source_and_launch(tmp_path):
    b = _bench()
    rec = {"kernel_source_sha": b.kernel_source_sha(), "block_size": 16, "num_workers": 0,
           "hbm_bytes_per_launch": 123456789}
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps(rec))
    b.TRAFFIC_FILE = str(f)
    assert b.measured_traffic(16, 0) == 123456789
    assert b.measured_traffic(32, 0) is None          # another block size
    assert b.measured_traffic(16, 512) is None        # another worker count
    f.write_text(json.dumps(dict(rec, kernel_source_sha="0" * 16)))
    assert b.measured_traffic(16, 0) is None          # kernel changed since the counters
    f.write_text("not json")
    assert b.measured_traffic(16, 0) is None
    b.TRAFFIC_FILE = str(tmp_path / "missing.json")
    assert b.measured_traffic(16, 0) is None


def test_committed_traffic_record_names_its_sources():
    b = _bench()
    with open(os.path.join(ROOT, "profiles", "decode_partial_mfma_gqa256_b16_traffic.json")) as f:
        t = json.load(f)
    assert len(t["kernel_source_sha"]) == 16
    assert t["block_size"] == 16
    assert t["hbm_bytes_per_launch"] > 0
    assert sorted(t["kernel_source_files"]) == sorted(b.KERNEL_SOURCES)
