"""Host-side logic of bench.py (no GPU): the single-GPU contract, the source hashes that
tie the committed rocprofv3 traffic counters to the kernels they were taken from, and
the rule that voids those counters once a kernel's sources change."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = run_bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_source_hashes_cover_every_measured_kernel():
    r = run_bench("--print-source-hashes")
    assert r.returncode == 0
    hashes = json.loads(r.stdout)
    assert set(hashes) == set(bench.KERNEL_SOURCES) == {"prefill", "decode_split", "window",
                                                     "short_split"}
    for kind, h in hashes.items():
        assert h == bench.source_hash(kind) and len(h) == 64
        for f in bench.KERNEL_SOURCES[kind]:
            assert os.path.exists(os.path.join(bench.CSRC, f)), f


def test_committed_traffic_counters_match_the_current_kernels():
    """profiles/traffic.json was taken from the kernels as they stand, so the bench
    line reports the measured HBM traffic instead of null."""
    with open(bench.TRAFFIC_FILE) as fh:
        t = json.load(fh)
    for kind in bench.KERNEL_SOURCES:
        assert t[kind]["source_sha256"] == bench.source_hash(kind), kind
        assert bench.measured_traffic(kind) > 0


@pytest.mark.parametrize("same_hash", [True, False])
def test_traffic_is_void_when_the_sources_changed(tmp_path, monkeypatch, same_hash):
    entry = {"kernel": "k", "fetch_kib": 1000.0, "write_kib": 500.0, "fetch_scale": 2.0,
             "write_scale": 1.0,
             "source_sha256": bench.source_hash("prefill") if same_hash else "0" * 64}
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps({"prefill": entry}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    got = bench.measured_traffic("prefill")
    assert got == ((1000.0 * 2.0 + 500.0) * 1024 if same_hash else None)
    assert bench.measured_traffic("decode_split") is None  # no entry at all
