"""Host-side checks of bench.py that need no GPU: the one-GPU guard, the
traffic record it reads from the committed counter summary (scaling by the
calibration copy, and None once the kernel's sources differ from the ones the
counters were taken on), and the shape of the CPU baseline entry on a tiny
sample of the step."""
import json
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

STAGE = "gemm_block_16384x2048x7168"


def test_more_than_one_gpu_is_refused():
    for argv, env in ((["--gpus", "2"], {}), (["--gpus", "1"], {"WORLD_SIZE": "4"})):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + argv, capture_output=True, text=True,
                           env={**os.environ, **env}, timeout=120)
        assert r.returncode == 2
        assert "one GPU" in r.stderr and r.stdout == ""


def _fake_tree(tmp_path, record):
    csrc = tmp_path / "fp8_scaled_matmul_amd" / "csrc"
    csrc.mkdir(parents=True)
    for f in bench.KERNEL_SOURCES[STAGE]:
        shutil.copy(os.path.join(ROOT, "fp8_scaled_matmul_amd", "csrc", f), csrc / f)
    prof = tmp_path / "profiles"
    prof.mkdir()
    if record is not None:
        (prof / f"{STAGE}_traffic.md").write_text("# summary\n\ntraffic-record: " + json.dumps(record) + "\n")
    return str(tmp_path)


def test_traffic_record_scaling(tmp_path, monkeypatch):
    # counters read half the true bytes on fetch and exactly on write for the
    # 1 GiB copy: the kernel's 1000 KiB fetched are 2000 KiB, 300 KiB written stay
    rec = {"kernel": "k", "fetch_kib": 1000.0, "write_kib": 300.0, "copy_fetch_kib": 524288.0,
           "copy_write_kib": 1048576.0, "copy_bytes": bench.COPY_BYTES}
    monkeypatch.setattr(bench, "ROOT", _fake_tree(tmp_path, None))
    assert bench.measured_traffic(STAGE) is None                       # no summary
    rec["sources_sha256"] = bench.sources_hash(STAGE)
    monkeypatch.setattr(bench, "ROOT", _fake_tree(tmp_path / "b", rec))
    assert bench.measured_traffic(STAGE) == (2000 + 300) * 1024
    assert bench.measured_traffic("no_such_stage") is None


def test_traffic_record_goes_stale_with_the_sources(tmp_path, monkeypatch):
    root = _fake_tree(tmp_path, None)
    monkeypatch.setattr(bench, "ROOT", root)
    rec = {"kernel": "k", "fetch_kib": 1.0, "write_kib": 1.0, "copy_fetch_kib": 1.0, "copy_write_kib": 1.0,
           "copy_bytes": bench.COPY_BYTES, "sources_sha256": bench.sources_hash(STAGE)}
    with open(os.path.join(root, "profiles", f"{STAGE}_traffic.md"), "w") as fh:
        fh.write("traffic-record: " + json.dumps(rec) + "\n")
    assert bench.measured_traffic(STAGE) is not None
    with open(os.path.join(root, "fp8_scaled_matmul_amd", "csrc", bench.KERNEL_SOURCES[STAGE][0]), "a") as fh:
        fh.write("\n// changed\n")
    assert bench.measured_traffic(STAGE) is None


def test_committed_traffic_record_is_well_formed():
    path = os.path.join(ROOT, "profiles", f"{STAGE}_traffic.md")
    if not os.path.exists(path):
        pytest.skip("no committed traffic summary")
    recs = [json.loads(l[len("traffic-record: "):]) for l in open(path) if l.startswith("traffic-record: ")]
    assert len(recs) == 1
    r = recs[0]
    assert r["copy_bytes"] == bench.COPY_BYTES
    assert r["fetch_kib"] > 0 and r["write_kib"] > 0
    # the block-scaled GEMM reads at least A and B once and writes its bf16 output once
    m, n, k = bench.FA_M, bench.FA_N, bench.FA_K
    fetch = r["fetch_kib"] * bench.COPY_BYTES / r["copy_fetch_kib"]
    write = r["write_kib"] * bench.COPY_BYTES / r["copy_write_kib"]
    assert fetch >= 0.99 * (m * k + n * k)
    assert write >= 0.99 * (2 * m * n)


def test_cpu_baseline_entry():
    out = bench.cpu_baseline(64, {})
    assert out["kind"] == "oracle" and out["unit"] == "TFLOP/s"
    assert out["value"] > 0 and out["cores"] >= 1
    assert "64 of 65536" in out["sample"]
