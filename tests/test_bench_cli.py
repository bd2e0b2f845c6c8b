"""bench.py's host-side contract (CPU only): more than one GPU is refused with a message and
exit status 2 before anything touches a device; the stored HBM-traffic figure of a workload is
read back only while the kernel sources still hash to the value its summary was taken with."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--steps", "1"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_stored_traffic_follows_the_source_hash(tmp_path, monkeypatch):
    h = bench.source_hash()
    assert len(h) == 16
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "dec_engine_x_traffic.md").write_text(f"# x\n\nsource_hash: {h}\ntraffic_bytes_per_launch: 1234\n")
    (prof / "dec_engine_y_traffic.md").write_text("# y\n\nsource_hash: 0000000000000000\ntraffic_bytes_per_launch: 99\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "source_hash", lambda: h)
    assert bench.stored_traffic("x") == 1234
    assert bench.stored_traffic("y") is None  # taken with other kernel sources
    assert bench.stored_traffic("z") is None  # no summary
