"""Host-side logic of bench.py that runs without a GPU."""
import hashlib
import subprocess
import sys

import bench


def test_counter_traffic_needs_matching_sources(tmp_path):
    (tmp_path / "a.hip").write_bytes(b"kernel a")
    (tmp_path / "b.h").write_bytes(b"header b")
    digest = hashlib.sha256(b"kernel a" + b"header b").hexdigest()
    summary = tmp_path / "s.md"
    body = "fetch-scale: 2.0\nwrite-scale: 1.0\nFETCH_SIZE_KiB: 100\nWRITE_SIZE_KiB: 50\n"
    summary.write_text(f"# x\n\nsource-sha256: {digest}\n" + body)
    assert bench.counter_traffic(["a.hip", "b.h"], str(summary), str(tmp_path)) == 1024 * 250
    summary.write_text("source-sha256: " + "0" * 64 + "\n" + body)
    assert bench.counter_traffic(["a.hip", "b.h"], str(summary), str(tmp_path)) is None
    assert bench.counter_traffic(["a.hip", "b.h"], str(tmp_path / "missing.md"), str(tmp_path)) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True, text=True)
    assert r.returncode != 0 and "one GPU" in (r.stdout + r.stderr)
