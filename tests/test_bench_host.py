"""Host-side checks of bench.py (no GPU): the one-GPU rule and where the
roofline's traffic figure may come from."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr


def test_traffic_only_for_the_counted_shape_and_source(tmp_path, monkeypatch):
    M, N, K = 65536, 5120, 1280                    # the d20 MLP up-projection
    alg = 2 * (M * K + N * K + M * N)
    import hashlib
    got = bench.measured_traffic(alg)
    fields = dict(line.split(":", 1) for line in open(bench.TRAFFIC_FILE) if ":" in line)
    assert int(fields["algorithmic bytes per launch"]) == alg
    sha = hashlib.sha256(open(bench.GEMM_SOURCE, "rb").read()).hexdigest()
    if fields["gemm.hip sha256"].strip() == sha:   # counters taken on this source
        assert got == pytest.approx(float(fields["hbm bytes per launch"]))
        assert got > alg                          # fetches include per-XCD re-reads
    else:
        assert got is None
    # another GEMM shape (d26) has no counters
    assert bench.measured_traffic(2 * (262144 * 1664 + 6656 * 1664 + 262144 * 6656)) is None
    # counters of another version of the GEMM source do not count
    other = tmp_path / "gemm.hip"
    other.write_text("// another version\n")
    monkeypatch.setattr(bench, "GEMM_SOURCE", str(other))
    assert bench.measured_traffic(alg) is None
