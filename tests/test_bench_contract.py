"""Host-side parts of the benchmark contract: one GPU only (--gpus N > 1
exits with a message), and the counter summary it reads is tied to the
kernel sources and the step's launch size."""

import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert p.returncode == 2
    assert "one GPU" in p.stderr and p.stdout == ""


def test_traffic_is_reported_only_for_the_measured_kernel_and_launch():
    fields = {}
    with open(bench.TRAFFIC_PROFILE) as f:
        for line in f:
            if line.startswith("- ") and ":" in line:
                k, v = line[2:].split(":", 1)
                fields[k.strip()] = v.strip()
    alg = int(fields["algorithmic_bytes_per_launch"])
    assert fields["source_sha256"] == bench.kernel_source_hash()
    assert bench.measured_traffic(alg) == float(fields["hbm_bytes_per_launch"])
    assert bench.measured_traffic(alg // 2) is None
    # within 1% of the algorithmic bytes: no re-reads, no write amplification
    assert abs(float(fields["hbm_bytes_per_launch"]) / alg - 1) < 0.01


def test_source_hash_ignores_comments_but_not_code(tmp_path, monkeypatch):
    """Editing a comment keeps the recorded counters valid; editing code
    invalidates them."""
    import shutil
    csrc = tmp_path / "gradient_all_reduce_allreduce_amd" / "csrc"
    shutil.copytree(os.path.join(ROOT, "gradient_all_reduce_allreduce_amd", "csrc"), csrc)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.kernel_source_hash()
    f = csrc / bench.KERNEL_SOURCES[0]
    f.write_text(f.read_text() + "\n// a new comment line\n/* and a block\n   comment */\n")
    assert bench.kernel_source_hash() == h0
    f.write_text(f.read_text() + "static const int kUnused = 1;\n")
    assert bench.kernel_source_hash() != h0
