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


def test_traffic_is_reported_only_for_the_measured_kernel_and_step(tmp_path, monkeypatch):
    """measured_traffic returns the recorded HBM bytes per launch only for
    the kernel source and step shape the counters were taken on."""
    prof = tmp_path / "traffic.md"
    prof.write_text("# counters\n\n- hbm_bytes_per_step: 3900\n- algorithmic_bytes_per_step: 3900\n"
                    "- launches_per_step: 39\n- source_sha256: " + bench.kernel_source_hash() + "\n")
    monkeypatch.setattr(bench, "TRAFFIC_PROFILE", str(prof))
    assert bench.measured_traffic(3900, 39) == 100.0
    assert bench.measured_traffic(3900, 38) is None
    assert bench.measured_traffic(3901, 39) is None
    prof.write_text(prof.read_text().replace(bench.kernel_source_hash(), "0" * 64))
    assert bench.measured_traffic(3900, 39) is None


def test_committed_traffic_profile_matches_the_headline_kernel():
    """The committed counter summary of the headline kernel was taken on the
    current kernel source and on the headline step: bytes per step are P * n
    * (2 + 4) over the transformer gradient set, one launch per bucket."""
    import math

    import workloads
    fields = bench.profile_fields(bench.TRAFFIC_PROFILE)
    assert fields["source_sha256"] == bench.kernel_source_hash()
    total = sum(math.prod(s) for s in workloads.model_shapes("transformer_2b"))
    alg = 8 * total * 6
    assert int(fields["algorithmic_bytes_per_step"]) == alg
    assert int(fields["launches_per_step"]) == -(-total // (100 * 2**20 // 2))
    traffic = bench.measured_traffic(alg, int(fields["launches_per_step"]))
    assert traffic is not None
    # within 1% of the algorithmic bytes: no re-reads, no write amplification
    assert abs(traffic * int(fields["launches_per_step"]) / alg - 1) < 0.01


def test_every_suite_workload_names_its_kernel():
    """Each workload of the suite states the kernel a profiler attributes its
    time and counters to (or None for multi-kernel steps)."""
    assert bench.HEADLINE_KERNEL.startswith("ring_reduce_kernel<8, true, false")
    assert "ring-transformer2b" in bench.WORKS and "pack-ragged2000" in bench.WORKS


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
