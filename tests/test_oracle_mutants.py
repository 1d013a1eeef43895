"""The oracle's pins catch plausible mistakes.

Each case below plants one mistake in a copy of the oracle package (on the
CPU, in a temporary directory): a wrong ring direction, start rank, owner or
chunk length, Mean taken by reciprocal or left out, wider accumulation, a
truncating or tie-breaking bf16 rounding, a lost quiet bit, a momentum step
with dampening or a fused multiply-add, a forward bucket order, a dropped tail
bucket, another tree, the levels of the two-level reduction swapped, the
ZeRO step gathering gradients instead of weights.  The copy is registered
as ``oracle`` in a fresh interpreter, which then runs the pin tests of that
part; each mistake must make at least one of them fail.  The unchanged copy
must pass the same pins, which shows that the harness runs the copy and
that a failure comes from the planted mistake.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.join(ROOT, "tests")

RING_PINS = ["test_oracle_ring.py"]
BF16_SGD_BUCKET_PINS = ["test_oracle_bf16_sgd_bucket.py"]

# (name, oracle module, text to replace (must occur once), replacement, pin files)
MUTANTS = [
    ("ring runs backwards", "ring.py",
     "            dst = (r + 1) % P\n            for j, (lo, hi) in enumerate(chunks):\n"
     "                if start[j] == (r - t) % P:",
     "            dst = (r + P - 1) % P\n            for j, (lo, hi) in enumerate(chunks):\n"
     "                if start[j] == (r + t) % P:",
     RING_PINS),
    ("chunk starts one rank late", "ring.py",
     "start = [j % P for j in range(C)]", "start = [(j + 1) % P for j in range(C)]", RING_PINS),
    ("owner is the start rank", "ring.py",
     "owner = [(s + P - 1) % P for s in start]", "owner = [s for s in start]", RING_PINS),
    ("chunk length rounded down", "ring.py",
     "return -(-n // chunking) if n > 0 else 0", "return max(1, n // chunking) if n > 0 else 0",
     RING_PINS),
    ("all-gather forwards from the wrong rank", "ring.py",
     "if owner[j] == (r - t) % P:", "if owner[j] == (r - t - 1) % P:", RING_PINS),
    ("Mean by the reciprocal", "ring.py",
     "A[owner[j], lo:hi] = A[owner[j], lo:hi] / div\n\n    _all_gather_steps",
     "A[owner[j], lo:hi] = A[owner[j], lo:hi] * (A.dtype.type(1) / div)\n\n    _all_gather_steps",
     RING_PINS),
    ("Mean left out", "ring.py",
     "    if op == MEAN:\n        div = A.dtype.type(P)\n        for j, (lo, hi) in enumerate(chunks):\n"
     "            A[owner[j], lo:hi] = A[owner[j], lo:hi] / div\n\n    _all_gather_steps",
     "    if False:\n        div = A.dtype.type(P)\n        for j, (lo, hi) in enumerate(chunks):\n"
     "            A[owner[j], lo:hi] = A[owner[j], lo:hi] / div\n\n    _all_gather_steps",
     RING_PINS),
    ("float32 inputs summed in float64", "ring.py",
     'if in_dtype == "f32":\n        return np.array(X, dtype=np.float32, copy=True)',
     'if in_dtype == "f32":\n        return np.array(X, dtype=np.float64, copy=True)',
     RING_PINS),
    ("sampled start ranks shifted", "ring.py",
     "return (idx // L) % P", "return (idx // L + 1) % P", RING_PINS),
    ("sampled ring walks the wrong way", "ring.py",
     "src = (start + t) % P", "src = (start - t) % P", RING_PINS),
    ("bf16 output truncated", "bf16.py",
     "out_mag = np.where(take_hi, hi_mag, lo_mag)", "out_mag = lo_mag", BF16_SGD_BUCKET_PINS),
    ("bf16 ties rounded up", "bf16.py",
     "take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ~lo_even)", "take_hi = d_hi <= d_lo",
     BF16_SGD_BUCKET_PINS),
    ("bf16 NaN not quieted", "bf16.py",
     "nan_out = ((u >> np.uint32(16)) | np.uint32(0x0040))", "nan_out = u >> np.uint32(16)",
     BF16_SGD_BUCKET_PINS),
    ("bf16 widened by the wrong shift", "bf16.py",
     "return (b << np.uint32(16)).view(np.float32)",
     "return ((b << np.uint32(16)) | np.uint32(0x8000)).view(np.float32)",
     BF16_SGD_BUCKET_PINS + RING_PINS),
    ("momentum with dampening", "sgd.py",
     "v_new = v_scaled + g ", "v_new = v_scaled + (np.float32(1) - mu32) * g ",
     BF16_SGD_BUCKET_PINS),
    ("weights moved up the gradient", "sgd.py",
     "w_new = w - step ", "w_new = w + step ", BF16_SGD_BUCKET_PINS),
    ("update fused into one rounding", "sgd.py",
     "w_new = w - step ",
     "w_new = (w.astype(np.float64) - np.float64(lr32) * v_new.astype(np.float64)).astype(np.float32) ",
     BF16_SGD_BUCKET_PINS),
    ("momentum fused into one rounding", "sgd.py",
     "v_new = v_scaled + g ",
     "v_new = (np.float64(mu32) * v.astype(np.float64) + g.astype(np.float64)).astype(np.float32) ",
     BF16_SGD_BUCKET_PINS),
    ("buckets planned in parameter order", "bucket.py",
     "    segments = []\n    flat = 0\n    for t in reversed(range(len(numels))):",
     "    segments = []\n    flat = 0\n    for t in range(len(numels)):",
     BF16_SGD_BUCKET_PINS),
    ("tensors packed in parameter order", "bucket.py",
     "flat = [np.asarray(t).reshape(-1) for t in reversed(list(tensors))]",
     "flat = [np.asarray(t).reshape(-1) for t in list(tensors)]",
     BF16_SGD_BUCKET_PINS),
    ("tail bucket dropped", "bucket.py",
     "n_buckets = -(-total // E)", "n_buckets = total // E", BF16_SGD_BUCKET_PINS),
    ("another tree", "tree.py",
     "(c - 1) // branching for c in range(1, P)", "c // branching for c in range(1, P)",
     ["test_oracle_tree.py"]),
    ("the two levels swapped", "hierarchical.py",
     "Y = _level_sum(A[g * Lr:(g + 1) * Lr], local[0], local[1], acc)",
     "Y = _level_sum(A[g * Lr:(g + 1) * Lr], global_[0], global_[1], acc)",
     ["test_oracle_hierarchical.py"]),
    ("two-level Mean over one node", "hierarchical.py",
     "total = total / A.dtype.type(P)", "total = total / A.dtype.type(Lr)",
     ["test_oracle_hierarchical.py"]),
    ("ZeRO gathers gradients, not weights", "zero.py",
     "B[r, mine] = w_new[mine]", "B[r, mine] = R[r, mine]", ["test_oracle_zero.py"]),
]

# Registers a package directory as ``oracle`` and runs pytest on the rest of
# the command line.
DRIVER = r"""
import importlib.util, sys
pkg = sys.argv[1]
spec = importlib.util.spec_from_file_location("oracle", pkg + "/__init__.py",
                                              submodule_search_locations=[pkg])
mod = importlib.util.module_from_spec(spec)
sys.modules["oracle"] = mod
spec.loader.exec_module(mod)
assert sys.modules["oracle"].__file__.startswith(pkg)
import pytest
sys.exit(pytest.main(sys.argv[2:]))
"""


def run_pins(pkg_dir, pin_files):
    cmd = [sys.executable, "-c", DRIVER, pkg_dir, "-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider"] \
        + [os.path.join(TESTS, f) for f in pin_files]
    env = dict(os.environ, PYTHONDONTWRITEBYTECODE="1", OMP_NUM_THREADS="1")
    p = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    return p.returncode, p.stdout[-3000:] + p.stderr[-2000:]


def copy_oracle(dst, mutant=None):
    pkg = os.path.join(dst, "oracle")
    shutil.copytree(os.path.join(ROOT, "oracle"), pkg, ignore=shutil.ignore_patterns("__pycache__"))
    if mutant is not None:
        _, module, old, new, _ = mutant
        path = os.path.join(pkg, module)
        with open(path) as f:
            text = f.read()
        assert text.count(old) == 1, f"{mutant[0]}: the text to replace occurs {text.count(old)} times"
        with open(path, "w") as f:
            f.write(text.replace(old, new))
    return pkg


def test_unchanged_copy_passes_every_pin(tmp_path):
    files = sorted({f for m in MUTANTS for f in m[4]})
    rc, out = run_pins(copy_oracle(str(tmp_path)), files)
    assert rc == 0, out


def test_every_planted_mistake_is_caught(tmp_path):
    def one(k):
        m = MUTANTS[k]
        return m[0], run_pins(copy_oracle(str(tmp_path / f"m{k}"), m), m[4])

    with ThreadPoolExecutor(max_workers=4) as pool:
        results = list(pool.map(one, range(len(MUTANTS))))
    # pytest's exit status 1 means "some tests failed": the pins ran and
    # rejected the mutant (2+ would be an interrupted or broken run).
    missed = [(name, rc, out) for name, (rc, out) in results if rc != 1]
    assert not missed, "\n\n".join(f"{name}: exit {rc}\n{out}" for name, rc, out in missed)
