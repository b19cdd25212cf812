"""Host-side checks of bench.py (no GPU): the byte accounting the roofline uses and the
refusal to run on more than one GPU."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from paged_kv_cache_288_amd.workloads import make_workload  # noqa: E402


def test_kv_bytes_logical_and_unique():
    w = make_workload("gqa70b", seed=2, B=5, lens=("uniform", 10, 300))
    per_token = 2 * w.Hkv * w.d * 2
    assert bench.kv_bytes(w) == int(w.context_lens.sum()) * per_token
    assert bench.kv_unique_bytes(w) == bench.kv_bytes(w)          # nothing shared
    f = make_workload("fp8prefix", seed=2, B=6, lens=("prefix", 256, 1, 90))
    per_token = 2 * f.Hkv * f.d * 1
    prefix = f.meta["prefix_blocks"] * f.bs
    assert bench.kv_bytes(f) == int(f.context_lens.sum()) * per_token
    assert bench.kv_unique_bytes(f) == (prefix + int((f.context_lens - prefix).sum())) * per_token
    m = make_workload("mla", seed=2, B=3, lens=("uniform", 64, 200))
    assert bench.kv_bytes(m) == int(m.context_lens.sum()) * 576 * 2


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stdout


def test_kernel_hash_ignores_comments():
    src = "int f(int x) { // the answer\n  return x; /* done */ }\n"
    assert bench._code_only(src) == bench._code_only("int f(int x) {\n  return x;  }\n")
    h = bench.kernel_hash("gqa")
    assert isinstance(h, str) and len(h) == 16 and h == bench.kernel_hash("gqa")
