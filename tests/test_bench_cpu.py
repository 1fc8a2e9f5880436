"""bench.py's contract pieces that run without a GPU: one GPU only (any other
count exits with a message that says so), and the oracle baseline's fields
(a bounded sample of the batched-decode workload on the host's cores)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--no-extra",
                        "--no-cpu-baseline"], capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in r.stderr and r.stdout.strip() == ""


def test_cpu_baseline_fields():
    sys.path.insert(0, ROOT)
    import bench
    rec = bench.cpu_baseline(bench.lengths_seed0(), seconds=0.5, threads=1)
    assert rec["kind"] == "oracle" and rec["unit"] == "GB/s" and rec["cores"] == 1
    assert rec["value"] > 0 and "decode steps" in rec["sample"]
    assert rec["tokens_per_s"] > 0 and rec["s_per_step"] > 0
