"""The decode work split's host arithmetic, checked natively (no GPU): the
slice table, the slice lookup, and the two divisions the kernels use in place
of 64-bit integer division."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "kv_cached_gqa_amd", "csrc")


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    pytest.skip("hipcc not found")


def test_split_arithmetic(tmp_path):
    exe = tmp_path / "split_check"
    src = os.path.join(ROOT, "tests", "native", "split_check.cpp")
    subprocess.run([_hipcc(), "-O2", "-std=c++17", f"-I{CSRC}", f"-I{os.path.join(ROOT, 'include')}", src,
                    "-o", str(exe)], check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-2000:]
    assert r.stdout.strip().endswith("ok: 0 failures")
