"""Host logic of bench.py (no GPU): the one-GPU contract and the source
fingerprint that decides whether the committed HBM counters still describe
the kernels."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=120)
    assert r.returncode == 2
    assert r.stdout == ""
    assert "one GPU" in r.stderr and "--gpus 2" in r.stderr


def test_kernel_fingerprint_ignores_comments_and_layout_only():
    src = "int f(int a) {\n  // scale\n  return a * 2; /* twice */\n}\n"
    same = "int f(int a) { /* other words */ return a * 2;   // changed comment\n}"
    other = "int f(int a) {\n  // scale\n  return a * 3; /* twice */\n}\n"
    assert bench.kernel_code_text(src) == bench.kernel_code_text(same)
    assert bench.kernel_code_text(src) != bench.kernel_code_text(other)
    assert "scale" not in bench.kernel_code_text(src)  # the comments are gone


def test_committed_counter_summary_names_its_fingerprint_and_kernels():
    import json
    rec = json.load(open(os.path.join(ROOT, "profiles", "dit32_1024px_hbm_traffic.json")))
    assert len(rec["kernel_source_sha256"]) == 64
    for kind in ("gemm_gate_up", "gemm_qkv", "gemm_down", "gemm_o", "attention"):
        ent = rec["kernels"][kind]["image-only"]
        assert int(ent["hbm_bytes"]) > 0
