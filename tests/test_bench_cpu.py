"""The benchmark's host-side contract, checked without a GPU: it refuses more than
one GPU, counts the algorithmic flops of each contraction launch, and reports HBM
traffic only from a counter summary taken on the current kernel source."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout.strip() == ""


def test_contraction_flops_per_launch():
    N, D, V = 16384, 2688, 131072
    for kind in ("forward", "dlogits", "d_hidden", "d_weight"):
        assert bench.contraction_flops(kind, N, D, V, 1) == 2.0 * N * D * V
    # a backward in several row chunks splits the rows over its launches
    assert bench.contraction_flops("dlogits", N, D, V, 4) == 2.0 * N * D * V / 4
    assert bench.contraction_flops("merge", N, D, V, 1) == 0.0


def test_traffic_only_for_the_current_kernel_source(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    entry = {"kernels": {"dlogits": {"hbm_bytes_per_launch": 123.0}}}
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_sha", lambda: "abc")
    assert bench.load_traffic("train_n16384", "dlogits") is None  # no summary at all
    (prof / "traffic_train_n16384.json").write_text(json.dumps({**entry, "kernel_source_sha": "abc"}))
    assert bench.load_traffic("train_n16384", "dlogits") == 123.0
    assert bench.load_traffic("train_n16384", "forward") is None  # kernel not in the summary
    (prof / "traffic_train_n16384.json").write_text(json.dumps({**entry, "kernel_source_sha": "old"}))
    assert bench.load_traffic("train_n16384", "dlogits") is None  # taken on other kernels


def test_kernel_source_sha_is_of_the_kernel_file():
    import hashlib
    p = os.path.join(ROOT, "lm_head_selected_bf16_amd", "csrc", "flp_kernels.hip")
    assert bench.kernel_source_sha() == hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]
