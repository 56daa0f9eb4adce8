"""Host-side checks of bench.py's contract that need no GPU: the one-GPU refusal, the
algorithmic byte counts it reports, and the committed traffic record it reads."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_algorithmic_bytes_per_element():
    M, K = 65536, 2048
    assert bench.mx_both_bytes(M, K) == M * K * (2 + 2 * (1 + 1 / 32))      # 4.0625 B / element
    assert bench.mx_dq_bytes(M, K) == M * K * (1 + 1 / 32 + 2)
    R = 524288
    assert bench.nv_bytes(R, K) == R * (2 * K + K // 2 + K // 16 + 4)   # the dominant kernel
    assert bench.nv_bytes(R, K) == 2753560576


def test_traffic_record_names_its_sources_and_scales():
    rec = json.load(open(bench.TRAFFIC_RECORD))
    assert rec["algorithmic_bytes_per_launch"] == bench.nv_bytes(524288, 2048)
    parts = rec["hbm_read_bytes_per_launch"] + rec["hbm_write_bytes_per_launch"]
    assert abs(rec["traffic_bytes_per_launch"] - parts) <= 1                # each figure rounded on its own
    assert abs(rec["traffic_bytes_per_launch"] / rec["algorithmic_bytes_per_launch"] - 1) < 0.01
    for p in rec["kernel_sources"]:
        assert os.path.exists(os.path.join(ROOT, p))
    assert abs(rec["fetch_size_scale"] - 2.0) < 0.01 and abs(rec["write_size_scale"] - 1.0) < 0.01


def test_cpu_baseline_reports_the_oracle_with_all_threads_and_with_one():
    import numpy as np
    import oracle
    import workloads
    rng = np.random.default_rng(5)
    a = workloads.bf16_bits_from_f32(rng.standard_normal((2048, 256)).astype(np.float32))
    w = workloads.bf16_bits_from_f32(rng.standard_normal((64, 512)).astype(np.float32))
    tok = rng.integers(0, 2048, size=4096)
    threads = oracle.max_threads()
    r = bench.cpu_baseline(a, w, tok, 1, 1)
    assert r["kind"] == "oracle" and r["unit"] == "GB/s" and r["value"] > 0
    assert r["cores"] == threads and "sample" in r
    st = r["single_thread"]
    assert st["cores"] == 1 and st["value"] > 0 and "1/32" in st["sample"]
    assert oracle.max_threads() == threads                    # restored afterwards
