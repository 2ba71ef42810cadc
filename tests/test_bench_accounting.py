"""The benchmark's own arithmetic, on the CPU: the algorithmic bytes behind the roofline
fraction, restated by hand from the cache and query layouts, and the one-GPU guard."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads as W  # noqa: E402


def test_algorithmic_bytes_by_hand():
    case = W.generate(W.config(1), 0)          # 4 rows, 16 blocks of 64, top-256
    ends = np.array([1000, 1024, 17, 0])
    # K: 64 bytes of e2m1 values + 4 UE8M0 bytes per valid column
    k_bytes = int(ends.sum()) * (64 + 4)
    # per row: the MXFP4 query (64 heads x (64 + 4) bytes), 64 fp32 weights, 12 bytes per
    # candidate block (id, schedule entry, block-table entry), 4 bytes per output slot
    row = 64 * 68 + 64 * 4 + 12 * 16 + 4 * 256
    assert bench.algorithmic_bytes(case, "mxfp4", ends) == k_bytes + 4 * row
    assert bench.algorithmic_bytes(case, "mxfp4", ends, with_output=False) == \
        k_bytes + 4 * (row - 4 * 256)
    # fp8 queries: 64 x 128 e4m3 bytes and one fp32 row scale
    row8 = 64 * 128 + 4 + 64 * 4 + 12 * 16 + 4 * 256
    assert bench.algorithmic_bytes(case, "fp8", ends) == k_bytes + 4 * row8


def test_gather_bytes_by_hand():
    case = W.generate(W.config(1), 0)          # 4 decode rows, one table row each, page 64
    case.row_ke[:] = [4096, 65, 1, 0]
    tables, lens, nbytes = bench.gather_workload(case)
    assert list(lens) == [4096, 65, 1, 0]
    # 68 bytes a position read and 68 written; block-table entries: 64 + 2 + 1 + 0 pages
    assert nbytes == (4096 + 65 + 1) * 136 + (64 + 2 + 1) * 4 + 8 * 4


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_source_bytes_by_hand():
    case = W.generate(W.config(1), 0)          # 4 rows, cbs 64, 16 blocks published a row
    case.row_ks[:] = [0, 10, 0, 0]
    case.row_ke[:] = [4096, 4096, 100, 0]
    ctx = 4096 + 4086 + 100 + 0
    parts = 4096 // 64                          # one part key a 64-token part of max_ctx
    row = 64 * 68 + 64 * 4 + 2 * 4 * parts + 4 * 16
    assert bench.source_bytes(case, "mxfp4", 4096) == ctx * 68 + 4 * row
    # bf16 weights: 2 bytes a head
    assert bench.source_bytes(case, "mxfp4", 4096, "bf16") == ctx * 68 + 4 * (row - 64 * 2)
