"""The benchmark's contract, checked on the CPU: the multi-GPU refusal, the
algorithmic work tables behind the roofline fractions, and the committed
traffic summary's parser (no GPU, no timing)."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert p.returncode != 0
    assert "one GPU" in (p.stdout + p.stderr)


def test_step_work_table():
    ops = bench.op_table()
    # NVFP4 = 0.5625 B per element; a bf16 input is read once (2 B)
    assert ops["attn_quantize"]["bytes"] == 4096 * 3072 * 2.5625 + 4
    assert ops["ffn_gemm1"]["flops"] == 2 * 8192 * 14336 * 3072
    assert ops["ffn_gemm2"]["flops"] == 2 * 8192 * 3072 * 14336
    # KV read: 30 layers x 68 pages x 884,736 B compressed + bf16 K^ and V^ written
    assert ops["kv_read"]["compressed_bytes"] == 30 * 68 * 884736
    assert ops["kv_read"]["bytes"] == 30 * (68 * 884736 + 2 * 68 * 256 * 24 * 128 * 2)
    # the step's roofline time: GEMMs on the fp16 MFMA peak, the rest on HBM
    roof = sum(bench.roofline_seconds(o) for o in ops.values())
    assert 1.6e-3 < roof < 1.8e-3


def test_next_rows_work_table():
    nxt = bench.next_op_table()
    assert nxt["kv_attention"]["flops"] == 4 * 880 * 68 * 256 * 128 * 24
    assert nxt["wgrad_gemm"]["flops"] == 2 * 14336 * 3072 * 8192
    assert nxt["window_pages"].get("launch_bound")
    for rec in nxt.values():
        assert rec["workload"]


def test_traffic_summary_matches_the_gemm_source():
    # the committed counter summary names the GEMM source it was taken with;
    # bench.py reports it only while that source is unchanged
    t = bench.measured_traffic()
    assert t is None or 2e8 < t < 2e9
