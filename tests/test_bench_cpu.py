"""The benchmark's arithmetic on the CPU: the algorithmic bytes and flops it
divides by, against the per-unit figures derived by hand for the K3 shapes
(bf16, d_k = d_v = 128), and its refusal of more than one GPU."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_prefill_bytes_per_token_head():
    # 2 (2 d_k + d_v) + 4 d_k + 4 + 2 d_v = 1540 B per (token, head), plus the
    # final state once per (sequence, head)
    b = bench.prefill_bytes(8192, 1, 96, 128, 128, 2, 2, False, True)
    assert b == 8192 * 96 * 1540 + 96 * 128 * 128 * 4 == 1217396736
    # an initial state adds one more state read
    assert bench.prefill_bytes(1, 1, 1, 128, 128, 2, 2, True, True) == 1540 + 2 * 65536


def test_prefill_flops_per_token_head():
    # C (2 d_k + 2 d_v) + 6 d_k d_v at C = 64: 131,072
    assert bench.prefill_flops(1, 1, 128, 128, 64) == 64 * 512 + 6 * 128 * 128 == 131072
    assert bench.prefill_flops(8192, 96, 128, 128, 64) == 103079215104


def test_decode_bytes_per_request_head():
    # 8 d_k d_v + 2 (2 d_k + d_v) + 4 d_k + 4 + 2 d_v = 132,612 B
    assert bench.decode_bytes(1, 1, 128, 128, 2, 2) == 132612
    assert bench.decode_bytes(256, 96, 128, 128, 2, 2) == 3259072512


def test_fused_prefill_bytes():
    # raw q, k and bf16 decay logits: 2 (3 d_k + d_v) + 4 + 2 d_v = 1284 B per
    # (token, head), plus the gate parameters and the final state
    b = bench.fused_prefill_bytes(8192, 1, 96, 128, 128, 2, False, True)
    assert b == 8192 * 96 * 1284 + 96 * (4 + 4 * 128) + 96 * 128 * 128 * 4


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]
