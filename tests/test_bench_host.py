"""bench.py's host-side logic, without a GPU: the algorithmic byte counts
that its roofline divides by a kernel's time, the committed-counter lookup,
and the refusal of more than one GPU."""
import json
import os
import subprocess
import sys

import bench
from synth import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# TinyLLaMA-1.1B geometry (hidden 2048, 22 layers, 32 query heads, 4 KV heads
# of 64 dims, SwiGLU width 5632, vocab 32000), counted by hand.  Q4_0 stores
# 32 weights in 18 bytes.
_PER_LAYER_WEIGHTS = ((32 + 2 * 4) * 64 * 2048    # W_q | W_k | W_v
                      + 2048 * 2048               # W_o
                      + 2 * 5632 * 2048           # W_gate | W_up
                      + 2048 * 5632)              # W_down
_WEIGHT_BYTES = (22 * _PER_LAYER_WEIGHTS + 32000 * 2048) * 18 // 32
_KV_ROW_BYTES = 22 * 2 * 4 * 64 * 2               # K and V rows, fp16, all layers
_NORM_BYTES = (2 * 22 + 1) * 2048 * 4 + 2048 * 4  # gammas + the embedding row


def test_tinyllama_weight_bytes_by_hand():
    assert _PER_LAYER_WEIGHTS == 44_040_192
    assert _WEIGHT_BYTES == 581_861_376


def test_decode_bytes_per_token():
    # context 2048, 128 steps: step j attends 2048 + j + 1 rows, mean 2112.5
    assert W.DECODE["context"] == 2048 and W.DECODE["steps"] == 128
    assert W.DECODE["cap"] >= 2048 + 128
    want = _WEIGHT_BYTES + _KV_ROW_BYTES * 2112.5 + _NORM_BYTES
    assert bench.decode_bytes_per_token(W.DECODE) == want == 629_828_608


def test_long_context_decode_bytes_per_token():
    # the 8192-row ring is full from the first step: every step reads all of it
    assert W.DECODE_LONG["context"] == W.DECODE_LONG["cap"] == 8192
    want = _WEIGHT_BYTES + _KV_ROW_BYTES * 8192 + _NORM_BYTES
    assert bench.decode_bytes_per_token(W.DECODE_LONG) == want == 766_787_584


def test_stored_traffic_requires_matching_source_hash():
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        t = json.load(f)
    for kernel, rec in t.items():
        assert bench.stored_traffic(kernel, rec["source_hash"]) == rec["bytes_per_launch"]
        assert bench.stored_traffic(kernel, "0" * 16) is None
        # counters scaled by the copy-kernel calibration give the stored bytes
        scaled = (rec["fetch_kib_per_launch"] * rec["fetch_scale"]
                  + rec["write_kib_per_launch"] * rec["write_scale"]) * 1024
        assert abs(scaled - rec["bytes_per_launch"]) < 1e-3 * rec["bytes_per_launch"]
    assert bench.stored_traffic("no such kernel", "0" * 16) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stdout
