"""bench.py on the CPU: the byte and flop accounting behind the roofline
figures, and the refusal of more than one GPU."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from w4a16_group_quantized_amd import inputs as synth  # noqa: E402


def test_expert_bytes_are_4625_bits_per_weight():
    # int4 codes (0.5 B/weight) + an fp16 scale and a packed 4-bit zero per 32
    # weights: 4.625 bits per weight.
    w13, w2 = bench.expert_bytes(2560, 640)
    assert (w13, w2) == (1_894_400, 947_200)
    assert (w13 + w2) * 8 == 4.625 * 3 * 2560 * 640
    w13, w2 = bench.expert_bytes(2560, 160)
    assert w13 + w2 == 710_400


def test_layer_work_of_the_decode_workload():
    shape = synth.WORKLOADS["decode_e512_k10_h2560_i640_t8"]
    work = bench.layer_work(shape, 73)
    io = 8 * 2560 * 2 + 8 * 512 * 4 + 8 * 2560 * 2
    assert work["layer_bytes"] == 73 * 2_841_600 + io
    assert work["gate_up_bytes"] == 73 * 1_894_400 + 8 * 2560 * 2
    assert work["flops"] == 6 * 8 * 10 * 2560 * 640
    assert work["gate_up_flops"] == 4 * 8 * 10 * 2560 * 640


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr or "single" in res.stderr
