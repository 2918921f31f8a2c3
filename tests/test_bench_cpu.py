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
    act = 80 * 640 * 2 * 2  # act as an fp16 hi/lo pair per sorted row
    assert work["layer_bytes"] == 73 * 2_841_600 + io
    assert work["gate_up_bytes"] == 73 * 1_894_400 + 8 * 2560 * 2 + act
    assert work["routed_gate_up_bytes"] == work["gate_up_bytes"] + 8 * 512 * 4
    assert work["down_bytes"] == 73 * 947_200 + act + 80 * 2560 * 4
    assert work["flops"] == 6 * 8 * 10 * 2560 * 640
    assert work["gate_up_flops"] == 4 * 8 * 10 * 2560 * 640


def test_routed_decode_follows_the_library_plan():
    """The one-call layer routes inside its first kernel where the plan table says so
    (GEMV sizes, T <= 32, E <= 1024)."""
    base = synth.WORKLOADS["decode_e512_k10_h2560_i640_t8"]
    assert bench.routed_decode(base) and bench.gemv_ffn(base)
    assert bench.routed_decode(synth.MoEShape(E=512, top_k=10, H=2560, I=640, T=32))
    assert not bench.routed_decode(synth.MoEShape(E=512, top_k=10, H=2560, I=640, T=33))
    assert not bench.gemv_ffn(synth.MoEShape(E=512, top_k=10, H=2560, I=640, T=33))
    assert not bench.routed_decode(synth.MoEShape(E=1025, top_k=10, H=2560, I=640, T=8))
    assert bench.routed_decode(synth.MoEShape(E=1024, top_k=10, H=2560, I=640, T=1))


def test_counter_lines_hold_only_for_their_sources(tmp_path, monkeypatch):
    """A traffic or MfmaUtil line is used only while the kernel sources hash as recorded."""
    import shutil

    for rel in bench.kernel_sources(True):
        dst = tmp_path / rel
        dst.parent.mkdir(parents=True, exist_ok=True)
        shutil.copy(os.path.join(ROOT, rel), dst)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    sha = bench.source_sha256(bench.kernel_sources(True))
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "counters_w.md").write_text(
        "text\n"
        f"traffic down fetch_kib=100 write_kib=10 fetch_scale=2 write_scale=1 source_sha256={sha}\n"
        f"mfma gate_up util_pct=31.5 source_sha256={sha}\n")
    assert bench.counter_traffic("w", "down", True) == (100 * 2 + 10) * 1024
    assert bench.mfma_util("w", "gate_up", True) == 31.5
    assert bench.counter_traffic("w", "gate_up", True) is None
    (tmp_path / bench.kernel_sources(True)[0]).write_text("// changed\n")
    assert bench.counter_traffic("w", "down", True) is None


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr or "single" in res.stderr


def test_option_defaults_and_block_only():
    """No flags: one GPU, the decode workload, the block and prefill objects
    on; --block-only is accepted and leaves the rest at its defaults."""
    a = bench.parse_args([])
    assert a.gpus == 1 and a.workload == bench.DEFAULT_WORKLOAD
    assert not a.block_only and not a.no_block and not a.no_prefill
    b = bench.parse_args(["--block-only", "--steps", "8"])
    assert b.block_only and b.steps == 8 and b.workload == bench.DEFAULT_WORKLOAD
