"""GPU parity of every plan (kernel variant and tile profile) the library
accepts: each candidate plan of the sweep behind the per-shape table gives the
oracle's routing exactly and its output within the layer tolerance
(tests/parity.py), at token counts on both sides of each threshold."""

from __future__ import annotations

import os
import sys

import numpy as np
import pytest

import oracle
from tests.parity import assert_fp16_close
from w4a16_group_quantized_amd import inputs as synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402  (the candidate plans of the sweep)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from w4a16_group_quantized_amd import ops

    ops.load_library()
    return torch.device("cuda:0")


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu-test] {request.node.nodeid}", flush=True)
    yield


@pytest.mark.parametrize("E,k,H,I,T", [
    (64, 6, 512, 160, 1), (64, 6, 512, 640, 8), (64, 6, 512, 640, 9), (64, 6, 512, 160, 64),
    (64, 6, 512, 640, 64), (64, 6, 512, 640, 100),
    (512, 10, 2560, 640, 8),   # model geometry: 2 lanes per w13 row copy scales synchronously
])
def test_every_plan_matches_oracle(dev, E, k, H, I, T):
    from w4a16_group_quantized_amd import ops

    shape = synth.MoEShape(E=E, top_k=k, H=H, I=I, T=T)
    host = synth.make_inputs(shape, 13)
    ref = oracle.layer(host, k)
    w = ops.weights_to_device(host, dev)
    logits = torch.from_numpy(host["logits"]).to(dev)
    x = torch.from_numpy(host["x"]).to(dev)
    ws = torch.empty(ops.layer_workspace_bytes(T, k, E, H, I), dtype=torch.uint8, device=dev)
    base, plans = bench.candidate_plans(T, E, k, H, I)
    assert base in plans
    for d in plans:
        plan = bench._plan(d)
        print(f"  plan {d}", flush=True)
        ws.fill_(255)
        out = torch.full((T, H), float("nan"), dtype=torch.float16, device=dev)
        ops.moe_layer_forward_plan(logits, x, k, w, plan, ws, out)
        torch.cuda.synchronize()
        views = ops.layer_workspace_views(ws, T, k, E, H, I)
        assert np.array_equal(views["topk_ids"].cpu().numpy(), ref["topk_ids"]), d
        assert np.array_equal(views["sorted_slots"].cpu().numpy(), ref["sorted_slots"]), d
        assert_fp16_close(out.cpu().numpy(), ref["out"], f"{shape} {d}")


def test_router_projection_on_matrix_cores_at_decode_sizes(dev):
    """The block with the projection's matrix-core variant forced at 8 tokens."""
    from w4a16_group_quantized_amd import ops

    shape = synth.MoEShape(E=512, top_k=10, H=2560, I=160, T=8)
    host = synth.make_block_inputs(shape, 14, shared=True)
    w = ops.weights_to_device(host, dev)
    x = torch.from_numpy(host["x"]).to(dev)
    gw = torch.from_numpy(host["gate_w"]).to(dev)
    base = ops.plan_default(8, 10, 512, 2560, 160, shared=True)
    assert base.router_gemv == 1
    logits = {}
    for gemv in (1, 0):
        plan = bench._plan(dict(base.as_dict(), router_gemv=gemv))
        ws = torch.empty(ops.block_workspace_bytes(8, 10, 512, True, 2560, 160), dtype=torch.uint8,
                         device=dev)
        lg = torch.full((8, 512), float("nan"), dtype=torch.float32, device=dev)
        out = torch.empty((8, 2560), dtype=torch.float16, device=dev)
        ops.moe_block_forward_plan(x, gw, 10, w, True, plan, ws, lg, out)
        torch.cuda.synchronize()
        logits[gemv] = lg.cpu().numpy().astype(np.float64)
    exact = oracle.router_logits(host["x"], host["gate_w"])
    mag = np.abs(host["x"].astype(np.float64)) @ np.abs(host["gate_w"].astype(np.float64)).T
    bound = (2560 / 16 + 64) * 2.0 ** -24 * mag
    for gemv, lg in logits.items():
        assert (np.abs(lg - exact) <= bound).all(), gemv
