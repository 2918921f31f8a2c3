"""GPU parity of the one-launch FFN plan (moe_plan.one_launch): gate/up and
down in one persistent launch give the oracle's routing and output, the same
bits as the two separate GEMV launches of the same plan, call after call (its
completion counts return to zero), and under HIP-graph replay."""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from tests.parity import assert_fp16_close
from w4a16_group_quantized_amd import inputs as synth

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


def _plans(T, E, k, H, I, rows):
    from w4a16_group_quantized_amd import ops

    d = ops.plan_default(T, k, E, H, I).as_dict()
    d.update(ffn=ops.FFN_GEMV, route=ops.ROUTE_IN_GATE_UP, cost_split=0, combine_in_down=0,
             rows_per_pass=rows, one_launch=0)
    two = ops.Plan()
    one = ops.Plan()
    for key, v in d.items():
        setattr(two, key, v)
        setattr(one, key, v)
    one.one_launch = 1
    return two, one


@pytest.mark.parametrize("E,k,H,I,T,rows", [
    (512, 10, 2560, 640, 8, 2),   # the model geometry at 8 tokens
    (512, 10, 2560, 160, 1, 1),
    (512, 10, 2560, 160, 2, 2),
    (64, 6, 512, 640, 33, 4),     # experts of several rows: more passes, 4 rows per pass
    (64, 6, 512, 256, 64, 1),     # one row per pass, up to 64 tokens
    (1000, 8, 256, 64, 64, 2),    # more than 512 experts: 16 logits per lane
    (37, 3, 96, 96, 9, 2),        # odd group counts, 3 groups per row
])
def test_one_launch_matches_two_launches_and_oracle(dev, E, k, H, I, T, rows):
    from w4a16_group_quantized_amd import ops

    shape = synth.MoEShape(E=E, top_k=k, H=H, I=I, T=T)
    host = synth.make_inputs(shape, 31)
    ref = oracle.layer(host, k)
    w = ops.weights_to_device(host, dev)
    logits = torch.from_numpy(host["logits"]).to(dev)
    x = torch.from_numpy(host["x"]).to(dev)
    ws = torch.empty(ops.layer_workspace_bytes(T, k, E, H, I), dtype=torch.uint8, device=dev)
    two, one = _plans(T, E, k, H, I, rows)

    def run(plan):
        ws.fill_(255)
        out = torch.full((T, H), float("nan"), dtype=torch.float16, device=dev)
        ops.moe_layer_forward_plan(logits, x, k, w, plan, ws, out)
        torch.cuda.synchronize()
        y = ops.layer_workspace_views(ws, T, k, E, H, I)["y_sorted"].clone()
        return out, y

    out2, y2 = run(two)
    for rep in range(3):  # the completion counts start from zero on every call
        print(f"  one launch, call {rep}", flush=True)
        out1, y1 = run(one)
        assert torch.equal(y1.view(torch.int32), y2.view(torch.int32)), f"y_sorted, call {rep}"
        assert torch.equal(out1.view(torch.int16), out2.view(torch.int16)), f"out, call {rep}"
    views = ops.layer_workspace_views(ws, T, k, E, H, I)
    assert np.array_equal(views["topk_ids"].cpu().numpy(), ref["topk_ids"])
    assert np.array_equal(views["sorted_slots"].cpu().numpy(), ref["sorted_slots"])
    assert np.array_equal(views["expert_offsets"].cpu().numpy(), ref["expert_offsets"])
    assert_fp16_close(out1.cpu().numpy(), ref["out"], f"{shape} one launch")


def test_one_launch_graph_replay(dev):
    """The one-launch layer captured in a HIP graph replays to its eager
    result, with eager work between replays."""
    from w4a16_group_quantized_amd import ops

    E, k, H, I, T = 512, 10, 2560, 640, 8
    shape = synth.MoEShape(E=E, top_k=k, H=H, I=I, T=T)
    host = synth.make_inputs(shape, 32)
    w = ops.weights_to_device(host, dev)
    logits = torch.from_numpy(host["logits"]).to(dev)
    x = torch.from_numpy(host["x"]).to(dev)
    ws = torch.empty(ops.layer_workspace_bytes(T, k, E, H, I), dtype=torch.uint8, device=dev)
    _, one = _plans(T, E, k, H, I, 2)
    out = torch.empty((T, H), dtype=torch.float16, device=dev)
    ops.moe_layer_forward_plan(logits, x, k, w, one, ws, out)
    eager = out.clone()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            ops.moe_layer_forward_plan(logits, x, k, w, one, ws, out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(4):
        out.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep}"
        _ = (out.float() * 2).sum().item()  # eager work between replays
    assert not torch.isnan(eager).any()
