"""moe_layer_forward_noalloc (the layer with the library's per-device scratch
instead of a workspace) against moe_layer_forward with a caller workspace:
two calls in a row, the second with a smaller input, at the decode workload
and at a matrix-core (prefill) size; the results must be equal bit for bit
(which meets the layer tolerance) and a size beyond the scratch is refused."""

from __future__ import annotations

import numpy as np
import pytest

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


def _pair(shape, seed, dev, T2):
    from w4a16_group_quantized_amd import ops

    host = synth.make_inputs(shape, seed)
    w = ops.weights_to_device(host, dev)
    for T in (shape.T, T2):   # the second call is smaller and reuses the scratch
        print(f"[no-alloc] {shape} T={T}", flush=True)
        logits = torch.from_numpy(np.ascontiguousarray(host["logits"][:T])).to(dev)
        x = torch.from_numpy(np.ascontiguousarray(host["x"][:T])).to(dev)
        ref = ops.moe_layer_forward(logits, x, shape.top_k, w)
        out = torch.full((T, shape.H), float("nan"), dtype=torch.float16, device=dev)
        got = ops.moe_layer_forward_noalloc(logits, x, shape.top_k, w, out)
        torch.cuda.synchronize()
        assert got.data_ptr() == out.data_ptr()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"T={T}"
        assert_fp16_close(got.cpu().numpy(), ref.float().cpu().numpy(), f"no-alloc T={T}")


def test_noalloc_decode_then_smaller(dev):
    _pair(synth.WORKLOADS["decode_e512_k10_h2560_i640_t8"], 0, dev, 3)   # 3 tokens: 16 lanes per w13 row


def test_noalloc_two_tokens_then_one(dev):
    # up to 2 tokens the combine runs inside the down launch
    _pair(synth.MoEShape(E=512, top_k=10, H=2560, I=160, T=2), 4, dev, 1)


def test_noalloc_prefill_then_smaller(dev):
    _pair(synth.MoEShape(E=64, top_k=6, H=512, I=256, T=200), 3, dev, 90)


def test_noalloc_refuses_sizes_beyond_the_scratch(dev):
    from w4a16_group_quantized_amd import ops

    shape = synth.WORKLOADS["decode_e512_k10_h2560_i640_t8"]
    T = 1024
    assert ops.layer_workspace_bytes(T, shape.top_k, shape.E, shape.H, shape.I) > ops.NOALLOC_SCRATCH_BYTES
    lib = ops.load_library()
    fake = 0x1000   # never dereferenced: the size check fails first
    st = lib.moe_layer_forward_noalloc(fake, fake, T, shape.E, shape.top_k, fake, fake, fake, fake,
                                       fake, fake, shape.H, shape.I, 32, fake, None)
    assert st == ops.MOE_ERR_WORKSPACE
