"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Bit-exact: top-k ids, expert offsets, sorted slots, slot rows, active experts
and their count.  Floating point: fp16 layer output within max |err| <= 2e-2
and relative RMS <= 1e-2 of the unrounded oracle (tests/parity.py), the fp32
router weights within 1e-6, and every row of the fp32 per-row expert outputs
y_sorted element by element (tests/parity.py states the bound).

Every output buffer is filled with NaN (and every workspace with 0xFF bytes)
before a call, so a row, tile or item the kernels never write fails the check
instead of passing on stale memory.  Each layer is run both as the four
separate calls and as the one-call moe_layer_forward, which must agree bit for
bit.

Sizes: every named workload at its full size (the two prefill workloads
against the fp32 oracle, every token and every y_sorted row), token counts
0/1/2/8/9/63/64/65/127/128, the 128-row M-tile path (S >= 64 E) with last
tiles of 1 to 4 live 32-row subtiles, and the degenerate cases (one expert,
k = E, E not a multiple of 64, every token on one expert, tied logits, the
largest E and k).
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from tests.parity import assert_fp16_close, assert_y_close
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


def _poison(layer):
    """NaN in every output, 0xFF bytes in every workspace (sentinels)."""
    nan = float("nan")
    layer.y_sorted.fill_(nan)
    layer.out.fill_(nan)
    layer.fused_out.fill_(nan)
    layer.weights.fill_(nan)
    layer.ids.fill_(-7)
    for v in layer.perm.values():
        v.fill_(-7)
    for ws in (layer.perm_ws, layer.ffn_ws, layer.layer_ws):
        ws.fill_(255)


def _run_layer(host, shape, dev):
    """The layer as the four calls and as moe_layer_forward (bit-equal), on
    poisoned buffers; returns the four calls' outputs as numpy arrays."""
    from w4a16_group_quantized_amd import ops

    w = ops.weights_to_device(host, dev)
    logits = torch.from_numpy(host["logits"]).to(dev)
    x = torch.from_numpy(host["x"]).to(dev)
    layer = ops.MoELayer(shape.T, shape.E, shape.top_k, shape.H, shape.I, dev)
    _poison(layer)
    torch.cuda.synchronize()
    out = layer(logits, x, w)
    fused = layer.forward(logits, x, w)
    torch.cuda.synchronize()
    res = {
        "topk_ids": layer.ids.cpu().numpy(),
        "topk_weights": layer.weights.cpu().numpy(),
        "y_sorted": layer.y_sorted.cpu().numpy(),
        "out": out.cpu().numpy(),
    }
    for k, v in layer.perm.items():
        res[k] = v.cpu().numpy()
    res["num_active"] = int(res["num_active"][0])
    if shape.T > 0:
        assert torch.equal(fused.view(torch.int16), out.view(torch.int16)), \
            "moe_layer_forward differs from the four calls"
        views = layer.forward_views()
        assert torch.equal(views["y_sorted"].view(torch.int32), layer.y_sorted.view(torch.int32))
        assert torch.equal(views["topk_ids"], layer.ids)
    return res


def _assert_routing_exact(got, ref):
    assert np.array_equal(got["topk_ids"], ref["topk_ids"]), "topk_ids"
    np.testing.assert_allclose(got["topk_weights"], ref["topk_weights"], rtol=0, atol=1e-6)
    for key in ("expert_offsets", "sorted_slots", "slot_rows", "active_experts"):
        assert np.array_equal(got[key], ref[key]), key
    assert got["num_active"] == int(ref["num_active"]), "num_active"


def _full_check(shape, seed, dev, host=None, dtype=np.float64):
    host = host if host is not None else synth.make_inputs(shape, seed)
    ref = oracle.layer(host, shape.top_k, dtype=dtype)
    got = _run_layer(host, shape, dev)
    if shape.T == 0:  # nothing is computed or written; outputs are empty
        assert got["topk_ids"].shape == (0, shape.top_k) and got["out"].shape == (0, shape.H)
        return got, ref
    _assert_routing_exact(got, ref)
    assert_y_close(got["y_sorted"], ref["y_sorted"], f"{shape} seed {seed}")
    assert_fp16_close(got["out"], ref["out"], f"{shape} seed {seed}")
    return got, ref


# --------------------------------------------------------------------------- #
# the named workloads
# --------------------------------------------------------------------------- #
def test_tiny_workload(dev):
    _full_check(synth.WORKLOADS["tiny_e8_k2_h256_i128_t4"], 0, dev)


def test_decode_workload_full(dev):
    _full_check(synth.WORKLOADS["decode_e512_k10_h2560_i640_t8"], 0, dev)


@pytest.mark.parametrize("T", [1, 2, 4, 8])
def test_decode_shard_token_sweep(dev, T):
    base = synth.WORKLOADS["decode_shard_e512_k10_h2560_i160_t8"]
    _full_check(synth.MoEShape(base.E, base.top_k, base.H, base.I, T), 0, dev)


def test_prefill_workload_full(dev):
    """1024 tokens: every token and every y_sorted row against the fp32 oracle."""
    _full_check(synth.WORKLOADS["prefill_e512_k10_h2560_i640_t1024"], 0, dev, dtype=np.float32)


def test_prefill_zipf_workload_full(dev):
    """4096 tokens with Zipf-skewed routing (the 128-row M-tile path): every
    token and every y_sorted row against the fp32 oracle."""
    shape = synth.WORKLOADS["prefill_zipf_e512_k10_h2560_i640_t4096"]
    got, _ = _full_check(shape, 0, dev, dtype=np.float32)
    # the skew is real: the hottest expert holds hundreds of rows
    counts = np.diff(got["expert_offsets"])
    assert counts.max() > 1000 and (counts == 0).sum() > 100


def test_layer_forward_decode_workload_against_oracle(dev):
    """The timed decode step (moe_layer_forward, 8 tokens, model geometry,
    seed 0) against the oracle directly, with its routing and y_sorted."""
    from w4a16_group_quantized_amd import ops

    shape = synth.WORKLOADS["decode_e512_k10_h2560_i640_t8"]
    host = synth.make_inputs(shape, 0)
    ref = oracle.layer(host, shape.top_k)
    w = ops.weights_to_device(host, dev)
    layer = ops.MoELayer(shape.T, shape.E, shape.top_k, shape.H, shape.I, dev)
    _poison(layer)
    out = layer.forward(torch.from_numpy(host["logits"]).to(dev),
                        torch.from_numpy(host["x"]).to(dev), w)
    torch.cuda.synchronize()
    v = layer.forward_views()
    got = {k: t.cpu().numpy() for k, t in v.items()}
    got["num_active"] = int(got["num_active"][0])
    _assert_routing_exact(got, ref)
    assert_y_close(got["y_sorted"], ref["y_sorted"], "moe_layer_forward decode")
    assert_fp16_close(out.cpu().numpy(), ref["out"], "moe_layer_forward decode")


def _last_tile_subtiles(counts):
    return {int(((c - 1) % 128) // 32 + 1) for c in counts if c > 0}


@pytest.mark.parametrize("E,k,H,I,T", [
    (8, 2, 256, 128, 256),    # S = 64 E exactly
    (8, 2, 288, 96, 300),     # odd group counts (9 and 3): no wide scale/zero loads
    (4, 2, 256, 128, 200),
    (4, 2, 256, 128, 256),
    (4, 2, 288, 96, 333),
])
def test_m128_tile_path_full(dev, E, k, H, I, T):
    """S >= 64 E selects 128-row M-tiles; whole outputs against the oracle."""
    shape = synth.MoEShape(E=E, top_k=k, H=H, I=I, T=T)
    assert T * k >= 64 * E
    got, _ = _full_check(shape, 5, dev)
    print(f"  last-tile live subtiles {sorted(_last_tile_subtiles(np.diff(got['expert_offsets'])))}")


def test_m128_tile_cases_cover_every_tail():
    """The cases above end experts in last M-tiles of 1, 2, 3 and 4 live subtiles."""
    seen = set()
    for (E, k, H, I, T) in [(8, 2, 256, 128, 256), (8, 2, 288, 96, 300), (4, 2, 256, 128, 200),
                            (4, 2, 256, 128, 256), (4, 2, 288, 96, 333)]:
        h = synth.make_activations(synth.MoEShape(E=E, top_k=k, H=H, I=I, T=T), 5)
        ids, _ = oracle.route(h["logits"], k)
        seen |= _last_tile_subtiles(np.bincount(ids.ravel(), minlength=E))
    assert seen == {1, 2, 3, 4}


def test_skewed_small_prefill(dev):
    """A few experts take most rows (many 128-row tiles), many take none."""
    shape = synth.MoEShape(E=32, top_k=3, H=256, I=128, T=700, zipf_s=1.1)
    got, _ = _full_check(shape, 4, dev)
    counts = np.diff(got["expert_offsets"])
    assert counts.max() > 256 and counts.min() < 32


# --------------------------------------------------------------------------- #
# token counts and degenerate cases
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("T", [0, 1, 2, 8, 9, 63, 64, 65, 127, 128])
def test_token_counts(dev, T):
    _full_check(synth.MoEShape(E=64, top_k=6, H=512, I=256, T=T), T, dev)


@pytest.mark.parametrize("E,k,H,I,T", [
    (1, 1, 256, 128, 5),      # one expert, top-1: the dense FFN
    (8, 8, 256, 128, 3),      # k = E: every expert on every token
    (37, 5, 256, 96, 70),     # E not a multiple of 64, ragged I tile, > 64 tokens
    (100, 3, 96, 32, 17),     # small odd geometry
    (4096, 64, 64, 32, 3),    # largest E and top_k
    (4, 2, 8192, 64, 4),      # decode, long K of gate/up: 32 steps per row block
    (4, 2, 128, 4096, 3),     # decode, long K of down: 16 steps per row block
    (6, 3, 96, 96, 2),        # decode, odd group counts: one lane per row
    (4, 4, 128, 128, 2),      # k = E at 2 tokens: every expert holds both rows, S > E
                              # (the combine inside the down launch)
    (2, 1, 16384, 64, 2),     # largest H, decode GEMV
    (2, 1, 64, 16384, 2),     # largest I at decode size: the down GEMV's A rows do not
                              # fit in LDS, so the matrix-core kernels take it
    (2, 2, 16384, 64, 40),    # largest H, matrix cores
    (2, 2, 64, 16384, 40),    # largest I, matrix cores
])
def test_degenerate_shapes(dev, E, k, H, I, T):
    _full_check(synth.MoEShape(E=E, top_k=k, H=H, I=I, T=T), 5, dev)


def _random_shapes(n, seed, t_max):
    """Seeded shapes across the supported ranges, small enough for the oracle
    (E * 2I * H at most 2^24 weights)."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        E = int(rng.integers(1, 300))
        k = int(rng.integers(1, min(E, 16) + 1))
        H = 32 * int(rng.integers(1, 41))
        I = 32 * int(rng.integers(1, 41))
        T = int(rng.integers(1, t_max + 1))
        if E * 2 * I * H <= 1 << 24:
            out.append((E, k, H, I, T))
    return out


# up to 300 tokens (mostly the matrix-core kernels), then up to 32 (the GEMV)
@pytest.mark.parametrize("E,k,H,I,T", _random_shapes(16, 2024, 300) + _random_shapes(10, 7, 32))
def test_random_shapes(dev, E, k, H, I, T):
    """Seeded random sizes (any E, top-k, H and I multiples of 32, T up to
    300): every output against the oracle, on whatever plan the table picks."""
    _full_check(synth.MoEShape(E=E, top_k=k, H=H, I=I, T=T), 11, dev)


def test_every_token_on_one_expert(dev):
    shape = synth.MoEShape(E=32, top_k=4, H=256, I=128, T=200)
    host = synth.make_inputs(shape, 9)
    host["logits"][:, 7] += 100.0
    got, ref = _full_check(shape, 9, dev, host)
    assert np.all(got["topk_ids"][:, 0] == 7)
    assert np.diff(got["expert_offsets"])[7] == shape.T


def test_tied_logits(dev):
    shape = synth.MoEShape(E=48, top_k=5, H=128, I=64, T=70)
    host = synth.make_inputs(shape, 2)
    host["logits"] = np.round(host["logits"], 0).astype(np.float32)  # many exact ties
    host["logits"][3] = 0.5  # a fully tied row
    host["logits"][4, :] = -0.0
    host["logits"][4, ::2] = 0.0
    got, ref = _full_check(shape, 2, dev, host)
    assert got["topk_ids"][3].tolist() == [0, 1, 2, 3, 4]
    assert got["topk_ids"][4].tolist() == [0, 1, 2, 3, 4]


def test_repeat_calls_are_bitwise_identical(dev):
    shape = synth.MoEShape(E=64, top_k=6, H=512, I=256, T=300)
    host = synth.make_inputs(shape, 3)
    a = _run_layer(host, shape, dev)
    b = _run_layer(host, shape, dev)
    for key in ("out", "y_sorted", "topk_weights", "sorted_slots"):
        assert np.array_equal(a[key], b[key]), key


# --------------------------------------------------------------------------- #
# single entry points in isolation
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("T,E", [(1, 1), (63, 7), (64, 512), (65, 512), (1000, 4096), (5000, 512)])
def test_permute_alone_bit_exact(dev, T, E):
    from w4a16_group_quantized_amd import ops

    k = min(E, 10)
    rng = np.random.default_rng(T + E)
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    ref = oracle.permute(ids, E)
    got = ops.moe_permute(torch.from_numpy(ids).to(dev), E)
    torch.cuda.synchronize()
    for key in ("expert_offsets", "sorted_slots", "slot_rows", "active_experts"):
        assert np.array_equal(got[key].cpu().numpy(), ref[key]), key
    assert int(got["num_active"].item()) == int(ref["num_active"])


@pytest.mark.parametrize("T,E,k", [
    (1, 512, 10), (8, 512, 10), (64, 1024, 64), (64, 64, 1), (5, 37, 5),
    (65, 512, 10),   # more than 64 tokens: the two-call path
    (3, 2048, 8),    # more than 1024 experts: the two-call path
])
def test_route_permute_matches_separate_calls(dev, T, E, k):
    """moe_route_permute returns what moe_route then moe_permute return, bit for bit,
    and the oracle's routing and permutation (ties included: logits repeat)."""
    from w4a16_group_quantized_amd import ops

    rng = np.random.default_rng(T * 7 + E)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[:, E // 3:E // 3 + 4] = logits[:, :4]          # equal logits on other experts
    lg = torch.from_numpy(logits).to(dev)
    ids_f, w_f, perm_f = ops.moe_route_permute(lg, k)
    ids_s, w_s = ops.moe_route(lg, k)
    perm_s = ops.moe_permute(ids_s, E)
    torch.cuda.synchronize()
    assert torch.equal(ids_f, ids_s)
    assert torch.equal(w_f.view(torch.int32), w_s.view(torch.int32))
    for key in perm_s:
        assert torch.equal(perm_f[key], perm_s[key]), key
    ref_ids, ref_w = oracle.route(logits, k)
    ref_perm = oracle.permute(ref_ids, E)
    assert np.array_equal(ids_f.cpu().numpy(), ref_ids)
    np.testing.assert_allclose(w_f.cpu().numpy(), ref_w, rtol=0, atol=1e-6)
    for key in ("expert_offsets", "sorted_slots", "slot_rows", "active_experts"):
        assert np.array_equal(perm_f[key].cpu().numpy(), ref_perm[key]), key
    assert int(perm_f["num_active"].item()) == int(ref_perm["num_active"])


@pytest.mark.parametrize("E,k,H,I,T", [
    (512, 10, 2560, 640, 8),    # the decode workload: routing inside the gate/up kernel
    (512, 10, 2560, 160, 1),
    (64, 6, 512, 256, 2),
    (2048, 8, 256, 128, 4),     # more than 1024 experts: routing as its own launch
    (64, 6, 512, 256, 9),       # more than 8 tokens: the matrix-core path
])
def test_layer_forward_matches_the_four_calls(dev, E, k, H, I, T):
    """moe_layer_forward gives the four calls' out, routing and y_sorted, bit for bit."""
    from w4a16_group_quantized_amd import ops

    shape = synth.MoEShape(E=E, top_k=k, H=H, I=I, T=T)
    host = synth.make_inputs(shape, 3)
    w = ops.weights_to_device(host, dev)
    logits = torch.from_numpy(host["logits"]).to(dev)
    x = torch.from_numpy(host["x"]).to(dev)
    layer = ops.MoELayer(T, E, k, H, I, dev)
    ref = layer(logits, x, w).clone()
    got = layer.forward(logits, x, w)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    v = layer.forward_views()
    assert torch.equal(v["topk_ids"], layer.ids)
    assert torch.equal(v["topk_weights"].view(torch.int32), layer.weights.view(torch.int32))
    for key in ("expert_offsets", "sorted_slots", "slot_rows", "active_experts", "num_active"):
        assert torch.equal(v[key], layer.perm[key]), key
    assert torch.equal(v["y_sorted"].view(torch.int32), layer.y_sorted.view(torch.int32))


def test_layer_forward_against_oracle(dev):
    from w4a16_group_quantized_amd import ops

    shape = synth.MoEShape(E=64, top_k=6, H=512, I=256, T=8)
    host = synth.make_inputs(shape, 11)
    ids, wts = oracle.route(host["logits"], shape.top_k)
    w = ops.weights_to_device(host, dev)
    out = ops.moe_layer_forward(torch.from_numpy(host["logits"]).to(dev),
                                torch.from_numpy(host["x"]).to(dev), shape.top_k, w)
    torch.cuda.synchronize()
    sub = oracle.token_outputs(host, ids, wts, np.arange(shape.T))
    assert_fp16_close(out.cpu().numpy(), sub, f"{shape} moe_layer_forward")


@pytest.mark.parametrize("E,k,H,I,T", [
    (8, 2, 256, 128, 4), (512, 10, 2560, 640, 8), (512, 10, 2560, 160, 1), (1024, 8, 512, 256, 8),
])
def test_route_gate_up_steps_match_layer_forward(dev, E, k, H, I, T):
    """moe_route_gate_up, moe_w4a16_down and moe_combine give moe_layer_forward's
    output bit for bit, and the routing of moe_route_permute."""
    from w4a16_group_quantized_amd import ops

    shape = synth.MoEShape(E=E, top_k=k, H=H, I=I, T=T)
    host = synth.make_inputs(shape, 12)
    w = ops.weights_to_device(host, dev)
    logits = torch.from_numpy(host["logits"]).to(dev)
    x = torch.from_numpy(host["x"]).to(dev)
    layer = ops.MoELayer(T, E, k, H, I, dev)
    _poison(layer)
    ops.moe_route_gate_up(logits, x, k, w, layer.ids, layer.weights, layer.perm, layer.ffn_ws)
    ops.moe_w4a16_down(T, k, layer.perm, w, layer.y_sorted, layer.ffn_ws)
    out = ops.moe_combine(layer.y_sorted, layer.weights, layer.perm["slot_rows"], layer.out)
    fused = layer.forward(logits, x, w)
    ids, wts, perm = ops.moe_route_permute(logits, k)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), fused.view(torch.int16))
    assert torch.equal(ids, layer.ids) and torch.equal(wts.view(torch.int32), layer.weights.view(torch.int32))
    for key, v in perm.items():
        assert torch.equal(v, layer.perm[key]), key
    ref = oracle.layer(host, k)
    assert_fp16_close(out.cpu().numpy(), ref["out"], f"{shape}")


def test_combine_alone(dev):
    from w4a16_group_quantized_amd import ops

    T, k, H = 33, 7, 320
    rng = np.random.default_rng(8)
    y = rng.standard_normal((T * k, H)).astype(np.float32) * 20
    w = rng.random((T, k)).astype(np.float32)
    w /= w.sum(axis=1, keepdims=True)
    slot_rows = rng.permutation(T * k).astype(np.int32)
    ref = oracle.combine(y.astype(np.float64), w.astype(np.float64), slot_rows)
    got = ops.moe_combine(torch.from_numpy(y).to(dev), torch.from_numpy(w).to(dev),
                          torch.from_numpy(slot_rows).to(dev))
    torch.cuda.synchronize()
    assert_fp16_close(got.cpu().numpy(), ref, "combine")


def test_gate_up_then_down_equals_grouped_ffn(dev):
    from w4a16_group_quantized_amd import ops

    shape = synth.MoEShape(E=64, top_k=6, H=512, I=256, T=8)
    host = synth.make_inputs(shape, 11)
    w = ops.weights_to_device(host, dev)
    logits = torch.from_numpy(host["logits"]).to(dev)
    x = torch.from_numpy(host["x"]).to(dev)
    ids, wts = ops.moe_route(logits, shape.top_k)
    perm = ops.moe_permute(ids, shape.E)
    y_a = ops.moe_w4a16_grouped_ffn(x, shape.top_k, perm, w)
    ws = torch.empty(ops.ffn_workspace_bytes(shape.T, shape.top_k, shape.E, shape.H, shape.I),
                     dtype=torch.uint8, device=dev)
    y_b = torch.empty_like(y_a)
    ops.moe_w4a16_gate_up(x, shape.top_k, perm, w, ws)
    ops.moe_w4a16_down(shape.T, shape.top_k, perm, w, y_b, ws)
    torch.cuda.synchronize()
    assert torch.equal(y_a, y_b)


@pytest.mark.parametrize("T", [1, 8])   # 1: the combine inside the down launch
def test_graph_replay_of_layer_forward(dev, T):
    """moe_layer_forward captured in a HIP graph replays to its eager result,
    with eager work between replays."""
    from w4a16_group_quantized_amd import ops

    shape = synth.MoEShape(E=64, top_k=6, H=512, I=256, T=T)
    host = synth.make_inputs(shape, 22)
    w = ops.weights_to_device(host, dev)
    logits = torch.from_numpy(host["logits"]).to(dev)
    x = torch.from_numpy(host["x"]).to(dev)
    layer = ops.MoELayer(shape.T, shape.E, shape.top_k, shape.H, shape.I, dev)
    eager = layer.forward(logits, x, w).clone()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            got = layer.forward(logits, x, w)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(4):
        got.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(got, eager), f"replay {rep}"
        _ = (got.float() * 2).sum().item()  # eager work between replays


@pytest.mark.parametrize("T", [8, 300])
def test_graph_replay_matches_eager(dev, T):
    """A captured layer call replays to the eager result, with eager work between replays."""
    from w4a16_group_quantized_amd import ops

    shape = synth.MoEShape(E=64, top_k=6, H=512, I=256, T=T)
    host = synth.make_inputs(shape, 21)
    w = ops.weights_to_device(host, dev)
    logits = torch.from_numpy(host["logits"]).to(dev)
    x = torch.from_numpy(host["x"]).to(dev)
    layer = ops.MoELayer(shape.T, shape.E, shape.top_k, shape.H, shape.I, dev)
    eager = layer(logits, x, w).clone()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            layer(logits, x, w)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(4):
        layer.out.fill_(7.0)
        layer.y_sorted.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(layer.out, eager), f"replay {rep}"
        _ = (layer.out.float() * 2).sum().item()  # eager work between replays
