"""GPU parity of the MoE block: the router gate projection, the routed layer
and the shared expert, through the C ABI, against the CPU oracle.

Logits.  The GPU forms each logit from exact fp16 x fp16 products summed in
fp32: the GEMV variant with one rounding per v_dot2 (two products) along a
lane and six in the cross-lane tree, the matrix-core variant with at least
one rounding per 16-product MFMA step.  Neither path rounds more than
H/16 + 64 times along any summation path, so

    |logit_gpu - logit_exact| <= (H/16 + 64) * 2^-24 * sum_h |x_h * w_h|

(the standard bound for recursive summation, with the unit roundoff 2^-24).
At H = 2560 that is 1.3e-5 of sum |x w|; a dropped or doubled term is about
1/H = 3.9e-4 of it, 30 times larger.

Routing decisions.  The router ranks fp32 logits, and the GPU's and the
oracle's fp32 logits may differ within the bound above.  A token whose k-th
and (k+1)-th largest oracle logits are closer than twice its bound may
legitimately pick either expert: its ids are checked for validity (every
choice within the bound of the k-th logit, every clearly larger logit chosen)
and its output is not compared; every other token's ids are compared exactly
and its output element by element (tests/parity.py tolerance).  Such tokens
must stay rare (5 % at most).
"""

from __future__ import annotations

import dataclasses

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


def _logit_bound(x, gate_w):
    H = x.shape[1]
    mag = np.abs(x.astype(np.float64)) @ np.abs(gate_w.astype(np.float64)).T
    return (H / 16 + 64) * 2.0 ** -24 * mag


def _assert_logits(got, exact, bound, label):
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - exact)
    assert np.isfinite(got).all(), f"{label}: non-finite logits"
    ratio = float((err / np.maximum(bound, 1e-300)).max()) if err.size else 0.0
    print(f"  {label}: logits max|err| {err.max() if err.size else 0:.3e}, "
          f"max err/bound {ratio:.3f}", flush=True)
    assert (err <= bound).all(), f"{label}: {int((err > bound).sum())} logits over the bound"


def _ambiguous_tokens(L32, bound, k):
    """Tokens whose k-th and (k+1)-th largest oracle fp32 logits are within
    twice the token's logit bound (either choice is a correct routing)."""
    T, E = L32.shape
    if k >= E:
        return np.zeros(T, dtype=bool)
    s = -np.sort(-L32.astype(np.float64), axis=1)
    gap = s[:, k - 1] - s[:, k]
    return gap <= 2 * bound.max(axis=1)


def _assert_valid_choice(ids, L32, bound, k):
    """The chosen k experts are a top-k of some logits within the bound."""
    L = L32.astype(np.float64)
    for t in range(L.shape[0]):
        kth = -np.sort(-L[t])[k - 1]
        tol = 2 * bound[t].max()
        chosen = set(int(e) for e in ids[t, :k])
        assert len(chosen) == k
        assert all(L[t, e] >= kth - tol for e in chosen), t
        must = set(np.nonzero(L[t] > kth + tol)[0].tolist())
        assert must <= chosen, t


def _shape(E, top_k, H, I, T):
    return synth.MoEShape(E=E, top_k=top_k, H=H, I=I, T=T)


# --------------------------------------------------------------------------- #
# the projection alone
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("T,E,H", [
    (1, 512, 2560), (2, 512, 2560), (8, 512, 2560), (16, 512, 2560),  # GEMV
    (17, 512, 2560), (1024, 512, 2560), (4096, 512, 2560),             # matrix cores
    (3, 96, 96), (40, 96, 96),        # 12 chunks per row (fewer than the lanes); a K tail of 32
    (100, 1, 32), (65, 200, 160),     # one expert; ragged expert and token tiles
    (2, 64, 16384), (5, 64, 16384),   # GEMV over 4 load windows; x too large for LDS -> MFMA
])
def test_router_gate_matches_oracle(dev, T, E, H):
    from w4a16_group_quantized_amd import ops

    shape = _shape(E, 1, H, 32, T)
    x = synth.make_activations(shape, 3)["x"]
    gw = synth.make_gate_weight(shape, 3)
    out = torch.full((T, E), float("nan"), dtype=torch.float32, device=dev)
    ops.moe_router_gate(torch.from_numpy(x).to(dev), torch.from_numpy(gw).to(dev), out)
    torch.cuda.synchronize()
    exact = oracle.router_logits(x, gw)
    _assert_logits(out.cpu().numpy(), exact, _logit_bound(x, gw), f"T={T} E={E} H={H}")


@pytest.mark.parametrize("T,H", [(16, 8192), (11, 4096)])   # x 256 KiB, 88 KiB
def test_router_gemv_beyond_the_default_x_size(dev, T, H):
    """The projection GEMV takes any H up to 16 tokens (x is read from global
    memory, not staged): forced by an explicit plan where the default picks
    the matrix cores (x over 80 KiB), against the oracle's logits."""
    from w4a16_group_quantized_amd import ops

    shape = _shape(64, 4, H, 64, T)
    host = synth.make_block_inputs(shape, 11, shared=True)
    base = ops.plan_default(T, 4, 64, H, 64, shared=True).as_dict()
    assert base["router_gemv"] == 0
    got, _ = _run_block(host, shape, dev, plan=dict(base, router_gemv=1))
    exact = oracle.router_logits(host["x"], host["gate_w"])
    _assert_logits(got["logits"], exact, _logit_bound(host["x"], host["gate_w"]), f"T={T} H={H} GEMV")


def test_router_gate_repeat_is_bitwise_identical(dev):
    from w4a16_group_quantized_amd import ops

    for T in (8, 300):
        shape = _shape(512, 1, 2560, 32, T)
        x = torch.from_numpy(synth.make_activations(shape, 4)["x"]).to(dev)
        gw = torch.from_numpy(synth.make_gate_weight(shape, 4)).to(dev)
        a = ops.moe_router_gate(x, gw).clone()
        b = ops.moe_router_gate(x, gw)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), T


# --------------------------------------------------------------------------- #
# routing with the shared slot
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("T,E,k", [(1, 8, 2), (8, 512, 10), (300, 512, 10), (70, 63, 63)])
def test_route_shared_matches_oracle(dev, T, E, k):
    from w4a16_group_quantized_amd import ops

    logits = synth.make_activations(_shape(E, k, 32, 32, T), 5)["logits"]
    ids, w = ops.moe_route_shared(torch.from_numpy(logits).to(dev), k)
    torch.cuda.synchronize()
    ids, w = ids.cpu().numpy(), w.cpu().numpy()
    ref_ids, ref_w = oracle.route(logits, k)
    assert np.array_equal(ids[:, :k], ref_ids)
    assert np.all(ids[:, k] == E) and np.all(w[:, k] == 1.0)
    np.testing.assert_allclose(w[:, :k], ref_w, rtol=0, atol=1e-6)


# --------------------------------------------------------------------------- #
# the whole block
# --------------------------------------------------------------------------- #
def _run_block(host, shape, dev, shared=True, plan=None):
    """The block on poisoned buffers, with the default plan or `plan` (a dict)."""
    from w4a16_group_quantized_amd import ops

    w = ops.weights_to_device(host, dev)
    x = torch.from_numpy(host["x"]).to(dev)
    gw = torch.from_numpy(host["gate_w"]).to(dev)
    blk = ops.MoEBlock(shape.T, shape.E, shape.top_k, shape.H, shape.I, shared, dev)
    blk.ws.fill_(255)
    blk.out.fill_(float("nan"))
    blk.logits.fill_(float("nan"))
    torch.cuda.synchronize()
    if plan is None:
        out = blk(x, gw, w)
    else:
        p = ops.Plan()
        for key, v in plan.items():
            setattr(p, key, v)
        out = ops.moe_block_forward_plan(x, gw, shape.top_k, w, shared, p, blk.ws, blk.logits,
                                         blk.out)
    torch.cuda.synchronize()
    v = blk.views()
    got = {"out": out.cpu().numpy(), "logits": blk.logits.cpu().numpy(),
           "topk_ids": v["topk_ids"].cpu().numpy(), "topk_weights": v["topk_weights"].cpu().numpy(),
           "expert_offsets": v["expert_offsets"].cpu().numpy(),
           "sorted_slots": v["sorted_slots"].cpu().numpy(), "y_sorted": v["y_sorted"].cpu().numpy()}
    return got, (x, gw, w, blk)


def _block_check(shape, seed, dev, dtype=np.float64):
    host = synth.make_block_inputs(shape, seed, shared=True)
    ref = oracle.block(host, shape.top_k, shared=True, dtype=dtype)
    got, _ = _run_block(host, shape, dev)
    label = f"{shape} seed {seed}"
    bound = _logit_bound(host["x"], host["gate_w"])
    _assert_logits(got["logits"], ref["logits_exact"], bound, label)
    k, E, T = shape.top_k, shape.E, shape.T
    amb = _ambiguous_tokens(ref["logits"], bound, k)
    print(f"  {label}: {int(amb.sum())} of {T} tokens with an ambiguous k-th choice", flush=True)
    assert amb.mean() <= 0.05
    clear = ~amb
    assert np.array_equal(got["topk_ids"][clear, :k], ref["topk_ids"][clear])
    # a logit error d moves a renormalised weight by at most about 2 d
    wtol = 1e-6 + 2 * bound.max(axis=1)[clear][:, None]
    assert (np.abs(got["topk_weights"][clear, :k] - ref["topk_weights"][clear]) <= wtol).all()
    if amb.any():
        _assert_valid_choice(got["topk_ids"][amb], ref["logits"][amb], bound[amb], k)
    # the shared slot, and the shared expert's segment: T rows, token order
    assert np.all(got["topk_ids"][:, k] == E) and np.all(got["topk_weights"][:, k] == 1.0)
    off = got["expert_offsets"]
    assert off[E + 1] - off[E] == T and off[E + 1] == T * (k + 1)
    assert np.array_equal(got["sorted_slots"][off[E]:off[E + 1]] // (k + 1), np.arange(T))
    assert_y_close(got["y_sorted"][off[E]:off[E + 1]], ref["y_shared"], f"{label} shared expert")
    assert_fp16_close(got["out"][clear], ref["out"][clear], label)
    return got, ref


@pytest.mark.parametrize("E,k,H,I,T", [
    (8, 2, 256, 128, 4),        # decode path, tiny
    (512, 10, 2560, 640, 1),    # decode path, one token
    (512, 10, 2560, 640, 8),    # decode path at the model geometry
    (512, 10, 2560, 160, 8),    # decode path at the per-rank shard
    (64, 6, 512, 256, 40),      # one-launch router + permutation, matrix-core FFN
    (64, 6, 512, 256, 300),     # router and permutation kernels, matrix-core FFN
    (63, 62, 256, 128, 9),      # top_k + 1 = 63 slots, E + 1 = 64 experts
    (64, 6, 512, 256, 20),      # shared expert on the matrix cores: a ragged 32-row tile
    (128, 4, 512, 160, 32),     # and a full one
    (8, 2, 288, 96, 5),         # odd group counts: K splits of 3, 3, 3, 0 and 2, 1 groups
    (512, 10, 2560, 640, 3),    # the fewest tokens with the shared expert on the matrix cores
    (512, 10, 2560, 640, 28),   # too many for its LDS: the matrix-core FFN takes the block
])
def test_block_matches_oracle(dev, E, k, H, I, T):
    _block_check(_shape(E, k, H, I, T), 7, dev)


def test_block_prefill_workload_full(dev):
    """1024 tokens at the model geometry with the shared expert, every token."""
    _block_check(_shape(512, 10, 2560, 640, 1024), 0, dev, dtype=np.float32)


@pytest.mark.parametrize("T", [2, 8, 40, 300])
def test_block_matches_its_steps(dev, T):
    """moe_block_forward equals moe_router_gate, moe_route_shared, moe_permute,
    moe_w4a16_grouped_ffn and moe_combine called one after another, bit for bit,
    when the shared expert runs in the FFN with the routed experts (the step
    calls know no shared expert; its matrix-core form is compared below)."""
    from w4a16_group_quantized_amd import ops

    shape = _shape(64, 6, 512, 256, T)
    host = synth.make_block_inputs(shape, 8, shared=True)
    plan = dict(ops.plan_default(T, 6, 64, 512, 256, shared=True).as_dict(), shared_mfma=0)
    got, (x, gw, w, blk) = _run_block(host, shape, dev, plan=plan)
    logits = ops.moe_router_gate(x, gw)
    ids, wts = ops.moe_route_shared(logits, shape.top_k)
    perm = ops.moe_permute(ids, shape.E + 1)
    y = ops.moe_w4a16_grouped_ffn(x, shape.top_k + 1, perm, w)
    out = ops.moe_combine(y, wts, perm["slot_rows"])
    torch.cuda.synchronize()
    assert np.array_equal(logits.cpu().numpy().view(np.int32), got["logits"].view(np.int32))
    assert np.array_equal(ids.cpu().numpy(), got["topk_ids"])
    assert np.array_equal(y.cpu().numpy().view(np.int32), got["y_sorted"].view(np.int32))
    assert np.array_equal(out.cpu().numpy().view(np.int16), got["out"].view(np.int16))


@pytest.mark.parametrize("E,k,H,I,T", [(512, 10, 2560, 640, 8), (64, 6, 512, 256, 1),
                                       (64, 6, 512, 160, 32),
                                       (512, 10, 2560, 640, 22)])   # the most LDS it takes
def test_shared_expert_on_matrix_cores_matches_the_gemv_form(dev, E, k, H, I, T):
    """The shared expert's rows on the matrix cores (extra workgroups) against
    the same rows in the GEMV with the routed experts: the routed rows bit for
    bit, the shared rows within the y_sorted bound (the order of fp32 sums
    differs), and both outputs within the layer tolerance of the oracle."""
    from w4a16_group_quantized_amd import ops

    shape = _shape(E, k, H, I, T)
    host = synth.make_block_inputs(shape, 15, shared=True)
    base = ops.plan_default(T, k, E, H, I, shared=True).as_dict()
    assert base["shared_mfma"] == (1 if T >= 3 else 0)   # the table's choice
    # (the combine folded into the down GEMV takes no shared-expert workgroups)
    mf, _ = _run_block(host, shape, dev, plan=dict(base, shared_mfma=1, combine_in_down=0))
    gv, _ = _run_block(host, shape, dev, plan=dict(base, shared_mfma=0))
    S = T * k
    assert np.array_equal(mf["topk_ids"], gv["topk_ids"])
    assert np.array_equal(mf["y_sorted"][:S].view(np.int32), gv["y_sorted"][:S].view(np.int32))
    assert_y_close(mf["y_sorted"][S:], gv["y_sorted"][S:], f"{shape} shared rows, MFMA vs GEMV")
    ref = oracle.block(host, k, shared=True)
    bound = _logit_bound(host["x"], host["gate_w"])
    clear = ~_ambiguous_tokens(ref["logits"], bound, k)
    assert_fp16_close(mf["out"][clear], ref["out"][clear], f"{shape} MFMA shared")
    assert_fp16_close(gv["out"][clear], ref["out"][clear], f"{shape} GEMV shared")


@pytest.mark.parametrize("T", [8, 300])
def test_block_without_shared_is_projection_plus_layer(dev, T):
    from w4a16_group_quantized_amd import ops

    shape = _shape(64, 6, 512, 256, T)
    host = synth.make_block_inputs(shape, 9, shared=False)
    got, (x, gw, w, blk) = _run_block(host, shape, dev, shared=False)
    logits = ops.moe_router_gate(x, gw)
    out = ops.moe_layer_forward(logits, x, shape.top_k, w)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.int16), got["out"].view(np.int16))


def test_block_graph_replay_matches_eager(dev):
    """A captured block call replays to the eager result, with eager work between replays."""
    shape = _shape(512, 10, 2560, 640, 8)
    host = synth.make_block_inputs(shape, 10, shared=True)
    got, (x, gw, w, blk) = _run_block(host, shape, dev)
    eager = blk.out.clone()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            blk(x, gw, w)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(4):
        blk.out.fill_(7.0)
        blk.logits.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(blk.out, eager), f"replay {rep}"
        _ = (blk.out.float() * 2).sum().item()  # eager work between replays
