"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Every check here is one of: a hand-built fixture whose expected value follows
from the definition by hand (tests/golden), a closed form of a special case, a
textbook library routine that the oracle does not use (stable argsort), an
invariant, or an independent scalar brute force on tiny inputs.  They are chosen
so that a dropped term, a wrong sign or index, a swapped gate/up half or a
transposed operand in the oracle fails at least one of them.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
from w4a16_group_quantized_amd import inputs as synth


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def _word(s):
    return np.array([int(s, 16)], dtype=np.uint32).view(np.int32)[0]


# --------------------------------------------------------------------------- #
# unpack and dequantise
# --------------------------------------------------------------------------- #
def test_weight_nibble_order_golden(golden_dir):
    g = _load(golden_dir, "handbuilt_int4.json")
    for case in g["weight_words"]:
        q = np.array([[_word(case["word"])]], dtype=np.int32)  # [N=1, K/8=1]
        assert oracle.unpack_weight_codes(q)[0].tolist() == case["codes"], case


def test_zero_nibble_order_golden(golden_dir):
    g = _load(golden_dir, "handbuilt_int4.json")
    for case in g["zero_words"]:
        z = np.array([[_word(case["word"])]], dtype=np.int32)  # [N/8=1, G=1]
        assert oracle.unpack_zero_codes(z)[:, 0].tolist() == case["rows"], case


def test_dequant_products_golden(golden_dir):
    g = _load(golden_dir, "handbuilt_int4.json")
    for case in g["dequant"]:
        # one 8-row x 32-col block; the case sits at row 5, column 13 (group 0)
        q = np.zeros((8, 4), dtype=np.uint32)
        q[5, 13 // 8] = case["q"] << (4 * (13 % 8))
        z = np.array([[case["z"] << (4 * 5)]], dtype=np.uint32)
        s = np.zeros((8, 1), dtype=np.float16)
        s[5, 0] = case["s"]
        W = oracle.dequantize(q.view(np.int32), z.view(np.int32), s)
        assert W.shape == (8, 32)
        assert W[5, 13] == case["w"], case
        # the rest of row 5 has q = 0, so it reads -z * s; other rows have s = 0
        rest = np.delete(W[5], 13)
        assert np.all(rest == -case["z"] * float(s[5, 0])), case
        assert np.all(np.delete(W, 5, axis=0) == 0.0)


def test_dequant_group_sums_closed_form():
    """x = ones over one group: sum_k W[n, k] = s * (sum_k q - 32 z), by hand."""
    # every word 0x76543210: each 8-nibble block sums to 0+1+..+7 = 28, a group to 112
    N, K = 16, 64  # two groups along K
    q = np.full((N, K // 8), _word("0x76543210"), dtype=np.int32)
    zeros = np.zeros((N, 2), dtype=np.int64)
    zeros[:, 0] = 3
    zeros[:, 1] = np.arange(N) % 16
    zw = np.zeros((N // 8, 2), dtype=np.int64)
    for n in range(N):
        for g in range(2):
            zw[n // 8, g] |= int(zeros[n, g]) << (4 * (n % 8))
    s = np.zeros((N, 2), dtype=np.float16)
    s[:, 0] = 0.5
    s[:, 1] = 2.0
    W = oracle.dequantize(q, zw.astype(np.uint32).view(np.int32), s)
    g0 = W[:, :32].sum(axis=1)
    g1 = W[:, 32:].sum(axis=1)
    assert np.all(g0 == 0.5 * (112 - 32 * 3))  # = 8
    assert np.all(g1 == 2.0 * (112 - 32 * (np.arange(N) % 16)))


def test_dequant_one_hot_picks_a_column():
    """x = e_k gives h = W[:, k] exactly: pins the operand orientation of x @ W^T."""
    shape = synth.MoEShape(E=1, top_k=1, H=64, I=32, T=1)
    w = synth.make_weights(shape, seed=3)
    W13 = oracle.dequantize(w["w13_q"][0], w["w13_z"][0], w["w13_s"][0])
    codes = oracle.unpack_weight_codes(w["w13_q"][0])
    zc = oracle.unpack_zero_codes(w["w13_z"][0])
    for k in (0, 7, 8, 31, 32, 63):
        x = np.zeros((1, 64))
        x[0, k] = 1.0
        h = (x @ W13.T)[0]
        expect = (codes[:, k].astype(np.float64) - zc[:, k // 32]) * w["w13_s"][0][:, k // 32].astype(np.float64)
        assert np.array_equal(h, expect)


# --------------------------------------------------------------------------- #
# router
# --------------------------------------------------------------------------- #
def test_route_golden(golden_dir):
    g = _load(golden_dir, "handbuilt_route.json")
    for case in g["cases"]:
        L = np.array([case["logits"]], dtype=np.float32)
        ids, w = oracle.route(L, case["top_k"])
        assert ids[0].tolist() == case["ids"], case
        np.testing.assert_allclose(w[0], case["weights"], rtol=0, atol=1e-6)


def test_route_matches_stable_argsort_with_ties():
    rng = np.random.default_rng(11)
    # round to one decimal so that many logits tie
    L = np.round(rng.standard_normal((300, 64)), 1).astype(np.float32)
    for k in (1, 2, 7, 64):
        ids, w = oracle.route(L, k)
        expect = np.argsort(-L, axis=1, kind="stable")[:, :k]
        assert np.array_equal(ids, expect)
        assert np.all(np.abs(w.sum(axis=1) - 1.0) < 1e-12)
        assert all(len(set(r)) == k for r in ids.tolist())
        # weights follow rank order (non-increasing)
        assert np.all(np.diff(w, axis=1) <= 1e-15)


def test_route_weights_are_softmax_ratios():
    rng = np.random.default_rng(5)
    L = rng.standard_normal((50, 32)).astype(np.float32)
    ids, w = oracle.route(L, 4)
    for t in range(50):
        e = [math.exp(float(L[t, i])) for i in ids[t]]
        assert w[t].tolist() == pytest.approx([v / sum(e) for v in e], rel=1e-12)


# --------------------------------------------------------------------------- #
# permutation
# --------------------------------------------------------------------------- #
def test_permute_golden(golden_dir):
    g = _load(golden_dir, "handbuilt_permute.json")
    p = oracle.permute(np.array(g["ids"], dtype=np.int32), g["E"])
    for key in ("expert_offsets", "sorted_slots", "slot_rows", "active_experts"):
        assert p[key].tolist() == g[key], key
    assert int(p["num_active"]) == g["num_active"]


@pytest.mark.parametrize("T,E,k", [(1, 8, 2), (9, 8, 8), (64, 512, 10), (65, 512, 10), (300, 37, 5)])
def test_permute_matches_textbook_sort(T, E, k):
    rng = np.random.default_rng(T * 1000 + E)
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    p = oracle.permute(ids, E)
    flat = ids.ravel()
    assert np.array_equal(p["sorted_slots"], np.argsort(flat, kind="stable"))
    counts = np.bincount(flat, minlength=E)
    assert np.array_equal(p["expert_offsets"], np.concatenate([[0], np.cumsum(counts)]))
    assert np.array_equal(p["slot_rows"][p["sorted_slots"]], np.arange(T * k))
    assert np.array_equal(p["sorted_slots"][p["slot_rows"]], np.arange(T * k))
    act = np.nonzero(counts)[0]
    assert int(p["num_active"]) == act.size
    assert np.array_equal(p["active_experts"][: act.size], act)
    assert np.all(p["active_experts"][act.size :] == -1)
    assert counts.max() <= T


# --------------------------------------------------------------------------- #
# FFN and combine
# --------------------------------------------------------------------------- #
def _pack_rows(codes):
    """[N, K] codes -> [N, K/8] words, low nibble first (test-side packer)."""
    N, K = codes.shape
    out = np.zeros((N, K // 8), dtype=np.uint64)
    for j in range(8):
        out |= codes[:, j::8].astype(np.uint64) << np.uint64(4 * j)
    return out.astype(np.uint32).view(np.int32)


def _pack_zero_rows(zc):
    """[N, G] zeros -> [N/8, G] words, row n in nibble n % 8."""
    N, G = zc.shape
    out = np.zeros((N // 8, G), dtype=np.uint64)
    for j in range(8):
        out |= zc[j::8, :].astype(np.uint64) << np.uint64(4 * j)
    return out.astype(np.uint32).view(np.int32)


def test_layer_gate_up_order_closed_form():
    """One expert, one token, x = e_0, gate pre-activation 2, up pre-activation -1.

    With every down weight (9 - 8) / 16 the output is I/16 * SiLU(2) * (-1) for
    every h; swapping gate and up would give I/16 * SiLU(-1) * 2 instead.
    """
    H, I = 32, 32
    c13 = np.zeros((2 * I, H), dtype=np.int64)
    c13[:I, 0] = 5  # gate: (5 - 1) * 0.5 = 2
    c13[I:, 0] = 0  # up:   (0 - 4) * 0.25 = -1
    z13 = np.zeros((2 * I, 1), dtype=np.int64)
    z13[:I] = 1
    z13[I:] = 4
    s13 = np.zeros((2 * I, 1), dtype=np.float16)
    s13[:I] = 0.5
    s13[I:] = 0.25
    c2 = np.full((H, I), 9, dtype=np.int64)
    z2 = np.full((H, 1), 8, dtype=np.int64)
    s2 = np.full((H, 1), 1.0 / 16, dtype=np.float16)
    x = np.zeros((1, H), dtype=np.float16)
    x[0, 0] = 1.0
    inp = {
        "logits": np.zeros((1, 1), dtype=np.float32), "x": x,
        "w13_q": _pack_rows(c13)[None], "w13_z": _pack_zero_rows(z13)[None], "w13_s": s13[None],
        "w2_q": _pack_rows(c2)[None], "w2_z": _pack_zero_rows(z2)[None], "w2_s": s2[None],
    }
    res = oracle.layer(inp, top_k=1)
    silu2 = 2.0 / (1.0 + math.exp(-2.0))
    expect = I / 16 * silu2 * -1.0
    assert np.allclose(res["out"], expect, rtol=1e-14, atol=0)
    assert res["topk_weights"][0, 0] == 1.0


def _brute_force_layer(inp, top_k):
    """Scalar-loop restatement of the layer, written apart from the oracle."""
    L = inp["logits"]
    T, E = L.shape
    H = inp["x"].shape[1]
    I = inp["w2_q"].shape[2] * 8

    def code(words, n, k):
        return (int(words[n, k // 8]) >> (4 * (k % 8))) & 0xF

    def zero(words, n, g):
        return (int(words[n // 8, g]) >> (4 * (n % 8))) & 0xF

    def wgt(e, which, n, k):
        q, z, s = inp[which + "_q"][e], inp[which + "_z"][e], inp[which + "_s"][e]
        return (code(q, n, k) - zero(z, n, k // 32)) * float(s[n, k // 32])

    out = [[0.0] * H for _ in range(T)]
    ids_all, w_all = [], []
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-float(L[t, e]), e))[:top_k]
        m = max(float(v) for v in L[t])
        den = sum(math.exp(float(v) - m) for v in L[t])
        p = [math.exp(float(L[t, e]) - m) / den for e in order]
        w = [v / sum(p) for v in p]
        ids_all.append(order)
        w_all.append(w)
        xt = [float(v) for v in inp["x"][t]]
        for j, e in enumerate(order):
            h = [sum(xt[k] * wgt(e, "w13", n, k) for k in range(H)) for n in range(2 * I)]
            a = [h[i] / (1.0 + math.exp(-h[i])) * h[I + i] for i in range(I)]
            for hh in range(H):
                y = sum(a[i] * wgt(e, "w2", hh, i) for i in range(I))
                out[t][hh] += w[j] * y
    return np.array(ids_all), np.array(w_all), np.array(out)


def test_layer_matches_scalar_brute_force():
    shape = synth.MoEShape(E=4, top_k=2, H=64, I=32, T=3)
    inp = synth.make_inputs(shape, seed=7)
    ids, w, out = _brute_force_layer(inp, shape.top_k)
    res = oracle.layer(inp, shape.top_k)
    assert np.array_equal(res["topk_ids"], ids)
    np.testing.assert_allclose(res["topk_weights"], w, rtol=1e-12, atol=0)
    np.testing.assert_allclose(res["out"], out, rtol=1e-9, atol=1e-9)


def test_single_expert_top1_is_dense_ffn():
    shape = synth.MoEShape(E=1, top_k=1, H=128, I=64, T=5)
    inp = synth.make_inputs(shape, seed=2)
    res = oracle.layer(inp, 1)
    W13 = oracle.dequantize(inp["w13_q"][0], inp["w13_z"][0], inp["w13_s"][0])
    W2 = oracle.dequantize(inp["w2_q"][0], inp["w2_z"][0], inp["w2_s"][0])
    x = inp["x"].astype(np.float64)
    g, u = x @ W13[:64].T, x @ W13[64:].T
    dense = (g * (1 / (1 + np.exp(-g))) * u) @ W2.T
    assert np.all(res["topk_weights"] == 1.0)
    np.testing.assert_allclose(res["out"], dense, rtol=1e-12, atol=1e-12)


def test_identical_experts_make_output_independent_of_routing():
    shape = synth.MoEShape(E=6, top_k=3, H=64, I=32, T=7)
    inp = synth.make_inputs(shape, seed=4)
    for key in ("w13_q", "w13_z", "w13_s", "w2_q", "w2_z", "w2_s"):
        inp[key] = np.repeat(inp[key][:1], shape.E, axis=0)
    res = oracle.layer(inp, shape.top_k)
    single = oracle.layer({**inp, "logits": np.zeros((shape.T, 1), np.float32),
                           **{k: inp[k][:1] for k in ("w13_q", "w13_z", "w13_s", "w2_q", "w2_z", "w2_s")}}, 1)
    np.testing.assert_allclose(res["out"], single["out"], rtol=1e-12, atol=1e-12)


def test_zero_scales_give_zero_output():
    shape = synth.MoEShape(E=8, top_k=2, H=256, I=128, T=4)
    inp = synth.make_inputs(shape, seed=0)
    inp["w2_s"] = np.zeros_like(inp["w2_s"])
    assert np.all(oracle.layer(inp, 2)["out"] == 0.0)


def test_doubling_down_scales_doubles_output():
    shape = synth.MoEShape(E=8, top_k=2, H=256, I=128, T=4)
    inp = synth.make_inputs(shape, seed=0)
    a = oracle.layer(inp, 2)["out"]
    inp["w2_s"] = (inp["w2_s"].astype(np.float32) * 2).astype(np.float16)  # exact in fp16
    b = oracle.layer(inp, 2)["out"]
    np.testing.assert_allclose(b, 2 * a, rtol=1e-13, atol=1e-13)


def test_fp32_variant_agrees_with_fp64():
    shape = synth.WORKLOADS["tiny_e8_k2_h256_i128_t4"]
    inp = synth.make_inputs(shape, seed=0)
    a = oracle.layer(inp, shape.top_k, np.float64)
    b = oracle.layer(inp, shape.top_k, np.float32)
    assert np.array_equal(a["topk_ids"], b["topk_ids"])
    err = np.abs(a["out"] - b["out"]).max() / np.abs(a["out"]).max()
    assert err < 1e-5


def test_combine_gathers_by_slot_rows():
    """Combine with one-hot y rows recovers the router weights at the right places."""
    T, k, H = 3, 2, 6
    slot_rows = np.array([4, 0, 1, 2, 5, 3])
    y = np.eye(6)  # y_sorted[r] = e_r
    w = np.array([[0.7, 0.3], [0.6, 0.4], [0.9, 0.1]])
    out = oracle.combine(y, w, slot_rows)
    expect = np.zeros((T, H))
    for t in range(T):
        for j in range(k):
            expect[t, slot_rows[t * k + j]] += w[t, j]
    assert np.array_equal(out, expect)


def test_token_outputs_match_layer():
    shape = synth.MoEShape(E=16, top_k=4, H=128, I=64, T=9)
    inp = synth.make_inputs(shape, seed=1)
    res = oracle.layer(inp, shape.top_k)
    sub = oracle.token_outputs(inp, res["topk_ids"], res["topk_weights"], [0, 4, 8])
    np.testing.assert_allclose(sub, res["out"][[0, 4, 8]], rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------- #
# the MoE block: router gate projection and shared expert
# --------------------------------------------------------------------------- #
def test_router_logits_one_hot_closed_form():
    """Row e of Wg holds c_e at column h(e) only, so logits[t, e] = c_e * x[t, h(e)] exactly."""
    T, E, H = 3, 6, 32
    rng = np.random.default_rng(11)
    x = rng.standard_normal((T, H)).astype(np.float16)
    h_of = [(5 * e + 3) % H for e in range(E)]
    c = [2.0 ** (e - 2) for e in range(E)]
    Wg = np.zeros((E, H), dtype=np.float16)
    for e in range(E):
        Wg[e, h_of[e]] = c[e]
    L = oracle.router_logits(x, Wg)
    assert L.shape == (T, E)
    for t in range(T):
        for e in range(E):
            assert L[t, e] == c[e] * float(x[t, h_of[e]]), (t, e)


def test_router_logits_match_exact_sums():
    """fp16 x fp16 products are exact in fp64; math.fsum rounds their sum once."""
    T, E, H = 3, 5, 96
    rng = np.random.default_rng(12)
    x = rng.standard_normal((T, H)).astype(np.float16)
    Wg = (rng.standard_normal((E, H)) / np.sqrt(H)).astype(np.float16)
    L = oracle.router_logits(x, Wg)
    for t in range(T):
        for e in range(E):
            terms = [float(x[t, h]) * float(Wg[e, h]) for h in range(H)]
            scale = math.fsum(abs(v) for v in terms)
            assert abs(L[t, e] - math.fsum(terms)) <= 1e-13 * scale, (t, e)


def _closed_form_expert(gate, up, H, I):
    """Codes of one expert whose gate/up pre-activations are `gate` and `up` for
    x = e_0 (each a (code, zero, scale) triple on column 0) and whose down
    weights are all (9 - 8) / 16."""
    c13 = np.zeros((2 * I, H), dtype=np.int64)
    z13 = np.zeros((2 * I, H // 32), dtype=np.int64)
    s13 = np.zeros((2 * I, H // 32), dtype=np.float16)
    for rows, (code, zero, scale) in ((slice(0, I), gate), (slice(I, 2 * I), up)):
        c13[rows, 0] = code
        z13[rows, 0] = zero
        s13[rows, 0] = scale
    c2 = np.full((H, I), 9, dtype=np.int64)
    z2 = np.full((H, I // 32), 8, dtype=np.int64)
    s2 = np.full((H, I // 32), 1.0 / 16, dtype=np.float16)
    return {"w13_q": _pack_rows(c13), "w13_z": _pack_zero_rows(z13), "w13_s": s13,
            "w2_q": _pack_rows(c2), "w2_z": _pack_zero_rows(z2), "w2_s": s2}


def test_shared_expert_closed_form():
    """Three identical routed experts (gate 2, up 1) and a shared expert (gate -1,
    up 2), x = e_0: out = I/16 * (SiLU(2) * 1 + SiLU(-1) * 2) for every h, since
    the routed weights sum to 1 and the shared expert has weight 1."""
    H, I, E, k = 32, 32, 3, 2
    routed = _closed_form_expert((5, 1, 0.5), (5, 1, 0.25), H, I)   # (5-1)*.5 = 2, (5-1)*.25 = 1
    shared = _closed_form_expert((2, 4, 0.5), (5, 1, 0.5), H, I)    # (2-4)*.5 = -1, (5-1)*.5 = 2
    inp = {key: np.stack([routed[key]] * E + [shared[key]]) for key in routed}
    x = np.zeros((2, H), dtype=np.float16)
    x[:, 0] = 1.0
    inp.update({"x": x, "logits": np.array([[0.5, -1.0, 2.0], [0.0, 0.0, 0.0]], np.float32)})
    res = oracle.layer_with_shared(inp, k)

    def silu(v):
        return v / (1.0 + math.exp(-v))

    expect = I / 16 * (silu(2.0) * 1.0 + silu(-1.0) * 2.0)
    assert np.allclose(res["out"], expect, rtol=1e-13, atol=0)
    assert np.allclose(res["y_shared"], I / 16 * silu(-1.0) * 2.0, rtol=1e-13, atol=0)


def _brute_force_block(inp, top_k):
    """Scalar restatement of the block: exact logits (fsum), rounded to fp32,
    the routed layer's scalar loops, plus the shared expert's."""
    x, Wg = inp["x"], inp["gate_w"]
    T, H = x.shape
    E = Wg.shape[0]
    L = np.zeros((T, E), dtype=np.float32)
    for t in range(T):
        for e in range(E):
            L[t, e] = np.float32(math.fsum(float(x[t, h]) * float(Wg[e, h]) for h in range(H)))
    ids, w, out = _brute_force_layer({**inp, "logits": L}, top_k)
    I = inp["w2_q"].shape[2] * 8

    def wgt(which, n, kk):
        q, z, s = inp[which + "_q"][E], inp[which + "_z"][E], inp[which + "_s"][E]
        code = (int(q[n, kk // 8]) >> (4 * (kk % 8))) & 0xF
        zero = (int(z[n // 8, kk // 32]) >> (4 * (n % 8))) & 0xF
        return (code - zero) * float(s[n, kk // 32])

    for t in range(T):
        xt = [float(v) for v in x[t]]
        h = [sum(xt[kk] * wgt("w13", n, kk) for kk in range(H)) for n in range(2 * I)]
        a = [h[i] / (1.0 + math.exp(-h[i])) * h[I + i] for i in range(I)]
        for hh in range(H):
            out[t][hh] += sum(a[i] * wgt("w2", hh, i) for i in range(I))
    return L, ids, w, out


def test_block_matches_scalar_brute_force():
    shape = synth.MoEShape(E=4, top_k=2, H=64, I=32, T=3)
    inp = synth.make_block_inputs(shape, seed=5)
    L, ids, w, out = _brute_force_block(inp, shape.top_k)
    res = oracle.block(inp, shape.top_k)
    assert np.array_equal(res["logits"], L)
    assert np.array_equal(res["topk_ids"], ids)
    np.testing.assert_allclose(res["topk_weights"], w, rtol=1e-12, atol=0)
    np.testing.assert_allclose(res["out"], out, rtol=1e-9, atol=1e-9)


def test_shared_expert_alone_is_the_single_expert_layer():
    """With every routed down scale zero the block is the shared expert alone,
    which is the one-expert top-1 layer over the shared expert's weights."""
    shape = synth.MoEShape(E=6, top_k=2, H=128, I=64, T=5)
    inp = synth.make_block_inputs(shape, seed=6)
    inp["w2_s"] = inp["w2_s"].copy()
    inp["w2_s"][: shape.E] = 0
    res = oracle.block(inp, shape.top_k)
    single = oracle.layer({"logits": np.zeros((shape.T, 1), np.float32), "x": inp["x"],
                           **{key: inp[key][shape.E:] for key in
                              ("w13_q", "w13_z", "w13_s", "w2_q", "w2_z", "w2_s")}}, 1)
    assert np.all(res["routed_out"] == 0.0)
    np.testing.assert_allclose(res["out"], single["out"], rtol=1e-13, atol=1e-13)
