"""CPU oracle for the routed-expert W4A16 group-32 MoE layer.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  The product path (the HIP library and
its Python binding) never calls it, and it imports nothing from the product.

What is computed.  The pages describe a 512-expert, top-10 routed-expert layer
with AWQ-style W4A16 group-32 weights ("[Model][SM70] Adapt Qwen3.8 Flash Next
NVFP4", section "Implemented route"; "[Perf][SM70] Narrow Qwen3.8 AWQ active
grouped decode", section "Purpose") whose experts are run per active expert
over multi-row segments located by offsets (same page, "Purpose").  The steps,
in order:

  1. route    softmax over the E router logits, top-k, weights renormalised to 1
  2. permute  stable counting sort of the T*k (token, choice) slots by expert:
              per-expert offsets, sorted slot list, its inverse, active experts
  3. gate/up  h = x[token] @ dequant(w13[e])^T                 (fp, [2I])
  4. act      a = SiLU(h[:I]) * h[I:]                          (fp, [I])
  5. down     y_sorted[row] = a @ dequant(w2[e])^T             (fp, [H])
  6. combine  out[t] = sum_j w[t, j] * y_sorted[row of slot t*k+j]

Dequantisation of a packed weight: w = (q - z) * s, with q the 4-bit code of
the weight, z the 4-bit zero and s the fp16 scale of its 32-wide group along K.

Precision: every floating-point step runs in ``dtype`` (fp64 by default; fp32
gives the "fp32 matmuls" variant).  Top-k ranks the fp32 logits themselves, so
the selection is the same in any dtype.

Around the routed layer (the MoE block): the router's gate projection makes
the logits from the activations, logits = x @ Wg^T, and a shared expert (one
more SwiGLU expert, in the same W4A16 format) runs on every token; its output
is added to the routed output before the one rounding to fp16.  The pages name
both only as the work beside the routed layer ("[Perf][SM70] Narrow Qwen3.8 AWQ
active grouped decode", sections "New-base bounded integration acceptance
(r2)", where the shared overlap is switched off, and "Capacity, startup, and
remaining limit", which names the shared projection costs); they give no
formula, so these are the plainest readings: an unquantised fp16 Wg [E, H]
without bias, fp32 logits, and a shared expert with weight 1 and no gate of
its own, stored as expert E after the E routed experts.

Readings of points the pages leave open (listed with reasons in the design
notes): weights are packed 8 per int32 along K, low nibble first, no column
interleave; zeros are packed 8 per int32 along N; w13 rows [0, I) are gate and
[I, 2I) are up; top-k ties go to the lower expert index and output columns are
in rank order; within an expert segment rows are in ascending slot order
(slot = t*k + j); ``active_experts`` lists active experts ascending, padded with
-1 to length E.
"""

from __future__ import annotations

import numpy as np

GROUP_SIZE = 32


# --------------------------------------------------------------------------- #
# 1. unpack and dequantise (AWQ-style W4A16, group size 32 along K)
# --------------------------------------------------------------------------- #
def unpack_weight_codes(qweight: np.ndarray) -> np.ndarray:
    """[..., N, K/8] int32 -> [..., N, K] uint8 codes; nibble j of word w is k = 8w + j."""
    words = qweight.astype(np.int64) & 0xFFFFFFFF
    fields = [((words >> (4 * j)) & 0xF) for j in range(8)]
    codes = np.stack(fields, axis=-1)  # [..., N, K/8, 8]
    return codes.reshape(*qweight.shape[:-1], qweight.shape[-1] * 8).astype(np.uint8)


def unpack_zero_codes(qzeros: np.ndarray) -> np.ndarray:
    """[..., N/8, G] int32 -> [..., N, G] uint8 zeros; nibble j of word w is row n = 8w + j."""
    words = qzeros.astype(np.int64) & 0xFFFFFFFF
    fields = [((words >> (4 * j)) & 0xF) for j in range(8)]
    z = np.stack(fields, axis=-2)  # [..., N/8, 8, G]
    return z.reshape(*qzeros.shape[:-2], qzeros.shape[-2] * 8, qzeros.shape[-1]).astype(np.uint8)


def dequantize(qweight: np.ndarray, qzeros: np.ndarray, scales: np.ndarray,
               dtype=np.float64) -> np.ndarray:
    """W[n, k] = (q[n, k] - z[n, k // 32]) * s[n, k // 32], shape [..., N, K]."""
    q = unpack_weight_codes(qweight).astype(dtype)
    z = unpack_zero_codes(qzeros).astype(dtype)
    s = scales.astype(dtype)
    K = q.shape[-1]
    group = np.arange(K) // GROUP_SIZE
    return (q - z[..., group]) * s[..., group]


# --------------------------------------------------------------------------- #
# 2. router: softmax, top-k, renormalise
# --------------------------------------------------------------------------- #
def route(logits: np.ndarray, top_k: int, dtype=np.float64):
    """Softmax over experts, pick the k largest, renormalise their weights to 1.

    Returns ``ids`` int32 [T, k] (rank order, ties to the lower expert index)
    and ``weights`` [T, k] in ``dtype``.
    """
    L = np.asarray(logits, dtype=np.float32)
    T, E = L.shape
    Ld = L.astype(dtype)
    p = np.exp(Ld - Ld.max(axis=1, keepdims=True))
    p = p / p.sum(axis=1, keepdims=True)

    ids = np.zeros((T, top_k), dtype=np.int32)
    taken = np.zeros((T, E), dtype=bool)
    rows = np.arange(T)
    for j in range(top_k):
        best = np.max(np.where(taken, -np.inf, L), axis=1)
        is_best = (~taken) & (L == best[:, None])
        pick = np.argmax(is_best, axis=1)  # first True: lowest expert index
        ids[:, j] = pick
        taken[rows, pick] = True

    sel = p[rows[:, None], ids]
    weights = sel / sel.sum(axis=1, keepdims=True)
    return ids, weights


# --------------------------------------------------------------------------- #
# 3. permutation: active-expert segments and offsets
# --------------------------------------------------------------------------- #
def permute(ids: np.ndarray, E: int):
    """Stable counting sort of slots s = t*k + j by expert id.

    Returns a dict with ``expert_offsets`` [E+1], ``sorted_slots`` [T*k]
    (slot held by each sorted row), ``slot_rows`` [T*k] (sorted row of each
    slot), ``active_experts`` [E] (ascending, -1 padded) and ``num_active``.
    """
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    S = flat.size
    counts = np.zeros(E, dtype=np.int64)
    for e in flat:
        counts[e] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]

    fill = offsets[:-1].copy()
    sorted_slots = np.zeros(S, dtype=np.int64)
    for s in range(S):
        e = flat[s]
        sorted_slots[fill[e]] = s
        fill[e] += 1

    slot_rows = np.zeros(S, dtype=np.int64)
    for r in range(S):
        slot_rows[sorted_slots[r]] = r

    active = [e for e in range(E) if counts[e] > 0]
    active_experts = np.full(E, -1, dtype=np.int64)
    active_experts[: len(active)] = active
    return {
        "expert_offsets": offsets.astype(np.int32),
        "sorted_slots": sorted_slots.astype(np.int32),
        "slot_rows": slot_rows.astype(np.int32),
        "active_experts": active_experts.astype(np.int32),
        "num_active": np.int32(len(active)),
    }


# --------------------------------------------------------------------------- #
# 4. expert FFN: gate/up, SiLU(gate) * up, down
# --------------------------------------------------------------------------- #
def silu(v: np.ndarray) -> np.ndarray:
    return v / (1.0 + np.exp(-v))


def expert_ffn(x_rows: np.ndarray, w13: np.ndarray, w2: np.ndarray) -> np.ndarray:
    """y = (SiLU(x W1^T) * (x W3^T)) W2^T for dequantised w13 = [W1; W3] and w2."""
    I = w13.shape[0] // 2
    h = x_rows @ w13.T
    act = silu(h[:, :I]) * h[:, I:]
    return act @ w2.T


def grouped_ffn(x: np.ndarray, top_k: int, perm: dict, weights: dict, dtype=np.float64) -> np.ndarray:
    """y_sorted [T*k, H]: every sorted row through its expert's FFN."""
    E = perm["expert_offsets"].size - 1
    H = x.shape[1]
    S = perm["sorted_slots"].size
    y_sorted = np.zeros((S, H), dtype=dtype)
    off = perm["expert_offsets"]
    for e in range(E):
        r0, r1 = int(off[e]), int(off[e + 1])
        if r1 == r0:
            continue
        tokens = perm["sorted_slots"][r0:r1] // top_k
        w13 = dequantize(weights["w13_q"][e], weights["w13_z"][e], weights["w13_s"][e], dtype)
        w2 = dequantize(weights["w2_q"][e], weights["w2_z"][e], weights["w2_s"][e], dtype)
        y_sorted[r0:r1] = expert_ffn(x[tokens].astype(dtype), w13, w2)
    return y_sorted


# --------------------------------------------------------------------------- #
# 5. combine back to token order
# --------------------------------------------------------------------------- #
def combine(y_sorted: np.ndarray, topk_weights: np.ndarray, slot_rows: np.ndarray) -> np.ndarray:
    """out[t] = sum over j ascending of w[t, j] * y_sorted[slot_rows[t*k + j]]."""
    T, k = topk_weights.shape
    out = np.zeros((T, y_sorted.shape[1]), dtype=y_sorted.dtype)
    for j in range(k):
        rows = slot_rows[np.arange(T) * k + j]
        out += topk_weights[:, j : j + 1].astype(y_sorted.dtype) * y_sorted[rows]
    return out


# --------------------------------------------------------------------------- #
# the whole layer, and a per-token version for sampled checks at large sizes
# --------------------------------------------------------------------------- #
def layer(inputs: dict, top_k: int, dtype=np.float64) -> dict:
    """Run all six steps; returns every intermediate the HIP path also exposes."""
    logits, x = inputs["logits"], inputs["x"]
    E = logits.shape[1]
    ids, w = route(logits, top_k, dtype)
    perm = permute(ids, E)
    y_sorted = grouped_ffn(x, top_k, perm, inputs, dtype)
    out = combine(y_sorted, w, perm["slot_rows"])
    res = {"topk_ids": ids, "topk_weights": w, "y_sorted": y_sorted, "out": out,
           "out_fp16": out.astype(np.float16)}
    res.update(perm)
    return res


def token_outputs(inputs: dict, ids: np.ndarray, weights: np.ndarray, tokens,
                  dtype=np.float64) -> np.ndarray:
    """out[t] for the listed tokens only, straight from the definition (no permutation)."""
    x = inputs["x"]
    tokens = np.asarray(tokens, dtype=np.int64)
    out = np.zeros((tokens.size, x.shape[1]), dtype=dtype)
    cache: dict[int, tuple[np.ndarray, np.ndarray]] = {}
    for i, t in enumerate(tokens):
        xt = x[t : t + 1].astype(dtype)
        for j in range(ids.shape[1]):
            e = int(ids[t, j])
            if e not in cache:
                cache[e] = (
                    dequantize(inputs["w13_q"][e], inputs["w13_z"][e], inputs["w13_s"][e], dtype),
                    dequantize(inputs["w2_q"][e], inputs["w2_z"][e], inputs["w2_s"][e], dtype),
                )
            w13, w2 = cache[e]
            out[i] += dtype(weights[t, j]) * expert_ffn(xt, w13, w2)[0]
    return out


# --------------------------------------------------------------------------- #
# the MoE block: router gate projection in front, shared expert beside
# --------------------------------------------------------------------------- #
_WEIGHT_KEYS = ("w13_q", "w13_z", "w13_s", "w2_q", "w2_z", "w2_s")


def router_logits(x: np.ndarray, gate_weight: np.ndarray, dtype=np.float64) -> np.ndarray:
    """logits[t, e] = sum_h x[t, h] * Wg[e, h], for x [T, H] and Wg [E, H] (fp16 values)."""
    return x.astype(dtype) @ gate_weight.astype(dtype).T


def shared_expert(x: np.ndarray, weights: dict, dtype=np.float64) -> np.ndarray:
    """The shared expert's FFN on every token: y [T, H].  It is the last expert
    (index E) of weight arrays that hold E + 1 experts."""
    e = weights["w13_q"].shape[0] - 1
    w13 = dequantize(weights["w13_q"][e], weights["w13_z"][e], weights["w13_s"][e], dtype)
    w2 = dequantize(weights["w2_q"][e], weights["w2_z"][e], weights["w2_s"][e], dtype)
    return expert_ffn(x.astype(dtype), w13, w2)


def layer_with_shared(inputs: dict, top_k: int, dtype=np.float64) -> dict:
    """The routed layer over experts [0, E) (E from the logits) plus the shared
    expert E: out = routed out + shared y, then one rounding to fp16."""
    E = inputs["logits"].shape[1]
    routed = layer({"logits": inputs["logits"], "x": inputs["x"],
                    **{k: inputs[k][:E] for k in _WEIGHT_KEYS}}, top_k, dtype)
    y_shared = shared_expert(inputs["x"], inputs, dtype)
    out = routed["out"] + y_shared
    res = dict(routed)
    res.update({"routed_out": routed["out"], "y_shared": y_shared, "out": out,
                "out_fp16": out.astype(np.float16)})
    return res


def block(inputs: dict, top_k: int, shared: bool = True, dtype=np.float64) -> dict:
    """The MoE block: logits = router_logits(x, gate_w), rounded to fp32 (the
    router ranks fp32 logits), then the routed layer, plus the shared expert
    when ``shared``.  ``logits`` in the result is the fp32 array routed on and
    ``logits_exact`` the projection before that rounding."""
    exact = router_logits(inputs["x"], inputs["gate_w"], dtype)
    logits = exact.astype(np.float32)
    E = logits.shape[1]
    inner = {"logits": logits, "x": inputs["x"], **{k: inputs[k] for k in _WEIGHT_KEYS}}
    if shared:
        res = layer_with_shared(inner, top_k, dtype)
    else:
        res = layer({**inner, **{k: inputs[k][:E] for k in _WEIGHT_KEYS}}, top_k, dtype)
    res["logits"] = logits
    res["logits_exact"] = exact
    return res
