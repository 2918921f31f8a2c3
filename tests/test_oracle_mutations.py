"""Plant plausible mistakes in the oracle (CPU only) and check the pins catch each.

Each mutation replaces one oracle function with a wrong variant, runs the pin
tests of ``test_oracle_pins`` and requires at least one of them to fail.
"""

import numpy as np
import pytest

import oracle
import oracle.moe_oracle as mo
from tests import test_oracle_pins as pins
from tests.conftest import GOLDEN

_orig = {name: getattr(mo, name) for name in
         ("unpack_weight_codes", "unpack_zero_codes", "dequantize", "route", "permute",
          "expert_ffn", "combine", "silu", "router_logits", "shared_expert")}


def _unpack_high_first(qweight):
    c = _orig["unpack_weight_codes"](qweight)
    K = c.shape[-1]
    return c.reshape(*c.shape[:-1], K // 8, 8)[..., ::-1].reshape(c.shape)


def _zeros_along_k(qzeros):
    z = _orig["unpack_zero_codes"](qzeros)
    return z[..., ::-1, :].copy()  # wrong row order inside the block


def _dequant_sign(qweight, qzeros, scales, dtype=np.float64):
    return -_orig["dequantize"](qweight, qzeros, scales, dtype)


def _dequant_no_zero(qweight, qzeros, scales, dtype=np.float64):
    q = _orig["unpack_weight_codes"](qweight).astype(dtype)
    g = np.arange(q.shape[-1]) // 32
    return q * scales.astype(dtype)[..., g]


def _dequant_group_mod(qweight, qzeros, scales, dtype=np.float64):
    q = _orig["unpack_weight_codes"](qweight).astype(dtype)
    z = _orig["unpack_zero_codes"](qzeros).astype(dtype)
    G = scales.shape[-1]
    g = np.arange(q.shape[-1]) % G  # wrong group index
    return (q - z[..., g]) * scales.astype(dtype)[..., g]


def _ffn_swapped(x_rows, w13, w2):
    I = w13.shape[0] // 2
    h = x_rows @ w13.T
    return (_orig["silu"](h[:, I:]) * h[:, :I]) @ w2.T


def _ffn_no_silu(x_rows, w13, w2):
    I = w13.shape[0] // 2
    h = x_rows @ w13.T
    return (h[:, :I] * h[:, I:]) @ w2.T


def _route_no_renorm(logits, top_k, dtype=np.float64):
    ids, _ = _orig["route"](logits, top_k, dtype)
    L = logits.astype(dtype)
    p = np.exp(L - L.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    return ids, p[np.arange(L.shape[0])[:, None], ids]


def _route_ties_high(logits, top_k, dtype=np.float64):
    # ties broken towards the higher expert index
    Lr = np.ascontiguousarray(logits[:, ::-1])
    ids, w = _orig["route"](Lr, top_k, dtype)
    return (logits.shape[1] - 1 - ids).astype(np.int32), w


def _permute_unstable(ids, E):
    p = _orig["permute"](ids, E)
    off = p["expert_offsets"]
    ss = p["sorted_slots"].copy()
    for e in range(E):
        ss[off[e]:off[e + 1]] = ss[off[e]:off[e + 1]][::-1]
    p["sorted_slots"] = ss
    p["slot_rows"] = np.argsort(ss).astype(np.int32)
    return p


def _combine_wrong_rows(y_sorted, w, slot_rows):
    T, k = w.shape
    out = np.zeros((T, y_sorted.shape[1]), y_sorted.dtype)
    for j in range(k):
        out += w[:, j:j + 1] * y_sorted[np.arange(T) * k + j]  # slot index, not its row
    return out


def _logits_gate_as_h_by_e(x, gate_weight, dtype=np.float64):
    E, H = gate_weight.shape
    return x.astype(dtype) @ gate_weight.reshape(H, E).astype(dtype)  # Wg read as [H, E]


def _logits_drop_last_column(x, gate_weight, dtype=np.float64):
    return x[:, :-1].astype(dtype) @ gate_weight[:, :-1].astype(dtype).T


def _logits_fp16_sum(x, gate_weight, dtype=np.float64):
    return (x @ gate_weight.T).astype(dtype)  # accumulated in fp16


def _shared_half_weight(x, weights, dtype=np.float64):
    return 0.5 * _orig["shared_expert"](x, weights, dtype)


def _shared_first_expert(x, weights, dtype=np.float64):
    first = {k: v[:1] for k, v in weights.items() if k.startswith("w")}
    return _orig["shared_expert"](x, first, dtype)


def _shared_dropped(x, weights, dtype=np.float64):
    return np.zeros_like(_orig["shared_expert"](x, weights, dtype))


MUTATIONS = {
    "nibbles high first": {"unpack_weight_codes": _unpack_high_first},
    "zero rows reversed": {"unpack_zero_codes": _zeros_along_k},
    "dequant sign flipped": {"dequantize": _dequant_sign},
    "zero point dropped": {"dequantize": _dequant_no_zero},
    "group index k % G": {"dequantize": _dequant_group_mod},
    "gate/up swapped": {"expert_ffn": _ffn_swapped},
    "SiLU dropped": {"expert_ffn": _ffn_no_silu},
    "no renormalisation": {"route": _route_no_renorm},
    "ties to higher index": {"route": _route_ties_high},
    "unstable segments": {"permute": _permute_unstable},
    "combine by slot not row": {"combine": _combine_wrong_rows},
    "gate projection read as [H, E]": {"router_logits": _logits_gate_as_h_by_e},
    "gate projection drops a column": {"router_logits": _logits_drop_last_column},
    "gate projection summed in fp16": {"router_logits": _logits_fp16_sum},
    "shared expert weight 1/2": {"shared_expert": _shared_half_weight},
    "shared expert taken from expert 0": {"shared_expert": _shared_first_expert},
    "shared expert dropped": {"shared_expert": _shared_dropped},
}

PINS = [
    lambda: pins.test_weight_nibble_order_golden(GOLDEN),
    lambda: pins.test_zero_nibble_order_golden(GOLDEN),
    lambda: pins.test_dequant_products_golden(GOLDEN),
    pins.test_dequant_group_sums_closed_form,
    pins.test_dequant_one_hot_picks_a_column,
    lambda: pins.test_route_golden(GOLDEN),
    pins.test_route_matches_stable_argsort_with_ties,
    lambda: pins.test_permute_golden(GOLDEN),
    lambda: pins.test_permute_matches_textbook_sort(65, 512, 10),
    pins.test_layer_gate_up_order_closed_form,
    pins.test_layer_matches_scalar_brute_force,
    pins.test_combine_gathers_by_slot_rows,
    pins.test_router_logits_one_hot_closed_form,
    pins.test_router_logits_match_exact_sums,
    pins.test_shared_expert_closed_form,
    pins.test_block_matches_scalar_brute_force,
]


@pytest.mark.parametrize("name", list(MUTATIONS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    for fn_name, repl in MUTATIONS[name].items():
        monkeypatch.setattr(mo, fn_name, repl)
        monkeypatch.setattr(oracle, fn_name, repl)
    failures = 0
    for pin in PINS:
        try:
            pin()
        except Exception:
            failures += 1
    assert failures > 0, f"no pin caught the planted mistake: {name}"
