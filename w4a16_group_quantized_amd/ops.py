"""Thin Python binding over libmoe_w4a16.so (C ABI in include/moe_w4a16.h).

Argument marshalling only: each function takes torch tensors, allocates its
outputs with torch (device memory is the caller's), and passes raw device
pointers plus torch's current HIP stream to the library.  Every step of the
layer runs in the library's HIP kernels; there is no fallback, and a missing
library or a non-OK status raises.
"""

from __future__ import annotations

import ctypes
import os

import torch

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libmoe_w4a16.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = 1
MOE_ERR_UNSUPPORTED = 2
MOE_ERR_WORKSPACE = 3
MOE_ERR_HIP = 4

GROUP_SIZE = 32

EXPORTED = (
    "moe_status_string",
    "moe_abi_version",
    "moe_route",
    "moe_permute_workspace_bytes",
    "moe_permute",
    "moe_route_permute",
    "moe_ffn_workspace_bytes",
    "moe_w4a16_grouped_ffn",
    "moe_w4a16_gate_up",
    "moe_w4a16_down",
    "moe_route_gate_up",
    "moe_combine",
    "moe_layer_workspace_bytes",
    "moe_layer_forward",
    "moe_layer_forward_noalloc",
    "moe_router_gate",
    "moe_route_shared",
    "moe_block_workspace_bytes",
    "moe_block_forward",
    "moe_plan_default",
    "moe_layer_forward_plan",
    "moe_block_forward_plan",
)

FFN_GEMV, FFN_MFMA = 0, 1
ROUTE_IN_GATE_UP, ROUTE_ONE_LAUNCH, ROUTE_SEPARATE = 0, 1, 2


class Plan(ctypes.Structure):
    """moe_plan: kernel variant and tile profile of a layer call."""

    _fields_ = [("ffn", ctypes.c_int32), ("route", ctypes.c_int32), ("msub", ctypes.c_int32),
                ("lanes_gate_up", ctypes.c_int32), ("lanes_down", ctypes.c_int32),
                ("rows_per_pass", ctypes.c_int32), ("cost_split", ctypes.c_int32),
                ("router_gemv", ctypes.c_int32), ("shared_mfma", ctypes.c_int32),
                ("combine_in_down", ctypes.c_int32), ("one_launch", ctypes.c_int32)]

    def as_dict(self) -> dict:
        return {name: int(getattr(self, name)) for name, _ in self._fields_}

    def __repr__(self):
        return f"Plan({self.as_dict()})"

NOALLOC_SCRATCH_BYTES = 32 << 20


class MoEError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_SZ = ctypes.c_size_t

_SIGNATURES = {
    "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "moe_abi_version": (ctypes.c_int, []),
    "moe_route": (ctypes.c_int, [_P, _I64, _I32, _I32, _P, _P, _P]),
    "moe_permute_workspace_bytes": (_SZ, [_I64, _I32, _I32]),
    "moe_permute": (ctypes.c_int, [_P, _I64, _I32, _I32, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_route_permute": (
        ctypes.c_int, [_P, _I64, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_ffn_workspace_bytes": (_SZ, [_I64, _I32, _I32, _I32, _I32]),
    "moe_w4a16_grouped_ffn": (
        ctypes.c_int,
        [_P, _I64, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _P, _P,
         _SZ, _P],
    ),
    "moe_w4a16_gate_up": (
        ctypes.c_int,
        [_P, _I64, _I32, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _P, _SZ, _P],
    ),
    "moe_w4a16_down": (
        ctypes.c_int,
        [_I64, _I32, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _P, _P, _SZ, _P],
    ),
    "moe_combine": (ctypes.c_int, [_P, _P, _P, _I64, _I32, _I32, _P, _P]),
    "moe_route_gate_up": (
        ctypes.c_int,
        [_P, _P, _I64, _I32, _I32, _P, _P, _P, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _P,
         _SZ, _P]),
    "moe_layer_workspace_bytes": (_SZ, [_I64, _I32, _I32, _I32, _I32]),
    "moe_layer_forward": (
        ctypes.c_int,
        [_P, _P, _I64, _I32, _I32, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _P, _P, _SZ, _P]),
    "moe_layer_forward_noalloc": (
        ctypes.c_int,
        [_P, _P, _I64, _I32, _I32, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _P, _P]),
    "moe_router_gate": (ctypes.c_int, [_P, _I64, _I32, _P, _I32, _P, _P]),
    "moe_route_shared": (ctypes.c_int, [_P, _I64, _I32, _I32, _P, _P, _P]),
    "moe_block_workspace_bytes": (_SZ, [_I64, _I32, _I32, _I32, _I32, _I32]),
    "moe_plan_default": (ctypes.c_int, [_I64, _I32, _I32, _I32, _I32, _I32, _P]),
    "moe_layer_forward_plan": (
        ctypes.c_int,
        [_P, _P, _I64, _I32, _I32, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _P, _P, _SZ, _P,
         _P]),
    "moe_block_forward_plan": (
        ctypes.c_int,
        [_P, _I64, _P, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _P, _P, _P,
         _SZ, _P, _P]),
    "moe_block_forward": (
        ctypes.c_int,
        [_P, _I64, _P, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _P, _P, _P,
         _SZ, _P]),
}


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Open the HIP library (once); raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m w4a16_group_quantized_amd.build_lib`"
        )
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().moe_status_string(status).decode()


def _check(fn: str, status: int) -> None:
    if status != MOE_OK:
        raise MoEError(fn, status, status_string(status))


def _ptr(t: torch.Tensor | None) -> int | None:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    return t.data_ptr() or None


def _stream() -> int | None:
    return torch.cuda.current_stream().cuda_stream or None


# --------------------------------------------------------------------------- #
# size queries
# --------------------------------------------------------------------------- #
def permute_workspace_bytes(T: int, top_k: int, E: int) -> int:
    return int(load_library().moe_permute_workspace_bytes(T, top_k, E))


def ffn_workspace_bytes(T: int, top_k: int, E: int, H: int, I: int) -> int:
    return int(load_library().moe_ffn_workspace_bytes(T, top_k, E, H, I))


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


# --------------------------------------------------------------------------- #
# the four layer calls (plus the two halves of the FFN)
# --------------------------------------------------------------------------- #
def moe_route(logits: torch.Tensor, top_k: int, out_ids=None, out_weights=None):
    """fp32 logits [T, E] -> (topk_ids int32 [T, k], topk_weights fp32 [T, k])."""
    lib = load_library()
    T, E = logits.shape
    dev = logits.device
    ids = out_ids if out_ids is not None else torch.empty((T, top_k), dtype=torch.int32, device=dev)
    w = out_weights if out_weights is not None else torch.empty((T, top_k), dtype=torch.float32, device=dev)
    _check("moe_route", lib.moe_route(_ptr(logits), T, E, top_k, _ptr(ids), _ptr(w), _stream()))
    return ids, w


def moe_permute(topk_ids: torch.Tensor, E: int, workspace: torch.Tensor | None = None,
                out: dict | None = None) -> dict:
    """topk_ids [T, k] -> dict of expert_offsets, sorted_slots, slot_rows, active_experts, num_active."""
    lib = load_library()
    T, k = topk_ids.shape
    dev = topk_ids.device
    S = T * k
    if out is None:
        out = {
            "expert_offsets": torch.empty(E + 1, dtype=torch.int32, device=dev),
            "sorted_slots": torch.empty(S, dtype=torch.int32, device=dev),
            "slot_rows": torch.empty(S, dtype=torch.int32, device=dev),
            "active_experts": torch.empty(E, dtype=torch.int32, device=dev),
            "num_active": torch.empty(1, dtype=torch.int32, device=dev),
        }
    need = permute_workspace_bytes(T, k, E)
    if workspace is None:
        workspace = _workspace(need, dev)
    _check("moe_permute", lib.moe_permute(
        _ptr(topk_ids), T, k, E, _ptr(out["expert_offsets"]), _ptr(out["sorted_slots"]),
        _ptr(out["slot_rows"]), _ptr(out["active_experts"]), _ptr(out["num_active"]),
        _ptr(workspace), workspace.numel(), _stream()))
    return out


def moe_route_permute(logits: torch.Tensor, top_k: int, workspace: torch.Tensor | None = None,
                      out_ids=None, out_weights=None, out: dict | None = None):
    """moe_route then moe_permute in one call (one launch for small T): (ids, weights, perm dict)."""
    lib = load_library()
    T, E = logits.shape
    dev = logits.device
    S = T * top_k
    ids = out_ids if out_ids is not None else torch.empty((T, top_k), dtype=torch.int32, device=dev)
    w = out_weights if out_weights is not None else torch.empty((T, top_k), dtype=torch.float32, device=dev)
    if out is None:
        out = {
            "expert_offsets": torch.empty(E + 1, dtype=torch.int32, device=dev),
            "sorted_slots": torch.empty(S, dtype=torch.int32, device=dev),
            "slot_rows": torch.empty(S, dtype=torch.int32, device=dev),
            "active_experts": torch.empty(E, dtype=torch.int32, device=dev),
            "num_active": torch.empty(1, dtype=torch.int32, device=dev),
        }
    need = permute_workspace_bytes(T, top_k, E)
    if workspace is None:
        workspace = _workspace(need, dev)
    _check("moe_route_permute", lib.moe_route_permute(
        _ptr(logits), T, E, top_k, _ptr(ids), _ptr(w), _ptr(out["expert_offsets"]),
        _ptr(out["sorted_slots"]), _ptr(out["slot_rows"]), _ptr(out["active_experts"]),
        _ptr(out["num_active"]), _ptr(workspace), workspace.numel(), _stream()))
    return ids, w, out


def _ffn_ws(T, k, E, H, I, workspace, dev):
    need = ffn_workspace_bytes(T, k, E, H, I)
    if workspace is None:
        workspace = _workspace(need, dev)
    return workspace


def moe_w4a16_grouped_ffn(x: torch.Tensor, top_k: int, perm: dict, w: dict,
                          y_sorted: torch.Tensor | None = None,
                          workspace: torch.Tensor | None = None) -> torch.Tensor:
    """x fp16 [T, H] -> y_sorted fp32 [T*k, H] (sorted-row order)."""
    lib = load_library()
    T, H = x.shape
    E = w["w13_q"].shape[0]
    I = w["w2_q"].shape[2] * 8
    dev = x.device
    if y_sorted is None:
        y_sorted = torch.empty((T * top_k, H), dtype=torch.float32, device=dev)
    workspace = _ffn_ws(T, top_k, E, H, I, workspace, dev)
    _check("moe_w4a16_grouped_ffn", lib.moe_w4a16_grouped_ffn(
        _ptr(x), T, top_k, _ptr(perm["expert_offsets"]), _ptr(perm["sorted_slots"]),
        _ptr(perm["active_experts"]), _ptr(perm["num_active"]),
        _ptr(w["w13_q"]), _ptr(w["w13_s"]), _ptr(w["w13_z"]),
        _ptr(w["w2_q"]), _ptr(w["w2_s"]), _ptr(w["w2_z"]),
        E, H, I, GROUP_SIZE, _ptr(y_sorted), _ptr(workspace), workspace.numel(), _stream()))
    return y_sorted


def moe_w4a16_gate_up(x: torch.Tensor, top_k: int, perm: dict, w: dict,
                      workspace: torch.Tensor) -> None:
    lib = load_library()
    T, H = x.shape
    E = w["w13_q"].shape[0]
    I = w["w2_q"].shape[2] * 8
    _check("moe_w4a16_gate_up", lib.moe_w4a16_gate_up(
        _ptr(x), T, top_k, _ptr(perm["expert_offsets"]), _ptr(perm["sorted_slots"]),
        _ptr(perm["active_experts"]), _ptr(perm["num_active"]),
        _ptr(w["w13_q"]), _ptr(w["w13_s"]), _ptr(w["w13_z"]),
        E, H, I, GROUP_SIZE, _ptr(workspace), workspace.numel(), _stream()))


def moe_w4a16_down(T: int, top_k: int, perm: dict, w: dict, y_sorted: torch.Tensor,
                   workspace: torch.Tensor) -> None:
    lib = load_library()
    E, H = w["w2_q"].shape[0], w["w2_q"].shape[1]
    I = w["w2_q"].shape[2] * 8
    _check("moe_w4a16_down", lib.moe_w4a16_down(
        T, top_k, _ptr(perm["expert_offsets"]), _ptr(perm["active_experts"]),
        _ptr(perm["num_active"]), _ptr(w["w2_q"]), _ptr(w["w2_s"]), _ptr(w["w2_z"]),
        E, H, I, GROUP_SIZE, _ptr(y_sorted), _ptr(workspace), workspace.numel(), _stream()))


def moe_route_gate_up(logits: torch.Tensor, x: torch.Tensor, top_k: int, w: dict,
                      ids: torch.Tensor, weights: torch.Tensor, perm: dict,
                      workspace: torch.Tensor) -> None:
    """Decode sizes (T <= 8): router, permutation and gate/up in one launch; the routing
    goes to ids, weights and perm (as moe_route_permute), act to the FFN workspace."""
    lib = load_library()
    T, E = logits.shape
    H = x.shape[1]
    I = w["w13_q"].shape[1] // 2
    _check("moe_route_gate_up", lib.moe_route_gate_up(
        _ptr(logits), _ptr(x), T, E, top_k, _ptr(w["w13_q"]), _ptr(w["w13_s"]), _ptr(w["w13_z"]),
        H, I, GROUP_SIZE, _ptr(ids), _ptr(weights), _ptr(perm["expert_offsets"]),
        _ptr(perm["sorted_slots"]), _ptr(perm["slot_rows"]), _ptr(perm["active_experts"]),
        _ptr(perm["num_active"]), _ptr(workspace), workspace.numel(), _stream()))


def moe_combine(y_sorted: torch.Tensor, topk_weights: torch.Tensor, slot_rows: torch.Tensor,
                out: torch.Tensor | None = None) -> torch.Tensor:
    """y_sorted fp32 [T*k, H] -> out fp16 [T, H]."""
    lib = load_library()
    T, k = topk_weights.shape
    H = y_sorted.shape[1]
    if out is None:
        out = torch.empty((T, H), dtype=torch.float16, device=y_sorted.device)
    _check("moe_combine", lib.moe_combine(
        _ptr(y_sorted), _ptr(topk_weights), _ptr(slot_rows), T, k, H, _ptr(out), _stream()))
    return out


def layer_workspace_bytes(T: int, top_k: int, E: int, H: int, I: int) -> int:
    return int(load_library().moe_layer_workspace_bytes(T, top_k, E, H, I))


def layer_workspace_views(ws: torch.Tensor, T: int, top_k: int, E: int, H: int, I: int) -> dict:
    """The routing and y_sorted inside a moe_layer_forward workspace (layout of the header)."""
    S = T * top_k

    def a256(n):
        return (n + 255) & ~255

    sizes = [("topk_ids", 4 * S), ("topk_weights", 4 * S), ("expert_offsets", 4 * (E + 1)),
             ("sorted_slots", 4 * S), ("slot_rows", 4 * S), ("active_experts", 4 * E),
             ("num_active", 4), ("perm_ws", permute_workspace_bytes(T, top_k, E)),
             ("ffn_ws", ffn_workspace_bytes(T, top_k, E, H, I)), ("y_sorted", 4 * S * H)]
    views, at = {}, 0
    for name, n in sizes:
        views[name] = ws[at:at + n]
        at += a256(n)
    out = {k: views[k].view(torch.int32) for k in ("topk_ids", "sorted_slots", "slot_rows",
                                                   "expert_offsets", "active_experts", "num_active")}
    out["topk_ids"] = out["topk_ids"].view(T, top_k)
    out["topk_weights"] = views["topk_weights"].view(torch.float32).view(T, top_k)
    out["y_sorted"] = views["y_sorted"].view(torch.float32).view(S, H)
    return out


def moe_layer_forward(logits: torch.Tensor, x: torch.Tensor, top_k: int, w: dict,
                      workspace: torch.Tensor | None = None, out: torch.Tensor | None = None):
    """The whole layer in one call: logits fp32 [T, E], x fp16 [T, H] -> out fp16 [T, H]."""
    lib = load_library()
    T, E = logits.shape
    H = x.shape[1]
    I = w["w2_q"].shape[2] * 8
    dev = x.device
    if workspace is None:
        workspace = _workspace(layer_workspace_bytes(T, top_k, E, H, I), dev)
    if out is None:
        out = torch.empty((T, H), dtype=torch.float16, device=dev)
    _check("moe_layer_forward", lib.moe_layer_forward(
        _ptr(logits), _ptr(x), T, E, top_k, _ptr(w["w13_q"]), _ptr(w["w13_s"]), _ptr(w["w13_z"]),
        _ptr(w["w2_q"]), _ptr(w["w2_s"]), _ptr(w["w2_z"]), H, I, GROUP_SIZE, _ptr(out),
        _ptr(workspace), workspace.numel(), _stream()))
    return out


def moe_layer_forward_noalloc(logits: torch.Tensor, x: torch.Tensor, top_k: int, w: dict,
                              out: torch.Tensor) -> torch.Tensor:
    """moe_layer_forward without a workspace: the library's per-device scratch is used.
    `out` fp16 [T, H] is the caller's (this call allocates nothing)."""
    lib = load_library()
    T, E = logits.shape
    H = x.shape[1]
    I = w["w2_q"].shape[2] * 8
    _check("moe_layer_forward_noalloc", lib.moe_layer_forward_noalloc(
        _ptr(logits), _ptr(x), T, E, top_k, _ptr(w["w13_q"]), _ptr(w["w13_s"]), _ptr(w["w13_z"]),
        _ptr(w["w2_q"]), _ptr(w["w2_s"]), _ptr(w["w2_z"]), H, I, GROUP_SIZE, _ptr(out), _stream()))
    return out


# --------------------------------------------------------------------------- #
# the MoE block: router gate projection, shared expert
# --------------------------------------------------------------------------- #
def moe_router_gate(x: torch.Tensor, gate_weight: torch.Tensor, out: torch.Tensor | None = None):
    """fp16 x [T, H], fp16 gate_weight [E, H] -> fp32 logits [T, E]."""
    lib = load_library()
    T, H = x.shape
    E = gate_weight.shape[0]
    if out is None:
        out = torch.empty((T, E), dtype=torch.float32, device=x.device)
    _check("moe_router_gate", lib.moe_router_gate(_ptr(x), T, H, _ptr(gate_weight), E, _ptr(out),
                                                  _stream()))
    return out


def moe_route_shared(logits: torch.Tensor, top_k: int):
    """fp32 logits [T, E] -> (ids int32 [T, k+1], weights fp32 [T, k+1]); column k is the
    shared expert E with weight 1."""
    lib = load_library()
    T, E = logits.shape
    dev = logits.device
    ids = torch.empty((T, top_k + 1), dtype=torch.int32, device=dev)
    w = torch.empty((T, top_k + 1), dtype=torch.float32, device=dev)
    _check("moe_route_shared", lib.moe_route_shared(_ptr(logits), T, E, top_k, _ptr(ids), _ptr(w),
                                                    _stream()))
    return ids, w


def block_workspace_bytes(T: int, top_k: int, E: int, shared: bool, H: int, I: int) -> int:
    return int(load_library().moe_block_workspace_bytes(T, top_k, E, int(shared), H, I))


def moe_block_forward(x: torch.Tensor, gate_weight: torch.Tensor, top_k: int, w: dict,
                      shared: bool = True, workspace: torch.Tensor | None = None,
                      logits: torch.Tensor | None = None, out: torch.Tensor | None = None):
    """The MoE block: projection, routed layer and (when ``shared``) the shared expert,
    stored as expert E of the weight arrays.  Returns (out fp16 [T, H], logits fp32 [T, E])."""
    lib = load_library()
    T, H = x.shape
    E = gate_weight.shape[0]
    I = w["w2_q"].shape[2] * 8
    dev = x.device
    if workspace is None:
        workspace = _workspace(block_workspace_bytes(T, top_k, E, shared, H, I), dev)
    if logits is None:
        logits = torch.empty((T, E), dtype=torch.float32, device=dev)
    if out is None:
        out = torch.empty((T, H), dtype=torch.float16, device=dev)
    _check("moe_block_forward", lib.moe_block_forward(
        _ptr(x), T, _ptr(gate_weight), E, top_k, int(shared), _ptr(w["w13_q"]), _ptr(w["w13_s"]),
        _ptr(w["w13_z"]), _ptr(w["w2_q"]), _ptr(w["w2_s"]), _ptr(w["w2_z"]), H, I, GROUP_SIZE,
        _ptr(logits), _ptr(out), _ptr(workspace), workspace.numel(), _stream()))
    return out, logits


def plan_default(T: int, top_k: int, E: int, H: int, I: int, shared: bool = False) -> Plan:
    """The plan the library uses for these sizes (routed top_k and E; `shared`: a shared expert)."""
    p = Plan()
    _check("moe_plan_default", load_library().moe_plan_default(T, top_k, E, int(shared), H, I,
                                                               ctypes.addressof(p)))
    return p


def _plan_ptr(plan):
    return None if plan is None else ctypes.addressof(plan)


def moe_layer_forward_plan(logits: torch.Tensor, x: torch.Tensor, top_k: int, w: dict,
                           plan: Plan | None, workspace: torch.Tensor | None = None,
                           out: torch.Tensor | None = None):
    """moe_layer_forward with an explicit plan (None: the default)."""
    lib = load_library()
    T, E = logits.shape
    H = x.shape[1]
    I = w["w2_q"].shape[2] * 8
    dev = x.device
    if workspace is None:
        workspace = _workspace(layer_workspace_bytes(T, top_k, E, H, I), dev)
    if out is None:
        out = torch.empty((T, H), dtype=torch.float16, device=dev)
    _check("moe_layer_forward_plan", lib.moe_layer_forward_plan(
        _ptr(logits), _ptr(x), T, E, top_k, _ptr(w["w13_q"]), _ptr(w["w13_s"]), _ptr(w["w13_z"]),
        _ptr(w["w2_q"]), _ptr(w["w2_s"]), _ptr(w["w2_z"]), H, I, GROUP_SIZE, _ptr(out),
        _ptr(workspace), workspace.numel(), _plan_ptr(plan), _stream()))
    return out


def moe_block_forward_plan(x: torch.Tensor, gate_weight: torch.Tensor, top_k: int, w: dict,
                           shared: bool, plan: Plan | None, workspace: torch.Tensor,
                           logits: torch.Tensor, out: torch.Tensor):
    """moe_block_forward with an explicit plan (None: the default)."""
    lib = load_library()
    T, H = x.shape
    E = gate_weight.shape[0]
    I = w["w2_q"].shape[2] * 8
    _check("moe_block_forward_plan", lib.moe_block_forward_plan(
        _ptr(x), T, _ptr(gate_weight), E, top_k, int(shared), _ptr(w["w13_q"]), _ptr(w["w13_s"]),
        _ptr(w["w13_z"]), _ptr(w["w2_q"]), _ptr(w["w2_s"]), _ptr(w["w2_z"]), H, I, GROUP_SIZE,
        _ptr(logits), _ptr(out), _ptr(workspace), workspace.numel(), _plan_ptr(plan), _stream()))
    return out


class MoEBlock:
    """Device-resident buffers for repeated block calls at one size (graph-capturable):
    the projection, the routed experts and the shared expert in one entry point."""

    def __init__(self, T: int, E: int, top_k: int, H: int, I: int, shared: bool = True,
                 device="cuda"):
        self.T, self.E, self.top_k, self.H, self.I, self.shared = T, E, top_k, H, I, shared
        dev = torch.device(device)
        self.ws = _workspace(block_workspace_bytes(T, top_k, E, shared, H, I), dev)
        self.logits = torch.empty((T, E), dtype=torch.float32, device=dev)
        self.out = torch.empty((T, H), dtype=torch.float16, device=dev)

    def __call__(self, x: torch.Tensor, gate_weight: torch.Tensor, w: dict) -> torch.Tensor:
        moe_block_forward(x, gate_weight, self.top_k, w, self.shared, self.ws, self.logits,
                          self.out)
        return self.out

    def views(self) -> dict:
        k, E = self.top_k + int(self.shared), self.E + int(self.shared)
        return layer_workspace_views(self.ws, self.T, k, E, self.H, self.I)


# --------------------------------------------------------------------------- #
# one whole layer call
# --------------------------------------------------------------------------- #
class MoELayer:
    """Device-resident buffers for repeated layer calls at one size (graph-capturable)."""

    def __init__(self, T: int, E: int, top_k: int, H: int, I: int, device="cuda"):
        self.T, self.E, self.top_k, self.H, self.I = T, E, top_k, H, I
        S = T * top_k
        dev = torch.device(device)
        self.ids = torch.empty((T, top_k), dtype=torch.int32, device=dev)
        self.weights = torch.empty((T, top_k), dtype=torch.float32, device=dev)
        self.perm = {
            "expert_offsets": torch.empty(E + 1, dtype=torch.int32, device=dev),
            "sorted_slots": torch.empty(S, dtype=torch.int32, device=dev),
            "slot_rows": torch.empty(S, dtype=torch.int32, device=dev),
            "active_experts": torch.empty(E, dtype=torch.int32, device=dev),
            "num_active": torch.empty(1, dtype=torch.int32, device=dev),
        }
        self.perm_ws = _workspace(permute_workspace_bytes(T, top_k, E), dev)
        self.ffn_ws = _workspace(ffn_workspace_bytes(T, top_k, E, H, I), dev)
        self.y_sorted = torch.empty((S, H), dtype=torch.float32, device=dev)
        self.out = torch.empty((T, H), dtype=torch.float16, device=dev)
        self.layer_ws = _workspace(layer_workspace_bytes(T, top_k, E, H, I), dev)
        self.fused_out = torch.empty((T, H), dtype=torch.float16, device=dev)

    def __call__(self, logits: torch.Tensor, x: torch.Tensor, w: dict) -> torch.Tensor:
        moe_route_permute(logits, self.top_k, self.perm_ws, self.ids, self.weights, self.perm)
        moe_w4a16_grouped_ffn(x, self.top_k, self.perm, w, self.y_sorted, self.ffn_ws)
        moe_combine(self.y_sorted, self.weights, self.perm["slot_rows"], self.out)
        return self.out

    def forward(self, logits: torch.Tensor, x: torch.Tensor, w: dict) -> torch.Tensor:
        """The same layer through moe_layer_forward (one call; routing kept in layer_ws)."""
        return moe_layer_forward(logits, x, self.top_k, w, self.layer_ws, self.fused_out)

    def forward_views(self) -> dict:
        return layer_workspace_views(self.layer_ws, self.T, self.top_k, self.E, self.H, self.I)


def weights_to_device(host: dict, device="cuda") -> dict:
    """numpy weight arrays -> device tensors (int32 and fp16 bit-compatible dtypes)."""
    out = {}
    for key in ("w13_q", "w13_z", "w2_q", "w2_z"):
        out[key] = torch.from_numpy(host[key]).to(device)
    for key in ("w13_s", "w2_s"):
        out[key] = torch.from_numpy(host[key]).to(device)
    return out
