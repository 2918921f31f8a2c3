"""CPU-only checks of the C ABI: the library loads, exports every symbol the
header declares, sizes workspaces, and rejects bad arguments before touching
the GPU (no compute call is made here).  The library is built first when it
is missing."""

import ctypes
import os
import re

import pytest

from w4a16_group_quantized_amd import ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_w4a16.h")



@pytest.fixture(scope="module", autouse=True)
def _built_library():
    """The library under test: built here with hipcc when it is missing (a
    failed build fails these tests instead of skipping them)."""
    if not os.path.exists(ops.LIB_PATH):
        from w4a16_group_quantized_amd import build_lib

        build_lib.build()
    assert os.path.exists(ops.LIB_PATH)


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_four_layer_calls():
    names = _declared_functions()
    for fn in ("moe_route", "moe_permute", "moe_w4a16_grouped_ffn", "moe_combine"):
        assert fn in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(ops.LIB_PATH)
    missing = [n for n in _declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    assert set(_declared_functions()) == set(ops.EXPORTED)


def test_status_strings_and_version():
    lib = ops.load_library()
    assert lib.moe_abi_version() == 102
    for st in range(5):
        assert len(ops.status_string(st)) > 0
    assert ops.status_string(99) == "unknown status"


def test_workspace_queries():
    assert ops.permute_workspace_bytes(64, 10, 512) == 0  # one workgroup, no scratch
    assert ops.permute_workspace_bytes(65, 10, 512) > 0
    assert ops.permute_workspace_bytes(4096, 10, 512) >= 64 * 512 * 12
    a = ops.ffn_workspace_bytes(8, 10, 512, 2560, 640)
    b = ops.ffn_workspace_bytes(4096, 10, 512, 2560, 640)
    assert a >= 2 * 80 * 640 * 2 and b >= 2 * 40960 * 640 * 2 and b > a
    # invalid sizes report 0
    assert ops.ffn_workspace_bytes(8, 10, 512, 2561, 640) == 0
    assert ops.permute_workspace_bytes(8, 0, 512) == 0


FAKE = 0x1000  # an aligned non-null value; never dereferenced because validation fails first


def test_route_rejects_bad_arguments():
    lib = ops.load_library()
    assert lib.moe_route(None, 4, 8, 2, None, None, None) == ops.MOE_ERR_INVALID_ARG
    assert lib.moe_route(FAKE, -1, 8, 2, FAKE, FAKE, None) == ops.MOE_ERR_INVALID_ARG
    assert lib.moe_route(FAKE, 4, 8, 9, FAKE, FAKE, None) == ops.MOE_ERR_INVALID_ARG
    assert lib.moe_route(FAKE, 4, 8, 0, FAKE, FAKE, None) == ops.MOE_ERR_INVALID_ARG
    assert lib.moe_route(FAKE, 4, 0, 1, FAKE, FAKE, None) == ops.MOE_ERR_INVALID_ARG
    assert lib.moe_route(FAKE, 4, 5000, 2, FAKE, FAKE, None) == ops.MOE_ERR_UNSUPPORTED
    assert lib.moe_route(FAKE, 4, 512, 65, FAKE, FAKE, None) == ops.MOE_ERR_UNSUPPORTED
    assert lib.moe_route(FAKE + 4, 4, 8, 2, FAKE, FAKE, None) == ops.MOE_ERR_INVALID_ARG  # misaligned
    assert lib.moe_route(None, 0, 8, 2, None, None, None) == ops.MOE_OK  # T = 0: nothing to do
    assert lib.moe_route(FAKE, 1 << 28, 512, 10, FAKE, FAKE, None) == ops.MOE_ERR_UNSUPPORTED


def test_permute_rejects_bad_arguments():
    lib = ops.load_library()
    args = [FAKE] * 6
    assert lib.moe_permute(FAKE, 100, 10, 512, *args[:5], None, 0, None) == ops.MOE_ERR_WORKSPACE
    assert lib.moe_permute(FAKE, 100, 10, 512, FAKE, None, FAKE, FAKE, FAKE, FAKE, 1 << 30,
                           None) == ops.MOE_ERR_INVALID_ARG
    assert lib.moe_permute(None, 0, 10, 512, None, None, None, None, None, None, 0, None) == ops.MOE_OK


def _ffn(lib, T=8, k=10, E=512, H=2560, I=640, gs=32, ws_bytes=1 << 30, y=FAKE, x=FAKE):
    p = [FAKE] * 10
    return lib.moe_w4a16_grouped_ffn(x, T, k, *p[:4], *p[4:10], E, H, I, gs, y, FAKE, ws_bytes, None)


def test_ffn_rejects_bad_arguments():
    lib = ops.load_library()
    assert _ffn(lib, gs=64) == ops.MOE_ERR_UNSUPPORTED
    assert _ffn(lib, gs=128) == ops.MOE_ERR_UNSUPPORTED
    assert _ffn(lib, H=2570) == ops.MOE_ERR_INVALID_ARG
    assert _ffn(lib, I=650) == ops.MOE_ERR_INVALID_ARG
    assert _ffn(lib, H=32768) == ops.MOE_ERR_UNSUPPORTED
    assert _ffn(lib, ws_bytes=16) == ops.MOE_ERR_WORKSPACE
    assert _ffn(lib, y=None) == ops.MOE_ERR_INVALID_ARG
    assert _ffn(lib, x=FAKE + 8) == ops.MOE_ERR_INVALID_ARG
    assert _ffn(lib, T=0, x=None, y=None) == ops.MOE_OK
    assert _ffn(lib, k=11, E=10) == ops.MOE_ERR_INVALID_ARG
    # x is addressed with 32-bit byte offsets: T * H < 2^31
    assert _ffn(lib, T=(1 << 31) // 2560 + 1, k=1) == ops.MOE_ERR_UNSUPPORTED


def test_gate_up_and_down_reject_bad_arguments():
    lib = ops.load_library()
    p = [FAKE] * 8
    assert lib.moe_w4a16_gate_up(FAKE, 8, 10, *p[:7], 512, 2560, 640, 16, FAKE, 1 << 30,
                                 None) == ops.MOE_ERR_UNSUPPORTED
    assert lib.moe_w4a16_gate_up(FAKE, 8, 10, *p[:7], 512, 2560, 640, 32, None, 1 << 30,
                                 None) == ops.MOE_ERR_INVALID_ARG
    assert lib.moe_w4a16_down(8, 10, *p[:6], 512, 2560, 640, 32, FAKE, FAKE, 8,
                              None) == ops.MOE_ERR_WORKSPACE


def test_route_gate_up_rejects_bad_arguments():
    lib = ops.load_library()
    p = [FAKE] * 8

    def call(T=8, E=512, k=10, H=2560, I=640, gs=32, ws_bytes=1 << 30, logits=FAKE):
        return lib.moe_route_gate_up(logits, FAKE, T, E, k, FAKE, FAKE, FAKE, H, I, gs, *p[:7],
                                     FAKE, ws_bytes, None)

    assert call(T=65) == ops.MOE_ERR_UNSUPPORTED       # 64-token routing masks
    assert call(T=9, ws_bytes=64) == ops.MOE_ERR_WORKSPACE  # 9..64 tokens are allowed
    assert call(E=1025) == ops.MOE_ERR_UNSUPPORTED
    assert call(gs=64) == ops.MOE_ERR_UNSUPPORTED
    assert call(ws_bytes=64) == ops.MOE_ERR_WORKSPACE
    assert call(logits=None) == ops.MOE_ERR_INVALID_ARG
    assert call(T=0, logits=None) == ops.MOE_OK


def test_combine_rejects_bad_arguments():
    lib = ops.load_library()
    assert lib.moe_combine(FAKE, FAKE, FAKE, 8, 10, 2561, FAKE, None) == ops.MOE_ERR_INVALID_ARG
    assert lib.moe_combine(FAKE, FAKE, None, 8, 10, 2560, FAKE, None) == ops.MOE_ERR_INVALID_ARG
    assert lib.moe_combine(FAKE, FAKE, FAKE, 8, 0, 2560, FAKE, None) == ops.MOE_ERR_INVALID_ARG
    assert lib.moe_combine(None, None, None, 0, 10, 2560, None, None) == ops.MOE_OK


def test_router_gate_rejects_bad_arguments():
    lib = ops.load_library()
    assert lib.moe_router_gate(FAKE, 8, 2570, FAKE, 512, FAKE, None) == ops.MOE_ERR_INVALID_ARG
    assert lib.moe_router_gate(FAKE, 8, 2560, FAKE, 0, FAKE, None) == ops.MOE_ERR_INVALID_ARG
    assert lib.moe_router_gate(FAKE, -1, 2560, FAKE, 512, FAKE, None) == ops.MOE_ERR_INVALID_ARG
    assert lib.moe_router_gate(FAKE, 8, 2560, FAKE, 5000, FAKE, None) == ops.MOE_ERR_UNSUPPORTED
    assert lib.moe_router_gate(FAKE, 8, 32768, FAKE, 512, FAKE, None) == ops.MOE_ERR_UNSUPPORTED
    # x is addressed with 32-bit byte offsets: T * H < 2^31
    assert lib.moe_router_gate(FAKE, (1 << 31) // 2560 + 1, 2560, FAKE, 512, FAKE,
                               None) == ops.MOE_ERR_UNSUPPORTED
    assert lib.moe_router_gate(None, 8, 2560, FAKE, 512, FAKE, None) == ops.MOE_ERR_INVALID_ARG
    assert lib.moe_router_gate(FAKE, 8, 2560, FAKE + 2, 512, FAKE, None) == ops.MOE_ERR_INVALID_ARG
    assert lib.moe_router_gate(FAKE, 8, 2560, FAKE, 512, None, None) == ops.MOE_ERR_INVALID_ARG
    assert lib.moe_router_gate(None, 0, 2560, None, 512, None, None) == ops.MOE_OK


def test_route_shared_rejects_bad_arguments():
    lib = ops.load_library()
    # the shared expert takes one more slot and one more expert id
    assert lib.moe_route_shared(FAKE, 4, 512, 64, FAKE, FAKE, None) == ops.MOE_ERR_UNSUPPORTED
    assert lib.moe_route_shared(FAKE, 4, 512, 63, None, FAKE, None) == ops.MOE_ERR_INVALID_ARG
    assert lib.moe_route_shared(FAKE, 4, 4096, 8, FAKE, FAKE, None) == ops.MOE_ERR_UNSUPPORTED
    assert lib.moe_route_shared(FAKE, 4, 8, 9, FAKE, FAKE, None) == ops.MOE_ERR_INVALID_ARG
    assert lib.moe_route_shared(None, 0, 8, 2, None, None, None) == ops.MOE_OK


def _block(lib, T=8, k=10, E=512, shared=1, H=2560, I=640, gs=32, ws_bytes=1 << 30,
           gate=FAKE, logits=FAKE):
    p = [FAKE] * 6
    return lib.moe_block_forward(FAKE, T, gate, E, k, shared, *p, H, I, gs, logits, FAKE, FAKE,
                                 ws_bytes, None)


def test_block_rejects_bad_arguments():
    lib = ops.load_library()
    assert _block(lib, shared=2) == ops.MOE_ERR_INVALID_ARG
    assert _block(lib, gs=64) == ops.MOE_ERR_UNSUPPORTED
    assert _block(lib, H=2570) == ops.MOE_ERR_INVALID_ARG
    assert _block(lib, ws_bytes=64) == ops.MOE_ERR_WORKSPACE
    assert _block(lib, gate=None) == ops.MOE_ERR_INVALID_ARG
    assert _block(lib, logits=FAKE + 4) == ops.MOE_ERR_INVALID_ARG
    assert _block(lib, k=64) == ops.MOE_ERR_UNSUPPORTED      # top_k + 1 slots > 64
    assert _block(lib, T=0) == ops.MOE_OK
    need1 = ops.block_workspace_bytes(8, 10, 512, True, 2560, 640)
    need0 = ops.block_workspace_bytes(8, 10, 512, False, 2560, 640)
    assert need0 == ops.layer_workspace_bytes(8, 10, 512, 2560, 640)
    assert need1 == ops.layer_workspace_bytes(8, 11, 513, 2560, 640) and need1 > need0
    assert _block(lib, ws_bytes=need1 - 1) == ops.MOE_ERR_WORKSPACE
    assert lib.moe_block_workspace_bytes(8, 10, 512, 2, 2560, 640) == 0
    assert lib.moe_block_workspace_bytes(8, 64, 512, 1, 2560, 640) == 0


def test_binding_refuses_to_run_without_library(tmp_path, monkeypatch):
    monkeypatch.setattr(ops, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        ops.load_library(str(tmp_path / "nope.so"))


def test_route_permute_rejects_bad_arguments():
    lib = ops.load_library()
    out = [FAKE] * 7
    assert lib.moe_route_permute(None, 4, 8, 2, *out, None, 0, None) == ops.MOE_ERR_INVALID_ARG
    assert lib.moe_route_permute(FAKE, 4, 8, 9, *out, None, 0, None) == ops.MOE_ERR_INVALID_ARG
    assert lib.moe_route_permute(FAKE, 4, 5000, 2, *out, None, 0, None) == ops.MOE_ERR_UNSUPPORTED
    # more than 64 tokens need the permutation workspace
    assert lib.moe_route_permute(FAKE, 100, 512, 10, *out, FAKE, 0, None) == ops.MOE_ERR_WORKSPACE
    assert lib.moe_route_permute(None, 0, 8, 2, *([None] * 7), None, 0, None) == ops.MOE_OK


def _layer(lib, T=8, E=512, k=10, H=2560, I=640, gs=32, ws_bytes=None, logits=FAKE, out=FAKE):
    need = ops.layer_workspace_bytes(T, k, E, H, I) if ws_bytes is None else ws_bytes
    w = [FAKE] * 6
    return lib.moe_layer_forward(logits, FAKE, T, E, k, *w, H, I, gs, out, FAKE, need, None)


def test_layer_workspace_and_arguments():
    lib = ops.load_library()
    need = ops.layer_workspace_bytes(8, 10, 512, 2560, 640)
    # routing, the FFN workspace and y_sorted [S, H] fp32 all live in it
    assert need >= ops.ffn_workspace_bytes(8, 10, 512, 2560, 640) + 80 * 2560 * 4
    assert ops.layer_workspace_bytes(8, 10, 512, 2561, 640) == 0
    assert _layer(lib, gs=64) == ops.MOE_ERR_UNSUPPORTED
    assert _layer(lib, H=2561) == ops.MOE_ERR_INVALID_ARG
    assert _layer(lib, k=0) == ops.MOE_ERR_INVALID_ARG
    assert _layer(lib, logits=None) == ops.MOE_ERR_INVALID_ARG
    assert _layer(lib, out=FAKE + 2) == ops.MOE_ERR_INVALID_ARG
    assert _layer(lib, ws_bytes=need - 1) == ops.MOE_ERR_WORKSPACE
    assert _layer(lib, T=0) == ops.MOE_OK
    assert _layer(lib, T=(1 << 31) // 2560 + 1, k=1) == ops.MOE_ERR_UNSUPPORTED
