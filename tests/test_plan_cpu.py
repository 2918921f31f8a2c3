"""The per-shape plan table (moe_plan_default) at every boundary, and the
rejection of plans the sizes do not allow, through the C ABI on the CPU (no
compute call is made)."""

import pytest

from w4a16_group_quantized_amd import ops

FAKE = 0x1000  # aligned, never dereferenced: validation fails or nothing is launched


@pytest.fixture(scope="module", autouse=True)
def _built_library():
    import os

    if not os.path.exists(ops.LIB_PATH):
        from w4a16_group_quantized_amd import build_lib

        build_lib.build()


def plan(T, k=10, E=512, H=2560, I=640, shared=False):
    return ops.plan_default(T, k, E, H, I, shared).as_dict()


def test_gemv_up_to_32_tokens_then_matrix_cores():
    assert plan(1)["ffn"] == ops.FFN_GEMV and plan(32)["ffn"] == ops.FFN_GEMV
    assert plan(33)["ffn"] == ops.FFN_MFMA and plan(4096)["ffn"] == ops.FFN_MFMA
    assert plan(32, I=160)["ffn"] == ops.FFN_GEMV


def test_routing_variant_boundaries():
    assert plan(1)["route"] == ops.ROUTE_IN_GATE_UP
    assert plan(32)["route"] == ops.ROUTE_IN_GATE_UP         # with the GEMV
    assert plan(33)["route"] == ops.ROUTE_SEPARATE           # matrix cores: two kernels
    assert plan(8, E=1024)["route"] == ops.ROUTE_IN_GATE_UP
    assert plan(8, E=1025)["route"] == ops.ROUTE_SEPARATE    # both one-launch forms stop at 1024
    assert plan(8, E=1025)["ffn"] == ops.FFN_GEMV
    # the standalone router + permutation call uses one launch up to 8 tokens
    assert plan(8, E=1025)["route"] != ops.ROUTE_ONE_LAUNCH
    assert plan(33, E=64)["route"] == ops.ROUTE_SEPARATE


def test_m_tile_switches_at_64_rows_per_expert():
    # S = T * k against 64 E = 32768 at E = 512, k = 10
    assert plan(3276)["msub"] == 1     # S = 32760
    assert plan(3277)["msub"] == 4     # S = 32770
    assert plan(64, k=2, E=2)["msub"] == 4   # S = 128 = 64 E
    assert plan(63, k=2, E=2)["msub"] == 1


def test_lanes_per_row_divide_the_groups():
    assert plan(8)["lanes_gate_up"] == 8     # H = 2560: 80 groups
    assert plan(5)["lanes_gate_up"] == 8
    assert plan(4)["lanes_gate_up"] == 16    # up to 4 tokens: 16 lanes where they divide
    assert plan(1, I=160)["lanes_gate_up"] == 16
    assert plan(4, H=2592)["lanes_gate_up"] == 1   # 81 groups
    assert plan(4, H=2624)["lanes_gate_up"] == 2   # 82 groups
    assert plan(8)["lanes_down"] == 4        # I = 640: 20 groups
    assert plan(8, I=160)["lanes_down"] == 1  # 5 groups
    assert plan(8, I=64)["lanes_down"] == 2   # 2 groups
    assert plan(8, H=96)["lanes_gate_up"] == 1


def test_router_projection_gemv_boundaries():
    assert plan(16)["router_gemv"] == 1      # x: 16 x 2560 x 2 = 80 KiB
    assert plan(17)["router_gemv"] == 0
    assert plan(2, H=16384)["router_gemv"] == 1   # 64 KiB
    assert plan(3, H=16384)["router_gemv"] == 0   # 96 KiB


def test_rows_per_pass_and_cost_split():
    assert plan(1)["rows_per_pass"] == 1 and plan(2)["rows_per_pass"] == 2
    assert plan(8)["rows_per_pass"] == 2 and plan(8)["cost_split"] == 0
    assert plan(9)["rows_per_pass"] == 2 and plan(9)["cost_split"] == 0
    assert plan(10)["rows_per_pass"] == 4 and plan(10)["cost_split"] == 1
    # a shared expert with the GEMV runs on the matrix cores in extra workgroups;
    # the GEMV's rows per pass and split then follow the routed experts
    assert plan(8, shared=True)["shared_mfma"] == 1 and plan(8, shared=True)["rows_per_pass"] == 2
    # from 3 tokens: with fewer the shared expert is one more expert of the GEMV
    assert plan(2, shared=True)["shared_mfma"] == 0 and plan(1, shared=True)["shared_mfma"] == 0
    assert plan(3, shared=True)["shared_mfma"] == 1
    assert plan(16, shared=True)["shared_mfma"] == 1
    # its A rows (T x H fp16) and the K-split partial sums share one
    # workgroup's LDS: 22 rows of 2560 fit, 23 do not
    assert plan(22, shared=True)["shared_mfma"] == 1
    assert plan(23, shared=True)["shared_mfma"] == 0
    # ... and then the matrix-core FFN takes the block (its rows one more M-tile)
    assert plan(22, shared=True)["ffn"] == ops.FFN_GEMV
    assert plan(23, shared=True)["ffn"] == ops.FFN_MFMA
    assert plan(23, shared=True)["route"] == ops.ROUTE_SEPARATE
    assert plan(32, shared=True)["ffn"] == ops.FFN_MFMA and plan(32)["ffn"] == ops.FFN_GEMV
    assert plan(2, shared=True)["ffn"] == ops.FFN_GEMV   # below 3 tokens the GEMV holds it
    assert plan(8, H=16384, shared=True)["shared_mfma"] == 0
    assert plan(33, shared=True)["shared_mfma"] == 0          # matrix-core FFN: in its tile list
    assert plan(8)["shared_mfma"] == 0
    # the shared expert counts for the one-launch routing limit and the M-tile switch
    assert plan(8, E=1024, shared=True)["route"] == ops.ROUTE_SEPARATE
    assert plan(8, E=1023, shared=True)["route"] == ops.ROUTE_IN_GATE_UP


def test_combine_inside_down_up_to_two_tokens():
    assert plan(1)["combine_in_down"] == 1 and plan(2)["combine_in_down"] == 1
    assert plan(3)["combine_in_down"] == 0 and plan(8)["combine_in_down"] == 0
    assert plan(1, I=160)["combine_in_down"] == 1
    assert plan(2, shared=True)["combine_in_down"] == 1   # the shared expert in the GEMV
    # more than 8 steps per lane (I = 16384 takes the matrix cores anyway) or no LDS room
    assert plan(1, I=4096)["combine_in_down"] == 0          # 128 groups / 8 lanes = 16 steps
    assert plan(33)["combine_in_down"] == 0


def test_plan_query_rejects_bad_sizes():
    p = ops.Plan()
    lib = ops.load_library()
    import ctypes

    a = ctypes.addressof(p)
    assert lib.moe_plan_default(8, 10, 512, 0, 2570, 640, a) == ops.MOE_ERR_INVALID_ARG
    assert lib.moe_plan_default(8, 11, 10, 0, 2560, 640, a) == ops.MOE_ERR_INVALID_ARG
    assert lib.moe_plan_default(8, 10, 512, 0, 2560, 640, None) == ops.MOE_ERR_INVALID_ARG
    assert lib.moe_plan_default(8, 10, 512, 2, 2560, 640, a) == ops.MOE_ERR_INVALID_ARG
    assert lib.moe_plan_default(8, 64, 512, 1, 2560, 640, a) == ops.MOE_ERR_UNSUPPORTED


def _layer(lib, d, T=8, E=512, k=10, H=2560, I=640, ws_bytes=1 << 40):
    p = ops.Plan()
    for key, v in d.items():
        setattr(p, key, v)
    ptrs = [FAKE] * 6
    import ctypes

    return lib.moe_layer_forward_plan(FAKE, FAKE, T, E, k, *ptrs, H, I, 32, FAKE, FAKE, ws_bytes,
                                      ctypes.addressof(p), None)


def test_layer_rejects_plans_the_sizes_do_not_allow():
    lib = ops.load_library()
    base = plan(8)
    assert _layer(lib, dict(base, msub=2)) == ops.MOE_ERR_INVALID_ARG
    assert _layer(lib, dict(base, lanes_gate_up=3)) == ops.MOE_ERR_INVALID_ARG
    assert _layer(lib, dict(base, lanes_down=8)) == ops.MOE_ERR_INVALID_ARG   # 20 groups
    assert _layer(lib, dict(base, lanes_down=16)) == ops.MOE_ERR_INVALID_ARG  # 20 groups
    assert _layer(lib, dict(base, lanes_gate_up=32)) == ops.MOE_ERR_INVALID_ARG
    assert _layer(lib, dict(base, ffn=2)) == ops.MOE_ERR_INVALID_ARG
    assert _layer(lib, dict(base, route=3)) == ops.MOE_ERR_INVALID_ARG
    assert _layer(lib, dict(base, rows_per_pass=3)) == ops.MOE_ERR_INVALID_ARG
    assert _layer(lib, dict(base, cost_split=2)) == ops.MOE_ERR_INVALID_ARG
    assert _layer(lib, dict(base, shared_mfma=1)) == ops.MOE_ERR_INVALID_ARG   # no shared expert
    assert _layer(lib, dict(base, combine_in_down=2)) == ops.MOE_ERR_INVALID_ARG
    assert _layer(lib, dict(base, combine_in_down=1)) == ops.MOE_ERR_UNSUPPORTED  # 8 tokens
    assert _layer(lib, dict(plan(2), combine_in_down=1, ffn=ops.FFN_MFMA,
                            route=ops.ROUTE_ONE_LAUNCH), T=2) == ops.MOE_ERR_UNSUPPORTED
    assert _layer(lib, dict(base, ffn=ops.FFN_MFMA)) == ops.MOE_ERR_UNSUPPORTED  # routing in gate/up
    big = plan(65)
    assert _layer(lib, dict(big, ffn=ops.FFN_GEMV), T=65) == ops.MOE_ERR_UNSUPPORTED
    assert _layer(lib, dict(big, route=ops.ROUTE_ONE_LAUNCH), T=65) == ops.MOE_ERR_UNSUPPORTED
    assert _layer(lib, dict(plan(33), route=ops.ROUTE_ONE_LAUNCH), T=33) != ops.MOE_ERR_UNSUPPORTED
    assert _layer(lib, dict(plan(8, E=1025), route=ops.ROUTE_IN_GATE_UP), E=1025) == \
        ops.MOE_ERR_UNSUPPORTED
    assert _layer(lib, dict(plan(17), router_gemv=1), T=17) == ops.MOE_ERR_UNSUPPORTED


def _block(lib, d, T=8, E=512, k=10, H=2560, I=640, shared=1):
    p = ops.Plan()
    for key, v in d.items():
        setattr(p, key, v)
    import ctypes

    return lib.moe_block_forward_plan(FAKE, T, FAKE, E, k, shared, *([FAKE] * 6), H, I, 32, FAKE,
                                      FAKE, FAKE, 1 << 40, ctypes.addressof(p), None)


def test_one_launch_ffn_limits():
    """The one-launch FFN is never a default (slower than two launches at every
    size swept) and is accepted only with the GEMV routing inside gate/up, no
    shared expert, an even split and a separate combine."""
    for T in (1, 2, 8, 9, 16, 32, 64, 1024):
        assert plan(T)["one_launch"] == 0
        assert plan(T, I=160, shared=True)["one_launch"] == 0
    lib = ops.load_library()
    base = dict(plan(8), cost_split=0)
    assert _layer(lib, dict(base, one_launch=2)) == ops.MOE_ERR_INVALID_ARG
    assert _layer(lib, dict(base, one_launch=-1)) == ops.MOE_ERR_INVALID_ARG
    assert _layer(lib, dict(base, one_launch=1, cost_split=1)) == ops.MOE_ERR_UNSUPPORTED
    assert _layer(lib, dict(base, one_launch=1, route=ops.ROUTE_ONE_LAUNCH)) == \
        ops.MOE_ERR_UNSUPPORTED
    assert _layer(lib, dict(base, one_launch=1, route=ops.ROUTE_SEPARATE)) == ops.MOE_ERR_UNSUPPORTED
    assert _layer(lib, dict(base, one_launch=1, ffn=ops.FFN_MFMA, route=ops.ROUTE_SEPARATE)) == \
        ops.MOE_ERR_UNSUPPORTED
    assert _layer(lib, dict(plan(1), one_launch=1), T=1) == ops.MOE_ERR_UNSUPPORTED  # folded combine
    assert _layer(lib, dict(plan(65), ffn=ops.FFN_GEMV, route=ops.ROUTE_IN_GATE_UP,
                            one_launch=1), T=65) == ops.MOE_ERR_UNSUPPORTED
    # the block with its shared expert
    blk = dict(plan(8, shared=True), shared_mfma=0, cost_split=0, one_launch=1)
    assert _block(lib, blk) == ops.MOE_ERR_UNSUPPORTED
    # both stages' LDS (a plan that passes stops at the 1-byte workspace, before
    # anything is enqueued): at I = 15360 the down stage's fragments fit beside
    # the routing tables of 8 experts, not beside those of 1024
    for E, ok in ((8, True), (1024, False)):
        two = dict(plan(8, E=E, k=2, H=256, I=15360), cost_split=0)
        assert two["ffn"] == ops.FFN_GEMV and two["route"] == ops.ROUTE_IN_GATE_UP
        assert _layer(lib, two, T=8, E=E, k=2, H=256, I=15360, ws_bytes=1) == ops.MOE_ERR_WORKSPACE
        assert _layer(lib, dict(two, one_launch=1), T=8, E=E, k=2, H=256, I=15360, ws_bytes=1) == \
            (ops.MOE_ERR_WORKSPACE if ok else ops.MOE_ERR_UNSUPPORTED)


def test_gemv_that_does_not_fit_lds_falls_back_or_is_refused():
    """At I = 16384 the down GEMV's A fragments alone need 160 KiB of LDS: the
    default plan takes the matrix cores, and an explicit GEMV plan is refused
    before anything is enqueued."""
    small = plan(8, E=8, k=2, H=256, I=15360)
    big = plan(8, E=8, k=2, H=256, I=16384)
    assert small["ffn"] == ops.FFN_GEMV
    assert big["ffn"] == ops.FFN_MFMA and big["route"] == ops.ROUTE_ONE_LAUNCH
    lib = ops.load_library()
    forced = dict(big, ffn=ops.FFN_GEMV, route=ops.ROUTE_IN_GATE_UP)
    assert _layer(lib, forced, T=8, E=8, k=2, H=256, I=16384) == ops.MOE_ERR_UNSUPPORTED
