"""CPU checks of the fp16 tolerance rule used by the GPU parity tests."""

import numpy as np

from tests.parity import fp16_check


def test_exact_and_close_values_pass():
    ref = np.array([0.0, 1.0, -3.25, 31.99, 63.9])
    got = ref.astype(np.float16)
    r = fp16_check(got, ref)
    assert r["ok"] and r["n_forced"] == 0


def test_error_above_bound_fails():
    ref = np.array([1.0, 2.0])
    got = np.array([1.0, 2.03], dtype=np.float16)  # 2.03 rounds to 2.0293 in fp16
    assert not fp16_check(got, ref)["ok"]


def test_representation_forced_elements_pass_only_when_bracketing():
    # fp16 spacing at 100 is 1/16: 100.03 has no fp16 value within 2e-2
    ref = np.array([100.03, 100.03, 100.03])
    got = np.array([100.0, 100.0625, 100.125], dtype=np.float16)
    r = fp16_check(got[:2], ref[:2])
    assert r["ok"] and r["n_forced"] == 2
    assert not fp16_check(got[2:], ref[2:])["ok"]


def test_relative_rms_bound():
    ref = np.full(1000, 1e-3)
    got = np.full(1000, 2e-3).astype(np.float16)  # abs error 1e-3 passes, rel-RMS 1.0 fails
    r = fp16_check(got, ref)
    assert r["max_abs"] < 2e-2 and not r["ok"]
