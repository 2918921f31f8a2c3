"""Shared helpers of the GPU parity tests: tolerance check and uploads.

Tolerance (stated for the fp16 layer output): max |err| <= 2e-2 absolute and
relative RMS <= 1e-2, where err = fp16 GPU output - unrounded fp64 oracle.  An
element whose exact value has no fp16 neighbour within 2e-2 (|y| >= 64, where
fp16 spacing is 1/16) passes when the GPU returned one of the two fp16 values
that bracket the exact value; such elements are counted and reported.
"""

from __future__ import annotations

import numpy as np

ABS_TOL = 2e-2
REL_RMS_TOL = 1e-2

# Per-row expert outputs y_sorted (fp32, not rounded to fp16).  Derivation:
# both paths keep B exact and scale per group in fp32.  The decode path
# multiplies biased codes (1024 + q) and removes the bias once per group, so
# each group partial is formed near 1024 * sum(a) (|.| up to ~10^4), whose
# fp32 spacing is ~5e-4-1e-3; scaled by s <= 0.02, summed over up to 80
# groups, carried through SiLU(gate) * up (|d act / d h| up to ~20 at the
# model geometry) and summed over the 640 terms of the down product, that is
# ~3e-3 absolute at most.  The matrix-core path has no bias and is ~10x
# tighter.  The bound below (1e-2 absolute plus 1e-5 relative) sits above
# both, far below |y| (rms ~20): it catches rows never written (the NaN
# sentinels) or written with a wrong operand, while the fp16 layer output
# carries the stated contract.
Y_ABS_TOL = 1e-2
Y_REL_TOL = 1e-5
Y_REL_RMS_TOL = 1e-4


def fp16_check(got_fp16: np.ndarray, ref: np.ndarray) -> dict:
    got = np.asarray(got_fp16, dtype=np.float16).astype(np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref)
    bad = err > ABS_TOL
    forced = np.zeros_like(bad)
    if bad.any():
        r16 = ref.astype(np.float16)
        below = r16.astype(np.float64) <= ref
        lo = np.where(below, r16, np.nextafter(r16, np.float16(-np.inf))).astype(np.float64)
        hi = np.where(below, np.nextafter(r16, np.float16(np.inf)), r16).astype(np.float64)
        no_close = ((ref - lo) > ABS_TOL) & ((hi - ref) > ABS_TOL)
        forced = bad & no_close & ((got == lo) | (got == hi))
    fails = bad & ~forced
    denom = np.sqrt((ref ** 2).sum())
    rel = float(np.sqrt((err ** 2).sum()) / denom) if denom > 0 else float(np.sqrt((err ** 2).sum()))
    return {
        "max_abs": float(err.max()) if err.size else 0.0,
        "rel_rms": rel,
        "n_fail": int(fails.sum()),
        "n_forced": int(forced.sum()),
        "ok": (not fails.any()) and rel <= REL_RMS_TOL and np.isfinite(got).all(),
    }


def assert_fp16_close(got_fp16, ref, label=""):
    r = fp16_check(got_fp16, ref)
    print(f"  {label}: max|err| {r['max_abs']:.3e} rel-RMS {r['rel_rms']:.3e} "
          f"forced {r['n_forced']} fail {r['n_fail']}", flush=True)
    assert r["ok"], f"{label}: {r}"
    return r


def assert_y_close(got, ref, label=""):
    """Every row and element of y_sorted against the oracle's."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, f"{label}: shape {got.shape} != {ref.shape}"
    finite = np.isfinite(got)
    err = np.abs(got - ref)
    bound = Y_ABS_TOL + Y_REL_TOL * np.abs(ref)
    bad = ~finite | (err > bound)
    denom = np.sqrt((ref ** 2).sum())
    rel = float(np.sqrt((np.where(finite, err, 0.0) ** 2).sum()) / denom) if denom > 0 else 0.0
    mx = float(np.where(finite, err, 0.0).max()) if err.size else 0.0
    print(f"  {label} y_sorted: max|err| {mx:.3e} rel-RMS {rel:.3e} non-finite "
          f"{int((~finite).sum())} over bound {int(bad.sum())} of {err.size}", flush=True)
    assert not bad.any() and rel <= Y_REL_RMS_TOL, f"{label}: y_sorted mismatch"
