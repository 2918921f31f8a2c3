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
