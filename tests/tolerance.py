"""Parity bar between the GPU path and the oracle.

Per output dtype (the GPU output widened to float64 against the float64
oracle on the same stored inputs):

* fp16: max |y - y_ref| <= 1e-3 over the tensor; every row sum within 1e-2 of 1.
* bf16: max |y - y_ref| <= 8e-3; every row sum within 1e-2 of 1.
* fp32: |y - y_ref| <= 1e-5 * y_ref + 1e-37 element by element (the floor
  covers results below the fp32 normal range, where the exponential may
  flush); every row sum within 1e-5 of 1.

A row sum is the sum of the *stored* outputs widened to float64.
"""
from __future__ import annotations

import numpy as np

TOL = {
    "f32": {"rel": 1e-5, "floor": 1e-37, "rowsum": 1e-5},
    "f16": {"abs": 1e-3, "rowsum": 1e-2},
    "bf16": {"abs": 8e-3, "rowsum": 1e-2},
}


def measure(y: np.ndarray, ref: np.ndarray, dtype: str) -> dict:
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(y - ref)
    out = {
        "max_abs": float(err.max()) if err.size else 0.0,
        "max_rowsum_dev": float(np.abs(y.sum(axis=-1) - 1.0).max()) if y.size else 0.0,
        "finite": bool(np.all(np.isfinite(y))),
    }
    if dtype == "f32":
        t = TOL["f32"]
        excess = err - (t["rel"] * ref + t["floor"])
        out["max_excess"] = float(excess.max()) if err.size else -1.0
        with np.errstate(divide="ignore", invalid="ignore"):
            rel = np.where(ref > 1e-30, err / ref, 0.0)
        out["max_rel"] = float(rel.max()) if err.size else 0.0
    return out


def check(y: np.ndarray, ref: np.ndarray, dtype: str, what: str = "") -> dict:
    m = measure(y, ref, dtype)
    assert m["finite"], f"{what}: non-finite output"
    t = TOL[dtype]
    if dtype == "f32":
        assert m["max_excess"] <= 0.0, f"{what}: fp32 relative error {m['max_rel']:.3e} > 1e-5 ({m})"
    else:
        assert m["max_abs"] <= t["abs"], f"{what}: max abs error {m['max_abs']:.3e} > {t['abs']}"
    assert m["max_rowsum_dev"] <= t["rowsum"], \
        f"{what}: row sum off by {m['max_rowsum_dev']:.3e} > {t['rowsum']}"
    return m


def rounded_rowsums(ref: np.ndarray, dtype: str) -> np.ndarray:
    """Row sums of the oracle's output rounded to the dtype (RNE): what the
    stored outputs of a correctly rounded result sum to.  For rows of
    millions of fp16 columns almost every output is an fp16 subnormal, and
    these sums fall short of 1 by more than the 1e-2 bar (fp16 [4, 8388608]:
    1 - 0.0192), so no fp16 output can meet the bar there."""
    import torch
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]
    return torch.from_numpy(np.ascontiguousarray(ref)).to(tdt).double().numpy().sum(axis=-1)


def check_long_rows(y: np.ndarray, ref: np.ndarray, dtype: str, what: str = "") -> dict:
    """The element bar of check(); the row-sum bar taken against the row sums
    of the correctly rounded result (rounded_rowsums) instead of 1."""
    m = measure(y, ref, dtype)
    assert m["finite"], f"{what}: non-finite output"
    t = TOL[dtype]
    if dtype == "f32":
        assert m["max_excess"] <= 0.0, f"{what}: fp32 relative error {m['max_rel']:.3e} > 1e-5"
    else:
        assert m["max_abs"] <= t["abs"], f"{what}: max abs error {m['max_abs']:.3e} > {t['abs']}"
    dev = np.abs(np.asarray(y, dtype=np.float64).sum(axis=-1) - rounded_rowsums(ref, dtype))
    m["max_rowsum_dev_vs_rounded"] = float(dev.max())
    assert dev.max() <= t["rowsum"], \
        f"{what}: row sum off the rounded result's by {dev.max():.3e} > {t['rowsum']}"
    return m
