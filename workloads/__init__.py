"""Seeded synthetic inputs for row-wise softmax and the row normalisations.

This module is shared by the oracle side and the GPU side and therefore holds
no softmax or normalisation arithmetic at all: it only draws numbers.  Every array comes back as
float64 in row-major ``[rows, cols]`` order; the caller rounds it to the storage
dtype (and both sides then read the *stored* values back).

Workloads, each named by what it is (dtype, shape, value distribution):

* ``fp32_worked_example``  -- the 2x3 example of the HIP tutorial page, section 1
  (rows [1,2,3] and [1,1,1]).
* ``fp32_64x1000``         -- fp32 [64, 1000], i.i.d. N(0, 1).
* ``fp16_attn_4x32x512x512`` -- fp16 attention scores [4,32,512,512] viewed as
  [65536, 512], i.i.d. N(0, 8^2) clipped to +-60 (large QK^T logits, the case
  study page, section 1).
* ``bf16_1Mx128``          -- bf16 [1048576, 128], i.i.d. U[-20, 20].
* ``fp16_8192x4097``       -- fp16 [8192, 4097], i.i.d. N(0, 4^2) with each entry
  independently replaced by +1e4 with probability 0.01.
* ``fp16_16x1M``           -- fp16 [16, 1048576], i.i.d. N(0, 3^2), then each
  row's (first) largest entry is swapped to a column drawn uniformly per row.
* ``ln_fp16_131040x192``, ``ln_fp16_32760x384`` (in ``NORM_WORKLOADS``, the
  inputs of the row normalisations) -- the two LayerNorm shapes
  of the Pangu-Weather profile page, section 3 ([1,131040,192] and
  [1,32760,384] tokens x hidden width), as activations with a per-row offset
  and spread: x = mu_r + sigma_r * z, mu_r ~ U[-4, 4], sigma_r ~ U[0.25, 4],
  z ~ N(0, 1).
* ``fp16_4x8M``, ``fp16_4x32M`` (in ``LONG_ROW_WORKLOADS``) -- the longest
  rows the CUDA safe-online-softmax page times its split-k on (section 4:
  [4, 8388608] and [4, 33554432] fp16), drawn like ``fp16_16x1M``.

Seeds are ``20260000 + k`` for the k-th workload of the list above (the worked
example shares k = 1 with the 64x1000 tensor but is not random).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "NORM_WORKLOADS",
    "LONG_ROW_WORKLOADS",
    "generate",
    "normal",
    "uniform",
    "spiked_normal",
    "argmax_moved_normal",
    "row_shifted_normal",
    "worked_example",
]


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def worked_example() -> np.ndarray:
    """The 2x3 input printed in section 1 of the HIP tutorial page."""
    return np.array([[1.0, 2.0, 3.0], [1.0, 1.0, 1.0]], dtype=np.float64)


def normal(rows: int, cols: int, seed: int, sigma: float = 1.0,
           clip: float | None = None) -> np.ndarray:
    """i.i.d. N(0, sigma^2), optionally clipped to [-clip, clip]."""
    x = _rng(seed).standard_normal((rows, cols)) * sigma
    if clip is not None:
        np.clip(x, -clip, clip, out=x)
    return x


def uniform(rows: int, cols: int, seed: int, lo: float, hi: float) -> np.ndarray:
    """i.i.d. U[lo, hi)."""
    return _rng(seed).uniform(lo, hi, size=(rows, cols))


def spiked_normal(rows: int, cols: int, seed: int, sigma: float = 4.0,
                  p: float = 0.01, spike: float = 1.0e4) -> np.ndarray:
    """N(0, sigma^2) with each entry independently set to ``spike`` w.p. ``p``.

    The Bernoulli mask is drawn after the normals from the same generator, so
    the count of spikes per row is random (not exactly p*cols).
    """
    g = _rng(seed)
    x = g.standard_normal((rows, cols)) * sigma
    mask = g.random((rows, cols)) < p
    x[mask] = spike
    return x


def argmax_moved_normal(rows: int, cols: int, seed: int, sigma: float = 3.0,
                        columns: np.ndarray | None = None) -> np.ndarray:
    """N(0, sigma^2); each row's first largest entry is swapped to column c_r.

    ``c_r`` is drawn uniformly from {0 .. cols-1} per row unless ``columns``
    fixes them (tests pin c_r to the first or last column or to a chunk edge).
    Swapping keeps the multiset of values in the row unchanged.
    """
    g = _rng(seed)
    x = g.standard_normal((rows, cols)) * sigma
    if columns is None:
        columns = g.integers(0, cols, size=rows)
    columns = np.asarray(columns, dtype=np.int64)
    if columns.shape != (rows,):
        raise ValueError("columns must have one entry per row")
    r = np.arange(rows)
    a = np.argmax(x, axis=1)
    va = x[r, a].copy()
    x[r, a] = x[r, columns]
    x[r, columns] = va
    return x


def row_shifted_normal(rows: int, cols: int, seed: int, mu_lo: float = -4.0, mu_hi: float = 4.0,
                       sigma_lo: float = 0.25, sigma_hi: float = 4.0) -> np.ndarray:
    """x = mu_r + sigma_r * z: per-row offset mu_r ~ U[mu_lo, mu_hi) and spread
    sigma_r ~ U[sigma_lo, sigma_hi), then z ~ N(0, 1) i.i.d. (drawn in that
    order from one generator)."""
    g = _rng(seed)
    mu = g.uniform(mu_lo, mu_hi, size=(rows, 1))
    sigma = g.uniform(sigma_lo, sigma_hi, size=(rows, 1))
    return mu + sigma * g.standard_normal((rows, cols))


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str  # "f32" | "f16" | "bf16"
    rows: int
    cols: int
    seed: int
    kind: str
    params: dict = field(default_factory=dict)
    description: str = ""

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def algorithmic_bytes(self) -> int:
        """One read of the input plus one write of the output."""
        return 2 * self.rows * self.cols * self.elem_bytes

    def generate(self, rows: int | None = None, row_offset: int = 0) -> np.ndarray:
        return generate(self, rows=rows, row_offset=row_offset)


WORKLOADS: dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("fp32_worked_example", "f32", 2, 3, 20260001, "worked_example",
                 description="[[1,2,3],[1,1,1]] fp32"),
        Workload("fp32_64x1000", "f32", 64, 1000, 20260001, "normal",
                 dict(sigma=1.0), "fp32 [64,1000] N(0,1)"),
        Workload("fp16_attn_4x32x512x512", "f16", 65536, 512, 20260002, "normal",
                 dict(sigma=8.0, clip=60.0),
                 "fp16 [4,32,512,512] = [65536,512] N(0,8^2) clipped +-60"),
        Workload("bf16_1Mx128", "bf16", 1048576, 128, 20260003, "uniform",
                 dict(lo=-20.0, hi=20.0), "bf16 [1048576,128] U[-20,20]"),
        Workload("fp16_8192x4097", "f16", 8192, 4097, 20260004, "spiked_normal",
                 dict(sigma=4.0, p=0.01, spike=1.0e4),
                 "fp16 [8192,4097] N(0,4^2), 1% entries +1e4"),
        Workload("fp16_16x1M", "f16", 16, 1048576, 20260005, "argmax_moved_normal",
                 dict(sigma=3.0), "fp16 [16,1048576] N(0,3^2), argmax at a random column"),
    ]
}

# Inputs of the row normalisations (LayerNorm, RMSNorm).
NORM_WORKLOADS: dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("ln_fp16_131040x192", "f16", 131040, 192, 20260006, "row_shifted_normal",
                 {}, "fp16 [1,131040,192] tokens, per-row offset/spread normal"),
        Workload("ln_fp16_32760x384", "f16", 32760, 384, 20260007, "row_shifted_normal",
                 {}, "fp16 [1,32760,384] tokens, per-row offset/spread normal"),
    ]
}


# Few rows of many millions of columns (more chunks per row than the
# single-launch split-k polls; the two-launch form runs them).
LONG_ROW_WORKLOADS: dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("fp16_4x8M", "f16", 4, 8388608, 20260008, "argmax_moved_normal",
                 dict(sigma=3.0), "fp16 [4,8388608] N(0,3^2), argmax at a random column"),
        Workload("fp16_4x32M", "f16", 4, 33554432, 20260009, "argmax_moved_normal",
                 dict(sigma=3.0), "fp16 [4,33554432] N(0,3^2), argmax at a random column"),
    ]
}


def generate(w: Workload, rows: int | None = None, row_offset: int = 0) -> np.ndarray:
    """Draw the workload's float64 input.

    ``rows``/``row_offset`` select a row range of the full tensor.  The full
    tensor is always drawn (the generator streams row-major), so a row range
    is bit-identical to the same rows of the full draw.
    """
    if w.kind == "worked_example":
        x = worked_example()
    elif w.kind == "normal":
        x = normal(w.rows, w.cols, w.seed, **w.params)
    elif w.kind == "uniform":
        x = uniform(w.rows, w.cols, w.seed, **w.params)
    elif w.kind == "spiked_normal":
        x = spiked_normal(w.rows, w.cols, w.seed, **w.params)
    elif w.kind == "argmax_moved_normal":
        x = argmax_moved_normal(w.rows, w.cols, w.seed, **w.params)
    elif w.kind == "row_shifted_normal":
        x = row_shifted_normal(w.rows, w.cols, w.seed, **w.params)
    else:  # pragma: no cover
        raise ValueError(w.kind)
    if rows is None:
        return x if row_offset == 0 else x[row_offset:]
    return x[row_offset:row_offset + rows]
