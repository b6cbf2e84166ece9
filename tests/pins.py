"""Pins for a row-wise softmax: checks against facts fixed by the pages and by
mathematics, not against another copy of the same formula.

``pin_failures(fn)`` runs every pin on a candidate ``fn(x2d_float64) ->
y2d_float64`` and returns the list of pins it fails (empty = all pass).  The
oracle must pass them all; deliberately broken variants (tests of the pins
themselves) must each fail at least one.

Pins, with what fixes each value:

* golden_worked_example  -- values printed in section 1 of the HIP softmax
  tutorial page (4 decimals).
* golden_ramp4            -- values printed in section 8 of the same page
  (6 significant digits; the input is a reading, see the fixture).
* golden_long_row         -- first 8 outputs of row 0 printed in section 8 of
  the same page (inferred input, see the fixture).
* constant_row            -- closed form 1/cols.
* two_entries_logistic    -- closed form: softmax([a, b]) = [expit(a-b),
  expit(b-a)] (scipy's logistic, a different formula).
* spikes_exact            -- k entries at +1e4 among N(0,16): outputs are
  exactly 1/k at the spikes and 0 elsewhere (e^-9900 underflows even in
  double); also shows that no overflow happens at +-1e4.
* high_precision_tiny     -- brute force: every row of length 1..3 over a grid
  of fp16 values, compared with the definition evaluated in 40-digit decimal
  arithmetic (no max subtraction needed there, the exponent range is huge).
* scipy_library           -- scipy.special.softmax on random matrices.
* row_sums / bounds / argmax -- invariants: sum 1, 0 <= y <= 1, the argmax
  keeps the largest output.
* shift_invariance        -- y(x + c) == y(x) for an exactly representable
  shift c (the CUDA safe-online-softmax page names the shift invariance).
* permutation             -- permuting a row's columns permutes its outputs.
* column_independence     -- each row is normalised on its own (catches a
  reduction along the wrong axis).
"""
from __future__ import annotations

from decimal import Decimal, getcontext
from itertools import product

import numpy as np
import scipy.special

from golden_io import load


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _hp_softmax_row(row):
    getcontext().prec = 40
    ex = [Decimal(float(v)).exp() for v in row]
    s = sum(ex)
    return [float(e / s) for e in ex]


def _pins():
    pins = {}

    def pin(f):
        pins[f.__name__] = f
        return f

    @pin
    def golden_worked_example(fn):
        g = load("worked_example_2x3.txt")
        y = fn(g["input"])
        return np.max(np.abs(y - g["output"])) <= 5e-5

    @pin
    def golden_ramp4(fn):
        g = load("ramp4_constant4.txt")
        y = fn(g["input"])
        ref = g["output"]
        # 6 significant digits: half a unit in the 6th digit of each value.
        tol = 0.5 * 10.0 ** (np.floor(np.log10(np.abs(ref))) - 5)
        return bool(np.all(np.abs(y - ref) <= tol * 1.0001))

    @pin
    def golden_long_row(fn):
        g = load("long_row_4x32768_row0_first8.txt")
        cols = int(g["cols"])
        x = (np.arange(cols) % 97 / 32.0).reshape(1, cols)
        y = fn(x)[0, :8]
        ref = g["output_first8"][0]
        return bool(np.all(np.abs(y - ref) <= float(g["relative_tolerance"]) * ref))

    @pin
    def constant_row(fn):
        ok = True
        for cols in (1, 2, 3, 7, 1000, 4097):
            x = np.full((3, cols), [[-5.0], [0.0], [123.25]])
            y = fn(x)
            ok &= bool(np.all(np.abs(y - 1.0 / cols) <= 4e-16 / cols + 1e-300))
        return ok

    @pin
    def two_entries_logistic(fn):
        g = _rng(1)
        a = g.normal(0, 5, 64)
        b = g.normal(0, 5, 64)
        y = fn(np.stack([a, b], axis=1))
        ref = np.stack([scipy.special.expit(a - b), scipy.special.expit(b - a)], axis=1)
        return bool(np.all(np.abs(y - ref) <= 1e-15 + 1e-14 * ref))

    @pin
    def spikes_exact(fn):
        g = _rng(2)
        rows, cols = 16, 4097
        x = g.normal(0, 4, (rows, cols))
        mask = g.random((rows, cols)) < 0.01
        x[mask] = 1.0e4
        mask[:, 0] = True  # every row has at least one spike
        x[:, 0] = 1.0e4
        y = fn(x)
        k = mask.sum(axis=1, keepdims=True).astype(np.float64)
        at_spikes = np.where(mask, np.abs(y - 1.0 / k) <= 2e-16 / k, True)
        elsewhere = np.where(~mask, y == 0.0, True)
        return bool(np.all(np.isfinite(y)) and np.all(at_spikes) and np.all(elsewhere))

    @pin
    def negative_spikes(fn):
        # rows of -1e4 with one far larger entry: all mass on it, no NaN
        x = np.full((2, 9), -1.0e4)
        x[0, 3] = 0.0
        x[1, 8] = -9000.0
        y = fn(x)
        ref = np.zeros_like(x)
        ref[0, 3] = 1.0
        ref[1, 8] = 1.0
        return bool(np.all(y == ref))

    @pin
    def high_precision_tiny(fn):
        grid = [-65504.0, -30.5, -3.0, -1.0, -0.5, -2.0 ** -14, 0.0, 2.0 ** -24,
                0.25, 1.0, 1.5, 2.0, 10.0, 11.0, 60.0, 65504.0]
        worst = 0.0
        for n in (1, 2, 3):
            rows = [list(r) for r in product(grid, repeat=n)]
            y = fn(np.array(rows, dtype=np.float64))
            for row, yr in zip(rows, y):
                ref = _hp_softmax_row(row)
                for a, b in zip(yr, ref):
                    worst = max(worst, abs(a - b) - 4e-15 * b)
        return worst <= 1e-300

    @pin
    def scipy_library(fn):
        g = _rng(3)
        ok = True
        for rows, cols, s in ((5, 1, 1.0), (7, 33, 3.0), (4, 1000, 8.0), (3, 5000, 30.0)):
            x = g.normal(0, s, (rows, cols))
            y = fn(x)
            ref = scipy.special.softmax(x, axis=1)
            ok &= bool(np.all(np.abs(y - ref) <= 1e-14 * ref + 1e-300))
        return ok

    @pin
    def row_sums_bounds_argmax(fn):
        g = _rng(4)
        x = g.normal(0, 8, (32, 777))
        y = fn(x)
        r = np.arange(32)
        a = np.argmax(x, axis=1)
        return bool(np.all(np.abs(y.sum(axis=1) - 1.0) <= 1e-13)
                    and np.all(y >= 0.0) and np.all(y <= 1.0)
                    and np.all(y[r, a] == y.max(axis=1)))

    @pin
    def shift_invariance(fn):
        g = _rng(5)
        # multiples of 2^-8 in [-64, 64): adding 512 is exact in double
        x = np.round(g.uniform(-64, 64, (8, 300)) * 256.0) / 256.0
        y0 = fn(x)
        y1 = fn(x + 512.0)
        return bool(np.all(np.abs(y0 - y1) <= 1e-15 * y0 + 1e-300))

    @pin
    def permutation(fn):
        g = _rng(6)
        x = g.normal(0, 2, (6, 257))
        p = g.permutation(257)
        y = fn(x)
        yp = fn(x[:, p])
        return bool(np.all(np.abs(yp - y[:, p]) <= 1e-13 * yp + 1e-300))

    @pin
    def column_independence(fn):
        g = _rng(7)
        x = g.normal(0, 1, (4, 5))
        y = fn(x)
        x2 = x.copy()
        x2[1] += 40.0  # another row: must not change row 0
        y2 = fn(x2)
        return bool(np.all(np.abs(y[0] - y2[0]) <= 1e-15) and abs(y2[1].sum() - 1) <= 1e-14)

    return pins


PINS = _pins()


def pin_failures(fn) -> list[str]:
    failed = []
    for name, check in PINS.items():
        try:
            with np.errstate(all="ignore"):
                ok = bool(check(fn))
        except Exception as e:  # a candidate that crashes fails the pin
            ok = False
            name = f"{name} ({type(e).__name__})"
        if not ok:
            failed.append(name)
    return failed

