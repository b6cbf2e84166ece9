"""Pins for the oracle's LayerNorm and RMSNorm (row normalisations with the
softmax structure, DCU case-study page, section 9; Pangu-Weather profile
page, section 3).  Closed forms, invariants, a 40-digit brute force, torch's
CPU float64 implementations, and planted mistakes that must fail."""
from decimal import Decimal, getcontext

import numpy as np
import pytest
import torch

import oracle


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _dec_layernorm(row, eps, w=None, b=None):
    getcontext().prec = 40
    xs = [Decimal(float(v)) for v in row]
    n = Decimal(len(xs))
    mu = sum(xs) / n
    var = sum((v - mu) * (v - mu) for v in xs) / n
    rstd = 1 / (var + Decimal(eps)).sqrt()
    out = []
    for j, v in enumerate(xs):
        o = (v - mu) * rstd
        if w is not None:
            o = o * Decimal(float(w[j]))
        if b is not None:
            o = o + Decimal(float(b[j]))
        out.append(float(o))
    return np.array(out), float(mu), float(rstd)


def _dec_rmsnorm(row, eps, w=None):
    getcontext().prec = 40
    xs = [Decimal(float(v)) for v in row]
    ms = sum(v * v for v in xs) / Decimal(len(xs))
    rstd = 1 / (ms + Decimal(eps)).sqrt()
    out = [float(v * rstd * (Decimal(float(w[j])) if w is not None else 1)) for j, v in enumerate(xs)]
    return np.array(out), float(rstd)


# ---------------------------------------------------------------------------
# LayerNorm pins.  fn(x, eps, weight, bias) -> (y, mean, rstd)
# ---------------------------------------------------------------------------
def layernorm_pins(fn):
    failed = []
    g = _rng(60)
    # 1. closed form: [1, 2, 3, 4], eps = 0 -> (2x - 5) / sqrt(5)
    y, mu, rs = fn(np.array([[1.0, 2.0, 3.0, 4.0]]), 0.0, None, None)
    if not np.allclose(y, np.array([[-3.0, -1.0, 1.0, 3.0]]) / np.sqrt(5.0), rtol=0, atol=1e-15):
        failed.append("closed_form_1234")
    if not (abs(mu[0] - 2.5) < 1e-15 and abs(rs[0] - 1.0 / np.sqrt(1.25)) < 1e-15):
        failed.append("closed_form_stats")
    # 2. two entries, eps = 0 -> -1 and +1 in the order of the entries
    y, _, _ = fn(np.array([[7.0, -2.0], [-1e-3, 5e3]]), 0.0, None, None)
    if not np.allclose(y, [[1.0, -1.0], [-1.0, 1.0]], rtol=0, atol=1e-15):
        failed.append("two_entries")
    # 3. output moments: mean 0, mean square var / (var + eps)
    x = g.normal(3.0, 2.0, (6, 257))
    eps = 0.25
    y, mu, rs = fn(x, eps, None, None)
    var = x.var(axis=1)
    if not np.all(np.abs(y.mean(axis=1)) < 1e-14):
        failed.append("output_mean_zero")
    if not np.allclose((y * y).mean(axis=1), var / (var + eps), rtol=1e-13, atol=0):
        failed.append("output_mean_square")
    # 4. statistics against numpy's mean and biased variance
    if not (np.allclose(mu, x.mean(axis=1), rtol=1e-14, atol=1e-14)
            and np.allclose(rs, 1.0 / np.sqrt(var + eps), rtol=1e-13, atol=0)):
        failed.append("numpy_stats")
    # 5. shift invariance of the normalised output
    y2, _, _ = fn(x + 1234.5, eps, None, None)
    if not np.allclose(y2, y, rtol=0, atol=1e-9):
        failed.append("shift_invariance")
    # 6. scale: LN(s x, s^2 eps) = sign(s) LN(x, eps)
    y3, _, _ = fn(-3.0 * x, 9.0 * eps, None, None)
    if not np.allclose(y3, -y, rtol=0, atol=1e-13):
        failed.append("scale_sign")
    # 7. affine: weight and bias apply per column after normalisation
    w = g.uniform(0.5, 2.0, 257)
    b = g.normal(0, 1, 257)
    ya, _, _ = fn(x, eps, w, b)
    if not np.allclose(ya, y * w[None, :] + b[None, :], rtol=1e-14, atol=1e-14):
        failed.append("affine")
    # 8. constant row, eps > 0 -> zeros; mean = the constant, rstd = 1/sqrt(eps)
    yc, mc, rc = fn(np.full((2, 33), -4.5), 1e-5, None, None)
    if not (np.all(yc == 0.0) and np.all(mc == -4.5) and np.allclose(rc, 1 / np.sqrt(1e-5), rtol=1e-15)):
        failed.append("constant_row")
    # 9. 40-digit brute force on small rows, with affine
    xs = g.normal(-1.0, 3.0, (3, 11))
    w = g.uniform(-2, 2, 11)
    b = g.normal(0, 1, 11)
    yb, mb, rb = fn(xs, 1e-3, w, b)
    for r in range(3):
        ref, mref, rref = _dec_layernorm(xs[r], 1e-3, w, b)
        if not (np.allclose(yb[r], ref, rtol=1e-14, atol=1e-15)
                and abs(mb[r] - mref) <= 1e-15 * max(1.0, abs(mref))
                and abs(rb[r] - rref) <= 1e-14 * rref):
            failed.append("brute_force")
            break
    # 10. torch.nn.functional.layer_norm on the CPU in float64
    x = g.normal(0.5, 4.0, (5, 100))
    w = g.uniform(0.1, 3.0, 100)
    b = g.normal(0, 2, 100)
    ref = torch.nn.functional.layer_norm(torch.tensor(x), (100,), torch.tensor(w), torch.tensor(b),
                                         eps=1e-5).numpy()
    yt, _, _ = fn(x, 1e-5, w, b)
    if not np.allclose(yt, ref, rtol=1e-12, atol=1e-13):
        failed.append("torch_layer_norm")
    # 11. rows are independent: permuting rows permutes outputs
    perm = g.permutation(5)
    yp, _, _ = fn(x[perm], 1e-5, w, b)
    if not np.array_equal(yp, yt[perm]):
        failed.append("row_independence")
    return failed


def _ln(x, eps, w, b):
    return oracle.layernorm(x, eps, w, b, return_stats=True)


def test_oracle_layernorm_passes_pins():
    assert layernorm_pins(_ln) == []


def _ln_unbiased(x, eps, w, b):
    x = np.asarray(x, dtype=np.float64)
    mu = x.mean(axis=1, keepdims=True)
    var = ((x - mu) ** 2).sum(axis=1, keepdims=True) / (x.shape[1] - 1)
    y = (x - mu) / np.sqrt(var + eps)
    y = y * (w if w is not None else 1) + (b if b is not None else 0)
    return y, mu[:, 0], 1 / np.sqrt(var[:, 0] + eps)


def _ln_eps_outside(x, eps, w, b):
    x = np.asarray(x, dtype=np.float64)
    mu = x.mean(axis=1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=1, keepdims=True)
    y = (x - mu) / (np.sqrt(var) + eps)
    y = y * (w if w is not None else 1) + (b if b is not None else 0)
    return y, mu[:, 0], 1 / (np.sqrt(var[:, 0]) + eps)


def _ln_not_centred_output(x, eps, w, b):
    x = np.asarray(x, dtype=np.float64)
    mu = x.mean(axis=1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=1, keepdims=True)
    y = x / np.sqrt(var + eps)
    y = y * (w if w is not None else 1) + (b if b is not None else 0)
    return y, mu[:, 0], 1 / np.sqrt(var[:, 0] + eps)


def _ln_bias_before_weight(x, eps, w, b):
    x = np.asarray(x, dtype=np.float64)
    mu = x.mean(axis=1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=1, keepdims=True)
    y = (x - mu) / np.sqrt(var + eps)
    y = (y + (b if b is not None else 0)) * (w if w is not None else 1)
    return y, mu[:, 0], 1 / np.sqrt(var[:, 0] + eps)


def _ln_no_eps(x, eps, w, b):
    return _ln(x, 0.0, w, b)


def _ln_stats_over_rows(x, eps, w, b):
    x = np.asarray(x, dtype=np.float64)
    if x.shape[0] == 1:
        return _ln(x, eps, w, b)
    mu = x.mean(axis=0, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=0, keepdims=True)
    y = (x - mu) / np.sqrt(var + eps)
    y = y * (w if w is not None else 1) + (b if b is not None else 0)
    return y, np.resize(mu[0], x.shape[0]), np.resize(1 / np.sqrt(var[0] + eps), x.shape[0])


def _ln_rms_instead(x, eps, w, b):
    y, rs = oracle.rmsnorm(x, eps, w, return_stats=True)
    if b is not None:
        y = y + b
    return y, np.asarray(x, dtype=np.float64).mean(axis=1), rs


@pytest.mark.parametrize("mutant", [_ln_unbiased, _ln_eps_outside, _ln_not_centred_output,
                                    _ln_bias_before_weight, _ln_no_eps, _ln_stats_over_rows,
                                    _ln_rms_instead])
def test_layernorm_mutants_fail(mutant):
    assert layernorm_pins(mutant) != []


# ---------------------------------------------------------------------------
# RMSNorm pins.  fn(x, eps, weight) -> (y, rstd)
# ---------------------------------------------------------------------------
def rmsnorm_pins(fn):
    failed = []
    g = _rng(61)
    # 1. closed form: [3, 4], eps = 0 -> [3, 4] / sqrt(12.5)
    y, rs = fn(np.array([[3.0, 4.0]]), 0.0, None)
    if not (np.allclose(y, [[3 / np.sqrt(12.5), 4 / np.sqrt(12.5)]], rtol=0, atol=1e-15)
            and abs(rs[0] - 1 / np.sqrt(12.5)) < 1e-15):
        failed.append("closed_form_34")
    # 2. one entry, eps = 0 -> its sign
    y, _ = fn(np.array([[-0.37], [12.0]]), 0.0, None)
    if not np.array_equal(y, [[-1.0], [1.0]]):
        failed.append("one_entry")
    # 3. output mean square ms / (ms + eps)
    x = g.normal(2.0, 3.0, (6, 300))
    eps = 0.5
    y, rs = fn(x, eps, None)
    ms = (x * x).mean(axis=1)
    if not np.allclose((y * y).mean(axis=1), ms / (ms + eps), rtol=1e-13, atol=0):
        failed.append("output_mean_square")
    if not np.allclose(rs, 1 / np.sqrt(ms + eps), rtol=1e-14, atol=0):
        failed.append("numpy_rstd")
    # 4. no centring: a shift changes the output (the mean is not removed)
    y_sh, _ = fn(x + 10.0, eps, None)
    if np.allclose(y_sh, y, atol=1e-3):
        failed.append("not_shift_invariant")
    # 5. zero-mean rows: RMSNorm == LayerNorm with the same eps
    xz = x - x.mean(axis=1, keepdims=True)
    yz, _ = fn(xz, eps, None)
    if not np.allclose(yz, oracle.layernorm(xz, eps), rtol=1e-13, atol=1e-14):
        failed.append("zero_mean_equals_layernorm")
    # 6. scale: RMS(s x, s^2 eps) = sign(s) RMS(x, eps)
    y3, _ = fn(-0.5 * x, 0.25 * eps, None)
    if not np.allclose(y3, -y, rtol=0, atol=1e-13):
        failed.append("scale_sign")
    # 7. 40-digit brute force with weight
    xs = g.normal(0.5, 2.0, (3, 13))
    w = g.uniform(-2, 2, 13)
    yb, rb = fn(xs, 1e-6, w)
    for r in range(3):
        ref, rref = _dec_rmsnorm(xs[r], 1e-6, w)
        if not (np.allclose(yb[r], ref, rtol=1e-14, atol=1e-15) and abs(rb[r] - rref) <= 1e-14 * rref):
            failed.append("brute_force")
            break
    # 8. torch.nn.functional.rms_norm on the CPU in float64
    x = g.normal(0, 5.0, (4, 96))
    w = g.uniform(0.2, 2.0, 96)
    ref = torch.nn.functional.rms_norm(torch.tensor(x), (96,), torch.tensor(w), eps=1e-5).numpy()
    yt, _ = fn(x, 1e-5, w)
    if not np.allclose(yt, ref, rtol=1e-12, atol=1e-13):
        failed.append("torch_rms_norm")
    # 9. zero row, eps > 0 -> zeros
    y0, r0 = fn(np.zeros((1, 17)), 1e-5, None)
    if not (np.all(y0 == 0.0) and abs(r0[0] - 1 / np.sqrt(1e-5)) < 1e-9):
        failed.append("zero_row")
    return failed


def _rms(x, eps, w):
    return oracle.rmsnorm(x, eps, w, return_stats=True)


def test_oracle_rmsnorm_passes_pins():
    assert rmsnorm_pins(_rms) == []


def _rms_centred(x, eps, w):
    y, _, rs = oracle.layernorm(x, eps, w, return_stats=True)
    return y, rs


def _rms_sum_not_mean(x, eps, w):
    x = np.asarray(x, dtype=np.float64)
    ss = (x * x).sum(axis=1, keepdims=True)
    y = x / np.sqrt(ss + eps) * (w if w is not None else 1)
    return y, 1 / np.sqrt(ss[:, 0] + eps)


def _rms_abs_mean(x, eps, w):
    x = np.asarray(x, dtype=np.float64)
    ma = np.abs(x).mean(axis=1, keepdims=True)
    y = x / (ma + eps) * (w if w is not None else 1)
    return y, 1 / (ma[:, 0] + eps)


def _rms_eps_squared(x, eps, w):
    x = np.asarray(x, dtype=np.float64)
    ms = (x * x).mean(axis=1, keepdims=True)
    y = x / np.sqrt(ms + eps * eps) * (w if w is not None else 1)
    return y, 1 / np.sqrt(ms[:, 0] + eps * eps)


@pytest.mark.parametrize("mutant", [_rms_centred, _rms_sum_not_mean, _rms_abs_mean,
                                    _rms_eps_squared])
def test_rmsnorm_mutants_fail(mutant):
    assert rmsnorm_pins(mutant) != []
