"""Pins for the oracle's scaled / masked / causal softmax (attention-score
fusion, DCU case-study page, section 9), against closed forms and scipy, and
a check that plausible mistakes in it fail those pins."""
import numpy as np
import pytest
import scipy.special

import oracle


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def masked_pins(fn):
    """fn(x, scale, mask, causal_q) -> y.  Returns the list of failed pins."""
    failed = []
    g = _rng(40)
    # reduces to the plain definition
    x = g.normal(0, 4, (7, 33))
    if not np.array_equal(fn(x, 1.0, None, 0), oracle.safe_softmax(x)):
        failed.append("identity")
    # causal on a constant matrix: uniform over the first i + 1 + cols - q columns
    for q, cols in ((5, 5), (4, 9), (1, 3)):
        rows = 2 * q
        y = fn(np.zeros((rows, cols)), 1.0, None, q)
        ref = np.zeros((rows, cols))
        for r in range(rows):
            n = (r % q) + 1 + cols - q
            ref[r, :n] = 1.0 / n
        if not np.allclose(y, ref, rtol=1e-15, atol=0):
            failed.append(f"causal_closed_form q={q} cols={cols}")
    # -inf mask entries drop those columns
    x = g.normal(0, 3, (4, 12))
    m = np.zeros((4, 12))
    m[:, [0, 5, 11]] = -np.inf
    y = fn(x, 1.0, m, 0)
    keep = [j for j in range(12) if j not in (0, 5, 11)]
    ok = np.all(y[:, [0, 5, 11]] == 0) and np.allclose(
        y[:, keep], scipy.special.softmax(x[:, keep], axis=1), rtol=1e-14, atol=0)
    if not ok:
        failed.append("neg_inf_mask_drops_columns")
    # additive log-weights on a zero input: y = w / sum(w)
    w = g.uniform(0.1, 5.0, (3, 10))
    y = fn(np.zeros((3, 10)), 1.0, np.log(w), 0)
    if not np.allclose(y, w / w.sum(axis=1, keepdims=True), rtol=1e-14, atol=0):
        failed.append("log_weights")
    # scale
    x = g.normal(0, 2, (5, 64))
    for s in (0.125, -2.0, 0.0):
        if not np.allclose(fn(x, s, None, 0), scipy.special.softmax(s * x, axis=1),
                           rtol=1e-14, atol=1e-300):
            failed.append(f"scale {s}")
    # mask rows broadcast: row r uses mask row r % mask_rows (mask [q, cols] over [b*q, cols])
    x = g.normal(0, 1, (12, 8))
    m = g.normal(0, 1, (3, 8))
    y = fn(x, 0.5, m, 0)
    ref = scipy.special.softmax(0.5 * x + m[np.arange(12) % 3], axis=1)
    if not np.allclose(y, ref, rtol=1e-14, atol=0):
        failed.append("broadcast")
    return failed


def test_oracle_masked_passes_pins():
    assert masked_pins(lambda x, s, m, q: oracle.masked_softmax(x, s, m, q)) == []


def _mut_causal_off_by_one(x, s, m, q):
    z = s * x + (0 if m is None else m[np.arange(x.shape[0]) % m.shape[0]])
    if q:
        r = np.arange(x.shape[0])[:, None] % q
        j = np.arange(x.shape[1])[None, :]
        z = np.where(j >= r + x.shape[1] - q, -np.inf, z)
    return oracle.safe_softmax(z)


def _mut_mask_row_div(x, s, m, q):
    mm = 0 if m is None else m[np.minimum(np.arange(x.shape[0]) // m.shape[0], m.shape[0] - 1)]
    return oracle.masked_softmax(s * x + mm, 1.0, None, q)


def _mut_scale_after_mask(x, s, m, q):
    return oracle.masked_softmax(x if m is None else x + m[np.arange(x.shape[0]) % m.shape[0]],
                                 s, None, q)


def _mut_causal_top_left(x, s, m, q):
    z = s * x + (0 if m is None else m[np.arange(x.shape[0]) % m.shape[0]])
    if q:
        r = np.arange(x.shape[0])[:, None] % q
        j = np.arange(x.shape[1])[None, :]
        z = np.where(j > r, -np.inf, z)
    return oracle.safe_softmax(z)


@pytest.mark.parametrize("mutant", [_mut_causal_off_by_one, _mut_mask_row_div,
                                    _mut_scale_after_mask, _mut_causal_top_left],
                         ids=lambda f: f.__name__.strip("_"))
def test_masked_mutants_fail(mutant):
    with np.errstate(all="ignore"):
        assert masked_pins(mutant) != []
