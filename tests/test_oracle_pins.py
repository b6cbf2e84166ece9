"""The CPU oracle against what the pages and mathematics fix (no GPU).

Every oracle routine that produces outputs runs the full pin set of
tests/pins.py; the statistics routines are pinned to scipy's logsumexp and to
each other; the merge rule is pinned by its algebra.
"""
import math

import numpy as np
import pytest
import scipy.special

import oracle
from pins import PINS, pin_failures

ROUTINES = {
    "definition": oracle.safe_softmax,
    "online_block256": lambda x: oracle.online_softmax(x, 256),
    "online_block1": lambda x: oracle.online_softmax(x, 1),
    "online_block7": lambda x: oracle.online_softmax(x, 7),
    "splitk_chunk1024": lambda x: oracle.splitk_softmax(x, 1024),
    "splitk_chunk3": lambda x: oracle.splitk_softmax(x, 3),
    "threads4": lambda x: oracle.safe_softmax_threads(x, 4)[0],
}


@pytest.mark.parametrize("name", sorted(ROUTINES))
def test_routine_passes_every_pin(name):
    assert pin_failures(ROUTINES[name]) == []


def test_pin_set_is_not_empty():
    assert len(PINS) >= 12


def test_worked_example_to_more_digits():
    # The page prints 4 decimals; the definition in double gives these.
    y = oracle.safe_softmax(np.array([[1.0, 2.0, 3.0], [1.0, 1.0, 1.0]]))
    e = [math.exp(-2), math.exp(-1), 1.0]
    s = math.fsum(e)
    assert np.allclose(y[0], [v / s for v in e], rtol=2e-16, atol=0)
    assert np.all(y[1] == 1.0 / 3.0)


def test_row_stats_log_sum_exp():
    g = np.random.Generator(np.random.PCG64(11))
    for rows, cols, s in ((3, 1, 1.0), (5, 100, 10.0), (2, 65536, 3.0)):
        x = g.normal(0, s, (rows, cols))
        m, d = oracle.row_stats(x)
        assert np.all(m == x.max(axis=1))
        lse = scipy.special.logsumexp(x, axis=1)
        assert np.allclose(m + np.log(d), lse, rtol=1e-14, atol=0)
        assert np.all(d >= 1.0) and np.all(d <= cols)


def test_elementwise_online_stats_match_definition():
    g = np.random.Generator(np.random.PCG64(12))
    x = g.normal(0, 6, (8, 3001))
    m0, d0 = oracle.row_stats(x)
    m1, d1 = oracle.online_stats_elementwise(x)
    assert np.all(m0 == m1)
    assert np.allclose(d0, d1, rtol=1e-12, atol=0)


@pytest.mark.parametrize("block", [1, 2, 255, 256, 257, 5000])
def test_online_equals_two_pass(block):
    g = np.random.Generator(np.random.PCG64(13))
    x = g.normal(0, 8, (6, 4097))
    y0 = oracle.safe_softmax(x)
    y1 = oracle.online_softmax(x, block)
    assert np.allclose(y0, y1, rtol=1e-12, atol=1e-300)


@pytest.mark.parametrize("chunk", [1, 8, 1000, 1024, 16384, 1 << 20])
def test_splitk_independent_of_chunk(chunk):
    g = np.random.Generator(np.random.PCG64(14))
    x = g.normal(0, 3, (2, 40000))
    y0 = oracle.safe_softmax(x)
    y1 = oracle.splitk_softmax(x, chunk)
    assert np.allclose(y0, y1, rtol=1e-12, atol=1e-300)


def test_merge_rule_algebra():
    ninf = -math.inf
    ident = (ninf, 0.0)
    assert oracle.md_merge(ident, ident) == (ninf, 0.0)  # no NaN
    a, b, c = (1.5, 3.0), (-2.0, 7.0), (4.25, 1.0)
    assert oracle.md_merge(ident, a) == a
    assert oracle.md_merge(a, ident) == a
    ab = oracle.md_merge(a, b)
    ba = oracle.md_merge(b, a)
    assert ab == ba
    left = oracle.md_merge(oracle.md_merge(a, b), c)
    right = oracle.md_merge(a, oracle.md_merge(b, c))
    assert left[0] == right[0] and math.isclose(left[1], right[1], rel_tol=1e-15)
    # merging the statistics of two halves gives those of the whole row
    g = np.random.Generator(np.random.PCG64(15))
    x = g.normal(0, 5, 1000)
    m1, d1 = oracle.row_stats(x[:313])
    m2, d2 = oracle.row_stats(x[313:])
    mm, dd = oracle.md_merge((m1[0], d1[0]), (m2[0], d2[0]))
    m, d = oracle.row_stats(x)
    assert mm == m[0] and math.isclose(dd, d[0], rel_tol=1e-14)


def test_overflow_safety_at_1e4():
    x = np.array([[1.0e4, 1.0e4 - 1.0, -1.0e4], [-1.0e4, -1.0e4 + 2.0, -1.0e4]])
    with np.errstate(over="ignore", invalid="ignore"):
        naive = np.exp(x) / np.exp(x).sum(axis=1, keepdims=True)
    assert not np.all(np.isfinite(naive))  # the unsafe form overflows
    y = oracle.safe_softmax(x)
    assert np.all(np.isfinite(y))
    assert np.allclose(y[0, :2], scipy.special.softmax([0.0, -1.0]), rtol=1e-15)
    assert y[0, 2] == 0.0


def test_nonfinite_readings():
    nan, inf = math.nan, math.inf
    y = oracle.safe_softmax(np.array([[1.0, nan, 2.0]]))
    assert np.all(np.isnan(y))
    y = oracle.safe_softmax(np.array([[1.0, inf, 2.0]]))
    assert np.all(np.isnan(y))
    y = oracle.safe_softmax(np.array([[0.0, -inf, math.log(3.0)]]))
    assert y[0, 1] == 0.0 and np.allclose(y[0, [0, 2]], [0.25, 0.75], rtol=1e-15)
    y = oracle.safe_softmax(np.array([[-inf, -inf]]))
    assert np.all(np.isnan(y))
    # online and split-k agree with the definition on these readings
    for x in ([[0.0, -inf, 1.0]], [[-inf] * 300 + [1.0, 2.0]]):
        x = np.array(x)
        y0 = oracle.safe_softmax(x)
        assert np.array_equal(oracle.online_softmax(x, 256), y0) or np.allclose(
            oracle.online_softmax(x, 256), y0, rtol=1e-15)
        assert np.allclose(oracle.splitk_softmax(x, 256), y0, rtol=1e-15)


def test_cols_one_is_one():
    y = oracle.safe_softmax(np.array([[-7.0], [0.0], [1e4]]))
    assert np.all(y == 1.0)


def test_threads_report_count():
    x = np.random.Generator(np.random.PCG64(16)).normal(0, 1, (10, 50))
    y, used = oracle.safe_softmax_threads(x, 4)
    assert used == 4
    assert np.array_equal(y, oracle.safe_softmax(x))
    y, used = oracle.safe_softmax_threads(x[:2], 8)
    assert used == 2
