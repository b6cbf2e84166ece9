"""The pins must catch plausible mistakes.

Each variant below is the oracle's definition with one mistake planted (a
dropped term, a wrong sign or index, the wrong axis, a missing rescale ...),
written in plain numpy on the CPU.  Every one must fail at least one pin of
tests/pins.py; otherwise the pin set would not protect the oracle.
"""
import numpy as np
import pytest

from pins import pin_failures


def _no_max_subtraction(x):
    e = np.exp(x)
    return e / e.sum(axis=1, keepdims=True)


def _min_instead_of_max(x):
    e = np.exp(x - x.min(axis=1, keepdims=True))
    return e / e.sum(axis=1, keepdims=True)


def _wrong_sign(x):
    e = np.exp(x.max(axis=1, keepdims=True) - x)
    return e / e.sum(axis=1, keepdims=True)


def _drop_last_from_sum(x):
    e = np.exp(x - x.max(axis=1, keepdims=True))
    return e / e[:, :-1].sum(axis=1, keepdims=True) if x.shape[1] > 1 else e


def _sum_of_inputs(x):
    e = np.exp(x - x.max(axis=1, keepdims=True))
    return e / np.abs(x).sum(axis=1, keepdims=True).clip(1e-300)


def _exp2_instead_of_exp(x):
    e = np.exp2(x - x.max(axis=1, keepdims=True))
    return e / e.sum(axis=1, keepdims=True)


def _wrong_axis(x):
    e = np.exp(x - x.max(axis=0, keepdims=True))
    return e / e.sum(axis=0, keepdims=True)


def _off_by_one_column(x):
    e = np.exp(x - x.max(axis=1, keepdims=True))
    y = e / e.sum(axis=1, keepdims=True)
    return np.roll(y, 1, axis=1)


def _first_element_as_max(x):
    e = np.exp(x - x[:, :1])
    return e / e.sum(axis=1, keepdims=True)


def _online_without_rescale(x, block=256):
    m = np.full((x.shape[0], 1), -np.inf)
    d = np.zeros((x.shape[0], 1))
    for i in range(0, x.shape[1], block):
        c = x[:, i:i + block]
        m_new = np.maximum(m, c.max(axis=1, keepdims=True))
        d = d + np.exp(c - m_new).sum(axis=1, keepdims=True)  # missing d*e^(m-m_new)
        m = m_new
    return np.exp(x - m) / d


def _plus_one_in_denominator(x):
    e = np.exp(x - x.max(axis=1, keepdims=True))
    return e / (e.sum(axis=1, keepdims=True) + 1.0)


def _float32_everywhere(x):
    x = x.astype(np.float32)
    e = np.exp(x - x.max(axis=1, keepdims=True))
    return (e / e.sum(axis=1, keepdims=True)).astype(np.float64)


def _mean_shift(x):
    e = np.exp(x - x.mean(axis=1, keepdims=True))
    return e / e.sum(axis=1, keepdims=True)


MUTANTS = [_no_max_subtraction, _min_instead_of_max, _wrong_sign, _drop_last_from_sum,
           _sum_of_inputs, _exp2_instead_of_exp, _wrong_axis, _off_by_one_column,
           _first_element_as_max, _online_without_rescale, _plus_one_in_denominator,
           _float32_everywhere, _mean_shift]


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda f: f.__name__.strip("_"))
def test_mutant_fails_some_pin(mutant):
    assert pin_failures(mutant) != []
