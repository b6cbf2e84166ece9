"""Pins for the oracle's softmax backward: the Jacobian of the (pinned)
forward oracle by central finite differences, closed forms, torch autograd on
the CPU in float64, invariants, and planted mistakes that must fail."""
import numpy as np
import pytest
import torch

import oracle


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def backward_pins(fn):
    failed = []
    g = _rng(50)
    # 1. J^T dy by central differences of the forward oracle (h = 1e-5)
    x = g.normal(0, 1.5, (3, 9))
    dy = g.normal(0, 1, (3, 9))
    y = oracle.safe_softmax(x)
    h = 1e-5
    fd = np.zeros_like(x)
    for j in range(9):
        e = np.zeros(9)
        e[j] = h
        yp = oracle.safe_softmax(x + e)
        ym = oracle.safe_softmax(x - e)
        fd[:, j] = ((yp - ym) / (2 * h) * dy).sum(axis=1)
    if not np.allclose(fn(y, dy), fd, rtol=0, atol=1e-8):
        failed.append("finite_differences")
    # 2. constant upstream gradient -> zero (softmax outputs sum to 1)
    x = g.normal(0, 3, (4, 50))
    y = oracle.safe_softmax(x)
    if not np.allclose(fn(y, np.full_like(y, 2.5)), 0.0, atol=1e-14):
        failed.append("constant_dy")
    # 3. one-hot upstream gradient e_k -> y_j (delta_jk - y_k)
    k = 7
    dyk = np.zeros_like(y)
    dyk[:, k] = 1.0
    ref = y * ((np.arange(50) == k)[None, :] - y[:, k:k + 1])
    if not np.allclose(fn(y, dyk), ref, rtol=1e-14, atol=1e-17):
        failed.append("one_hot")
    # 4. torch autograd (CPU, float64)
    x = g.normal(0, 2, (5, 33))
    dy = g.normal(0, 1, (5, 33))
    xt = torch.tensor(x, requires_grad=True)
    torch.softmax(xt, dim=-1).backward(torch.tensor(dy))
    if not np.allclose(fn(oracle.safe_softmax(x), dy), xt.grad.numpy(), rtol=1e-12, atol=1e-15):
        failed.append("torch_autograd")
    # 5. sum of dx over a row is zero when y sums to one
    dy = g.normal(0, 1, (4, 50))
    if not np.all(np.abs(fn(y, dy).sum(axis=1)) < 1e-14):
        failed.append("row_sum_zero")
    return failed


def test_oracle_backward_passes_pins():
    assert backward_pins(oracle.softmax_backward) == []


def _mut_sign(y, dy):
    return y * (oracle.safe_softmax(np.zeros_like(y)) * 0 + dy + (dy * y).sum(axis=1, keepdims=True))


def _mut_no_dot(y, dy):
    return y * dy


def _mut_sum_dy(y, dy):
    return y * (dy - dy.sum(axis=1, keepdims=True))


def _mut_missing_y(y, dy):
    return dy - (dy * y).sum(axis=1, keepdims=True)


def _mut_dot_wrong_axis(y, dy):
    return y * (dy - (dy * y).sum(axis=0, keepdims=True))


@pytest.mark.parametrize("mutant", [_mut_sign, _mut_no_dot, _mut_sum_dy, _mut_missing_y,
                                    _mut_dot_wrong_axis], ids=lambda f: f.__name__.strip("_"))
def test_backward_mutants_fail(mutant):
    assert backward_pins(mutant) != []
