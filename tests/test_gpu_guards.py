"""GPU: no byte outside the output rows is written by the masked softmax, the
softmax backward, LayerNorm and RMSNorm, for every kernel family they have.

The output sits inside a buffer filled with a sentinel, with 64 guard
elements on each side.  The input starts 3 elements into its buffer (rows of
every 16-byte phase); the output at guard + 0 elements (another phase: every
partial granule is stored element by element) or guard + 3 (the input's
phase: partial granules go out as naturally aligned 2-, 4- and 8-byte
pieces).  Values are checked against the oracle with the tolerances of the
respective parity tests.
"""
import numpy as np
import pytest
import torch

import oracle
import row_wise_safe_amd as rws
from gpu_util import have_gpu, supports, to_device
from test_gpu_backward import _check as check_backward
from test_gpu_norm import _check as check_norm
from tolerance import check

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not have_gpu(), reason="needs an MI355X GPU")]

DTYPES = ["f32", "f16", "bf16"]
KERNELS = ["auto", "wave_row", "block_onepass", "two_pass"]
ROWS, GUARD, X_OFF = 7, 64, 3


def _guarded(like, off):
    buf = torch.full((like.numel() + 2 * GUARD + off,), -7.0, dtype=like.dtype, device="cuda")
    before = buf.clone()
    out = buf[GUARD + off:GUARD + off + like.numel()].view(like.shape)
    return buf, before, out


def _assert_guards(buf, before, off, n, what):
    torch.cuda.synchronize()
    lo, hi = GUARD + off, GUARD + off + n
    assert torch.equal(buf[:lo], before[:lo]), f"{what}: head guard written"
    assert torch.equal(buf[hi:], before[hi:]), f"{what}: tail guard written"


def _x(cols, dtype, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    return to_device(g.normal(0.0, 3.0, (ROWS, cols)), dtype, offset=X_OFF)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("cols", [3, 129, 4097])
@pytest.mark.parametrize("off", [0, 3])
def test_masked_guards(dtype, cols, off):
    x, xs = _x(cols, dtype, seed=cols + 11)
    g = np.random.Generator(np.random.PCG64(cols + 12))
    mask, ms = to_device(g.normal(0.0, 1.0, (3, cols)), dtype, offset=1)
    causal = min(cols, 5)
    ref = oracle.masked_softmax(xs, 0.5, ms, causal_q=causal)
    for kernel in KERNELS:
        if kernel != "auto" and not supports(kernel, cols, dtype, False):
            continue
        buf, before, out = _guarded(x, off)
        rws.softmax_masked(x, 0.5, mask, causal_q=causal, out=out, kernel=kernel)
        what = f"masked {kernel} {dtype} cols={cols} out+{off}"
        _assert_guards(buf, before, off, x.numel(), what)
        check(out.double().cpu().numpy(), ref, dtype, what)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("cols", [3, 129, 4097])
@pytest.mark.parametrize("off", [0, 3])
def test_backward_guards(dtype, cols, off):
    g = np.random.Generator(np.random.PCG64(cols + 21))
    y, ys = to_device(oracle.safe_softmax(g.normal(0.0, 2.0, (ROWS, cols))), dtype, offset=X_OFF)
    dy, gs = to_device(g.normal(0.0, 1.0, (ROWS, cols)), dtype, offset=X_OFF)
    for kernel in KERNELS:
        if kernel != "auto" and not supports(kernel, cols, dtype, False):
            continue
        buf, before, out = _guarded(y, off)
        rws.softmax_backward(y, dy, out=out, kernel=kernel)
        what = f"backward {kernel} {dtype} cols={cols} out+{off}"
        _assert_guards(buf, before, off, y.numel(), what)
        check_backward(out.double().cpu().numpy(), ys, gs, dtype, what)


@pytest.mark.parametrize("mode", ["layernorm", "rmsnorm"])
@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("cols", [3, 129, 4097])
@pytest.mark.parametrize("off", [0, 3])
def test_norm_guards(mode, dtype, cols, off):
    x, xs = _x(cols, dtype, seed=cols + 31)
    for kernel in KERNELS:
        if kernel != "auto" and not supports(kernel, cols, dtype, False):
            continue
        buf, before, out = _guarded(x, off)
        if mode == "layernorm":
            rws.layer_norm(x, 1e-5, out=out, kernel=kernel)
        else:
            rws.rms_norm(x, 1e-5, out=out, kernel=kernel)
        what = f"{mode} {kernel} {dtype} cols={cols} out+{off}"
        _assert_guards(buf, before, off, x.numel(), what)
        check_norm(mode, dtype, out.double().cpu().numpy(), xs, 1e-5, None, None, what)
