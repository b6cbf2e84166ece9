"""GPU parity on rows shifted far from zero, through every form that merges
partial (m, d) pairs taken against different maxima: the running update of
two_pass (and its masked form), and the three split-k forms.

Softmax is shift invariant (CUDA safe-online-softmax page, section 1: the
maximum is subtracted for exactly that reason), so x + c must give the same
outputs as x.  Each kernel subtracts fl(m * log2 e) in the exponent; partial
sums taken against different chunk maxima m_c each carry the rounding error
of their own product, which the merge has to account for.  With fp32 rows of
c + N(0, 1), c in {1e3, 1e4, 1e5}, a merge that ignored it was off by about
1e-5, 1e-4 and 2e-3 relative; the bar is 1e-5.
"""
import numpy as np
import pytest
import torch

import oracle
import row_wise_safe_amd as rws
from gpu_util import NotCoResident, have_gpu, run, to_device
from tolerance import check

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not have_gpu(), reason="needs an MI355X GPU")]

MERGING = ["two_pass", "splitk", "splitk_ordered", "splitk_fused", "auto"]


@pytest.fixture(scope="module", autouse=True)
def _lib():
    rws.load_library()
    yield


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shift", [1.0e3, 1.0e4, 1.0e5, -1.0e5])
@pytest.mark.parametrize("rows,cols", [(4, 200003), (2, 1 << 20), (33, 5000)])
def test_shifted_rows_every_merging_kernel(dtype, shift, rows, cols):
    g = np.random.Generator(np.random.PCG64(int(abs(shift)) + cols))
    x64 = shift + g.normal(0.0, 1.0, (rows, cols))
    x, stored = to_device(x64, dtype)
    ref = oracle.safe_softmax(stored)
    for kernel in MERGING:
        print(f"shifted {dtype} {shift:g} [{rows},{cols}] {kernel}", flush=True)
        try:
            y = run(x, torch.empty_like(x), kernel)
        except NotCoResident:
            continue
        check(y, ref, dtype, f"{kernel} shift={shift:g} [{rows},{cols}]")


@pytest.mark.parametrize("shift", [1.0e4, 1.0e5])
def test_shifted_rows_masked_two_pass(shift):
    # the masked form's running update: scale 1, a mask of zeros except a
    # few -inf, rows long enough for two_pass
    rows, cols = 6, 70001
    g = np.random.Generator(np.random.PCG64(int(shift) + 7))
    x, xs = to_device(shift + g.normal(0.0, 1.0, (rows, cols)), "f32")
    m64 = np.zeros((2, cols))
    m64[0, ::101] = -np.inf
    mask, ms = to_device(m64, "f32")
    print(f"shifted masked {shift:g}", flush=True)
    y = rws.softmax_masked(x, 1.0, mask, kernel="two_pass")
    torch.cuda.synchronize()
    ref = oracle.masked_softmax(xs, 1.0, ms)
    check(y.double().cpu().numpy(), ref, "f32", f"masked two_pass shift={shift:g}")
