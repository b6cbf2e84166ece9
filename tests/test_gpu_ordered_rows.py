"""GPU parity of the single-launch split-k forms of the softmax backward
(bwd_ordered) and of LayerNorm / RMSNorm (norm_ordered), which the
dispatcher takes for few long rows.

Cases: the dispatcher's choice on fp16 [16, 2^20] (128 chunks per row);
the forms forced on short and ragged rows of every dtype, with unaligned and
split-phase pointers, weight and bias on and off the rows' phase, and the
statistics outputs; back-to-back calls on one stream interleaved with the
forward's ordered split-k, which shares the epoch-tagged words.  Tolerances
are the backward's and the normalisations' (test_gpu_backward,
test_gpu_norm): the partials only regroup the same fp32 sums."""
import numpy as np
import pytest
import torch

import oracle
import row_wise_safe_amd as rws
from gpu_util import empty_like_at, have_gpu, to_device
from test_gpu_backward import _check as check_backward
from test_gpu_norm import _case as norm_case
from tolerance import check

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not have_gpu(), reason="needs an MI355X GPU")]

CODE = {"f32": rws.RWS_F32, "f16": rws.RWS_F16, "bf16": rws.RWS_BF16}


def _bwd_inputs(rows, cols, dtype, seed, offs=(0, 0)):
    g = np.random.Generator(np.random.PCG64(seed))
    y, ys = to_device(oracle.safe_softmax(g.normal(0.0, 2.0, (rows, cols))), dtype, offset=offs[0])
    dy, gs = to_device(g.normal(0.0, 1.0, (rows, cols)), dtype, offset=offs[1])
    return y, ys, dy, gs


def test_backward_few_long_rows_auto():
    rows, cols = 16, 1 << 20
    y, ys, dy, gs = _bwd_inputs(rows, cols, "f16", 5)
    desc = rws.softmax_bwd_describe_launch(rows, cols, rws.RWS_F16, y.data_ptr(), y.data_ptr())
    assert desc.startswith("bwd_ordered") and "P=128" in desc, desc
    dx = rws.softmax_backward(y, dy)
    torch.cuda.synchronize()
    check_backward(dx.double().cpu().numpy(), ys, gs, "f16", desc)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("cols", [1, 1000, 5003, 70001])
@pytest.mark.parametrize("offs", [(0, 0, 0), (3, 3, 1), (1, 2, 0)])
def test_backward_forced(dtype, cols, offs):
    rows = 7
    y, ys, dy, gs = _bwd_inputs(rows, cols, dtype, cols + offs[0], offs[:2])
    out = empty_like_at(y, offs[2])
    rws.softmax_backward(y, dy, out=out, kernel="splitk_ordered")
    torch.cuda.synchronize()
    check_backward(out.double().cpu().numpy(), ys, gs, dtype,
                   f"bwd_ordered {dtype} cols={cols} offs={offs}")


@pytest.mark.parametrize("mode", ["layernorm", "rmsnorm"])
def test_norm_few_long_rows_auto(mode):
    rows, cols = 16, 1 << 20
    desc = rws.norm_describe_launch(rows, cols, rws.RWS_F16, 256, 512, affine=True)
    assert desc.startswith("norm_ordered") and "P=128" in desc, desc
    norm_case(mode, "f16", rows, cols, "auto", seed=11)


@pytest.mark.parametrize("mode", ["layernorm", "rmsnorm"])
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("cols", [1, 999, 5003, 70001])
def test_norm_forced(mode, dtype, cols):
    for i, (affine, x_off, out_off, w_off) in enumerate(
            [(False, 0, 0, 0), (True, 0, 0, 0), (True, 3, 3, 2), (True, 1, 0, 0)]):
        norm_case(mode, dtype, 9, cols, "splitk_ordered", seed=cols * 4 + i, affine=affine,
                  x_off=x_off, out_off=out_off, w_off=w_off)


def test_back_to_back_with_forward_ordered():
    # the three ordered forms share one stream's tag words and epoch counter
    rows, cols = 12, 300000
    g = np.random.Generator(np.random.PCG64(3))
    x, xs = to_device(g.normal(0.0, 3.0, (rows, cols)), "f16")
    y, ys, dy, gs = _bwd_inputs(rows, cols, "f16", 4)
    ref_fwd = oracle.safe_softmax(xs)
    for it in range(3):
        out = rws.softmax(x, kernel="splitk_ordered")
        dx = rws.softmax_backward(y, dy, kernel="splitk_ordered")
        ln = rws.layer_norm(x, 1e-5, kernel="splitk_ordered")
        torch.cuda.synchronize()
        check(out.double().cpu().numpy(), ref_fwd, "f16", f"forward, call {it}")
        check_backward(dx.double().cpu().numpy(), ys, gs, "f16", f"backward, call {it}")
        ref_ln = oracle.layernorm(xs, 1e-5)
        err = np.abs(ln.double().cpu().numpy() - ref_ln).max()
        assert err <= 2.0 ** -8 * 2, f"layernorm, call {it}: max abs error {err:.3e}"
