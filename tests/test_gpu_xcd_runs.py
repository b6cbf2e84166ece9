"""GPU: the workgroup-per-row kernels that give each XCD runs of consecutive
rows (block_onepass, masked block_onepass, the backward's bwd_block) cover
every row exactly once and match the oracle.

Rows of 1000 fp16 values (2000 bytes, not line-aligned) go in runs of 128
rows, spans of 8 * 128 = 1024 rows; the row counts cover a partial span only,
exactly one and two spans, and spans plus a partial one.  The output starts
inside a sentinel-filled buffer, so a row left unwritten, or written past the
tensor, fails."""
import numpy as np
import pytest
import torch

import oracle
import row_wise_safe_amd as rws
from gpu_util import have_gpu, to_device
from test_gpu_backward import _check as check_backward
from tolerance import check

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not have_gpu(), reason="needs an MI355X GPU")]

COLS, RUN, GUARD = 1000, 128, 64
ROWS = [1023, 1024, 1025, 2048, 2048 + 577]


def _guarded_out(like):
    buf = torch.full((like.numel() + 2 * GUARD,), -5.0, dtype=like.dtype, device="cuda")
    return buf, buf[GUARD:GUARD + like.numel()].view(like.shape)


def _guards_intact(buf, n):
    torch.cuda.synchronize()
    return bool(torch.all(buf[:GUARD] == -5.0)) and bool(torch.all(buf[GUARD + n:] == -5.0))


def test_run_length_is_described():
    rws.load_library()
    desc = rws.softmax_describe_launch(4096, COLS, rws.RWS_F16, 256, 512)
    assert desc.startswith("block_onepass") and f"xcd_run={RUN}" in desc, desc


@pytest.mark.parametrize("rows", ROWS)
def test_forward_rows_once(rows):
    g = np.random.Generator(np.random.PCG64(rows))
    x, xs = to_device(g.normal(0.0, 4.0, (rows, COLS)), "f16")
    buf, out = _guarded_out(x)
    rws.softmax(x, out=out)
    assert _guards_intact(buf, x.numel())
    check(out.double().cpu().numpy(), oracle.safe_softmax(xs), "f16", f"rows={rows}")


@pytest.mark.parametrize("rows", ROWS)
def test_masked_rows_once(rows):
    g = np.random.Generator(np.random.PCG64(rows + 1))
    x, xs = to_device(g.normal(0.0, 4.0, (rows, COLS)), "f16")
    mask, ms = to_device(g.normal(0.0, 1.0, (7, COLS)), "f16")
    buf, out = _guarded_out(x)
    rws.softmax_masked(x, 0.5, mask, causal_q=300, out=out)
    assert _guards_intact(buf, x.numel())
    ref = oracle.masked_softmax(xs, 0.5, ms, causal_q=300)
    check(out.double().cpu().numpy(), ref, "f16", f"masked rows={rows}")


@pytest.mark.parametrize("rows", ROWS)
def test_backward_rows_once(rows):
    g = np.random.Generator(np.random.PCG64(rows + 2))
    y, ys = to_device(oracle.safe_softmax(g.normal(0.0, 2.0, (rows, COLS))), "f16")
    dy, gs = to_device(g.normal(0.0, 1.0, (rows, COLS)), "f16")
    buf, out = _guarded_out(y)
    rws.softmax_backward(y, dy, out=out)
    assert _guards_intact(buf, y.numel())
    check_backward(out.double().cpu().numpy(), ys, gs, "f16", f"backward rows={rows}")
