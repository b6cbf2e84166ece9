"""GPU parity for every launch shape the dispatcher can choose for rows held
by one workgroup (block_onepass: one granule per thread when a launch has few
waves, 2-5 granules per thread with the fewest idle slots for many rows, the
long-row shapes), plain and masked.

The shapes are found on the host: row lengths are scanned and the first
(rows, cols) for which the dispatcher describes each shape is kept; rows are
16 (few waves) or just above the few-waves limit (many rows).  Each case runs
through the dispatcher and is compared with the oracle on every row.
"""
import re

import numpy as np
import pytest
import torch

import oracle
import row_wise_safe_amd as rws
from gpu_util import have_gpu, run, to_device
from tolerance import check

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not have_gpu(), reason="needs an MI355X GPU")]

ES = {"f32": 4, "f16": 2, "bf16": 2}
CODE = {"f32": rws.RWS_F32, "f16": rws.RWS_F16, "bf16": rws.RWS_BF16}
FEW_WAVES = 32 * 256  # the dispatcher's limit for 256 CUs, in waves


def _cases(dtype: str, few: bool, masked: bool):
    """{(B, KR, KL): (rows, cols)} over row windows up to 16384 granules."""
    es = ES[dtype]
    seen = {}
    step = 16 // es  # one granule more per step
    for cols in range(step, 16384 * step, step):
        w = (cols * es + 143) // 16
        rows = 16 if few else FEW_WAVES // min((w + 63) // 64, 16) + 1
        desc = rws.softmax_describe_launch(rows, cols, CODE[dtype], 256, 512, 0, masked=masked)
        m = re.match(r"block_onepass<[^>]*B=(\d+),KR=(\d+),KL=(\d+)>", desc)
        if m:
            seen.setdefault(tuple(int(v) for v in m.groups()), (rows, cols))
    return seen


@pytest.fixture(scope="module", autouse=True)
def _lib():
    rws.load_library()
    yield


@pytest.mark.parametrize("dtype", ["f16", "f32"])
@pytest.mark.parametrize("few", [True, False])
def test_every_block_shape(dtype, few):
    cases = _cases(dtype, few, masked=False)
    assert len(cases) >= (6 if few else 10), cases
    for (b, kr, kl), (rows, cols) in sorted(cases.items()):
        x64 = np.random.Generator(np.random.PCG64(rows * 31 + cols)).normal(0.0, 4.0, (rows, cols))
        x, stored = to_device(x64, dtype)
        desc = rws.softmax_describe_launch(rows, cols, CODE[dtype], x.data_ptr(), x.data_ptr())
        assert f"B={b},KR={kr},KL={kl}" in desc, desc
        y = run(x, torch.empty_like(x))
        check(y, oracle.safe_softmax(stored), dtype, f"{desc} rows={rows} cols={cols}")
        del x, y


@pytest.mark.parametrize("few", [True, False])
def test_every_masked_block_shape(few):
    dtype = "f16"
    cases = _cases(dtype, few, masked=True)
    assert len(cases) >= (6 if few else 10), cases
    for (b, kr, kl), (rows, cols) in sorted(cases.items()):
        assert kl == 0
        g = np.random.Generator(np.random.PCG64(rows * 37 + cols))
        x, xs = to_device(g.normal(0.0, 4.0, (rows, cols)), dtype)
        mask, ms = to_device(g.normal(0.0, 1.0, (5, cols)), dtype)
        causal = min(cols, 7)
        y = rws.softmax_masked(x, 0.25, mask, causal_q=causal)
        torch.cuda.synchronize()
        ref = oracle.masked_softmax(xs, 0.25, ms, causal_q=causal)
        check(y.double().cpu().numpy(), ref, dtype, f"masked B={b},KR={kr} rows={rows} cols={cols}")
        del x, y


def _norm_cases(dtype: str, few: bool):
    """{(B, KR): (rows, cols)} of the normalisations' workgroup-per-row shapes."""
    es = ES[dtype]
    seen = {}
    step = 16 // es
    for cols in range(step, 4096 * step, step):
        w = (cols * es + 143) // 16
        rows = 16 if few else FEW_WAVES // min((w + 63) // 64, 16) + 1
        desc = rws.norm_describe_launch(rows, cols, CODE[dtype], 256, 512)
        m = re.match(r"norm_block<[^>]*B=(\d+),KR=(\d+)>", desc)
        if m:
            seen.setdefault(tuple(int(v) for v in m.groups()), (rows, cols))
    return seen


@pytest.mark.parametrize("dtype", ["f16", "f32"])
@pytest.mark.parametrize("few", [True, False])
def test_every_norm_block_shape(dtype, few):
    from test_gpu_norm import _case
    cases = _norm_cases(dtype, few)
    assert len(cases) >= (6 if few else 10), cases
    for (b, kr), (rows, cols) in sorted(cases.items()):
        for mode in ("layernorm", "rmsnorm"):
            _case(mode, dtype, rows, cols, "auto", seed=rows * 7 + cols + kr)


def _bwd_cases(dtype: str):
    """{(B, KR): (rows, cols)} of the backward's workgroup-per-row shapes."""
    es = ES[dtype]
    seen = {}
    step = 16 // es
    for cols in range(step, 4096 * step, step):
        # 192 rows: beyond the few-rows limit of the ordered split-k
        desc = rws.softmax_bwd_describe_launch(192, cols, CODE[dtype], 256, 512)
        m = re.match(r"bwd_block<[^>]*B=(\d+),KR=(\d+)>", desc)
        if m:
            seen.setdefault(tuple(int(v) for v in m.groups()), (192, cols))
    return seen


@pytest.mark.parametrize("dtype", ["f16", "f32"])
def test_every_bwd_block_shape(dtype):
    from test_gpu_backward import _check as check_backward
    cases = _bwd_cases(dtype)
    assert len(cases) >= 13, cases
    for (b, kr), (rows, cols) in sorted(cases.items()):
        g = np.random.Generator(np.random.PCG64(rows * 11 + cols))
        y, ys = to_device(oracle.safe_softmax(g.normal(0.0, 2.0, (rows, cols))), dtype)
        dy, gs = to_device(g.normal(0.0, 1.0, (rows, cols)), dtype)
        desc = rws.softmax_bwd_describe_launch(rows, cols, CODE[dtype], y.data_ptr(), y.data_ptr())
        assert f"B={b},KR={kr}" in desc, desc
        dx = rws.softmax_backward(y, dy)
        torch.cuda.synchronize()
        check_backward(dx.double().cpu().numpy(), ys, gs, dtype, f"{desc} rows={rows} cols={cols}")


# Long 16-bit rows at 8 register granules per thread take the raw-granule
# form (k_block_onepass_raw), with and without LDS parking, on line-aligned
# rows and on rows that are not; a row of -inf except one entry, and a ragged
# tail, are in every case.
@pytest.mark.parametrize("dtype,cols", [("bf16", 50257), ("f16", 49153), ("f16", 65536),
                                        ("bf16", 65536), ("f16", 128256), ("bf16", 120000)])
def test_raw_long_rows(dtype, cols):
    rows = 6
    g = np.random.Generator(np.random.PCG64(cols))
    x64 = g.normal(0.0, 3.0, (rows, cols))
    x64[2, :] = -np.inf
    x64[2, cols // 3] = 1.0
    x, xs = to_device(x64, dtype)
    desc = rws.softmax_describe_launch(rows, cols, CODE[dtype], x.data_ptr(), x.data_ptr(),
                                       rws.KERNEL_IDS["block_onepass"])
    assert "KR=8" in desc, desc
    y = run(x, torch.empty_like(x), "block_onepass")
    check(y, oracle.safe_softmax(xs), dtype, f"{desc} cols={cols}")
