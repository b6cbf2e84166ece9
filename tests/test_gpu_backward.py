"""GPU parity of softmax_bwd against the oracle's softmax_backward.

Tolerance (derived from the arithmetic, the pages state none for the
backward): the kernels accumulate the row's dot product and evaluate
y*(dy - dot) in fp32 and round once to the output dtype, so per element
    |dx - ref| <= r * |ref| + 2e-5 * y * (|dy| + sum_i |y_i dy_i|) + floor
with r the output's half-ulp (fp32 0, fp16 2^-11, bf16 2^-8) and floor its
smallest step (fp16 2^-25, otherwise 1e-37).  The middle term bounds the fp32
cancellation in dy - dot and the rounding of the dot product."""
import numpy as np
import pytest
import torch

import oracle
import row_wise_safe_amd as rws
from gpu_util import empty_like_at, have_gpu, to_device

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not have_gpu(), reason="needs an MI355X GPU")]

DTYPES = ["f32", "f16", "bf16"]
KERNELS = ["auto", "wave_row", "block_onepass", "two_pass"]
HALF_ULP = {"f32": 0.0, "f16": 2.0 ** -11, "bf16": 2.0 ** -8}
FLOOR = {"f32": 1e-37, "f16": 2.0 ** -25, "bf16": 1e-37}


def _supports(kernel, cols, dtype):
    es = 4 if dtype == "f32" else 2
    w = (cols * es + 143) // 16
    if kernel == "wave_row":
        return w <= 512
    if kernel == "block_onepass":
        return w <= 4096
    return True


def _inputs(rows, cols, dtype, seed, offs=(0, 0)):
    g = np.random.Generator(np.random.PCG64(seed))
    y64 = oracle.safe_softmax(g.normal(0.0, 2.0, (rows, cols)))
    y, ys = to_device(y64, dtype, offset=offs[0])
    dy, gs = to_device(g.normal(0.0, 1.0, (rows, cols)), dtype, offset=offs[1])
    return y, ys, dy, gs


def _check(dx, ys, gs, dtype, what):
    ref = oracle.softmax_backward(ys, gs)
    s_abs = np.abs(ys * gs).sum(axis=1, keepdims=True)
    bound = HALF_ULP[dtype] * np.abs(ref) + 2e-5 * ys * (np.abs(gs) + s_abs) + FLOOR[dtype]
    err = np.abs(dx - ref)
    assert np.all(np.isfinite(dx)), f"{what}: non-finite"
    worst = np.max(err - bound)
    assert worst <= 0.0, f"{what}: error exceeds bound by {worst:.3e} (max err {err.max():.3e})"
    # sum_j dx_j = dot * (1 - sum_j y_j): small when the stored y sums to ~1
    lhs = np.abs(dx.sum(axis=1))
    rhs = np.abs((ys * gs).sum(axis=1) * (1.0 - ys.sum(axis=1))) + bound.sum(axis=1)
    assert np.all(lhs <= rhs), f"{what}: row sums"


def _run(y, dy, out, kernel):
    rws.softmax_backward(y, dy, out=out, kernel=kernel)
    torch.cuda.synchronize()
    return out.double().cpu().numpy()


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("cols", [1, 3, 8, 64, 65, 129, 512, 1000, 1025, 4097, 8193, 40000,
                                  300001])
def test_backward_sweep(dtype, cols):
    rows = 67 if cols <= 1025 else 3
    y, ys, dy, gs = _inputs(rows, cols, dtype, seed=cols)
    for kernel in KERNELS:
        if not _supports(kernel, cols, dtype):
            continue
        dx = _run(y, dy, torch.empty_like(y), kernel)
        _check(dx, ys, gs, dtype, f"{kernel} cols={cols}")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("offs", [(1, 1), (0, 1), (3, 0)])
def test_backward_phases(dtype, offs):
    rows, cols = 9, 777
    y, ys, dy, gs = _inputs(rows, cols, dtype, seed=5, offs=offs)
    for kernel in KERNELS:
        for oo in (0, 2):
            dx = _run(y, dy, empty_like_at(y, oo), kernel)
            _check(dx, ys, gs, dtype, f"{kernel} offs={offs} out+{oo}")


@pytest.mark.parametrize("kernel", KERNELS)
def test_backward_in_place(kernel):
    y, ys, dy, gs = _inputs(33, 2049, "f16", seed=6, offs=(1, 1))
    dx = _run(y, dy, dy, kernel)  # dx overwrites dy
    _check(dx, ys, gs, "f16", f"in place {kernel}")


def test_backward_attention_workload():
    w = __import__("workloads").WORKLOADS["fp16_attn_4x32x512x512"]
    x64 = w.generate(rows=8192)
    ys64 = oracle.safe_softmax(torch.from_numpy(x64).half().double().numpy())
    y, ys = to_device(ys64, "f16")
    dy, gs = to_device(np.random.Generator(np.random.PCG64(7)).normal(0, 1, ys.shape), "f16")
    dx = _run(y, dy, torch.empty_like(y), "auto")
    _check(dx, ys, gs, "f16", "attention rows")


def test_backward_rejects_split_kernels():
    # the two-launch and fused split-k forms exist for the forward only
    # (the backward's split-k is the ordered form)
    y = torch.zeros(2, 64, dtype=torch.float16, device="cuda")
    for kernel in ("splitk", "splitk_fused"):
        st = rws.softmax_bwd_kernel(y.data_ptr(), y.data_ptr(), y.data_ptr(), 2, 64, rws.RWS_F16,
                                    0, rws.KERNEL_IDS[kernel])
        assert st == rws.RWS_ERR_INVALID_ARG


# --------------------------------------------------------------------------
# tile_rows: several short rows per wave as one 16-byte-aligned range
# --------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("cols", [9, 33, 100, 250, 333, 500, 1001])
def test_tile_rows_form(dtype, cols):
    from gpu_util import tile_supports
    if not tile_supports(cols, dtype):
        pytest.skip("outside the tile rows")
    es = 4 if dtype == "f32" else 2
    for rows in (64, 67, 777):
        y, ys, dy, gs = _inputs(rows, cols, dtype, seed=cols * 13 + rows)
        dx = empty_like_at(y)
        desc = rws.softmax_bwd_describe_launch(rows, cols, rws.dtype_code(y.dtype), y.data_ptr(),
                                               dx.data_ptr())
        rb = cols * es
        if rb <= 2048 and rb % 128 and (rb % 16 or rb > 128):
            assert desc.startswith("bwd_tile<"), desc
        for kernel in ("auto", "tile_rows"):
            _run(y, dy, dx, kernel)
            torch.cuda.synchronize()
            _check(dx.double().cpu().numpy(), ys, gs, dtype, f"{kernel} {desc} rows={rows}")


def test_tile_rows_form_in_place_and_refusals():
    rows, cols = 70, 77
    y, ys, dy, gs = _inputs(rows, cols, "f16", seed=5)
    _run(y, dy, dy, "tile_rows")  # dx aliases dy
    torch.cuda.synchronize()
    _check(dy.double().cpu().numpy(), ys, gs, "f16", "tile_rows in place")
    # dy that is not 16-byte aligned: refused by the tile form, another form for auto
    y2, ys2, dy2, gs2 = _inputs(rows, cols, "f16", seed=6, offs=(0, 1))
    dx2 = empty_like_at(y2)
    st = rws.softmax_bwd_kernel(y2.data_ptr(), dy2.data_ptr(), dx2.data_ptr(), rows, cols,
                                rws.RWS_F16, torch.cuda.current_stream().cuda_stream,
                                rws.KERNEL_IDS["tile_rows"])
    assert st == rws.RWS_ERR_UNSUPPORTED_SHAPE
    _run(y2, dy2, dx2, "auto")
    torch.cuda.synchronize()
    _check(dx2.double().cpu().numpy(), ys2, gs2, "f16", "auto, dy unaligned")


@pytest.mark.parametrize("dtype,rows,cols", [("f16", 1000003, 33), ("f16", 1048583, 100),
                                             ("bf16", 262147, 120)])
def test_tile_rows_form_large_launch_sampled_rows(dtype, rows, cols):
    # the dispatcher's tile at full size: sampled rows (both ends, the
    # partial last tile among them, and seeded random rows) against the oracle
    from gpu_util import TORCH_DTYPE
    gen = torch.Generator(device="cuda").manual_seed(rows * 5 + cols)
    tdt = TORCH_DTYPE[dtype]
    y = torch.softmax(torch.randn(rows, cols, generator=gen, device="cuda") * 2.0, dim=1).to(tdt)
    dy = torch.randn(rows, cols, generator=gen, device="cuda").to(tdt)
    dx = torch.empty_like(y)
    desc = rws.softmax_bwd_describe_launch(rows, cols, rws.dtype_code(tdt), y.data_ptr(),
                                           dx.data_ptr())
    assert desc.startswith("bwd_tile<"), desc
    rws.softmax_backward(y, dy, out=dx)
    torch.cuda.synchronize()
    print(desc, flush=True)
    rng = np.random.Generator(np.random.PCG64(rows))
    idx = np.unique(np.concatenate([np.arange(200), np.arange(rows - 200, rows),
                                    rng.integers(0, rows, 600)]))
    ti = torch.from_numpy(idx).cuda()
    ys = y.index_select(0, ti).double().cpu().numpy()
    gs = dy.index_select(0, ti).double().cpu().numpy()
    _check(dx.index_select(0, ti).double().cpu().numpy(), ys, gs, dtype, f"{desc} sampled rows")
