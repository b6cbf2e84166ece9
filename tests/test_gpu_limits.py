"""GPU parity at the size limits: the longest row the library takes
(cols = 2^30), row counts that need several launches (beyond 2^31 rows for
the lane-group kernels, 2^22 for the workgroup-per-row kernels) and masked
rows past 2^32 (64-bit row arithmetic).

Inputs that large cannot go through the host oracle element by element, so
they are built on the GPU from closed-form patterns with few distinct rows
(or a period that tiles the row); the oracle computes each distinct pattern
once, and the comparison with that table runs on the GPU over every output
element, in slices.  The 2^22-row cases are small enough to check in full
against the oracle on the host."""
import numpy as np
import pytest
import torch

import oracle
import row_wise_safe_amd as rws
from gpu_util import have_gpu, to_device

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not have_gpu(), reason="needs an MI355X GPU")]

SLICE = 1 << 27


def _free_gib():
    free, _ = torch.cuda.mem_get_info()
    return free / 2 ** 30


def _max_err_vs_table(y, table):
    """max |y[r] - table[r mod period]| over all rows (period = rows of the
    table), on strided views of y, in slices."""
    period = table.shape[0]
    worst = 0.0
    t = torch.from_numpy(table).to("cuda")
    for k in range(period):
        v = y[k::period]
        for r0 in range(0, v.shape[0], SLICE):
            sl = v[r0:r0 + SLICE].to(torch.float64)
            worst = max(worst, float((sl - t[k][None, :]).abs().max()))
            del sl
    return worst


def test_longest_row_fp32():
    # cols = 2^30 (the limit), one row: split-k with 131072 chunks.  The row
    # tiles a 1024-value period, so y = softmax(period) / 2^20 tiled.
    if _free_gib() < 12:
        pytest.skip("needs 12 GiB of free device memory")
    cols, period = 1 << 30, 1024
    g = np.random.Generator(np.random.PCG64(4242))
    p, ps = to_device(g.normal(0.0, 2.0, (1, period)), "f32")
    x = p.reshape(-1).repeat(cols // period).view(1, cols)
    y = torch.empty_like(x)
    print(f"\nlongest row: {rws.softmax_describe_launch(1, cols, rws.RWS_F32, x.data_ptr(), y.data_ptr())}",
          flush=True)
    rws.softmax(x, out=y)
    torch.cuda.synchronize()
    ref = oracle.safe_softmax(ps)[0] / (cols // period)
    refd = torch.from_numpy(ref).to("cuda")[None, :]
    yv = y.view(cols // period, period)
    excess = -1.0
    for r0 in range(0, yv.shape[0], 1 << 16):
        sl = yv[r0:r0 + (1 << 16)].to(torch.float64)
        excess = max(excess, float(((sl - refd).abs() - (1e-5 * refd + 1e-37)).max()))
    assert excess <= 0.0, f"fp32 relative error above 1e-5 (excess {excess:.3e})"
    assert abs(float(torch.sum(y, dtype=torch.float64)) - 1.0) <= 1e-5


def test_rows_beyond_one_grid_fp16():
    # 2^31 + 37 rows of 3 columns: wave_row with 16 rows per wave takes at most
    # 2^29 rows per launch (2^23 workgroups), so five launches.
    # x[r, j] = ((3r + j) mod 13)/4 - 1.5 (exact in fp16): 13 distinct rows.
    rows, cols = (1 << 31) + 37, 3
    if _free_gib() < 30:
        pytest.skip("needs 30 GiB of free device memory")
    x = torch.empty((rows, cols), dtype=torch.float16, device="cuda")
    j = torch.arange(cols, device="cuda", dtype=torch.int64)
    for r0 in range(0, rows, SLICE):
        r1 = min(rows, r0 + SLICE)
        r = torch.arange(r0, r1, device="cuda", dtype=torch.int64)
        x[r0:r1] = (((3 * r[:, None] + j[None, :]) % 13).to(torch.float32) / 4 - 1.5).half()
        del r
    y = torch.empty_like(x)
    print(f"\nrows beyond one grid: "
          f"{rws.softmax_describe_launch(rows, cols, rws.RWS_F16, x.data_ptr(), y.data_ptr())}",
          flush=True)
    rws.softmax(x, out=y)
    torch.cuda.synchronize()
    # row r depends on r mod 13 only
    table = oracle.safe_softmax(
        np.array([[((3 * k + c) % 13) / 4 - 1.5 for c in range(cols)] for k in range(13)]))
    err = _max_err_vs_table(y, table)
    assert err <= 1e-3, f"max abs error {err:.3e}"
    del x, y
    torch.cuda.empty_cache()


def test_masked_rows_beyond_2_32():
    # 2^32 + 5 rows of 2 columns with a [3, 2] mask and causal q = 2: rows
    # past 2^32 take the 64-bit row arithmetic.  x[r, j] = (2 (r mod 7) + j)/4
    # - 1; the output depends on r mod 42 (lcm of 7, 3 and 2).
    rows, cols = (1 << 32) + 5, 2
    if _free_gib() < 45:
        pytest.skip("needs 45 GiB of free device memory")
    x = torch.empty((rows, cols), dtype=torch.float16, device="cuda")
    j = torch.arange(cols, device="cuda", dtype=torch.int64)
    for r0 in range(0, rows, SLICE):
        r1 = min(rows, r0 + SLICE)
        r = torch.arange(r0, r1, device="cuda", dtype=torch.int64)
        x[r0:r1] = ((2 * (r[:, None] % 7) + j[None, :]).to(torch.float32) / 4 - 1).half()
        del r
    mask64 = np.array([[0.5, -0.25], [-1.0, 0.75], [0.0, 1.5]])
    mask, mask_s = to_device(mask64, "f16")
    y = torch.empty_like(x)
    rws.softmax_masked(x, 0.5, mask, causal_q=2, out=y)
    torch.cuda.synchronize()
    xt = np.array([[(2 * (k % 7) + c) / 4 - 1 for c in range(cols)] for k in range(42)])
    table = oracle.masked_softmax(xt, 0.5, mask_s, causal_q=2)
    err = _max_err_vs_table(y, table)
    assert err <= 1e-3, f"max abs error {err:.3e}"
    # rows with r mod 2 == 0 see column 0 only: exactly [1, 0]
    assert float(y[-5, 0]) == 1.0 and float(y[-5, 1]) == 0.0  # row 2^32 is even
    del x, y
    torch.cuda.empty_cache()


ROWS_BLOCK = (1 << 22) + 5  # one more batch than a workgroup-per-row launch takes


@pytest.mark.parametrize("kernel", ["block_onepass", "two_pass"])
def test_block_families_beyond_one_batch(kernel):
    g = np.random.Generator(np.random.PCG64(77))
    x64 = g.normal(0.0, 3.0, (ROWS_BLOCK, 24))
    x, xs = to_device(x64, "f16")
    y = torch.empty_like(x)
    rws.softmax(x, out=y, kernel=kernel)
    torch.cuda.synchronize()
    err = np.abs(y.to(torch.float64).cpu().numpy() - oracle.safe_softmax(xs)).max()
    assert err <= 1e-3, f"{kernel}: max abs error {err:.3e}"


@pytest.mark.parametrize("kernel", ["block_onepass", "two_pass"])
def test_backward_and_norms_beyond_one_batch(kernel):
    g = np.random.Generator(np.random.PCG64(78))
    cols = 24
    y64 = oracle.safe_softmax(g.normal(0.0, 2.0, (ROWS_BLOCK, cols)))
    yd, ys = to_device(y64, "f32")
    dyd, gs = to_device(g.normal(0.0, 1.0, (ROWS_BLOCK, cols)), "f32")
    dx = rws.softmax_backward(yd, dyd, kernel=kernel)
    torch.cuda.synchronize()
    ref = oracle.softmax_backward(ys, gs)
    s_abs = np.abs(ys * gs).sum(axis=1, keepdims=True)
    bound = 2e-5 * ys * (np.abs(gs) + s_abs) + 1e-37
    assert np.all(np.abs(dx.double().cpu().numpy() - ref) <= bound), f"backward {kernel}"
    del yd, dyd, dx

    x64 = g.normal(1.0, 2.0, (ROWS_BLOCK, cols))
    x, xs = to_device(x64, "f32")
    out = rws.layer_norm(x, 1e-5, kernel=kernel)
    torch.cuda.synchronize()
    ref = oracle.layernorm(xs, 1e-5)
    c = 256 * 2.0 ** -24
    mu_bound = c * np.abs(xs).mean(axis=1, keepdims=True)
    rs = oracle.layernorm(xs, 1e-5, return_stats=True)[2][:, None]
    bound = mu_bound * rs + (c + 0.5 * (mu_bound * rs) ** 2) * np.abs(ref) + 2.0 ** -23 * np.abs(ref)
    assert np.all(np.abs(out.double().cpu().numpy() - ref) <= bound + 1e-37), f"layernorm {kernel}"
