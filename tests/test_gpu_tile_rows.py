"""GPU parity of tile_rows (several short rows per wave as one 16-byte-aligned
range, rows reduced across the lanes that hold them) against the oracle.

Every compiled (rows per tile, granules per lane) shape in three dtypes,
row lengths that put the row boundaries at every position inside a granule,
row counts that leave a partial last tile (and a tensor end inside a
granule), in place, extreme and non-finite values, the dispatcher's choice,
and the refusals (pointers not 16-byte aligned, rows too short or too long).
"""
import numpy as np
import pytest
import torch

import oracle
import row_wise_safe_amd as rws
from gpu_util import empty_like_at, have_gpu, tile_supports, to_device
from tolerance import check

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not have_gpu(), reason="needs an MI355X GPU")]

DTYPES = ["f32", "f16", "bf16"]
ES = {"f32": 4, "f16": 2, "bf16": 2}
TILE = rws.KERNEL_IDS["tile_rows"]


@pytest.fixture(scope="module", autouse=True)
def _lib():
    rws.load_library()
    yield


def _describe(rows, cols, dtype, x, y, variant=None):
    code = rws.dtype_code(x.dtype)
    if variant is None:
        return rws.softmax_describe_launch(rows, cols, code, x.data_ptr(), y.data_ptr(), TILE)
    return rws.softmax_describe_variant(rows, cols, code, x.data_ptr(), y.data_ptr(), TILE, variant)


def _run_variant(x, y, variant):
    rows, cols = x.shape
    st = rws.softmax_fwd_variant(x.data_ptr(), y.data_ptr(), rows, cols, rws.dtype_code(x.dtype),
                                 torch.cuda.current_stream().cuda_stream, TILE, variant)
    assert st == rws.RWS_OK, rws.softmax_last_error()


def _period(cols, es):
    """Rows after which a row starts on the same 16-byte phase again."""
    g = 16
    while (cols * es) % g:
        g //= 2
    return 16 // g


def _rows_per_tile(cols, es, K):
    """The tile height the library takes for K granules per lane: the largest
    multiple of the rows' 16-byte period, at most 64, whose tile fits 64*K
    granules (0 below 4 rows)."""
    if cols * es > 1024 or cols < 16 // es:
        return 0
    p0 = _period(cols, es)
    t = min(64, 64 * K * 16 // (cols * es))
    t -= t % p0
    return t if t >= 4 else 0


@pytest.mark.parametrize("dtype", DTYPES)
def test_every_variant_and_tile_height(dtype):
    # every compiled K (granules per lane) over row lengths whose tiles range
    # from 64 rows (one lane folds a row) down to 4 (sixteen lanes), row
    # boundaries inside granules, three tiles and a partial fourth
    es = ES[dtype]
    vec = 16 // es
    n = rws.softmax_variant_count(TILE)
    assert n == 4
    lengths = [vec + 1, 13, 25, 33, 60, 100, 250 if es == 2 else 125, 500 if es == 2 else 250]
    seen = set()
    for v in range(n):
        K = v + 1
        for cols in lengths:
            T = _rows_per_tile(cols, es, K)
            rows = 3 * max(T, 4) + max(T, 4) // 2 + 1
            g = np.random.Generator(np.random.PCG64(700 + v * 31 + cols))
            x, xs = to_device(g.normal(0.0, 4.0, (rows, cols)), dtype)
            y = empty_like_at(x)
            if T == 0:
                st = rws.softmax_fwd_variant(x.data_ptr(), y.data_ptr(), rows, cols,
                                             rws.dtype_code(x.dtype),
                                             torch.cuda.current_stream().cuda_stream, TILE, v)
                assert st == rws.RWS_ERR_UNSUPPORTED_SHAPE, (cols, K)
                continue
            desc = _describe(rows, cols, dtype, x, y, v)
            assert f"T={T},K={K}>" in desc, (desc, T, K)
            seen.add(T)
            _run_variant(x, y, v)
            torch.cuda.synchronize()
            print(f"{desc} rows={rows} cols={cols}", flush=True)
            check(y.double().cpu().numpy(), oracle.safe_softmax(xs), dtype, f"{desc} cols={cols}")
    # heights with 1, 2, 4, 8 and 16 lanes per row all ran
    assert any(t > 32 for t in seen) and any(16 < t <= 32 for t in seen)
    assert any(8 < t <= 16 for t in seen) and any(4 < t <= 8 for t in seen) and 4 in seen


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("cols", [9, 15, 17, 33, 60, 63, 65, 100, 127, 129, 250, 255, 257,
                                  333, 500, 511, 513, 1000, 1023, 1025])
def test_row_lengths(dtype, cols):
    es = ES[dtype]
    # a tile of at least max(4, period) rows must fit 64 * 4 granules
    if cols * es > 2048 or cols < 16 // es or max(4, _period(cols, es)) * cols * es > 4096:
        pytest.skip("outside the tile rows")
    for rows in (64, 67, 1000):
        g = np.random.Generator(np.random.PCG64(cols * 1009 + rows))
        x, xs = to_device(g.normal(0.0, 5.0, (rows, cols)), dtype)
        y = empty_like_at(x)
        desc = rws.softmax_describe_launch(rows, cols, rws.dtype_code(x.dtype), x.data_ptr(),
                                           y.data_ptr())
        if (cols * es) % 16:
            assert desc.startswith("tile_rows<"), desc
        rws.softmax(x, out=y, kernel="tile_rows")
        torch.cuda.synchronize()
        check(y.double().cpu().numpy(), oracle.safe_softmax(xs), dtype, f"{desc} rows={rows}")


@pytest.mark.parametrize("dtype", DTYPES)
def test_in_place_and_guards(dtype):
    rows, cols = 77, 131
    g = np.random.Generator(np.random.PCG64(5))
    x, xs = to_device(g.normal(0.0, 3.0, (rows, cols)), dtype)
    # guard zones around the output
    buf = torch.full((rows * cols + 64,), 7.0, dtype=x.dtype, device="cuda")
    y = buf[32:32 + rows * cols].view(rows, cols)
    rws.softmax(x, out=y, kernel="tile_rows")
    rws.softmax(x, out=x, kernel="tile_rows")
    torch.cuda.synchronize()
    ref = oracle.safe_softmax(xs)
    check(y.double().cpu().numpy(), ref, dtype, "out of place")
    check(x.double().cpu().numpy(), ref, dtype, "in place")
    assert torch.all(buf[:32] == 7.0) and torch.all(buf[32 + rows * cols:] == 7.0)


def test_extremes_and_non_finite():
    rows, cols = 64, 75
    g = np.random.Generator(np.random.PCG64(6))
    x64 = g.normal(0.0, 2.0, (rows, cols))
    x64[0, 5] = np.nan            # NaN row
    x64[1, :] = -np.inf           # all -inf: NaN row (0/0)
    x64[2, 74] = np.inf           # +inf: NaN row
    x64[3, :] += 1e4              # large shift
    x64[4, 0] = -np.inf           # a -inf entry under a finite max: 0
    x64[5, :] = 3.0               # constant row
    x64[6, :] += 3e7              # maximum past the FMA form's range (exact form)
    x64[7, :] = -3e7 + x64[7, :]  # the same, negative
    x, xs = to_device(x64, "f32")
    y = torch.empty_like(x)
    rws.softmax(x, out=y, kernel="tile_rows")
    torch.cuda.synchronize()
    got = y.double().cpu().numpy()
    ref = oracle.safe_softmax(xs)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref).any(axis=1)
    check(got[ok], ref[ok], "f32", "finite rows")
    assert got[4, 0] == 0.0
    assert np.allclose(got[5], 1.0 / cols, rtol=1e-6)


def test_refusals():
    x = torch.zeros(2 * 4098 + 64 * 100 + 8, dtype=torch.float16, device="cuda")
    # pointers that are not 16-byte aligned
    st = rws.softmax_fwd_kernel(x.data_ptr() + 2, x.data_ptr() + 2, 64, 100, rws.RWS_F16,
                                torch.cuda.current_stream().cuda_stream, TILE)
    assert st == rws.RWS_ERR_UNSUPPORTED_SHAPE
    # rows shorter than a granule, and rows longer than a tile holds
    for cols in (7, 2049 * 2):
        st = rws.softmax_fwd_kernel(x.data_ptr(), x.data_ptr(), 2, cols, rws.RWS_F16,
                                    torch.cuda.current_stream().cuda_stream, TILE)
        assert st == rws.RWS_ERR_UNSUPPORTED_SHAPE
    # the masked form takes the same tile
    desc = rws.softmax_describe_launch(1000, 100, rws.RWS_F16, x.data_ptr(), x.data_ptr(),
                                       masked=True)
    assert desc.startswith("tile_rows<"), desc


def _sample_rows(rows, seed, n_ends=200, n_random=600):
    """Both ends of the tensor (the first tiles, and the partial last tile)
    and seeded random rows in between."""
    rng = np.random.Generator(np.random.PCG64(seed))
    idx = np.concatenate([np.arange(min(rows, n_ends)), np.arange(max(0, rows - n_ends), rows),
                          rng.integers(0, rows, n_random)])
    return np.unique(idx)


@pytest.mark.parametrize("dtype,rows,cols", [("f16", 1000003, 33), ("f16", 1048583, 100),
                                             ("bf16", 262147, 120), ("f32", 131075, 125)])
def test_large_launch_sampled_rows(dtype, rows, cols):
    # the dispatcher's tile at full size (tens of thousands of tiles in XCD
    # runs, a partial last tile): every row sum on the device, sampled rows
    # against the oracle row by row
    from gpu_util import TORCH_DTYPE
    from tolerance import TOL
    gen = torch.Generator(device="cuda").manual_seed(rows * 7 + cols)
    x = (torch.randn(rows, cols, generator=gen, device="cuda") * 4.0).to(TORCH_DTYPE[dtype])
    y = torch.empty_like(x)
    desc = rws.softmax_describe_launch(rows, cols, rws.dtype_code(x.dtype), x.data_ptr(),
                                       y.data_ptr())
    assert desc.startswith("tile_rows<"), desc
    rws.softmax(x, out=y)
    torch.cuda.synchronize()
    print(desc, flush=True)
    assert torch.isfinite(y).all().item()
    dev = (y.double().sum(dim=1) - 1.0).abs().max().item()
    assert dev <= TOL[dtype]["rowsum"], f"{desc}: row sum off by {dev:.3e}"
    idx = _sample_rows(rows, rows + cols)
    ti = torch.from_numpy(idx).cuda()
    xs = x.index_select(0, ti).double().cpu().numpy()
    check(y.index_select(0, ti).double().cpu().numpy(), oracle.safe_softmax(xs), dtype,
          f"{desc} sampled rows")


@pytest.mark.parametrize("dtype", DTYPES)
def test_fewer_rows_than_one_tile(dtype):
    # forced onto tiles of 12 to 56 rows, tensors of 1..17 rows: mostly a
    # single partial tile, the tensor ending inside its last granule
    es = ES[dtype]
    for cols in (9, 33, 77):
        if not tile_supports(cols, dtype):
            continue
        for rows in (1, 2, 5, 17):
            g = np.random.Generator(np.random.PCG64(rows * 101 + cols))
            x, xs = to_device(g.normal(0.0, 3.0, (rows, cols)), dtype)
            y = empty_like_at(x)
            desc = rws.softmax_describe_launch(rows, cols, rws.dtype_code(x.dtype), x.data_ptr(),
                                               y.data_ptr(), TILE)
            assert desc.startswith("tile_rows<"), desc
            rws.softmax(x, out=y, kernel="tile_rows")
            torch.cuda.synchronize()
            check(y.double().cpu().numpy(), oracle.safe_softmax(xs), dtype,
                  f"{desc} rows={rows} es={es}")
