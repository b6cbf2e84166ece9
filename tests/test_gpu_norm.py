"""GPU parity of layernorm_fwd / rmsnorm_fwd against the oracle's layernorm /
rmsnorm, through the C ABI.

Tolerance (derived from the arithmetic; the pages state none for the row
normalisations).  The kernels form the row's sums in fp32 with at most ~90
roundings in any chain (up to 64 values per lane, then at most 22 tree and
fold steps; the streaming form adds a few pairwise merges), so with
u = 2^-24 and c = 256u:
    e = |mu_k - mu|     <= c * mean|x|
    |rstd_k - rstd|     <= rstd * (c + s),   s = (e * rstd)^2 / 2
(the centred sum of squares about mu_k exceeds the one about mu by n e^2, a
second-order term that matters only when |mean| dwarfs the spread), and each
output, rounded once to its dtype,
    |y - ref| <= h*|ref| + |w| * (c * rstd * mean|x| + (c + s) * |n|)
                 + 2u * (|ref| + |b|) + floor
where n = (x - mu) * rstd is the normalised value, h the output's half-ulp
(fp32 0, fp16 2^-11, bf16 2^-8) and floor its smallest step.  For RMSNorm
there is no mean (e = 0).  The first term is the final rounding; the second
the fp32 error of the statistics carried through the normalisation (it grows
with |mean| / sigma: fp32 cannot centre a row whose mean dwarfs its spread
more exactly)."""
import numpy as np
import pytest
import torch

import oracle
import row_wise_safe_amd as rws
import workloads
from gpu_util import empty_like_at, have_gpu, to_device

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not have_gpu(), reason="needs an MI355X GPU")]

DTYPES = ["f32", "f16", "bf16"]
KERNELS = ["auto", "wave_row", "block_onepass", "two_pass"]
MODES = ["layernorm", "rmsnorm"]
HALF_ULP = {"f32": 0.0, "f16": 2.0 ** -11, "bf16": 2.0 ** -8}
FLOOR = {"f32": 1e-37, "f16": 2.0 ** -25, "bf16": 1e-37}
U32 = 2.0 ** -24
C = 256 * U32


def _supports(kernel, cols, dtype):
    es = 4 if dtype == "f32" else 2
    w = (cols * es + 143) // 16
    if kernel == "wave_row":
        return w <= 512
    if kernel == "block_onepass":
        return w <= 4096
    return True


def _ref(mode, xs, eps, ws, bs):
    if mode == "layernorm":
        y, mu, rs = oracle.layernorm(xs, eps, ws, bs, return_stats=True)
        n = oracle.layernorm(xs, eps)
    else:
        y, rs = oracle.rmsnorm(xs, eps, ws, return_stats=True)
        mu = None
        n = oracle.rmsnorm(xs, eps)
    return y, mu, rs, n


def _mean_err(mode, xs):
    return C * np.abs(xs).mean(axis=1) if mode == "layernorm" else np.zeros(xs.shape[0])


def _rstd_rel(mode, xs, rs):
    return C + 0.5 * (_mean_err(mode, xs) * rs) ** 2


def _bound(mode, dtype, xs, ref, n, rs, ws, bs):
    wabs = np.abs(ws)[None, :] if ws is not None else 1.0
    babs = np.abs(bs)[None, :] if bs is not None else 0.0
    stat = (_mean_err(mode, xs) * rs)[:, None] + _rstd_rel(mode, xs, rs)[:, None] * np.abs(n)
    return (HALF_ULP[dtype] * np.abs(ref) + wabs * stat + 2 * U32 * (np.abs(ref) + babs)
            + FLOOR[dtype])


def _check(mode, dtype, y, xs, eps, ws, bs, what, mean=None, rstd=None):
    ref, mu, rs, n = _ref(mode, xs, eps, ws, bs)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    err = np.abs(y - ref)
    bound = _bound(mode, dtype, xs, ref, n, rs, ws, bs)
    worst = np.max(err - bound) if err.size else -1.0
    assert worst <= 0.0, f"{what}: error exceeds bound by {worst:.3e} (max err {err.max():.3e})"
    if mean is not None:
        assert np.all(np.abs(mean - mu) <= _mean_err(mode, xs) + 1e-37), f"{what}: mean"
    if rstd is not None:
        assert np.all(np.abs(rstd - rs) <= _rstd_rel(mode, xs, rs) * rs), f"{what}: rstd"
    return float(err.max()) if err.size else 0.0


def _call(mode, x, out, eps, w, b, mean, rstd, kernel):
    if mode == "layernorm":
        rws.layer_norm(x, eps, w, b, out=out, mean=mean, rstd=rstd, kernel=kernel)
    else:
        rws.rms_norm(x, eps, w, out=out, rstd=rstd, kernel=kernel)
    torch.cuda.synchronize()


def _case(mode, dtype, rows, cols, kernel, seed, affine=True, x_off=0, out_off=0, w_off=0,
          eps=1e-5, x64=None, stats=True):
    g = np.random.Generator(np.random.PCG64(seed))
    if x64 is None:
        x64 = workloads.row_shifted_normal(rows, cols, seed)
    x, xs = to_device(x64, dtype, offset=x_off)
    w = b = None
    ws = bs = None
    if affine:
        w, ws = to_device(g.uniform(0.25, 2.0, (1, cols)), dtype, offset=w_off)
        w, ws = w.view(cols), ws[0]
        if mode == "layernorm":
            b, bs = to_device(g.normal(0.0, 1.0, (1, cols)), dtype, offset=w_off)
            b, bs = b.view(cols), bs[0]
    out = empty_like_at(x, out_off)
    mean = torch.full((rows,), float("nan"), device="cuda") if stats and mode == "layernorm" else None
    rstd = torch.full((rows,), float("nan"), device="cuda") if stats else None
    _call(mode, x, out, eps, w, b, mean, rstd, kernel)
    y = out.to(torch.float64).cpu().numpy()
    what = (f"{mode} {dtype} [{rows},{cols}] {kernel} affine={affine} offs=({x_off},{out_off},"
            f"{w_off}) eps={eps}")
    return _check(mode, dtype, y, xs, eps, ws, bs, what,
                  mean.double().cpu().numpy() if mean is not None else None,
                  rstd.double().cpu().numpy() if rstd is not None else None)


# --------------------------------------------------------------------------
# the two LayerNorm shapes of the Pangu-Weather profile page, full size, in
# the benchmarked launch (dispatcher's choice, no affine: the page folds the
# affine parameters into the next Linear)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("name", list(workloads.NORM_WORKLOADS))
def test_norm_workload_full_size(name, mode):
    wl = workloads.NORM_WORKLOADS[name]
    x, xs = to_device(wl.generate(), wl.dtype)
    out = torch.empty_like(x)
    _call(mode, x, out, 1e-5, None, None, None, None, "auto")
    y = out.to(torch.float64).cpu().numpy()
    e = _check(mode, wl.dtype, y, xs, 1e-5, None, None, f"{name} {mode}")
    print(f"\n{name} {mode}: max abs err {e:.3e}", flush=True)
    # one fp16 ulp at |y| < 4 is 2^-8; within the bound above every error is
    # at most one ulp of the output
    assert e <= 2.0 ** -8 * 2


# the same shapes with weight and bias (RMSNorm: weight) in the lane groups
# taken with them, the vectors at the rows' 16-byte phase (the phase-matched
# kernels) and 2 elements off it (element loads)
@pytest.mark.parametrize("w_off", [0, 2])
@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("name", list(workloads.NORM_WORKLOADS))
def test_norm_workload_affine(name, mode, w_off):
    wl = workloads.NORM_WORKLOADS[name]
    desc = rws.norm_describe_launch(wl.rows, wl.cols, rws.RWS_F16, 256, 512, affine=True)
    print(f"\n{name} {mode} w_off={w_off}: {desc}", flush=True)
    _case(mode, wl.dtype, wl.rows, wl.cols, "auto", seed=wl.seed + 1, affine=True, w_off=w_off,
          x64=wl.generate())


# --------------------------------------------------------------------------
# sweep: row lengths across the three families' ranges and their ragged
# edges, every dtype, each family forced, both modes
# --------------------------------------------------------------------------
SWEEP_COLS = [1, 2, 3, 7, 8, 15, 16, 31, 33, 64, 100, 127, 128, 192, 255, 384, 500, 512, 768,
              1000, 1024, 2047, 2048, 4096, 4097, 8192, 10000, 16384, 33000]


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("dtype", DTYPES)
def test_norm_sweep(dtype, kernel, mode):
    for i, cols in enumerate(SWEEP_COLS):
        if not _supports(kernel, cols, dtype):
            continue
        rows = 37 if cols <= 4096 else 5
        _case(mode, dtype, rows, cols, kernel, seed=7000 + i, affine=(i % 2 == 1))


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("kernel", KERNELS)
def test_norm_unaligned_and_split_phase(kernel, mode):
    for dtype in DTYPES:
        for cols in (61, 192, 385, 1999, 5003):
            if not _supports(kernel, cols, dtype):
                continue
            for offs in ((1, 1, 0), (3, 0, 1), (0, 5, 2), (2, 2, 3)):
                _case(mode, dtype, 23, cols, kernel, seed=cols + offs[0], affine=True,
                      x_off=offs[0], out_off=offs[1], w_off=offs[2])


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("kernel", KERNELS)
def test_norm_in_place(kernel, mode):
    for dtype in DTYPES:
        for cols in (96, 1000, 3000):
            if not _supports(kernel, cols, dtype):
                continue
            x64 = workloads.row_shifted_normal(19, cols, 99 + cols)
            x, xs = to_device(x64, dtype)
            _call(mode, x, x, 1e-5, None, None, None, None, kernel)
            _check(mode, dtype, x.to(torch.float64).cpu().numpy(), xs, 1e-5, None, None,
                   f"in place {mode} {dtype} {cols} {kernel}")


@pytest.mark.parametrize("kernel", KERNELS)
def test_layernorm_large_mean(kernel):
    # mean/sigma up to 1e4: the centring cancels most digits; the bound grows
    # with rstd * mean|x| as fp32 allows
    for dtype in ("f32", "bf16"):
        for cols in (256, 2500):
            if not _supports(kernel, cols, dtype):
                continue
            x64 = workloads.row_shifted_normal(11, cols, 5, mu_lo=-1e4, mu_hi=1e4,
                                               sigma_lo=0.5, sigma_hi=2.0)
            _case("layernorm", dtype, 11, cols, kernel, seed=5, x64=x64, affine=False)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("kernel", KERNELS)
def test_norm_constant_and_zero_rows(kernel, mode):
    for dtype in DTYPES:
        cols = 300
        if not _supports(kernel, cols, dtype):
            continue
        x64 = np.zeros((4, cols))
        x64[1] = 2.5
        x64[2] = -0.1
        x64[3, ::3] = 1.0
        x, xs = to_device(x64, dtype)
        out = torch.empty_like(x)
        _call(mode, x, out, 1e-5, None, None, None, None, kernel)
        y = out.to(torch.float64).cpu().numpy()
        _check(mode, dtype, y, xs, 1e-5, None, None, f"constant rows {mode} {dtype} {kernel}")
        if mode == "layernorm":
            assert np.all(y[0] == 0.0) and np.all(y[1] == 0.0)
        else:
            assert np.all(y[0] == 0.0)


@pytest.mark.parametrize("mode", MODES)
def test_norm_eps_zero_constant_row_is_nan(mode):
    # var + eps == 0: 0 * inf = NaN, as the definition gives
    x, _ = to_device(np.zeros((3, 64)), "f32")
    out = torch.empty_like(x)
    _call(mode, x, out, 0.0, None, None, None, None, "auto")
    assert torch.isnan(out).all()


@pytest.mark.parametrize("mode", MODES)
def test_norm_eps_values(mode):
    for eps in (0.0, 1e-12, 1e-3, 10.0):
        _case(mode, "f32", 9, 777, "auto", seed=31, eps=eps)


def test_norm_empty_is_noop():
    x = torch.empty((0, 64), dtype=torch.float16, device="cuda")
    rws.layer_norm(x)
    rws.rms_norm(x)
    x = torch.empty((5, 0), dtype=torch.float16, device="cuda")
    rws.layer_norm(x)


def test_norm_on_a_stream():
    s = torch.cuda.Stream()
    x64 = workloads.row_shifted_normal(1024, 384, 3)
    x, xs = to_device(x64, "f16")
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        out = torch.empty_like(x)
        rws.layer_norm(x, 1e-5, out=out, stream=s)
    s.synchronize()
    _check("layernorm", "f16", out.to(torch.float64).cpu().numpy(), xs, 1e-5, None, None,
           "stream")


def test_norm_rejects_split_kernels():
    # the two-launch and fused split-k forms exist for the forward only
    # (the normalisations' split-k is the ordered form)
    x = torch.zeros((4, 64), dtype=torch.float16, device="cuda")
    with pytest.raises(rws.SoftmaxError):
        rws.layer_norm(x, kernel="splitk")
    with pytest.raises(rws.SoftmaxError):
        rws.rms_norm(x, kernel="splitk_fused")


def test_norm_deterministic():
    x64 = workloads.row_shifted_normal(513, 4001, 8)
    x, _ = to_device(x64, "bf16")
    a = rws.layer_norm(x)
    b = rws.layer_norm(x)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# --------------------------------------------------------------------------
# tile_rows: several short rows per wave as one 16-byte-aligned range (no
# weight or bias)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("mode", ["layernorm", "rmsnorm"])
@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("cols", [9, 33, 100, 250, 333, 500, 1001])
def test_tile_rows_form(mode, dtype, cols):
    from gpu_util import tile_supports
    if not tile_supports(cols, dtype):
        pytest.skip("outside the tile rows")
    es = 4 if dtype == "f32" else 2
    for rows in (64, 67, 777):
        g = np.random.Generator(np.random.PCG64(cols * 17 + rows))
        x, xs = to_device(g.normal(0.5, 2.0, (rows, cols)), dtype)
        out = empty_like_at(x)
        mean = torch.empty(rows, dtype=torch.float32, device="cuda")
        rstd = torch.empty(rows, dtype=torch.float32, device="cuda")
        desc = rws.norm_describe_launch(rows, cols, rws.dtype_code(x.dtype), x.data_ptr(),
                                        out.data_ptr())
        rb = cols * es
        if rb <= 2048 and rb % 128 and (rb % 16 or rb > 128):
            assert desc.startswith("norm_tile<"), desc
        for kernel in ("auto", "tile_rows"):
            _call(mode, x, out, 1e-5, None, None, mean, rstd, kernel)
            _check(mode, dtype, out.double().cpu().numpy(), xs, 1e-5, None, None,
                   f"{mode} {kernel} {desc} rows={rows}",
                   mean=mean.double().cpu().numpy() if mode == "layernorm" else None,
                   rstd=rstd.double().cpu().numpy())


def test_tile_rows_form_affine_and_constant_rows():
    rows, cols = 66, 100
    g = np.random.Generator(np.random.PCG64(9))
    x, xs = to_device(g.normal(0.0, 1.0, (rows, cols)), "f16")
    w, ws = to_device(g.uniform(0.5, 1.5, (1, cols)), "f16")
    # with a weight the dispatcher keeps the lane groups; the tile form refuses it
    desc = rws.norm_describe_launch(rows, cols, rws.RWS_F16, x.data_ptr(), x.data_ptr(),
                                    affine=True)
    assert not desc.startswith("norm_tile<"), desc
    with pytest.raises(rws.SoftmaxError):
        rws.layer_norm(x, 1e-5, w.view(cols), None, kernel="tile_rows")
    # constant rows normalise to exact zeros
    c, cs = to_device(np.full((rows, cols), 3.25), "f16")
    y = rws.layer_norm(c, 1e-5, kernel="tile_rows")
    torch.cuda.synchronize()
    assert torch.all(y == 0)


@pytest.mark.parametrize("mode", ["layernorm", "rmsnorm"])
@pytest.mark.parametrize("dtype,rows,cols", [("f16", 1000003, 33), ("f16", 1048583, 100),
                                             ("bf16", 262147, 120)])
def test_tile_rows_form_large_launch_sampled_rows(mode, dtype, rows, cols):
    # the dispatcher's tile at full size with the statistics outputs: sampled
    # rows (both ends, the partial last tile among them, and seeded random
    # rows) against the oracle
    from gpu_util import TORCH_DTYPE
    gen = torch.Generator(device="cuda").manual_seed(rows * 3 + cols)
    tdt = TORCH_DTYPE[dtype]
    x = (torch.randn(rows, cols, generator=gen, device="cuda") * 2.0 + 0.5).to(tdt)
    out = torch.empty_like(x)
    mean = torch.empty(rows, dtype=torch.float32, device="cuda")
    rstd = torch.empty(rows, dtype=torch.float32, device="cuda")
    desc = rws.norm_describe_launch(rows, cols, rws.dtype_code(tdt), x.data_ptr(), out.data_ptr())
    assert desc.startswith("norm_tile<"), desc
    _call(mode, x, out, 1e-5, None, None, mean, rstd, "auto")
    print(desc, flush=True)
    rng = np.random.Generator(np.random.PCG64(rows + 1))
    idx = np.unique(np.concatenate([np.arange(200), np.arange(rows - 200, rows),
                                    rng.integers(0, rows, 600)]))
    ti = torch.from_numpy(idx).cuda()
    xs = x.index_select(0, ti).double().cpu().numpy()
    _check(mode, dtype, out.index_select(0, ti).double().cpu().numpy(), xs, 1e-5, None, None,
           f"{mode} {desc} sampled rows",
           mean=mean.index_select(0, ti).double().cpu().numpy() if mode == "layernorm" else None,
           rstd=rstd.index_select(0, ti).double().cpu().numpy())
