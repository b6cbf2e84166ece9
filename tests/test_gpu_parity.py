"""GPU parity: the HIP library, called through its C ABI, against the CPU
oracle on the same seeded inputs (tolerances in tests/tolerance.py).

Covers the five workloads at full size in the dispatcher's launch (the one
bench.py times), every kernel family forced over a sweep of row lengths that
crosses lane-group, wave, workgroup and chunk boundaries with ragged tails,
unaligned base pointers, in/out with different 16-byte phases, in-place,
guard zones around the output, determinism and the degenerate shapes.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import row_wise_safe_amd as rws
import workloads
from golden_io import load
from gpu_util import (NotCoResident, empty_like_at, have_gpu, run, supports, tile_supports,
                      to_device)
from tolerance import check, check_long_rows

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not have_gpu(), reason="needs an MI355X GPU")]

DTYPES = ["f32", "f16", "bf16"]
KERNELS = ["wave_row", "block_onepass", "two_pass", "splitk", "splitk_fused", "splitk_ordered"]


@pytest.fixture(scope="module", autouse=True)
def _lib():
    rws.load_library()
    yield


def _gen(rows, cols, seed, sigma=4.0):
    return np.random.Generator(np.random.PCG64(seed)).normal(0.0, sigma, (rows, cols))


# --------------------------------------------------------------------------
# worked example (HIP softmax tutorial page, section 1)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("kernel", ["auto"] + KERNELS)
def test_worked_example(kernel):
    g = load("worked_example_2x3.txt")
    x, stored = to_device(g["input"], "f32")
    y = run(x, empty_like_at(x), kernel)  # P = 1: always co-resident
    assert np.max(np.abs(y - g["output"])) <= 5e-5
    check(y, oracle.safe_softmax(stored), "f32", f"worked example / {kernel}")


# --------------------------------------------------------------------------
# the five workloads at full size, dispatcher's choice (the benchmarked launch)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("name", [n for n in workloads.WORKLOADS])
def test_workload_full_size(name):
    w = workloads.WORKLOADS[name]
    x, stored = to_device(w.generate(), w.dtype)
    desc = rws.softmax_describe_launch(w.rows, w.cols, rws.dtype_code(x.dtype), x.data_ptr(),
                                       x.data_ptr())
    print(f"\n{name}: {desc}", flush=True)
    y = run(x, torch.empty_like(x))
    ref = oracle.safe_softmax(stored)
    m = check(y, ref, w.dtype, name)
    print(f"{name}: {m}", flush=True)
    if name == "fp16_8192x4097":
        # closed form: spikes at +1e4 carry 1/k each, everything else is 0
        spikes = stored == 1.0e4
        k = spikes.sum(axis=1, keepdims=True)
        assert np.all(k > 0)
        assert np.max(np.abs(np.where(spikes, y - 1.0 / k, 0.0))) <= 1e-3
        assert np.all(np.where(~spikes, y == 0.0, True))


@pytest.mark.parametrize("name", list(workloads.LONG_ROW_WORKLOADS))
def test_long_row_workload_full_size(name):
    # rows of 8M and 32M columns: inputs of 64 and 256 MiB, more than the
    # ordered launch's re-read keeps in L2.  The fused single launch's grid
    # fits the device at once for 64 MiB (one read per element); 256 MiB
    # takes the two launches
    w = workloads.LONG_ROW_WORKLOADS[name]
    x, stored = to_device(w.generate(), w.dtype)
    desc = rws.softmax_describe_launch(w.rows, w.cols, rws.RWS_F16, x.data_ptr(), x.data_ptr())
    print(f"\n{name}: {desc}", flush=True)
    expected = {"fp16_4x8M": "splitk_fused<", "fp16_4x32M": "splitk<"}[name]
    assert desc.startswith(expected), desc
    y = run(x, torch.empty_like(x))
    del x
    m = check_long_rows(y, oracle.safe_softmax(stored), w.dtype, name)
    print(f"{name}: {m}", flush=True)


@pytest.mark.parametrize("kernel", KERNELS)
def test_workload_attn_each_kernel(kernel):
    w = workloads.WORKLOADS["fp16_attn_4x32x512x512"]
    x, stored = to_device(w.generate(rows=4099 if kernel != "splitk_fused" else 257), w.dtype)
    y = run(x, torch.empty_like(x), kernel)
    check(y, oracle.safe_softmax(stored), w.dtype, kernel)


@pytest.mark.parametrize("kernel", ["splitk", "splitk_fused", "splitk_ordered", "two_pass", "auto"])
def test_long_rows_max_at_chunk_edges(kernel):
    cols = 1 << 20
    columns = np.array([0, cols - 1, 16383, 16384, 8191, 131072])
    x64 = workloads.argmax_moved_normal(len(columns), cols, 20260005, 3.0, columns=columns)
    assert np.all(np.argmax(x64, axis=1) == columns)
    x, stored = to_device(x64, "f16")
    y = run(x, torch.empty_like(x), kernel)
    check(y, oracle.safe_softmax(stored), "f16", kernel)


# --------------------------------------------------------------------------
# forced kernels over a sweep of row lengths
# --------------------------------------------------------------------------
SWEEP_COLS = [1, 2, 3, 7, 8, 9, 15, 16, 17, 31, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257,
              511, 512, 513, 1000, 1023, 1024, 1025, 2047, 2049, 4095, 4096, 4097, 8191, 8193,
              16385, 32767, 32769, 65537, 131073, (1 << 20) - 1]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("cols", SWEEP_COLS)
def test_sweep_all_kernels(dtype, cols):
    rows = 67 if cols <= 1025 else 3
    x64 = _gen(rows, cols, seed=1000 + cols, sigma=4.0)
    x, stored = to_device(x64, dtype)
    ref = oracle.safe_softmax(stored)
    aligned = (cols * x.element_size()) % 16 == 0
    ran = 0
    for kernel in ["auto"] + KERNELS + ["tile_rows"]:
        if kernel == "tile_rows":
            if not tile_supports(cols, dtype):  # the base here is 16-byte aligned
                continue
        elif kernel != "auto" and not supports(kernel, cols, dtype, aligned):
            continue
        try:
            y = run(x, torch.empty_like(x), kernel)
        except NotCoResident:
            continue
        check(y, ref, dtype, f"{kernel} cols={cols}")
        ran += 1
    assert ran >= 3


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("rows", [1, 2, 3, 15, 17, 63, 65, 4097])
def test_ragged_row_counts(dtype, rows):
    for cols in (24, 128, 512, 1000):
        x, stored = to_device(_gen(rows, cols, seed=rows * 7 + cols), dtype)
        ref = oracle.safe_softmax(stored)
        for kernel in ["auto", "wave_row", "block_onepass"]:
            try:
                y = run(x, torch.empty_like(x), kernel)
            except NotCoResident:
                continue
            check(y, ref, dtype, f"{kernel} rows={rows} cols={cols}")


# --------------------------------------------------------------------------
# alignment, phases, aliasing, guard zones
# --------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("in_off,out_off", [(1, 1), (3, 3), (1, 0), (0, 5), (2, 7)])
@pytest.mark.parametrize("cols", [5, 64, 100, 513, 4097, 40000])
def test_unaligned_and_split_phase(dtype, in_off, out_off, cols):
    rows = 9
    x, stored = to_device(_gen(rows, cols, seed=cols + in_off), dtype, offset=in_off)
    ref = oracle.safe_softmax(stored)
    aligned = False
    for kernel in ["auto"] + KERNELS:
        if kernel != "auto" and not supports(kernel, cols, dtype, aligned):
            continue
        out = empty_like_at(x, out_off)
        try:
            y = run(x, out, kernel)
        except NotCoResident:
            continue
        check(y, ref, dtype, f"{kernel} in+{in_off} out+{out_off} cols={cols}")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("cols", [3, 512, 4097, 70000])
def test_in_place(dtype, cols):
    rows = 5
    for kernel in ["auto"] + KERNELS:
        if kernel != "auto" and not supports(kernel, cols, dtype, False):
            continue
        x, stored = to_device(_gen(rows, cols, seed=cols), dtype, offset=1)
        try:
            y = run(x, x, kernel)
        except NotCoResident:
            continue
        check(y, oracle.safe_softmax(stored), dtype, f"in-place {kernel} cols={cols}")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("cols", [3, 129, 4097, 33000])
def test_guard_zones_untouched(dtype, cols):
    rows, guard = 7, 64
    x, stored = to_device(_gen(rows, cols, seed=cols * 3), dtype, offset=3)
    for kernel in ["auto"] + KERNELS:
        if kernel != "auto" and not supports(kernel, cols, dtype, False):
            continue
        # off 3: the output has the input's 16-byte phase, so partial
        # granules go out as aligned pieces; 0 and 1: element stores
        for off in (0, 1, 3):
            buf = torch.full((rows * cols + 2 * guard + off,), -7.0, dtype=x.dtype, device="cuda")
            before = buf.clone()
            out = buf[guard + off:guard + off + rows * cols].view(rows, cols)
            rws.softmax(x, out=out, kernel=kernel)  # 7 rows: always co-resident
            torch.cuda.synchronize()
            assert torch.equal(buf[:guard + off], before[:guard + off]), f"{kernel}: head guard"
            assert torch.equal(buf[guard + off + rows * cols:], before[guard + off + rows * cols:]), \
                f"{kernel}: tail guard"
            check(out.double().cpu().numpy(), oracle.safe_softmax(stored), dtype, kernel)


# --------------------------------------------------------------------------
# values: large magnitudes, constants, non-finite readings, determinism
# --------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", DTYPES)
def test_plus_minus_1e4(dtype):
    x64 = _gen(16, 3000, seed=5)
    x64[:, ::97] = 1.0e4
    x64[3] = -1.0e4
    x64[3, 17] = -9990.0
    x, stored = to_device(x64, dtype)
    ref = oracle.safe_softmax(stored)
    for kernel in ["auto"] + KERNELS:
        if kernel != "auto" and not supports(kernel, 3000, dtype, False):
            continue
        try:
            y = run(x, torch.empty_like(x), kernel)
        except NotCoResident:
            continue
        check(y, ref, dtype, kernel)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_huge_magnitudes(dtype):
    # rows whose max is far beyond fp16 range: the exp argument must not
    # carry an offset of half an ulp of max*log2(e)
    cols = 2000
    g = np.random.Generator(np.random.PCG64(21))
    x64 = g.normal(0, 4, (8, cols))
    x64[0] += 1.0e10
    x64[1] -= 1.0e10
    x64[2] = -1.0e30
    x64[2, 1500:] = g.normal(0, 4, cols - 1500)
    x64[3] += 3.0e6
    x64[4] = g.normal(0, 1e5, cols)
    x64[5] = 1.0e30 * g.normal(0, 1, cols)
    x64[6] = -3.0e38 + 1e32 * g.uniform(0, 1, cols)
    x, stored = to_device(x64, dtype)
    ref = oracle.safe_softmax(stored)
    for kernel in ["auto"] + KERNELS:
        if kernel != "auto" and not supports(kernel, cols, dtype, False):
            continue
        try:
            y = run(x, torch.empty_like(x), kernel)
        except NotCoResident:
            continue
        check(y, ref, dtype, kernel)


@pytest.mark.parametrize("dtype", DTYPES)
def test_constant_rows_and_single_column(dtype):
    for cols in (1, 2, 1000, 5000):
        x, stored = to_device(np.full((4, cols), 3.0), dtype)
        ref = oracle.safe_softmax(stored)
        assert np.all(ref == 1.0 / cols)
        for kernel in ["auto"] + KERNELS:
            if kernel != "auto" and not supports(kernel, cols, dtype, False):
                continue
            try:
                y = run(x, torch.empty_like(x), kernel)
            except NotCoResident:
                continue
            check(y, ref, dtype, f"{kernel} constant cols={cols}")
            if cols == 1:
                assert np.all(y == 1.0)


@pytest.mark.parametrize("dtype", DTYPES)
def test_nonfinite_rows(dtype):
    cols = 700
    x64 = _gen(6, cols, seed=9)
    x64[1, 5] = math.nan
    x64[2, 600] = math.inf
    x64[3, :] = -math.inf
    x64[4, ::3] = -math.inf
    x, stored = to_device(x64, dtype)
    ref = oracle.safe_softmax(stored)
    for kernel in ["auto"] + KERNELS:
        if kernel != "auto" and not supports(kernel, cols, dtype, False):
            continue
        try:
            y = run(x, torch.empty_like(x), kernel)
        except NotCoResident:
            continue
        for r in (1, 2, 3):
            assert np.all(np.isnan(y[r])), f"{kernel}: row {r} should be NaN"
        assert np.all(np.isnan(ref[[1, 2, 3]]))
        check(y[[0, 4, 5]], ref[[0, 4, 5]], dtype, kernel)
        assert np.all(y[4, ::3] == 0.0)


@pytest.mark.parametrize("kernel", KERNELS)
def test_deterministic(kernel):
    cols = 3990 if kernel == "wave_row" else 4097  # wave_row holds <= 512 granules
    x, _ = to_device(_gen(33, cols, seed=77), "f16", offset=1)
    a = torch.empty_like(x)
    b = torch.empty_like(x)
    rws.softmax(x, out=a, kernel=kernel)
    rws.softmax(x, out=b, kernel=kernel)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_empty_shapes_are_noops():
    for shape in [(0, 5), (5, 0), (0, 0)]:
        x = torch.empty(shape, dtype=torch.float16, device="cuda")
        y = rws.softmax(x)
        assert y.shape == x.shape
    assert rws.softmax_fwd(0, 0, 0, 10, rws.RWS_F16, 0) == rws.RWS_OK


def test_forced_kernel_rejects_too_long_rows():
    x = torch.zeros(2, 600 * 8, dtype=torch.float16, device="cuda")
    with pytest.raises(rws.SoftmaxError) as e:
        rws.softmax(x, kernel="wave_row")
    assert e.value.status == rws.RWS_ERR_UNSUPPORTED_SHAPE


def test_stream_argument_is_used():
    s = torch.cuda.Stream()
    x, stored = to_device(_gen(64, 512, seed=3), "f16")
    out = torch.empty_like(x)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        rws.softmax(x, out=out)
    s.synchronize()
    check(out.double().cpu().numpy(), oracle.safe_softmax(stored), "f16", "side stream")


def test_copy_bytes():
    a = torch.randint(-1000, 1000, (1 << 20,), dtype=torch.int32, device="cuda")
    b = torch.zeros_like(a)
    rws.copy_bytes(a, b)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_read_and_write_references():
    # the write reference fills granule i with (i, i >> 32, 0x5a5a5a5a, ~i); the
    # read reference leaves its input and everything else untouched
    n16 = 1 << 16
    buf = torch.zeros(4 * n16 + 64, dtype=torch.int32, device="cuda")
    out = buf[32:32 + 4 * n16]  # 128-byte aligned: written through
    s = torch.cuda.current_stream().cuda_stream
    assert rws.softmax_write_bytes(out.data_ptr(), 16 * n16, s) == rws.RWS_OK
    before = buf.clone()
    assert rws.softmax_read_bytes(out.data_ptr(), 16 * n16, s) == rws.RWS_OK
    torch.cuda.synchronize()
    assert torch.equal(buf, before)
    got = out.view(n16, 4).cpu().numpy().view(np.uint32)
    i = np.arange(n16, dtype=np.uint64)
    assert np.array_equal(got[:, 0], (i & 0xffffffff).astype(np.uint32))
    assert np.array_equal(got[:, 1], (i >> 32).astype(np.uint32))
    assert np.all(got[:, 2] == 0x5a5a5a5a)
    assert np.array_equal(got[:, 3], (~i & 0xffffffff).astype(np.uint32))
    assert torch.all(buf[:32] == 0) and torch.all(buf[32 + 4 * n16:] == 0)
