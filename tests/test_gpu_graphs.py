"""Graph capture and replay.  The single-launch split-k forms of the forward,
backward and normalisations tell one launch's partials from the previous
one's by an epoch passed as a kernel argument, which a replayed graph would
repeat.  Under capture the forward takes the two-launch split-k; the
backward and normalisations keep the single launch with an epoch that a
recorded kernel advances in device memory on every replay (or, with no tag
buffer on the stream yet, take one workgroup per row).  Each graph is
captured after an eager call on its stream (which sizes the workspace),
replayed several times on fresh input contents with eager library work and
synchronisations between the replays, and every replay is checked against
the CPU oracle.  Nothing in these graphs is a memset node (the library
clears nothing while capturing)."""
import os

import numpy as np
import pytest
import torch

import oracle
import row_wise_safe_amd as rws
from gpu_util import TORCH_DTYPE, FreshStream, have_gpu
from test_gpu_backward import _check as check_backward
from test_gpu_norm import _check as check_norm
from tolerance import check

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not have_gpu(), reason="needs an MI355X GPU")]

REPLAYS = 3


def _host(rows, cols, seed, sigma=3.0):
    return np.random.Generator(np.random.PCG64(seed)).normal(0.0, sigma, (rows, cols))


def _fill(t: torch.Tensor, x64: np.ndarray) -> np.ndarray:
    """Write x64 (rounded to t's dtype) into t in place; return the stored values."""
    h = torch.from_numpy(np.ascontiguousarray(x64)).to(t.dtype)
    t.copy_(h.to(t.device))
    return h.to(torch.float64).numpy()


def _dev(rows, cols, dtype):
    return torch.empty((rows, cols), dtype=TORCH_DTYPE[dtype], device="cuda")


def _capture(fn, stream):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        fn()
    return g


def _eager_noise(stream, seed):
    """Library calls between replays on the capture stream: an ordered split-k
    forward (advances the epochs of that stream's tag words) and a two-launch
    split-k forward larger than any captured one (grows that stream's partials
    buffer, which a captured graph must keep using)."""
    out = []
    with torch.cuda.stream(stream):
        a = _dev(8, 400000, "f16")
        sa = _fill(a, _host(8, 400000, seed))
        out.append((rws.softmax(a, kernel="splitk_ordered"), sa))
        b = _dev(64 + seed % 7, 300001, "bf16")
        sb = _fill(b, _host(b.shape[0], b.shape[1], seed + 1))
        out.append((rws.softmax(b, kernel="splitk"), sb))
    return out


def _check_noise(noise):
    for y, stored in noise:
        dt = "f16" if y.dtype == torch.float16 else "bf16"
        check(y.double().cpu().numpy(), oracle.safe_softmax(stored), dt, "eager call between replays")


@pytest.mark.parametrize("kernel", ["auto", "splitk_ordered", "splitk_fused"])
def test_forward_few_long_rows(kernel):
    rows, cols = 16, 1 << 20
    s = torch.cuda.Stream()
    x, y = _dev(rows, cols, "f16"), _dev(rows, cols, "f16")
    desc = rws.softmax_describe_launch(rows, cols, rws.RWS_F16, x.data_ptr(), y.data_ptr(),
                                       rws.KERNEL_IDS[kernel])
    with torch.cuda.stream(s):
        stored = _fill(x, _host(rows, cols, 300))
        try:
            rws.softmax(x, out=y, kernel=kernel)
        except rws.SoftmaxError as e:
            if kernel == "splitk_fused" and e.status == rws.RWS_ERR_UNSUPPORTED_SHAPE:
                pytest.skip(f"fused row not co-resident here: {e}")
            raise
    torch.cuda.synchronize()
    check(y.double().cpu().numpy(), oracle.safe_softmax(stored), "f16", f"eager {desc}")
    g = _capture(lambda: rws.softmax(x, out=y, kernel=kernel), s)
    for i in range(REPLAYS):
        # on the capturing stream, with eager split-k calls queued behind the
        # replay (they share its workspace) and one synchronisation for both
        with torch.cuda.stream(s):
            stored = _fill(x, _host(rows, cols, 301 + i, sigma=1.0 + i))
            y.fill_(float("nan"))
            g.replay()
            noise = _eager_noise(s, 310 + 2 * i)
        torch.cuda.synchronize()
        check(y.double().cpu().numpy(), oracle.safe_softmax(stored), "f16",
              f"replay {i} of {kernel} ({desc})")
        _check_noise(noise)


@pytest.mark.parametrize("rows,cols,dtype,masked", [
    (4096, 512, "f16", False),     # wave_row
    (256, 5000, "bf16", False),    # block_onepass, unaligned rows
    (1024, 1024, "f32", True),     # masked, causal
])
def test_forward_row_kernels(rows, cols, dtype, masked):
    s = torch.cuda.Stream()
    x, y = _dev(rows, cols, dtype), _dev(rows, cols, dtype)
    mask = None
    if masked:
        mask = _dev(64, cols, dtype)
        m64 = np.where(_host(64, cols, 320) > 1.5, -np.inf, 0.0)
        m64[:, 0] = 0.0  # with the causal limit, row 0 keeps key 0
        mstored = _fill(mask, m64)

    def call():
        if masked:
            rws.softmax_masked(x, scale=0.125, mask=mask, causal_q=rows, out=y)
        else:
            rws.softmax(x, out=y)

    def ref(stored):
        if masked:
            return oracle.masked_softmax(stored, scale=0.125, mask=mstored, causal_q=rows)
        return oracle.safe_softmax(stored)

    with torch.cuda.stream(s):
        _fill(x, _host(rows, cols, 321))
        call()
    torch.cuda.synchronize()
    g = _capture(call, s)
    for i in range(REPLAYS):
        with torch.cuda.stream(s):
            stored = _fill(x, _host(rows, cols, 322 + i))
            g.replay()
            noise = _eager_noise(s, 330 + 2 * i)
        torch.cuda.synchronize()
        check(y.double().cpu().numpy(), ref(stored), dtype, f"replay {i} of [{rows},{cols}]")
        _check_noise(noise)


@pytest.mark.parametrize("kernel", ["auto", "splitk_ordered"])
def test_backward_few_long_rows(kernel):
    rows, cols, dtype = 16, 300000, "f16"
    s = torch.cuda.Stream()
    y, dy, dx = _dev(rows, cols, dtype), _dev(rows, cols, dtype), _dev(rows, cols, dtype)
    eager = rws.softmax_bwd_describe_launch(rows, cols, rws.RWS_F16, y.data_ptr(), dx.data_ptr(),
                                            rws.KERNEL_IDS[kernel])
    assert eager.startswith("bwd_ordered"), eager
    with torch.cuda.stream(s):
        _fill(y, oracle.safe_softmax(_host(rows, cols, 340)))
        _fill(dy, _host(rows, cols, 341, sigma=1.0))
        rws.softmax_backward(y, dy, out=dx, kernel=kernel)
    torch.cuda.synchronize()
    g = _capture(lambda: rws.softmax_backward(y, dy, out=dx, kernel=kernel), s)
    for i in range(REPLAYS):
        with torch.cuda.stream(s):
            sy = _fill(y, oracle.safe_softmax(_host(rows, cols, 342 + i, sigma=1.0 + i)))
            sdy = _fill(dy, _host(rows, cols, 350 + i, sigma=1.0))
            dx.fill_(float("nan"))
            g.replay()
        torch.cuda.synchronize()
        check_backward(dx.double().cpu().numpy(), sy, sdy, dtype,
                       f"replay {i} of backward ({eager} eagerly)")
        with torch.cuda.stream(s):  # eager ordered backward between replays
            rws.softmax_backward(y, dy, out=dx, kernel="splitk_ordered")
        torch.cuda.synchronize()
        check_backward(dx.double().cpu().numpy(), sy, sdy, dtype,
                       f"eager backward after replay {i}")


@pytest.mark.parametrize("mode", ["layernorm", "rmsnorm"])
def test_norm_few_long_rows(mode):
    rows, cols, dtype = 16, 300000, "bf16"
    eps = 1e-5
    s = torch.cuda.Stream()
    x, out = _dev(rows, cols, dtype), _dev(rows, cols, dtype)
    w = torch.empty(cols, dtype=TORCH_DTYPE[dtype], device="cuda")
    b = torch.empty(cols, dtype=TORCH_DTYPE[dtype], device="cuda")
    sw = _fill(w.view(1, cols), 1.0 + 0.1 * _host(1, cols, 360))[0]
    sb = _fill(b.view(1, cols), 0.1 * _host(1, cols, 361))[0] if mode == "layernorm" else None
    rstd = torch.empty(rows, dtype=torch.float32, device="cuda")
    mean = torch.empty(rows, dtype=torch.float32, device="cuda") if mode == "layernorm" else None
    eager = rws.norm_describe_launch(rows, cols, rws.RWS_BF16, x.data_ptr(), out.data_ptr(),
                                     kernel_id=0, affine=True)
    assert eager.startswith("norm_ordered"), eager

    def call():
        if mode == "layernorm":
            rws.layer_norm(x, eps, w, b, out=out, mean=mean, rstd=rstd)
        else:
            rws.rms_norm(x, eps, w, out=out, rstd=rstd)

    def verify(stored, what):
        check_norm(mode, dtype, out.double().cpu().numpy(), stored, eps, sw, sb, what,
                   mean=mean.double().cpu().numpy() if mean is not None else None,
                   rstd=rstd.double().cpu().numpy())

    with torch.cuda.stream(s):
        _fill(x, _host(rows, cols, 362))
        call()
    torch.cuda.synchronize()
    g = _capture(call, s)
    for i in range(REPLAYS):
        with torch.cuda.stream(s):
            stored = _fill(x, 2.0 + _host(rows, cols, 363 + i, sigma=1.0 + i))
            out.fill_(float("nan"))
            g.replay()
        torch.cuda.synchronize()
        verify(stored, f"replay {i} of {mode}")
        with torch.cuda.stream(s):  # eager ordered normalisation between replays
            call()
        torch.cuda.synchronize()
        verify(stored, f"eager {mode} after replay {i}")


def test_capture_without_workspace_fails_cleanly():
    # a stream whose split-k partials were never sized: the capture reports
    # an error instead of allocating, and the stream works eagerly afterwards
    rows, cols = 16, 1 << 20
    x, y = _dev(rows, cols, "f16"), _dev(rows, cols, "f16")
    stored = _fill(x, _host(rows, cols, 370))
    torch.cuda.synchronize()
    with FreshStream() as s:
        g = torch.cuda.CUDAGraph()
        with pytest.raises(rws.SoftmaxError, match="graph capture"):
            with torch.cuda.graph(g, stream=s):
                y.zero_()
                rws.softmax(x, out=y)
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            rws.softmax(x, out=y)
        torch.cuda.synchronize()
        check(y.double().cpu().numpy(), oracle.safe_softmax(stored), "f16",
              "eager after failed capture")


def test_backward_capture_without_tag_buffer():
    # no tag buffer on the stream: the captured backward takes one workgroup
    # per row and needs no workspace at all
    rows, cols, dtype = 16, 300000, "f16"
    y, dy, dx = _dev(rows, cols, dtype), _dev(rows, cols, dtype), _dev(rows, cols, dtype)
    with FreshStream() as s:
        g = _capture(lambda: rws.softmax_backward(y, dy, out=dx), s)
        for i in range(REPLAYS):
            with torch.cuda.stream(s):
                sy = _fill(y, oracle.safe_softmax(_host(rows, cols, 380 + i)))
                sdy = _fill(dy, _host(rows, cols, 385 + i, sigma=1.0))
                dx.fill_(float("nan"))
                g.replay()
            torch.cuda.synchronize()
            check_backward(dx.double().cpu().numpy(), sy, sdy, dtype,
                           f"replay {i} of a backward captured without tags")


def test_device_epoch_wrap():
    # a fresh tag buffer whose device epoch starts 3 below the end of its
    # range (test hook read at allocation): replays 3 and on cross the end,
    # where the recorded kernel zeroes the tag words and restarts the range;
    # eager ordered calls on the same buffer run between the replays
    rows, cols, dtype = 16, 300000, "f16"
    y, dy, dx = _dev(rows, cols, dtype), _dev(rows, cols, dtype), _dev(rows, cols, dtype)
    x, out = _dev(rows, cols, dtype), _dev(rows, cols, dtype)
    os.environ["RWS_TEST_DEVICE_EPOCH"] = str(0xFFFFFFFF - 3)
    try:
        with FreshStream() as s:
            with torch.cuda.stream(s):
                sy = _fill(y, oracle.safe_softmax(_host(rows, cols, 390)))
                sdy = _fill(dy, _host(rows, cols, 391, sigma=1.0))
                rws.softmax_backward(y, dy, out=dx)  # allocates the tag buffer
            torch.cuda.synchronize()
            g = _capture(lambda: rws.softmax_backward(y, dy, out=dx), s)
            for i in range(8):
                with torch.cuda.stream(s):
                    sy = _fill(y, oracle.safe_softmax(_host(rows, cols, 392 + i)))
                    sdy = _fill(dy, _host(rows, cols, 400 + i, sigma=1.0))
                    dx.fill_(float("nan"))
                    g.replay()
                torch.cuda.synchronize()
                check_backward(dx.double().cpu().numpy(), sy, sdy, dtype,
                               f"replay {i} across the device epoch wrap")
                with torch.cuda.stream(s):
                    sx = _fill(x, _host(rows, cols, 410 + i))
                    rws.layer_norm(x, 1e-5, out=out)
                torch.cuda.synchronize()
                check_norm("layernorm", dtype, out.double().cpu().numpy(), sx, 1e-5, None, None,
                           f"eager LayerNorm after replay {i}")
    finally:
        del os.environ["RWS_TEST_DEVICE_EPOCH"]


def _dev_at(rows, cols, dtype, offset):
    """[rows, cols] view `offset` elements into a fresh buffer (offset 1: no
    row starts on a 16-byte boundary)."""
    buf = torch.empty(rows * cols + offset, dtype=TORCH_DTYPE[dtype], device="cuda")
    return buf[offset:].view(rows, cols)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("offset", [0, 1])
def test_captured_ordered_dtypes(dtype, offset):
    # the captured ordered backward and RMSNorm (device epochs) in every dtype,
    # on line-aligned and unaligned rows, replays interleaved with eager
    # ordered calls of both on the same tag buffer
    rows = 8
    cols = 200064 if offset == 0 else 200001  # line-aligned rows / no row on a 16-byte boundary
    y, dy, dx = (_dev_at(rows, cols, dtype, offset) for _ in range(3))
    x, out = _dev_at(rows, cols, dtype, offset), _dev_at(rows, cols, dtype, offset)
    rstd = torch.empty(rows, dtype=torch.float32, device="cuda")
    code = rws.dtype_code(TORCH_DTYPE[dtype])
    assert rws.softmax_bwd_describe_launch(rows, cols, code, y.data_ptr(), dx.data_ptr()) \
        .startswith("bwd_ordered")
    assert rws.norm_describe_launch(rows, cols, code, x.data_ptr(), out.data_ptr()) \
        .startswith("norm_ordered")
    s = torch.cuda.Stream()

    def call():
        rws.softmax_backward(y, dy, out=dx)
        rws.rms_norm(x, 1e-5, out=out, rstd=rstd)

    with torch.cuda.stream(s):
        _fill(y, oracle.safe_softmax(_host(rows, cols, 420)))
        _fill(dy, _host(rows, cols, 421, sigma=1.0))
        _fill(x, _host(rows, cols, 422))
        call()
    torch.cuda.synchronize()
    g = _capture(call, s)
    for i in range(REPLAYS):
        with torch.cuda.stream(s):
            sy = _fill(y, oracle.safe_softmax(_host(rows, cols, 423 + i, sigma=2.0)))
            sdy = _fill(dy, _host(rows, cols, 430 + i, sigma=1.0))
            sx = _fill(x, 1.0 + _host(rows, cols, 440 + i))
            dx.fill_(float("nan"))
            out.fill_(float("nan"))
            g.replay()
        torch.cuda.synchronize()
        what = f"{dtype} offset {offset} replay {i}"
        check_backward(dx.double().cpu().numpy(), sy, sdy, dtype, f"backward {what}")
        check_norm("rmsnorm", dtype, out.double().cpu().numpy(), sx, 1e-5, None, None,
                   f"rmsnorm {what}", rstd=rstd.double().cpu().numpy())
        with torch.cuda.stream(s):  # eager ordered calls on the same tag words
            call()
        torch.cuda.synchronize()
        check_backward(dx.double().cpu().numpy(), sy, sdy, dtype, f"eager backward {what}")
        check_norm("rmsnorm", dtype, out.double().cpu().numpy(), sx, 1e-5, None, None,
                   f"eager rmsnorm {what}", rstd=rstd.double().cpu().numpy())
