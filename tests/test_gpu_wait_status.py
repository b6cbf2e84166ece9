"""The single-launch split-k forms report a wait that gave up.

Their waiting workgroups (the ordered form's stage 2, every workgroup of the
fused form) poll the row's partials with a bounded wait (they rely on
workgroups being dispatched in index order within each XCD; a wait that runs
out means that order did not hold).  Such a workgroup writes NaN
for its chunk and sets the stream's status word; softmax_stream_status then
returns RWS_ERR_WAIT_TIMEOUT once and clears it.  The tests force the
give-up from the host by setting the wait limit to 0 tries, so every
waiting workgroup gives up without polling and every kernel still ends
normally; then the default limit is restored and the same call must match
the oracle with a clean status.
"""
import numpy as np
import pytest
import torch

import oracle
import row_wise_safe_amd as rws
from gpu_util import FreshStream, have_gpu, to_device
from tolerance import check

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not have_gpu(), reason="needs an MI355X GPU")]

ROWS, COLS = 4, 1 << 18  # few long rows: P = 64 chunks of 256 x 4 granules (fp16)


@pytest.fixture(scope="module", autouse=True)
def _lib():
    rws.load_library()
    yield
    rws.softmax_set_wait_limit(-1)


def _status(s):
    return rws.softmax_stream_status(int(s.cuda_stream))


def _forced_give_up_then_clean(call, ref_check):
    with FreshStream() as s:
        with torch.cuda.stream(s):
            assert _status(s) == rws.RWS_OK  # nothing ran on this stream yet
            try:
                assert rws.softmax_set_wait_limit(0) == rws.RWS_OK
                out = call()
            finally:
                rws.softmax_set_wait_limit(-1)
            assert _status(s) == rws.RWS_ERR_WAIT_TIMEOUT
            assert "gave up" in rws.softmax_last_error()
            assert torch.isnan(out).all()
            assert _status(s) == rws.RWS_OK  # the query cleared it
            out = call()
            assert _status(s) == rws.RWS_OK
            ref_check(out)


def test_forward_ordered_reports_give_up():
    x64 = np.random.Generator(np.random.PCG64(61)).normal(0.0, 3.0, (ROWS, COLS))
    x, xs = to_device(x64, "f16")
    assert "splitk_ordered" in rws.softmax_describe_launch(
        ROWS, COLS, rws.RWS_F16, x.data_ptr(), x.data_ptr(), rws.KERNEL_IDS["splitk_ordered"])
    print("forward ordered give-up", flush=True)
    _forced_give_up_then_clean(
        lambda: rws.softmax(x, kernel="splitk_ordered"),
        lambda y: check(y.double().cpu().numpy(), oracle.safe_softmax(xs), "f16", "ordered"))


def test_forward_fused_reports_give_up():
    # four long rows: the dispatcher's fused single launch, whose every
    # workgroup waits for its row's partials
    x64 = np.random.Generator(np.random.PCG64(64)).normal(0.0, 3.0, (ROWS, COLS))
    x, xs = to_device(x64, "f16")
    assert "splitk_fused" in rws.softmax_describe_launch(ROWS, COLS, rws.RWS_F16, x.data_ptr(),
                                                         x.data_ptr())
    print("forward fused give-up", flush=True)
    _forced_give_up_then_clean(
        lambda: rws.softmax(x),
        lambda y: check(y.double().cpu().numpy(), oracle.safe_softmax(xs), "f16", "fused"))


def test_backward_ordered_reports_give_up():
    g = np.random.Generator(np.random.PCG64(62))
    y, ys = to_device(oracle.safe_softmax(g.normal(0.0, 2.0, (ROWS, COLS))), "f32")
    dy, gs = to_device(g.normal(0.0, 1.0, (ROWS, COLS)), "f32")
    assert rws.softmax_bwd_describe_launch(ROWS, COLS, rws.RWS_F32, y.data_ptr(),
                                           y.data_ptr()).startswith("bwd_ordered")
    ref = oracle.softmax_backward(ys, gs)
    bound = 2e-5 * ys * (np.abs(gs) + np.abs(ys * gs).sum(axis=1, keepdims=True)) + 1e-37
    print("backward ordered give-up", flush=True)
    _forced_give_up_then_clean(
        lambda: rws.softmax_backward(y, dy),
        lambda dx: np.testing.assert_array_less(np.abs(dx.double().cpu().numpy() - ref),
                                                bound + 1e-300))


@pytest.mark.parametrize("mode", ["layernorm", "rmsnorm"])
def test_norm_ordered_reports_give_up(mode):
    x64 = np.random.Generator(np.random.PCG64(63)).normal(1.0, 2.0, (ROWS, COLS))
    x, xs = to_device(x64, "f32")
    assert rws.norm_describe_launch(ROWS, COLS, rws.RWS_F32, x.data_ptr(),
                                    x.data_ptr()).startswith("norm_ordered")
    fn = rws.layer_norm if mode == "layernorm" else rws.rms_norm
    ref = (oracle.layernorm if mode == "layernorm" else oracle.rmsnorm)(xs, 1e-5)
    print(f"{mode} ordered give-up", flush=True)
    _forced_give_up_then_clean(
        lambda: fn(x, 1e-5),
        lambda y: np.testing.assert_array_less(np.abs(y.double().cpu().numpy() - ref), 1e-4))


def test_status_is_per_stream():
    # a give-up on one stream is not reported on another
    x64 = np.random.Generator(np.random.PCG64(64)).normal(0.0, 3.0, (ROWS, COLS))
    x, _ = to_device(x64, "f16")
    with FreshStream() as a, FreshStream() as b:
        with torch.cuda.stream(b):
            rws.softmax(x)  # b has a status word too
        with torch.cuda.stream(a):
            try:
                rws.softmax_set_wait_limit(0)
                rws.softmax(x)
            finally:
                rws.softmax_set_wait_limit(-1)
        assert _status(b) == rws.RWS_OK
        assert _status(a) == rws.RWS_ERR_WAIT_TIMEOUT
        with pytest.raises(rws.SoftmaxError):
            with torch.cuda.stream(a):
                rws.softmax_set_wait_limit(0)
                try:
                    rws.softmax(x)
                finally:
                    rws.softmax_set_wait_limit(-1)
                rws.stream_status()
