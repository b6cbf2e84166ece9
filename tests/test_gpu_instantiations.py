"""GPU parity of every lane-group kernel instantiation the library can
launch, and of the exact launches the benchmark lines time.

The lane-group kernels (one row per group of G lanes, K granules per lane,
U row sets per wave) are compiled per (dtype, line-aligned or not, G, K, U);
their stores take one of three paths at run time (write-through on
line-aligned rows, 128-bit non-temporal, element stores when in and out
have different 16-byte phases).  The cases are found on the host: row
lengths, row counts and pointer offsets are scanned through the describe
calls (no GPU work), the first (smallest) shape that reaches each
(dtype, alignment, G, K, U, store path) is kept, and that shape runs on the
GPU against the oracle -- for the forward softmax (dispatcher's choice and
the forced wave_row family), its masked form (with mask and causal limit),
the backward, and LayerNorm / RMSNorm with and without weight and bias.
"""
import re

import numpy as np
import pytest
import torch

import oracle
import row_wise_safe_amd as rws
import workloads
from gpu_util import empty_like_at, have_gpu, to_device
from tolerance import check

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not have_gpu(), reason="needs an MI355X GPU")]

DTYPES = ["f32", "f16", "bf16"]
ES = {"f32": 4, "f16": 2, "bf16": 2}
CODE = {"f32": rws.RWS_F32, "f16": rws.RWS_F16, "bf16": rws.RWS_BF16}
# (input offset, output offset) in elements from a 256-byte aligned base:
# line-aligned rows, unaligned rows with one phase, split phases
OFFSETS = [(0, 0), (1, 1), (1, 0)]
ROWS = [16, 4100]  # few waves; beyond the few-waves limit of 256 CUs
LANES = re.compile(r"^(\w+)<(\w+),(aligned|unaligned|unaligned,split-phase),"
                   r"G=(\d+),K=(\d+),U=(\d+)>.*?( store=wt)?$")


def _scan(describe, dtype, kernels, extra=(None,)):
    """{key: (rows, cols, offsets, kernel)} for the first shape that reaches
    each lane-group key; key = (name, dtype, alignment, G, K, U, wt, extra)."""
    es = ES[dtype]
    found = {}
    max_cols = 512 * 16 // es
    for kernel in kernels:
        for ex in extra:
            for offs in OFFSETS:
                for rows in ROWS:
                    for cols in range(1, max_cols + 1):
                        desc = describe(rows, cols, CODE[dtype], 256 + offs[0] * es,
                                        256 + 4096 + offs[1] * es, rws.KERNEL_IDS[kernel], ex)
                        m = LANES.match(desc)
                        if not m:
                            continue
                        key = (m.group(1), m.group(2), m.group(3), int(m.group(4)),
                               int(m.group(5)), int(m.group(6)), bool(m.group(7)), ex)
                        found.setdefault(key, (rows, cols, offs, kernel))
    return found


def _fwd_describe(rows, cols, code, ip, op, kid, masked):
    try:
        return rws.softmax_describe_launch(rows, cols, code, ip, op, kid, masked=bool(masked))
    except rws.SoftmaxError:
        return ""


def _bwd_describe(rows, cols, code, ip, op, kid, _):
    try:
        return rws.softmax_bwd_describe_launch(rows, cols, code, ip, op, kid)
    except rws.SoftmaxError:
        return ""


def _norm_describe(rows, cols, code, ip, op, kid, affine):
    try:
        return rws.norm_describe_launch(rows, cols, code, ip, op, kid, affine=bool(affine))
    except rws.SoftmaxError:
        return ""


@pytest.fixture(scope="module", autouse=True)
def _lib():
    rws.load_library()
    yield


def _confirm(key, desc):
    m = LANES.match(desc)
    assert m, desc
    got = (m.group(1), m.group(2), m.group(3), int(m.group(4)), int(m.group(5)),
           int(m.group(6)), bool(m.group(7)))
    assert got == key[:7], (got, key)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("masked", [False, True])
def test_every_forward_lane_group(dtype, masked):
    cases = _scan(_fwd_describe, dtype, ["auto", "wave_row"], extra=(masked,))
    groups = {k[3:6] for k in cases}
    assert len(groups) >= 8, sorted(groups)
    if masked:  # the masked line's launch: two granules per lane on 32 lanes
        assert (32, 2, 1) in groups
    for key, (rows, cols, offs, kernel) in sorted(cases.items()):
        g = np.random.Generator(np.random.PCG64(rows * 131 + cols + offs[0] * 7 + offs[1]))
        x, xs = to_device(g.normal(0.0, 4.0, (rows, cols)), dtype, offset=offs[0])
        out = empty_like_at(x, offs[1])
        desc = _fwd_describe(rows, cols, CODE[dtype], x.data_ptr(), out.data_ptr(),
                             rws.KERNEL_IDS[kernel], masked)
        _confirm(key, desc)
        print(f"{'masked ' if masked else ''}{desc} rows={rows} cols={cols} offs={offs}",
              flush=True)
        if masked:
            mask, ms = to_device(g.normal(0.0, 1.0, (5, cols)), dtype)
            causal = max(1, min(cols, 7))
            rws.softmax_masked(x, 0.125, mask, causal_q=causal, out=out, kernel=kernel)
            ref = oracle.masked_softmax(xs, 0.125, ms, causal_q=causal)
        else:
            rws.softmax(x, out=out, kernel=kernel)
            ref = oracle.safe_softmax(xs)
        torch.cuda.synchronize()
        y = out.double().cpu().numpy()
        if masked:
            # rows whose every key is masked out are NaN on both sides
            dead = np.all(np.isnan(ref), axis=1)
            assert np.all(np.isnan(y[dead]))
            y, ref = y[~dead], ref[~dead]
        check(y, ref, dtype, f"{desc} rows={rows} cols={cols} offs={offs}")
        del x, out


@pytest.mark.parametrize("dtype", DTYPES)
def test_every_backward_lane_group(dtype):
    from test_gpu_backward import _check as check_backward
    cases = _scan(_bwd_describe, dtype, ["auto", "wave_row"])
    groups = {k[3:6] for k in cases}
    assert len(groups) >= 8, sorted(groups)
    for key, (rows, cols, offs, kernel) in sorted(cases.items()):
        g = np.random.Generator(np.random.PCG64(rows * 17 + cols + offs[0] * 5 + offs[1]))
        y, ys = to_device(oracle.safe_softmax(g.normal(0.0, 2.0, (rows, cols))), dtype,
                          offset=offs[0])
        dy, gs = to_device(g.normal(0.0, 1.0, (rows, cols)), dtype, offset=offs[0])
        dx = empty_like_at(y, offs[1])
        desc = _bwd_describe(rows, cols, CODE[dtype], y.data_ptr(), dx.data_ptr(),
                             rws.KERNEL_IDS[kernel], None)
        _confirm(key, desc)
        print(f"{desc} rows={rows} cols={cols} offs={offs}", flush=True)
        rws.softmax_backward(y, dy, out=dx, kernel=kernel)
        torch.cuda.synchronize()
        check_backward(dx.double().cpu().numpy(), ys, gs, dtype,
                       f"{desc} rows={rows} cols={cols} offs={offs}")
        del y, dy, dx


@pytest.mark.parametrize("dtype", DTYPES)
def test_every_norm_lane_group(dtype):
    from test_gpu_norm import _case
    cases = _scan(_norm_describe, dtype, ["auto", "wave_row"], extra=(False, True))
    groups = {k[3:6] for k in cases}
    assert len(groups) >= 8, sorted(groups)
    for key, (rows, cols, offs, kernel) in sorted(cases.items()):
        affine = key[7]
        print(f"{key} rows={rows} cols={cols} offs={offs}", flush=True)
        for mode in ("layernorm", "rmsnorm"):
            _case(mode, dtype, rows, cols, kernel, seed=rows * 3 + cols + offs[1],
                  affine=bool(affine), x_off=offs[0], out_off=offs[1], w_off=offs[0])


# --------------------------------------------------------------------------
# the benchmarked launches of the masked and backward lines, at full size
# --------------------------------------------------------------------------
def test_masked_bench_line_full_size():
    # softmax(x/8 + mask[512,512] + causal 512) over fp16 [4,32,512,512]
    w = workloads.WORKLOADS["fp16_attn_4x32x512x512"]
    x, xs = to_device(w.generate(), w.dtype)
    g = np.random.Generator(np.random.PCG64(w.seed + 100))
    mask, ms = to_device(g.normal(0.0, 1.0, (w.cols, w.cols)), w.dtype)
    out = torch.empty_like(x)
    desc = rws.softmax_describe_launch(w.rows, w.cols, rws.RWS_F16, x.data_ptr(), out.data_ptr(),
                                       masked=True)
    print(desc, flush=True)
    assert desc.startswith("wave_row<f16,aligned,G=32,K=2,U=1>") and desc.endswith("store=wt")
    rws.softmax_masked(x, 0.125, mask, causal_q=w.cols, out=out)
    torch.cuda.synchronize()
    ref = oracle.masked_softmax(xs, 0.125, ms, causal_q=w.cols)
    m = check(out.double().cpu().numpy(), ref, "f16", "masked fp16 [65536,512]")
    print(m, flush=True)
    # the causal limit: query r % 512 sees keys j <= r % 512
    y = out[:1024].double().cpu().numpy()
    r = np.arange(1024)[:, None] % w.cols
    assert np.all(y[np.arange(w.cols)[None, :] > r] == 0.0)


@pytest.mark.parametrize("name", ["bf16_1Mx128", "fp16_attn_4x32x512x512"])
def test_backward_bench_line_full_size(name):
    from test_gpu_backward import _check as check_backward
    w = workloads.WORKLOADS[name]
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16}[w.dtype]
    # as the benchmark: y = the library's forward output, dy ~ N(0, 1)
    x, _ = to_device(w.generate(), w.dtype)
    y = rws.softmax(x)
    g = np.random.Generator(np.random.PCG64(w.seed + 200))
    dy, gs = to_device(g.standard_normal((w.rows, w.cols)), w.dtype)
    dx = torch.empty_like(y)
    desc = rws.softmax_bwd_describe_launch(w.rows, w.cols, rws.dtype_code(tdt), y.data_ptr(),
                                           dx.data_ptr())
    print(desc, flush=True)
    want = {"bf16_1Mx128": "bwd_wave<bf16,aligned,G=16,K=1,U=1>",
            "fp16_attn_4x32x512x512": "bwd_wave<f16,aligned,G=64,K=1,U=1>"}[name]
    assert desc.startswith(want), desc
    rws.softmax_backward(y, dy, out=dx)
    torch.cuda.synchronize()
    ys = y.double().cpu().numpy()
    check_backward(dx.double().cpu().numpy(), ys, gs, w.dtype, f"backward {name}")
