"""GPU parity of the masked/scaled softmax (softmax_fwd_masked) against the
oracle's masked_softmax: attention-score shapes [B, H, S, S] with a [S, S]
mask broadcast over B and H, causal limits (keys may outnumber queries),
scales, -inf mask entries, a mask whose rows have another 16-byte phase than
the input's, every kernel family that has a masked form."""
import math

import numpy as np
import pytest
import torch

import oracle
import row_wise_safe_amd as rws
from gpu_util import TORCH_DTYPE, have_gpu, tile_supports, to_device
from tolerance import check

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not have_gpu(), reason="needs an MI355X GPU")]

DTYPES = ["f32", "f16", "bf16"]
KERNELS = ["auto", "wave_row", "block_onepass", "two_pass"]


def _supports(kernel, cols, dtype):
    es = 4 if dtype == "f32" else 2
    w = (cols * es + 143) // 16
    return kernel != "wave_row" or w <= 512


def _masked(x, scale, mask, causal_q, kernel):
    out = torch.empty_like(x)
    rws.softmax_masked(x, scale=scale, mask=mask, causal_q=causal_q, out=out, kernel=kernel)
    torch.cuda.synchronize()
    return out.double().cpu().numpy()


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("S", [64, 100, 1000])
def test_attention_scores_mask_and_causal(dtype, S):
    B, H = 2, 3
    g = np.random.Generator(np.random.PCG64(S))
    x64 = g.normal(0.0, 4.0, (B * H * S, S))
    m64 = g.normal(0.0, 2.0, (S, S))
    m64[:, 3::7] = -math.inf if dtype != "bf16" else -1.0e30  # key 0 stays visible
    x, xs = to_device(x64, dtype)
    m, ms = to_device(m64, dtype)
    scale = 1.0 / math.sqrt(64.0)
    for causal in (0, S):
        ref = oracle.masked_softmax(xs, scale, ms, causal)
        for kernel in KERNELS:
            if not _supports(kernel, S, dtype):
                continue
            y = _masked(x, scale, m, causal, kernel)
            check(y, ref, dtype, f"{kernel} S={S} causal={causal}")


@pytest.mark.parametrize("dtype", DTYPES)
def test_causal_more_keys_than_queries(dtype):
    q, cols = 17, 33
    x, xs = to_device(np.random.Generator(np.random.PCG64(1)).normal(0, 3, (4 * q, cols)), dtype)
    ref = oracle.masked_softmax(xs, 0.7, None, q)
    for kernel in KERNELS:
        y = _masked(x, 0.7, None, q, kernel)
        check(y, ref, dtype, kernel)
        r = np.arange(4 * q)[:, None] % q
        j = np.arange(cols)[None, :]
        assert np.all(y[j > r + cols - q] == 0.0)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("scale", [1.0, -1.5, 0.0, 0.125])
def test_scale_only(dtype, scale):
    x, xs = to_device(np.random.Generator(np.random.PCG64(2)).normal(0, 5, (37, 777)), dtype)
    ref = oracle.masked_softmax(xs, scale, None, 0)
    for kernel in KERNELS:
        check(_masked(x, scale, None, 0, kernel), ref, dtype, f"{kernel} scale={scale}")


def _plain_same_launch(x, kernel):
    """The plain softmax through the compiled variant the masked form picks
    (the masked form prefers other lane groups than the plain one)."""
    rows, cols = x.shape
    code = rws.dtype_code(x.dtype)
    desc = rws.softmax_describe_launch(rows, cols, code, x.data_ptr(), x.data_ptr(),
                                       rws.KERNEL_IDS[kernel], masked=True)
    family, shape = desc.split("<")[0], desc.split(">")[0].split(",", 2)[2]
    kid = rws.KERNEL_IDS[family]
    y = torch.empty_like(x)
    for v in range(rws.softmax_variant_count(kid)):
        try:
            d = rws.softmax_describe_variant(rows, cols, code, x.data_ptr(), y.data_ptr(), kid, v)
        except rws.SoftmaxError:
            continue
        if d.split(">")[0].split(",", 2)[2] == shape:
            st = rws.softmax_fwd_variant(x.data_ptr(), y.data_ptr(), rows, cols, code,
                                         torch.cuda.current_stream().cuda_stream, kid, v)
            assert st == rws.RWS_OK
            return y
    raise AssertionError(f"no plain variant of {desc}")


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("cols", [512, 256, 128])
def test_identity_prologue_equals_plain(kernel, cols):
    # scale 1, no mask, no causal limit: bit-identical to the plain kernel of
    # the same shape
    x, _ = to_device(np.random.Generator(np.random.PCG64(3)).normal(0, 4, (65, cols)), "f16")
    a = _masked(x, 1.0, None, 0, kernel)
    b = _plain_same_launch(x, kernel)
    torch.cuda.synchronize()
    assert np.array_equal(a, b.double().cpu().numpy())


@pytest.mark.parametrize("dtype", DTYPES)
def test_mask_with_other_phase(dtype):
    rows, cols = 24, 1001
    g = np.random.Generator(np.random.PCG64(4))
    x, xs = to_device(g.normal(0, 2, (rows, cols)), dtype)
    m, ms = to_device(g.normal(0, 2, (5, cols)), dtype, offset=1)  # mask rows misaligned
    ref = oracle.masked_softmax(xs, 2.0, ms, 0)
    for kernel in KERNELS:
        check(_masked(x, 2.0, m, 0, kernel), ref, dtype, kernel)


@pytest.mark.parametrize("dtype", DTYPES)
def test_mask_at_every_phase(dtype):
    # mask rows at every 16-byte phase against the input rows: the mask
    # granules are then read as aligned pairs and shifted into place, and
    # element by element where such a pair would leave the mask (its first
    # and last rows); input rows start at every phase too (odd cols)
    vec = 4 if dtype == "f32" else 8
    g = np.random.Generator(np.random.PCG64(14))
    rows, mask_rows = 16, 7
    for cols in (577, 1000, 3001):
        for xoff in (0, 3):
            x, xs = to_device(g.normal(0, 3, (rows, cols)), dtype, offset=xoff)
            for moff in range(vec):
                m, ms = to_device(g.normal(0, 2, (mask_rows, cols)), dtype, offset=moff)
                for causal in (0, rows):
                    ref = oracle.masked_softmax(xs, 0.5, ms, causal)
                    for kernel in KERNELS:
                        if _supports(kernel, cols, dtype):
                            check(_masked(x, 0.5, m, causal, kernel), ref, dtype,
                                  f"{kernel} cols={cols} x+{xoff} mask+{moff} causal={causal}")


def test_fully_masked_rows_are_nan():
    x, xs = to_device(np.zeros((6, 4)), "f32")
    y = _masked(x, 1.0, None, 6, "auto")  # q > cols: queries 0 and 1 see no key
    ref = oracle.masked_softmax(xs, 1.0, None, 6)
    assert np.all(np.isnan(y[[0, 1]])) and np.all(np.isnan(ref[[0, 1]]))
    check(y[2:], ref[2:], "f32", "partly masked rows")


def test_masked_rejects_splitk_and_bad_args():
    x = torch.zeros(4, 1 << 16, dtype=torch.float16, device="cuda")
    for kernel in ("splitk", "splitk_fused", "splitk_ordered"):
        with pytest.raises(rws.SoftmaxError) as e:
            rws.softmax_masked(x, kernel=kernel)
        assert e.value.status == rws.RWS_ERR_UNSUPPORTED_SHAPE
    st = rws.softmax_fwd_masked(x.data_ptr(), x.data_ptr(), 4, 1 << 16, rws.RWS_F16, 1.0, 0, 0,
                                -1, 0, 0)
    assert st == rws.RWS_ERR_INVALID_ARG


def test_long_rows_masked_use_two_pass():
    x, xs = to_device(np.random.Generator(np.random.PCG64(5)).normal(0, 2, (3, 300001)), "f16")
    assert rws.softmax_describe_launch(3, 300001, rws.RWS_F16, x.data_ptr(), x.data_ptr()) \
        .startswith("splitk")
    check(_masked(x, 0.5, None, 0, "auto"), oracle.masked_softmax(xs, 0.5, None, 0), "f16", "auto")


def test_out_on_the_host_is_rejected_before_any_launch():
    # a host tensor's pointer handed to a kernel would fault the GPU: every
    # tensor-level entry point checks out's device first
    x = torch.zeros(4, 64, dtype=torch.float16, device="cuda")
    host = torch.empty(4, 64, dtype=torch.float16)
    for call in (lambda: rws.softmax_masked(x, 0.5, out=host),
                 lambda: rws.softmax(x, out=host),
                 lambda: rws.softmax_backward(x, x, out=host),
                 lambda: rws.layer_norm(x, out=host),
                 lambda: rws.rms_norm(x, out=host)):
        with pytest.raises(ValueError):
            call()


# --------------------------------------------------------------------------
# tile_rows: short rows that are not line-aligned, several per wave
# --------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("S", [9, 33, 77, 197, 200, 250, 500])
def test_tile_rows_attention_scores(dtype, S):
    # [B*H*S, S] scores with a [S, S] mask (rows of it wrap inside most
    # tiles when S is not a multiple of the tile height), causal or not
    if not tile_supports(S, dtype):
        pytest.skip("outside the tile rows")
    BH = 6
    g = np.random.Generator(np.random.PCG64(S * 3 + 1))
    x64 = g.normal(0.0, 4.0, (BH * S, S))
    m64 = g.normal(0.0, 2.0, (S, S))
    m64[:, 3::7] = -math.inf if dtype != "bf16" else -1.0e30  # key 0 stays visible
    x, xs = to_device(x64, dtype)
    m, ms = to_device(m64, dtype)
    scale = 0.125
    es = 4 if dtype == "f32" else 2
    for causal in (0, S):
        ref = oracle.masked_softmax(xs, scale, ms, causal)
        desc = rws.softmax_describe_launch(BH * S, S, rws.dtype_code(x.dtype), x.data_ptr(),
                                           x.data_ptr(), masked=True)
        if (S * es) % 128 and ((S * es) % 16 or S * es > 128) and BH * S >= 64:
            assert desc.startswith("tile_rows<"), desc
        for kernel in ("auto", "tile_rows"):
            y = _masked(x, scale, m, causal, kernel)
            check(y, ref, dtype, f"{kernel} {desc} S={S} causal={causal}")


@pytest.mark.parametrize("dtype", DTYPES)
def test_tile_rows_mask_phase_rows_and_limits(dtype):
    # a mask 16-byte aligned or not (one element in: two loads and a byte
    # shift per granule, element loads where the pair would leave the mask),
    # mask rows that do not divide the rows (a wrap in most tiles, or none
    # when one row is broadcast), causal limits with more keys than queries,
    # a partial last tile, no mask
    cols = 77
    rows = 3 * 7 * 24 + 5
    g = np.random.Generator(np.random.PCG64(77))
    x64 = g.normal(0.0, 3.0, (rows, cols))
    x, xs = to_device(x64, dtype)
    for mask_rows in (1, 5, 24, 77, 100):
        m64 = g.normal(0.0, 2.0, (mask_rows, cols))
        for moff in (0, 1):
            m, ms = to_device(m64, dtype, offset=moff)
            for causal in (0, 17, 77):
                ref = oracle.masked_softmax(xs, 0.5, ms, causal)
                y = _masked(x, 0.5, m, causal, "tile_rows")
                check(y, ref, dtype, f"mask_rows={mask_rows} offset={moff} causal={causal}")
    for causal in (0, 17):
        ref = oracle.masked_softmax(xs, -1.25, None, causal)
        check(_masked(x, -1.25, None, causal, "tile_rows"), ref, dtype, f"no mask causal={causal}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_tile_rows_masked_full_size_vit_scores(dtype):
    # ViT-like scores: 64 x 12 heads of 197 x 197, a [197,197] mask, causal;
    # sampled rows (both ends and seeded random ones) against the oracle,
    # every row sum on the device
    S, BH = 197, 64 * 12
    rows = BH * S
    gen = torch.Generator(device="cuda").manual_seed(197)
    x = (torch.randn(rows, S, generator=gen, device="cuda") * 4.0).to(TORCH_DTYPE[dtype])
    m = (torch.randn(S, S, generator=gen, device="cuda") * 2.0).to(TORCH_DTYPE[dtype])
    desc = rws.softmax_describe_launch(rows, S, rws.dtype_code(x.dtype), x.data_ptr(),
                                       x.data_ptr(), masked=True)
    assert desc.startswith("tile_rows<"), desc
    out = torch.empty_like(x)
    rws.softmax_masked(x, scale=0.125, mask=m, causal_q=S, out=out)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all().item()
    assert (out.double().sum(dim=1) - 1.0).abs().max().item() <= 1e-2
    rng = np.random.Generator(np.random.PCG64(5))
    idx = np.unique(np.concatenate([np.arange(300), np.arange(rows - 300, rows),
                                    rng.integers(0, rows, 600)]))
    ti = torch.from_numpy(idx).cuda()
    xs = x.index_select(0, ti).double().cpu().numpy()
    ms = m.double().cpu().numpy()
    # the oracle over the sampled rows: each keeps its global row's mask row
    # and causal limit
    ref = np.empty((idx.size, S))
    for k, r in enumerate(idx):
        full = oracle.masked_softmax(np.vstack([np.zeros((r % S, S)), xs[k:k + 1]]), 0.125, ms, S)
        ref[k] = full[-1]
    check(out.index_select(0, ti).double().cpu().numpy(), ref, dtype, f"{desc} sampled rows")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("S,heads,family", [(577, 96, "wave_row<"), (1001, 32, "block_onepass<")])
def test_long_masked_rows_full_size(dtype, S, heads, family):
    # score rows longer than a tile holds, at full size: S = 577 (two rows
    # per wave, three granules per lane) and S = 1001 (a workgroup per row),
    # where most heads' mask rows have another 16-byte phase than their
    # input rows (aligned mask pairs and a shift) and the mask's first and
    # last rows read element by element; a [S,S] mask, causal.  Sampled rows
    # (the ends of every eighth head, seeded random ones) against the oracle,
    # every row sum on the device.
    rows = heads * S
    gen = torch.Generator(device="cuda").manual_seed(S)
    x = (torch.randn(rows, S, generator=gen, device="cuda") * 4.0).to(TORCH_DTYPE[dtype])
    m = (torch.randn(S, S, generator=gen, device="cuda") * 2.0).to(TORCH_DTYPE[dtype])
    desc = rws.softmax_describe_launch(rows, S, rws.dtype_code(x.dtype), x.data_ptr(),
                                       x.data_ptr(), masked=True)
    assert desc.startswith(family), desc
    out = torch.empty_like(x)
    rws.softmax_masked(x, scale=0.125, mask=m, causal_q=S, out=out)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all().item()
    assert (out.double().sum(dim=1) - 1.0).abs().max().item() <= 1e-2
    rng = np.random.Generator(np.random.PCG64(S + 1))
    ends = [h * S + r for h in range(0, heads, 8) for r in (0, 1, S - 2, S - 1)]
    idx = np.unique(np.concatenate([np.array(ends), rng.integers(0, rows, 300)]))
    ti = torch.from_numpy(idx).cuda()
    xs = x.index_select(0, ti).double().cpu().numpy()
    ms = m.double().cpu().numpy()
    ref = np.empty((idx.size, S))
    for k, r in enumerate(idx):
        # the oracle on a block whose last row is global row r: same mask row
        # and causal limit
        full = oracle.masked_softmax(np.vstack([np.zeros((r % S, S)), xs[k:k + 1]]), 0.125, ms, S)
        ref[k] = full[-1]
    check(out.index_select(0, ti).double().cpu().numpy(), ref, dtype, f"{desc} sampled rows")
