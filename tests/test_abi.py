"""The C ABI without a GPU: the library loads, exports every symbol that
include/row_wise_softmax.h declares, and its host-side logic (argument
checks, status strings, kernel names, the dispatcher's choices) behaves as
documented.  No call here reaches a kernel launch."""
import ctypes
import os
import re

import numpy as np
import pytest

import row_wise_safe_amd as rws

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "row_wise_softmax.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(rws.library_path()):
        from row_wise_safe_amd import build
        build.build()
    return rws.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b((?:softmax|layernorm|rmsnorm)_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("softmax_fwd", "softmax_fwd_kernel", "softmax_select_kernel",
              "softmax_describe_launch", "softmax_describe_launch_masked",
              "softmax_kernel_name", "softmax_status_string",
              "softmax_last_error", "softmax_copy_bytes", "layernorm_fwd", "rmsnorm_fwd",
              "layernorm_fwd_kernel", "rmsnorm_fwd_kernel"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    path = rws.library_path()
    raw = ctypes.CDLL(path)
    for n in declared_functions():
        assert hasattr(raw, n), f"{n} not exported"


def test_binding_mirrors_the_abi():
    for n in declared_functions():
        assert callable(getattr(rws, n)), n


def test_status_strings_and_names(lib):
    assert rws.softmax_status_string(rws.RWS_OK) == "ok"
    for st in range(1, 7):
        assert rws.softmax_status_string(st) not in ("", "ok", "unknown status")
    assert rws.softmax_status_string(99) == "unknown status"
    assert [rws.softmax_kernel_name(i) for i in range(8)] == \
        ["auto", "wave_row", "block_onepass", "two_pass", "splitk", "splitk_fused",
         "splitk_ordered", "tile_rows"]
    assert rws.softmax_kernel_name(17) == "unknown"


@pytest.mark.parametrize("args,status", [
    ((0, 0, -1, 3, rws.RWS_F16, 0), rws.RWS_ERR_INVALID_ARG),
    ((0, 0, 3, -1, rws.RWS_F16, 0), rws.RWS_ERR_INVALID_ARG),
    ((0, 0, 3, 4, 3, 0), rws.RWS_ERR_UNSUPPORTED_DTYPE),
    ((0, 0, 3, 4, -1, 0), rws.RWS_ERR_UNSUPPORTED_DTYPE),
    ((0, 0, 3, 4, rws.RWS_F16, 0), rws.RWS_ERR_INVALID_ARG),        # NULL pointers
    ((16, 0, 3, 4, rws.RWS_F16, 0), rws.RWS_ERR_INVALID_ARG),       # NULL out
    ((17, 32, 3, 4, rws.RWS_F16, 0), rws.RWS_ERR_MISALIGNED),       # odd address for fp16
    ((32, 18, 3, 4, rws.RWS_F32, 0), rws.RWS_ERR_MISALIGNED),       # 2-byte aligned fp32
    ((32, 32, 3, (1 << 30) + 1, rws.RWS_F16, 0), rws.RWS_ERR_UNSUPPORTED_SHAPE),
])
def test_argument_checks_never_launch(lib, args, status):
    assert rws.softmax_fwd(*args) == status
    assert rws.softmax_last_error() != ""


def test_empty_is_success_without_pointers(lib):
    assert rws.softmax_fwd(0, 0, 0, 5, rws.RWS_F16, 0) == rws.RWS_OK
    assert rws.softmax_fwd(0, 0, 5, 0, rws.RWS_BF16, 0) == rws.RWS_OK
    assert rws.softmax_last_error() == ""


def test_bad_kernel_id(lib):
    assert rws.softmax_fwd_kernel(32, 32, 2, 2, rws.RWS_F32, 0, 9) == rws.RWS_ERR_INVALID_ARG
    assert rws.softmax_fwd_kernel(32, 32, 2, 2, rws.RWS_F32, 0, 8) == rws.RWS_ERR_INVALID_ARG
    assert rws.softmax_fwd_kernel(32, 32, 2, 2, rws.RWS_F32, 0, -1) == rws.RWS_ERR_INVALID_ARG


def test_copy_argument_checks(lib):
    assert rws.softmax_copy_bytes(16, 32, 15, 0) == rws.RWS_ERR_MISALIGNED
    assert rws.softmax_copy_bytes(16, 32, -16, 0) == rws.RWS_ERR_INVALID_ARG
    assert rws.softmax_copy_bytes(0, 0, 0, 0) == rws.RWS_OK
    for fn in (rws.softmax_read_bytes, rws.softmax_write_bytes):
        assert fn(16, 15, 0) == rws.RWS_ERR_MISALIGNED
        assert fn(24, 32, 0) == rws.RWS_ERR_MISALIGNED
        assert fn(16, -16, 0) == rws.RWS_ERR_INVALID_ARG
        assert fn(0, 16, 0) == rws.RWS_ERR_INVALID_ARG
        assert fn(0, 0, 0) == rws.RWS_OK


def test_forced_wave_row_rejects_long_rows(lib):
    buf = ctypes.create_string_buffer(256)
    st = lib.softmax_describe_launch(2, 4800, rws.RWS_F16, 256, 256, 1, buf, 256)
    assert st == rws.RWS_ERR_UNSUPPORTED_SHAPE


# The dispatcher's routing for the five workloads (16-byte aligned pointers).
@pytest.mark.parametrize("rows,cols,dtype,family", [
    (2, 3, rws.RWS_F32, "wave_row"),
    (64, 1000, rws.RWS_F32, "block_onepass"),  # few waves: one granule per thread
    (65536, 512, rws.RWS_F16, "wave_row"),
    (1 << 20, 128, rws.RWS_BF16, "wave_row"),
    (8192, 4097, rws.RWS_F16, "block_onepass"),
    (16, 1 << 20, rws.RWS_F16, "splitk_ordered"),
    (3, (1 << 20) - 1, rws.RWS_F16, "splitk_fused"),  # at most four rows
    (1, 1 << 30, rws.RWS_F32, "splitk"),  # P = 131072 chunks: two launches
    (4096, 1 << 20, rws.RWS_F16, "two_pass"),
    # few long rows, from the measured crossovers (256 CUs assumed): split-k
    # below half the CUs, or at half of them when block_onepass would park in LDS
    (64, 65536, rws.RWS_F16, "splitk_ordered"),
    (128, 65536, rws.RWS_F16, "block_onepass"),
    (128, 131072, rws.RWS_F16, "splitk_ordered"),
    (256, 131072, rws.RWS_F16, "block_onepass"),
    (256, 16384, rws.RWS_F16, "block_onepass"),
    (384, 65536, rws.RWS_F16, "block_onepass"),
    # ordered single launch while the input fits 32 MiB and P <= 512, from
    # eight rows; the fused single launch while its whole grid fits at once
    # (64 MiB of line-aligned 16-bit input; capacity from the compiled waves
    # per SIMD without a device); two launches beyond
    (8, 1 << 21, rws.RWS_F16, "splitk_ordered"),   # 32 MiB, P = 256
    (8, 1 << 20, rws.RWS_F16, "splitk_ordered"),   # 16 MiB
    (4, 1 << 22, rws.RWS_F16, "splitk_fused"),     # 32 MiB, four rows
    (4, 1 << 20, rws.RWS_F16, "splitk_fused"),     # 8 MiB, four rows
    (2, 1 << 23, rws.RWS_F16, "splitk_fused"),     # 32 MiB, P = 1024 ordered
    (16, 1 << 21, rws.RWS_F16, "splitk_fused"),    # 64 MiB
    (4, 1 << 23, rws.RWS_F16, "splitk_fused"),     # 64 MiB
    (128, 1 << 18, rws.RWS_F16, "splitk_fused"),   # 64 MiB
    (16, 1 << 20, rws.RWS_F32, "splitk_fused"),    # 64 MiB
    (4, 1 << 25, rws.RWS_F16, "splitk"),           # 256 MiB: several passes
    (16, 1 << 22, rws.RWS_F16, "splitk"),          # 128 MiB
])
def test_dispatch_routes(lib, rows, cols, dtype, family):
    kid = rws.softmax_select_kernel(rows, cols, dtype, 256, 512)
    assert rws.softmax_kernel_name(kid) == family
    desc = rws.softmax_describe_launch(rows, cols, dtype, 256, 512)
    assert desc.startswith(family)


# The launch shape chosen for rows held by one workgroup (16-byte aligned
# pointers, 256 CUs assumed without a device): one granule per thread when the
# launch has few waves, else 2-5 granules per thread with the fewest idle
# slots -- the fastest shapes of sweeps on MI355X.
@pytest.mark.parametrize("rows,cols,dtype,shape", [
    (64, 1000, rws.RWS_F32, "B=320,KR=1"),
    (1024, 2000, rws.RWS_F16, "B=320,KR=1"),
    (64, 8000, rws.RWS_F16, "B=1024,KR=1"),
    (32768, 1000, rws.RWS_F16, "B=64,KR=3"),
    (16384, 2000, rws.RWS_F16, "B=64,KR=5"),
    (8192, 4000, rws.RWS_F16, "B=256,KR=2"),
    (8192, 4097, rws.RWS_F16, "B=192,KR=3"),
    (4096, 8000, rws.RWS_F16, "B=512,KR=2"),
])
def test_block_shape_choice(lib, rows, cols, dtype, shape):
    desc = rws.softmax_describe_launch(rows, cols, dtype, 256, 512)
    assert desc.startswith("block_onepass") and shape in desc, desc


def test_many_rows_of_two_granules_stay_on_one_wave(lib):
    # fp16 rows of 960 columns (1920 bytes, line-aligned): 120 granules, two per lane
    desc = rws.softmax_describe_launch(65536, 960, rws.RWS_F16, 256, 512)
    assert desc.startswith("wave_row<f16,aligned,G=64,K=2"), desc
    # few rows of the same length: a workgroup of one granule per thread
    assert "KR=1" in rws.softmax_describe_launch(64, 960, rws.RWS_F16, 256, 512)


# Write-through stores only where every output line is written by one wave:
# wave_row on line-aligned rows (plain and masked), not on rows that start
# mid-line, and never for the other families.
@pytest.mark.parametrize("rows,cols,dtype,inp,out,masked,wt", [
    (65536, 512, rws.RWS_F16, 256, 512, False, True),
    (65536, 512, rws.RWS_F16, 256, 512, True, True),
    (1 << 20, 128, rws.RWS_BF16, 256, 512, False, True),
    (65536, 512, rws.RWS_F16, 256 + 16, 512 + 16, False, False),  # 16-byte aligned only
    (65536, 504, rws.RWS_F16, 256, 512, False, False),  # rows of 1008 bytes
    (8192, 4097, rws.RWS_F16, 256, 512, False, False),  # block_onepass
    (16, 1 << 20, rws.RWS_F16, 256, 512, False, False),  # split-k
])
def test_write_through_only_on_line_aligned_wave_rows(lib, rows, cols, dtype, inp, out,
                                                      masked, wt):
    desc = rws.softmax_describe_launch(rows, cols, dtype, inp, out, masked=masked)
    assert ("store=wt" in desc) == wt, desc
    if wt:
        assert desc.startswith("wave_row<") and ",aligned," in desc, desc


# Normalisation shapes: the tuned lane groups, then the forward's workgroup
# shapes (exact-fit two-granule shapes at common fp16 hidden sizes).
@pytest.mark.parametrize("rows,cols,shape", [
    (131040, 192, "norm_wave<f16,aligned,G=16,K=2,U=1>"),
    (32760, 384, "norm_wave<f16,aligned,G=8,K=6,U=1>"),
    (43690, 768, "norm_block<f16,aligned,B=64,KR=2>"),
    (32768, 1024, "norm_block<f16,aligned,B=64,KR=2>"),
    (16384, 2048, "norm_block<f16,aligned,B=128,KR=2>"),
    (8192, 4096, "norm_block<f16,aligned,B=256,KR=2>"),
    (4096, 8192, "norm_block<f16,aligned,B=512,KR=2>"),
    (32768, 1000, "norm_block<f16,unaligned,B=64,KR=3>"),
    (8192, 4097, "norm_block<f16,unaligned,B=192,KR=3>"),
    (64, 1000, "norm_block<f16,unaligned,B=192,KR=1>"),
    (1024, 40000, "norm_stream<f16,aligned,B=1024,U=4>"),
])
def test_norm_shape_choice(lib, rows, cols, shape):
    desc = rws.norm_describe_launch(rows, cols, rws.RWS_F16, 256, 512)
    assert desc.startswith(shape), desc


# With weight and/or bias the two tuned widths take groups of fewer rows.
@pytest.mark.parametrize("rows,cols,shape", [
    (131040, 192, "norm_wave<f16,aligned,G=8,K=3,U=1>"),
    (32760, 384, "norm_wave<f16,aligned,G=16,K=3,U=1>"),
    # line window 31: (8,3) too small; 16-byte aligned rows with a weight or
    # bias take windows that start at the row
    (131040, 184, "norm_wave<f16,aligned,G=16,K=2,U=1>"),
    (8192, 4096, "norm_block<f16,aligned,B=256,KR=2>"),
])
def test_norm_affine_shape_choice(lib, rows, cols, shape):
    desc = rws.norm_describe_launch(rows, cols, rws.RWS_F16, 256, 512, affine=True)
    assert desc.startswith(shape), desc


# Backward block shapes: the smallest capacity, at equal capacity the one
# with more granules per thread.
@pytest.mark.parametrize("rows,cols,shape", [
    (65536, 512, "bwd_wave<f16,aligned,G=64,K=1,U=1>"),
    (32768, 1000, "bwd_block<f16,unaligned,B=64,KR=3> grid=32768 block=64 xcd_run=128"),
    (32768, 1024, "bwd_block<f16,aligned,B=128,KR=1>"),
    (16384, 2000, "bwd_block<f16,unaligned,B=320,KR=1>"),
    (8192, 4096, "bwd_block<f16,aligned,B=512,KR=1>"),
    (8192, 4097, "bwd_block<f16,unaligned,B=192,KR=3> grid=8192 block=192 xcd_run=16"),
    (1024, 40000, "bwd_stream<f16,aligned,B=1024,U=4>"),
])
def test_bwd_shape_choice(lib, rows, cols, shape):
    desc = rws.softmax_bwd_describe_launch(rows, cols, rws.RWS_F16, 256, 512)
    assert desc.startswith(shape), desc


# Few long rows: the backward and the normalisations take the single-launch
# split-k (chunks of 1024 granules) for rows their one-workgroup-per-row
# register form cannot hold (more than 4096 granules) and fewer rows than
# CUs (256 assumed without a device); where that form holds the row, it is
# kept at any row count.
@pytest.mark.parametrize("rows,cols,P", [(16, 1 << 20, 128), (64, 1 << 18, 32),
                                         (192, 65536, 8)])
def test_few_long_rows_take_ordered_split_k(lib, rows, cols, P):
    b = rws.softmax_bwd_describe_launch(rows, cols, rws.RWS_F16, 256, 512)
    n = rws.norm_describe_launch(rows, cols, rws.RWS_F16, 256, 512)
    assert b.startswith("bwd_ordered") and f" P={P} " in b, b
    assert n.startswith("norm_ordered") and f" P={P} " in n, n
    # from one row per CU on, the streaming form
    assert rws.softmax_bwd_describe_launch(256, cols, rws.RWS_F16, 256, 512).startswith("bwd_stream")
    assert rws.norm_describe_launch(256, cols, rws.RWS_F16, 256, 512).startswith("norm_stream")


@pytest.mark.parametrize("rows,cols", [(16, 16384), (128, 16384), (8, 32768), (64, 32768)])
def test_rows_the_register_form_holds_keep_it(lib, rows, cols):
    assert rws.softmax_bwd_describe_launch(rows, cols, rws.RWS_F16, 256, 512).startswith("bwd_block")
    assert rws.norm_describe_launch(rows, cols, rws.RWS_F16, 256, 512).startswith("norm_block")


# Runs of consecutive rows per XCD for block_onepass on rows that are not
# line-aligned: the smallest power of two of at least 128 KiB of rows.
@pytest.mark.parametrize("rows,cols,inp,run", [
    (8192, 4097, 256, 16),      # 8194-byte rows
    (16384, 2001, 256, 64),     # 4002-byte rows
    (32768, 1000, 256, 128),    # 2000-byte rows
    (4096, 8000, 256, None),    # 16000-byte rows, line-aligned
    (8192, 4096, 256, None),    # 8192-byte rows, line-aligned
    (8192, 4096, 256 + 2, 16),  # the same rows starting mid-line
])
def test_xcd_run_length(lib, rows, cols, inp, run):
    desc = rws.softmax_describe_launch(rows, cols, rws.RWS_F16, inp, inp + 256)
    assert desc.startswith("block_onepass"), desc
    if run is None:
        assert "xcd_run" not in desc, desc
    else:
        assert desc.endswith(f" xcd_run={run}"), desc


@pytest.mark.parametrize("rows,cols", [((1 << 22) + 5, 12000), ((1 << 22) + 5, 24)])
def test_block_launch_stays_below_2_32_threads(lib, rows, cols):
    # the grid of one launch times its workgroup size must fit the 32-bit grid size
    for kernel in (2, 3):  # block_onepass, two_pass
        desc = rws.softmax_describe_launch(rows, cols, rws.RWS_F16, 256, 512, kernel)
        grid = int(re.search(r"grid=(\d+)", desc).group(1))
        block = int(re.search(r"block=(\d+)", desc).group(1))
        assert grid * block < 1 << 32, desc


def test_select_rejects_bad_args(lib):
    assert rws.softmax_select_kernel(-1, 4, rws.RWS_F16) < 0
    assert rws.softmax_select_kernel(4, 4, 5) < 0


def test_describe_mentions_alignment(lib):
    assert "unaligned" in rws.softmax_describe_launch(8, 100, rws.RWS_F16, 258, 258)
    assert "split-phase" in rws.softmax_describe_launch(8, 100, rws.RWS_F16, 258, 256)
    assert ",aligned" in rws.softmax_describe_launch(8, 128, rws.RWS_F16, 256, 512)


@pytest.mark.parametrize("cols,plain_group,masked_group", [
    (512, "G=64,K=1,U=1", "G=32,K=2,U=1"),
    (384, "G=64,K=1,U=1", "G=32,K=2,U=1"),
    (256, "G=32,K=1,U=1", "G=16,K=2,U=1"),
    (192, "G=32,K=1,U=1", "G=16,K=2,U=1"),
    (128, "G=16,K=1,U=1", "G=8,K=2,U=1"),
    (768, "G=64,K=2,U=1", "G=32,K=3,U=1"),
    (1024, "G=64,K=2,U=1", "G=64,K=2,U=1"),
])
def test_masked_launch_choice(lib, cols, plain_group, masked_group):
    # one granule per lane for plain softmax where it holds the row; two
    # granules per lane on half the lanes for the masked form (each measured
    # fastest on MI355X); two granules on full waves for both past 64
    rows = 64 * cols
    plain = rws.softmax_describe_launch(rows, cols, rws.RWS_F16, 256, 512)
    masked = rws.softmax_describe_launch(rows, cols, rws.RWS_F16, 256, 512, masked=True)
    assert plain_group in plain and "block=64" in plain, plain
    assert masked_group in masked and "block=64" in masked, masked


@pytest.mark.parametrize("cols,dtype", [(577, "f16"), (600, "f16"), (700, "f16"), (300, "f32")])
def test_three_granule_lane_groups(lib, cols, dtype):
    # rows of 65-96 granules that are not line-aligned: two rows per wave,
    # three granules per lane on 32 lanes (plain and masked)
    code = rws.RWS_F16 if dtype == "f16" else rws.RWS_F32
    for masked in (False, True):
        d = rws.softmax_describe_launch(64 * cols, cols, code, 256, 512, masked=masked)
        assert d.startswith("wave_row<") and "G=32,K=3,U=1" in d, d


def test_masked_argument_checks(lib):
    f16 = rws.RWS_F16
    assert rws.softmax_fwd_masked(256, 256, 2, 8, f16, 1.0, 0, 0, -1, 0, 0) == rws.RWS_ERR_INVALID_ARG
    assert rws.softmax_fwd_masked(256, 256, 2, 8, f16, 1.0, 257, 2, 0, 0, 0) == rws.RWS_ERR_MISALIGNED
    assert rws.softmax_fwd_masked(256, 256, 2, 8, f16, 1.0, 512, 0, 0, 0, 0) == rws.RWS_ERR_INVALID_ARG
    assert rws.softmax_fwd_masked(0, 0, 0, 8, f16, 1.0, 0, 0, 0, 0, 0) == rws.RWS_OK
    assert rws.softmax_fwd_masked(256, 256, 2, 8, 9, 1.0, 0, 0, 0, 0, 0) == \
        rws.RWS_ERR_UNSUPPORTED_DTYPE


def test_backward_argument_checks(lib):
    f16 = rws.RWS_F16
    assert rws.softmax_bwd(256, 0, 256, 2, 8, f16, 0) == rws.RWS_ERR_INVALID_ARG   # NULL dy
    assert rws.softmax_bwd(256, 257, 256, 2, 8, f16, 0) == rws.RWS_ERR_MISALIGNED
    assert rws.softmax_bwd(0, 0, 0, 0, 8, f16, 0) == rws.RWS_OK
    assert rws.softmax_bwd_kernel(256, 256, 256, 2, 8, f16, 0, 4) == rws.RWS_ERR_INVALID_ARG
    assert rws.softmax_bwd(256, 256, 256, 2, 8, 7, 0) == rws.RWS_ERR_UNSUPPORTED_DTYPE


def test_norm_argument_checks(lib):
    f16 = rws.RWS_F16
    ok = rws.RWS_OK
    assert rws.layernorm_fwd(256, 256, 2, 8, f16, -1.0, 0, 0, 0, 0, 0) == rws.RWS_ERR_INVALID_ARG
    assert rws.layernorm_fwd(256, 256, 2, 8, f16, float("nan"), 0, 0, 0, 0, 0) == \
        rws.RWS_ERR_INVALID_ARG
    assert rws.layernorm_fwd(256, 256, 2, 8, f16, float("inf"), 0, 0, 0, 0, 0) == \
        rws.RWS_ERR_INVALID_ARG
    assert rws.layernorm_fwd(256, 256, 2, 8, f16, 1e-5, 257, 0, 0, 0, 0) == rws.RWS_ERR_MISALIGNED
    assert rws.layernorm_fwd(256, 256, 2, 8, f16, 1e-5, 0, 259, 0, 0, 0) == rws.RWS_ERR_MISALIGNED
    assert rws.layernorm_fwd(256, 256, 2, 8, f16, 1e-5, 0, 0, 258, 0, 0) == rws.RWS_ERR_MISALIGNED
    assert rws.rmsnorm_fwd(256, 256, 2, 8, f16, 1e-5, 0, 2, 0) == rws.RWS_ERR_MISALIGNED
    assert rws.layernorm_fwd(0, 0, 0, 8, f16, 1e-5, 0, 0, 0, 0, 0) == ok
    assert rws.rmsnorm_fwd(0, 0, 3, 0, f16, 1e-5, 0, 0, 0) == ok
    assert rws.layernorm_fwd(256, 256, 2, 8, 7, 1e-5, 0, 0, 0, 0, 0) == rws.RWS_ERR_UNSUPPORTED_DTYPE
    assert rws.layernorm_fwd(0, 256, 2, 8, f16, 1e-5, 0, 0, 0, 0, 0) == rws.RWS_ERR_INVALID_ARG
    for kid in (4, 5, 9, -1):
        assert rws.layernorm_fwd_kernel(256, 256, 2, 8, f16, 1e-5, 0, 0, 0, 0, 0, kid) == \
            rws.RWS_ERR_INVALID_ARG
        assert rws.rmsnorm_fwd_kernel(256, 256, 2, 8, f16, 1e-5, 0, 0, 0, kid) == \
            rws.RWS_ERR_INVALID_ARG
    # rows too long for the register-held families are refused before any launch
    assert rws.layernorm_fwd_kernel(256, 256, 2, 8192, f16, 1e-5, 0, 0, 0, 0, 0, 1) == \
        rws.RWS_ERR_UNSUPPORTED_SHAPE
    assert rws.rmsnorm_fwd_kernel(256, 256, 2, 70000, f16, 1e-5, 0, 0, 0, 2) == \
        rws.RWS_ERR_UNSUPPORTED_SHAPE


def test_plan_cache_keeps_calls_apart(lib):
    # the dispatcher keeps its last plans per thread, keyed on everything a
    # plan depends on: the same queries in any order give the same answers
    cases = []
    for rows, cols in [(65536, 512), (64, 1000), (16, 1 << 20), (8192, 4097), (4096, 8000)]:
        for dtype in (rws.RWS_F32, rws.RWS_F16):
            for inp, out in [(256, 512), (258, 514), (256, 272)]:
                for kid in (0, 2):
                    for masked in (False, True):
                        cases.append((rows, cols, dtype, inp, out, kid, masked))

    def ask(c):
        try:
            return rws.softmax_describe_launch(*c[:6], masked=c[6])
        except rws.SoftmaxError as e:
            return f"error {e.status}"

    first = [ask(c) for c in cases]
    rng = np.random.Generator(np.random.PCG64(0))
    for _ in range(3):
        order = rng.permutation(len(cases))
        for i in order:
            assert ask(cases[i]) == first[i], cases[i]


def test_wait_limit_argument_checks(lib):
    # host-only setter: default (< 0), an explicit count, and out of range
    assert rws.softmax_set_wait_limit(-1) == rws.RWS_OK
    assert rws.softmax_set_wait_limit(1000) == rws.RWS_OK
    assert rws.softmax_set_wait_limit(1 << 32) == rws.RWS_ERR_INVALID_ARG
    assert "2^32" in rws.softmax_last_error()
    assert rws.softmax_set_wait_limit(-1) == rws.RWS_OK


@pytest.mark.parametrize("args,status", [
    ((0, 0, -1, 3, rws.RWS_F16, 0), rws.RWS_ERR_INVALID_ARG),
    ((0, 0, 3, 4, 3, 0), rws.RWS_ERR_UNSUPPORTED_DTYPE),
    ((0, 0, 3, 4, rws.RWS_F16, 0), rws.RWS_ERR_INVALID_ARG),        # NULL pointers
    ((17, 32, 3, 4, rws.RWS_F16, 0), rws.RWS_ERR_MISALIGNED),
    ((32, 32, 3, (1 << 30) + 1, rws.RWS_F16, 0), rws.RWS_ERR_UNSUPPORTED_SHAPE),
])
def test_noalloc_argument_checks_never_launch(lib, args, status):
    assert rws.softmax_fwd_noalloc(*args) == status
    assert rws.softmax_last_error() != ""
    assert rws.softmax_fwd_noalloc(0, 0, 0, 5, rws.RWS_F32, 0) == rws.RWS_OK  # empty: no-op


def test_variant_forcing_host_checks(lib):
    counts = {k: rws.softmax_variant_count(rws.KERNEL_IDS[k]) for k in rws.KERNELS}
    assert all(c > 0 for c in counts.values()), counts
    assert rws.softmax_variant_count(0) == 0 and rws.softmax_variant_count(42) == 0
    code, ip, op = rws.RWS_F16, 256, 256 + 4096
    # every block_onepass shape that holds an fp16 row of 4097 describes itself
    held = 0
    for v in range(counts["block_onepass"]):
        try:
            d = rws.softmax_describe_variant(8192, 4097, code, ip, op, 2, v)
        except rws.SoftmaxError as e:
            assert e.status == rws.RWS_ERR_UNSUPPORTED_SHAPE
            continue
        assert d.startswith("block_onepass<f16,"), d
        held += 1
    assert held >= 5
    # the dispatcher's own choice is one of them
    auto = rws.softmax_describe_launch(8192, 4097, code, ip, op)
    assert any(rws.softmax_describe_variant(8192, 4097, code, ip, op, 2, v) == auto
               for v in range(counts["block_onepass"])
               if "B=" in _try_describe(8192, 4097, code, ip, op, 2, v))
    # a 4-lane group cannot hold 4097 columns; auto and negative ids are refused
    with pytest.raises(rws.SoftmaxError) as e:
        rws.softmax_describe_variant(8, 4097, code, ip, op, 1, 0)
    assert e.value.status == rws.RWS_ERR_UNSUPPORTED_SHAPE
    for kid, v in ((0, 0), (2, -1)):
        assert rws.softmax_fwd_variant(16, 16, 4, 8, code, 0, kid, v) == rws.RWS_ERR_INVALID_ARG
    assert rws.softmax_fwd_variant(16, 16, 4, 8, code, 0, 2, 10 ** 6) == \
        rws.RWS_ERR_UNSUPPORTED_SHAPE


def _try_describe(*args):
    try:
        return rws.softmax_describe_variant(*args)
    except rws.SoftmaxError:
        return ""


def _tile_choice(rows, cols, es):
    """The tile the dispatcher takes for rows of cols elements of es bytes,
    restated from its rule: for each K (granules per lane) the largest
    multiple of the rows' 16-byte period, at most 64, whose tile fits 64*K
    granules; then the K with the least weighted slots per row,
    64*K*w(K) / T.  Up to 2^27 bytes per direction w = 1.30, 1.00, 1.02,
    1.07 for K = 1..4 and the smaller K at equal cost; beyond, w = 1.30,
    1, 1, 1 and the larger tile at equal cost."""
    small = rows * cols * es <= 1 << 27
    weight = {1: 130, 2: 100, 3: 102, 4: 107} if small else {1: 130, 2: 100, 3: 100, 4: 100}
    rb = cols * es
    if cols < 16 // es or rb > 1024:
        return None
    g = 16
    while rb % g:
        g //= 2
    p0 = 16 // g
    best = None
    for K in (1, 2, 3, 4):
        T = min(64, 64 * K * 16 // rb)
        T -= T % p0
        if T < 4:
            continue
        if best is not None:
            lhs, rhs = K * weight[K] * best[0], best[1] * weight[best[1]] * T
            if lhs > rhs or (lhs == rhs and (small or T <= best[0])):
                continue
        best = (T, K)
    return best


@pytest.mark.parametrize("dtype,es", [(rws.RWS_F16, 2), (rws.RWS_BF16, 2), (rws.RWS_F32, 4)])
def test_tile_height_choice(lib, dtype, es):
    # every row length the tile form takes, plain softmax, backward and the
    # normalisations: the height and K follow the rule, and the tile starts
    # on a 16-byte boundary and holds at most 64*K granules
    seen = set()
    for rows, cols in [(4096, c) for c in range(16 // es, 1024 // es + 1)] + \
                      [((1 << 28) // (c * es), c) for c in range(16 // es, 1024 // es + 1, 7)]:
        rb = cols * es
        want = _tile_choice(rows, cols, es)
        fits = want is not None and rb % 128 != 0 and (rb % 16 != 0 or rb > 128)
        desc = rws.softmax_describe_launch(rows, cols, dtype, 256, 512)
        bwd = rws.softmax_bwd_describe_launch(rows, cols, dtype, 256, 512)
        norm = rws.norm_describe_launch(rows, cols, dtype, 256, 512)
        if not fits:
            assert not desc.startswith("tile_rows<"), (cols, desc)
            continue
        T, K = want
        assert (T * rb) % 16 == 0 and T * rb // 16 <= 64 * K and 4 <= T <= 64
        tag = f"T={T},K={K}>"
        assert desc.startswith("tile_rows<") and tag in desc, (cols, desc, want)
        assert bwd.startswith("bwd_tile<") and tag in bwd, (cols, bwd, want)
        assert norm.startswith("norm_tile<") and tag in norm, (cols, norm, want)
        seen.add((T > 32, K))
    # short rows take one lane per row, and K = 2..4 are each chosen somewhere
    assert {2, 3, 4} <= {k for _, k in seen} and any(big for big, _ in seen)


def test_masked_form_takes_the_same_tiles(lib):
    for cols in (33, 77, 197, 250):
        plain = rws.softmax_describe_launch(4096, cols, rws.RWS_F16, 256, 512)
        masked = rws.softmax_describe_launch(4096, cols, rws.RWS_F16, 256, 512, masked=True)
        assert plain.startswith("tile_rows<") and masked == plain, (plain, masked)


def test_tile_needs_enough_rows_and_aligned_pointers(lib):
    assert rws.softmax_describe_launch(64, 250, rws.RWS_F16, 256, 512).startswith("tile_rows<")
    assert not rws.softmax_describe_launch(63, 250, rws.RWS_F16, 256, 512).startswith("tile_rows<")
    assert not rws.softmax_describe_launch(4096, 250, rws.RWS_F16, 258, 512).startswith("tile_rows<")
    assert not rws.softmax_describe_launch(4096, 250, rws.RWS_F16, 256, 520).startswith("tile_rows<")
