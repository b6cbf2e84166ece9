"""GPU parity of every compiled variant of every forward kernel family
(softmax_fwd_variant), not only the ones the dispatcher picks: lane groups
and granules per lane of wave_row, workgroup shapes of block_onepass and
two_pass, chunk shapes of the three split-k forms, each on the shapes it can
hold -- aligned and unaligned rows, three dtypes -- against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import row_wise_safe_amd as rws
from gpu_util import have_gpu, to_device
from tolerance import check

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not have_gpu(), reason="needs an MI355X GPU")]

# (dtype, rows, cols, input offset in elements)
SHAPES = {
    "wave_row": [("f16", 67, 512, 0), ("f32", 33, 1000, 1), ("bf16", 9, 4001, 0)],
    "block_onepass": [("f16", 67, 4097, 0), ("f32", 9, 2000, 1), ("bf16", 5, 65536, 0)],
    "two_pass": [("f16", 17, 4097, 1), ("f32", 5, 70001, 0), ("bf16", 3, 300001, 0)],
    "splitk": [("f16", 4, 300001, 1), ("f32", 3, 1 << 20, 0), ("bf16", 2, 2000003, 0)],
    "splitk_ordered": [("f16", 4, 300001, 1), ("f32", 3, 1 << 20, 0), ("bf16", 2, 2000003, 0)],
    "splitk_fused": [("f16", 4, 300001, 1), ("f32", 2, 1 << 19, 0)],
}


@pytest.fixture(scope="module", autouse=True)
def _lib():
    rws.load_library()
    yield


@pytest.mark.parametrize("family", list(SHAPES))
def test_every_variant_of_every_family(family):
    kid = rws.KERNEL_IDS[family]
    n = rws.softmax_variant_count(kid)
    ran = set()
    for dtype, rows, cols, off in SHAPES[family]:
        g = np.random.Generator(np.random.PCG64(rows * 7919 + cols))
        x, xs = to_device(g.normal(0.0, 4.0, (rows, cols)), dtype, offset=off)
        ref = oracle.safe_softmax(xs)
        code = rws.dtype_code(x.dtype)
        s = torch.cuda.current_stream().cuda_stream
        for v in range(n):
            out = torch.full_like(x, float("nan"))
            try:
                desc = rws.softmax_describe_variant(rows, cols, code, x.data_ptr(), out.data_ptr(),
                                                    kid, v)
            except rws.SoftmaxError as e:
                assert e.status == rws.RWS_ERR_UNSUPPORTED_SHAPE
                continue
            print(f"{family} v{v}: {desc}", flush=True)
            st = rws.softmax_fwd_variant(x.data_ptr(), out.data_ptr(), rows, cols, code, s, kid, v)
            assert st == rws.RWS_OK, rws.softmax_last_error()
            torch.cuda.synchronize()
            check(out.double().cpu().numpy(), ref, dtype, f"{desc} [{rows},{cols}] +{off}")
            ran.add(v)
    assert len(ran) >= min(n, 2), (family, sorted(ran))
