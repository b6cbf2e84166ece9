"""Python binding of librws_softmax.so -- row-wise safe softmax on MI355X,
with its backward and the LayerNorm / RMSNorm row normalisations.

Argument marshalling only: every step of the computation runs in the
library's gfx950 HIP kernels.  The functions named ``softmax_*``,
``layernorm_*`` and ``rmsnorm_*`` mirror the C ABI of
``include/row_wise_softmax.h`` one to one (plain integers for pointers,
sizes and the stream); :func:`softmax` is the tensor-level convenience that
fills them in from a torch tensor and the current stream.

torch is imported first so that the process has a single HIP runtime (the
library then binds to the one torch loaded).  If the library has not been
built, every entry point raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "RWS_F32", "RWS_F16", "RWS_BF16",
    "RWS_OK", "RWS_ERR_INVALID_ARG", "RWS_ERR_UNSUPPORTED_DTYPE", "RWS_ERR_MISALIGNED",
    "RWS_ERR_HIP", "RWS_ERR_UNSUPPORTED_SHAPE", "RWS_ERR_WAIT_TIMEOUT",
    "KERNELS", "KERNEL_IDS",
    "library_path", "load_library",
    "softmax_fwd", "softmax_fwd_kernel", "softmax_fwd_noalloc", "softmax_fwd_masked",
    "softmax_bwd",
    "softmax_bwd_kernel", "softmax_select_kernel",
    "softmax_describe_launch",
    "softmax_describe_launch_masked",
    "norm_describe_launch",
    "softmax_bwd_describe_launch",
    "softmax_kernel_name", "softmax_status_string", "softmax_last_error", "softmax_copy_bytes",
    "softmax_stream_status", "softmax_set_wait_limit", "stream_status",
    "softmax_read_bytes", "softmax_write_bytes",
    "softmax_fwd_variant", "softmax_variant_count", "softmax_describe_variant",
    "layernorm_fwd", "layernorm_fwd_kernel", "rmsnorm_fwd", "rmsnorm_fwd_kernel",
    "softmax", "softmax_masked", "softmax_backward", "layer_norm", "rms_norm", "copy_bytes",
    "dtype_code", "SoftmaxError",
]

RWS_F32, RWS_F16, RWS_BF16 = 0, 1, 2
RWS_OK = 0
RWS_ERR_INVALID_ARG = 1
RWS_ERR_UNSUPPORTED_DTYPE = 2
RWS_ERR_MISALIGNED = 3
RWS_ERR_HIP = 4
RWS_ERR_UNSUPPORTED_SHAPE = 5
RWS_ERR_WAIT_TIMEOUT = 6

KERNEL_IDS = {"auto": 0, "wave_row": 1, "block_onepass": 2, "two_pass": 3, "splitk": 4,
              "splitk_fused": 5, "splitk_ordered": 6, "tile_rows": 7}
KERNELS = tuple(k for k in KERNEL_IDS if k != "auto")

_DTYPES = {torch.float32: RWS_F32, torch.float16: RWS_F16, torch.bfloat16: RWS_BF16}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


class SoftmaxError(RuntimeError):
    def __init__(self, status: int, detail: str = ""):
        self.status = status
        text = softmax_status_string(status) if _LIB is not None else f"status {status}"
        super().__init__(f"{text}: {detail}" if detail else text)


def library_path() -> str:
    return os.path.join(_HERE, "librws_softmax.so")


def load_library():
    """Load librws_softmax.so; raises if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it first (python row_wise_safe_amd/build.py or "
            "__graft_entry__.build()); there is no non-HIP fallback")
    lib = ctypes.CDLL(path)
    i64, vp, cint = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    lib.softmax_fwd.argtypes = [vp, vp, i64, i64, cint, vp]
    lib.softmax_fwd.restype = cint
    lib.softmax_fwd_kernel.argtypes = [vp, vp, i64, i64, cint, vp, cint]
    lib.softmax_fwd_kernel.restype = cint
    lib.softmax_fwd_noalloc.argtypes = [vp, vp, i64, i64, cint, vp]
    lib.softmax_fwd_noalloc.restype = cint
    lib.softmax_fwd_masked.argtypes = [vp, vp, i64, i64, cint, ctypes.c_float, vp, i64, i64, vp,
                                       cint]
    lib.softmax_fwd_masked.restype = cint
    lib.softmax_bwd.argtypes = [vp, vp, vp, i64, i64, cint, vp]
    lib.softmax_bwd.restype = cint
    lib.softmax_bwd_kernel.argtypes = [vp, vp, vp, i64, i64, cint, vp, cint]
    lib.softmax_bwd_kernel.restype = cint
    lib.softmax_select_kernel.argtypes = [i64, i64, cint, vp, vp]
    lib.softmax_select_kernel.restype = cint
    lib.softmax_describe_launch.argtypes = [i64, i64, cint, vp, vp, cint, ctypes.c_char_p, i64]
    lib.softmax_describe_launch.restype = cint
    lib.softmax_describe_launch_masked.argtypes = [i64, i64, cint, vp, vp, cint,
                                                   ctypes.c_char_p, i64]
    lib.softmax_describe_launch_masked.restype = cint
    lib.norm_describe_launch.argtypes = [i64, i64, cint, vp, vp, cint, cint, ctypes.c_char_p, i64]
    lib.norm_describe_launch.restype = cint
    lib.softmax_bwd_describe_launch.argtypes = [i64, i64, cint, vp, vp, cint, ctypes.c_char_p, i64]
    lib.softmax_bwd_describe_launch.restype = cint
    lib.softmax_kernel_name.argtypes = [cint]
    lib.softmax_kernel_name.restype = ctypes.c_char_p
    lib.softmax_status_string.argtypes = [cint]
    lib.softmax_status_string.restype = ctypes.c_char_p
    lib.softmax_last_error.argtypes = []
    lib.softmax_last_error.restype = ctypes.c_char_p
    lib.softmax_copy_bytes.argtypes = [vp, vp, i64, vp]
    lib.softmax_copy_bytes.restype = cint
    lib.softmax_fwd_variant.argtypes = [vp, vp, i64, i64, cint, vp, cint, cint]
    lib.softmax_fwd_variant.restype = cint
    lib.softmax_variant_count.argtypes = [cint]
    lib.softmax_variant_count.restype = cint
    lib.softmax_describe_variant.argtypes = [i64, i64, cint, vp, vp, cint, cint, ctypes.c_char_p,
                                             i64]
    lib.softmax_describe_variant.restype = cint
    lib.softmax_read_bytes.argtypes = [vp, i64, vp]
    lib.softmax_read_bytes.restype = cint
    lib.softmax_write_bytes.argtypes = [vp, i64, vp]
    lib.softmax_write_bytes.restype = cint
    lib.softmax_stream_status.argtypes = [vp]
    lib.softmax_stream_status.restype = cint
    lib.softmax_set_wait_limit.argtypes = [i64]
    lib.softmax_set_wait_limit.restype = cint
    f32 = ctypes.c_float
    lib.layernorm_fwd.argtypes = [vp, vp, i64, i64, cint, f32, vp, vp, vp, vp, vp]
    lib.layernorm_fwd.restype = cint
    lib.layernorm_fwd_kernel.argtypes = [vp, vp, i64, i64, cint, f32, vp, vp, vp, vp, vp, cint]
    lib.layernorm_fwd_kernel.restype = cint
    lib.rmsnorm_fwd.argtypes = [vp, vp, i64, i64, cint, f32, vp, vp, vp]
    lib.rmsnorm_fwd.restype = cint
    lib.rmsnorm_fwd_kernel.argtypes = [vp, vp, i64, i64, cint, f32, vp, vp, vp, cint]
    lib.rmsnorm_fwd_kernel.restype = cint
    _LIB = lib
    return lib


# --- the C ABI, one to one --------------------------------------------------

def softmax_fwd(in_ptr: int, out_ptr: int, rows: int, cols: int, dtype: int, stream: int) -> int:
    return load_library().softmax_fwd(in_ptr, out_ptr, rows, cols, dtype, stream)


def softmax_fwd_kernel(in_ptr: int, out_ptr: int, rows: int, cols: int, dtype: int, stream: int,
                       kernel_id: int) -> int:
    return load_library().softmax_fwd_kernel(in_ptr, out_ptr, rows, cols, dtype, stream,
                                             kernel_id)


def softmax_fwd_noalloc(in_ptr: int, out_ptr: int, rows: int, cols: int, dtype: int,
                        stream: int) -> int:
    return load_library().softmax_fwd_noalloc(in_ptr, out_ptr, rows, cols, dtype, stream)


def softmax_fwd_masked(in_ptr: int, out_ptr: int, rows: int, cols: int, dtype: int, scale: float,
                       mask_ptr: int, mask_rows: int, causal_q: int, stream: int,
                       kernel_id: int = 0) -> int:
    return load_library().softmax_fwd_masked(in_ptr, out_ptr, rows, cols, dtype, scale,
                                             mask_ptr or None, mask_rows, causal_q, stream,
                                             kernel_id)


def softmax_bwd(y_ptr: int, dy_ptr: int, dx_ptr: int, rows: int, cols: int, dtype: int,
                stream: int) -> int:
    return load_library().softmax_bwd(y_ptr, dy_ptr, dx_ptr, rows, cols, dtype, stream)


def softmax_bwd_kernel(y_ptr: int, dy_ptr: int, dx_ptr: int, rows: int, cols: int, dtype: int,
                       stream: int, kernel_id: int) -> int:
    return load_library().softmax_bwd_kernel(y_ptr, dy_ptr, dx_ptr, rows, cols, dtype, stream,
                                             kernel_id)


def layernorm_fwd(in_ptr: int, out_ptr: int, rows: int, cols: int, dtype: int, eps: float,
                  weight_ptr: int, bias_ptr: int, mean_ptr: int, rstd_ptr: int,
                  stream: int) -> int:
    return load_library().layernorm_fwd(in_ptr, out_ptr, rows, cols, dtype, eps, weight_ptr or None,
                                        bias_ptr or None, mean_ptr or None, rstd_ptr or None,
                                        stream)


def layernorm_fwd_kernel(in_ptr: int, out_ptr: int, rows: int, cols: int, dtype: int, eps: float,
                         weight_ptr: int, bias_ptr: int, mean_ptr: int, rstd_ptr: int,
                         stream: int, kernel_id: int) -> int:
    return load_library().layernorm_fwd_kernel(in_ptr, out_ptr, rows, cols, dtype, eps,
                                               weight_ptr or None, bias_ptr or None,
                                               mean_ptr or None, rstd_ptr or None, stream,
                                               kernel_id)


def rmsnorm_fwd(in_ptr: int, out_ptr: int, rows: int, cols: int, dtype: int, eps: float,
                weight_ptr: int, rstd_ptr: int, stream: int) -> int:
    return load_library().rmsnorm_fwd(in_ptr, out_ptr, rows, cols, dtype, eps, weight_ptr or None,
                                      rstd_ptr or None, stream)


def rmsnorm_fwd_kernel(in_ptr: int, out_ptr: int, rows: int, cols: int, dtype: int, eps: float,
                       weight_ptr: int, rstd_ptr: int, stream: int, kernel_id: int) -> int:
    return load_library().rmsnorm_fwd_kernel(in_ptr, out_ptr, rows, cols, dtype, eps,
                                             weight_ptr or None, rstd_ptr or None, stream,
                                             kernel_id)


def softmax_select_kernel(rows: int, cols: int, dtype: int, in_ptr: int = 0,
                          out_ptr: int = 0) -> int:
    return load_library().softmax_select_kernel(rows, cols, dtype, in_ptr, out_ptr)


def softmax_describe_launch(rows: int, cols: int, dtype: int, in_ptr: int = 0, out_ptr: int = 0,
                            kernel_id: int = 0, masked: bool = False) -> str:
    buf = ctypes.create_string_buffer(256)
    lib = load_library()
    fn = lib.softmax_describe_launch_masked if masked else lib.softmax_describe_launch
    st = fn(rows, cols, dtype, in_ptr, out_ptr, kernel_id, buf, len(buf))
    if st != RWS_OK:
        raise SoftmaxError(st, softmax_last_error())
    return buf.value.decode()


def softmax_describe_launch_masked(rows: int, cols: int, dtype: int, in_ptr: int = 0,
                                   out_ptr: int = 0, kernel_id: int = 0) -> str:
    return softmax_describe_launch(rows, cols, dtype, in_ptr, out_ptr, kernel_id, masked=True)


def softmax_bwd_describe_launch(rows: int, cols: int, dtype: int, y_ptr: int = 0, dx_ptr: int = 0,
                                kernel_id: int = 0) -> str:
    """The launch softmax_backward would make (kernel_id: KERNEL_IDS)."""
    buf = ctypes.create_string_buffer(256)
    st = load_library().softmax_bwd_describe_launch(rows, cols, dtype, y_ptr, dx_ptr, kernel_id,
                                                    buf, len(buf))
    if st != RWS_OK:
        raise SoftmaxError(st, softmax_last_error())
    return buf.value.decode()


def norm_describe_launch(rows: int, cols: int, dtype: int, in_ptr: int = 0, out_ptr: int = 0,
                         kernel_id: int = 0, affine: bool = False) -> str:
    """The launch layer_norm / rms_norm would make (kernel_id: KERNEL_IDS;
    affine: a weight and/or bias is passed)."""
    buf = ctypes.create_string_buffer(256)
    st = load_library().norm_describe_launch(rows, cols, dtype, in_ptr, out_ptr, int(affine),
                                             kernel_id, buf, len(buf))
    if st != RWS_OK:
        raise SoftmaxError(st, softmax_last_error())
    return buf.value.decode()


def softmax_kernel_name(kernel_id: int) -> str:
    return load_library().softmax_kernel_name(kernel_id).decode()


def softmax_status_string(status: int) -> str:
    return load_library().softmax_status_string(status).decode()


def softmax_last_error() -> str:
    return load_library().softmax_last_error().decode()


def softmax_copy_bytes(in_ptr: int, out_ptr: int, nbytes: int, stream: int) -> int:
    return load_library().softmax_copy_bytes(in_ptr, out_ptr, nbytes, stream)


def softmax_fwd_variant(in_ptr: int, out_ptr: int, rows: int, cols: int, dtype: int, stream: int,
                        kernel_id: int, variant: int) -> int:
    return load_library().softmax_fwd_variant(in_ptr, out_ptr, rows, cols, dtype, stream,
                                              kernel_id, variant)


def softmax_variant_count(kernel_id: int) -> int:
    return load_library().softmax_variant_count(kernel_id)


def softmax_describe_variant(rows: int, cols: int, dtype: int, in_ptr: int = 0, out_ptr: int = 0,
                             kernel_id: int = 1, variant: int = 0) -> str:
    buf = ctypes.create_string_buffer(256)
    st = load_library().softmax_describe_variant(rows, cols, dtype, in_ptr, out_ptr, kernel_id,
                                                 variant, buf, len(buf))
    if st != RWS_OK:
        raise SoftmaxError(st, softmax_last_error())
    return buf.value.decode()


def softmax_read_bytes(in_ptr: int, nbytes: int, stream: int) -> int:
    return load_library().softmax_read_bytes(in_ptr, nbytes, stream)


def softmax_write_bytes(out_ptr: int, nbytes: int, stream: int) -> int:
    return load_library().softmax_write_bytes(out_ptr, nbytes, stream)


def softmax_stream_status(stream: int) -> int:
    return load_library().softmax_stream_status(stream)


def softmax_set_wait_limit(tries: int) -> int:
    return load_library().softmax_set_wait_limit(tries)


# --- tensor convenience -----------------------------------------------------

def dtype_code(dtype: torch.dtype) -> int:
    try:
        return _DTYPES[dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {dtype}; expected float32, float16 or bfloat16")


def _stream_handle(device: torch.device, stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def softmax(x: torch.Tensor, out: torch.Tensor | None = None, kernel: str = "auto",
            stream=None) -> torch.Tensor:
    """Softmax of ``x`` along its last dimension (any contiguous GPU tensor).

    ``out`` (same shape and dtype, contiguous) may be ``x`` itself (in place).
    ``kernel`` forces a family (``"wave_row"``, ``"block_onepass"``,
    ``"two_pass"``, ``"splitk"``, ``"splitk_fused"``, ``"splitk_ordered"``) instead of the
    dispatcher's choice.
    Work is enqueued on ``stream`` (default: the current stream of x's
    device); the call runs with x's device current, as the C ABI requires.
    """
    if not x.is_cuda:
        raise ValueError("x must be a GPU tensor")
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    code = dtype_code(x.dtype)
    if out is None:
        out = torch.empty_like(x)
    if out.shape != x.shape or out.dtype != x.dtype or not out.is_contiguous() or \
            out.device != x.device:
        raise ValueError("out must be a contiguous tensor of x's shape, dtype and device")
    cols = x.shape[-1] if x.dim() > 0 else 1
    rows = x.numel() // cols if cols > 0 else 0
    with torch.cuda.device(x.device):
        st = load_library().softmax_fwd_kernel(x.data_ptr(), out.data_ptr(), rows, cols, code,
                                               _stream_handle(x.device, stream),
                                               KERNEL_IDS[kernel])
    if st != RWS_OK:
        raise SoftmaxError(st, softmax_last_error())
    return out


def softmax_masked(x: torch.Tensor, scale: float = 1.0, mask: torch.Tensor | None = None,
                   causal_q: int = 0, out: torch.Tensor | None = None, kernel: str = "auto",
                   stream=None) -> torch.Tensor:
    """softmax(scale * x + mask (+ causal limit)) along the last dimension.

    ``mask`` (optional) has x's dtype and last dimension; its rows are
    broadcast cyclically over x's rows (row r uses mask row r % mask_rows), so
    a [S, S] mask serves [B, H, S, S] scores.  ``causal_q`` > 0 excludes keys
    j > (r % causal_q) + cols - causal_q.
    """
    if not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous GPU tensor")
    code = dtype_code(x.dtype)
    if out is None:
        out = torch.empty_like(x)
    if out.shape != x.shape or out.dtype != x.dtype or not out.is_contiguous() or \
            out.device != x.device:
        raise ValueError("out must be a contiguous tensor of x's shape, dtype and device")
    cols = x.shape[-1] if x.dim() > 0 else 1
    rows = x.numel() // cols if cols > 0 else 0
    mask_ptr, mask_rows = None, 0
    if mask is not None:
        if mask.dtype != x.dtype or not mask.is_contiguous() or mask.shape[-1] != cols or \
                mask.device != x.device:
            raise ValueError("mask must be contiguous, on x's device, with x's dtype and columns")
        mask_ptr, mask_rows = mask.data_ptr(), mask.numel() // cols
    with torch.cuda.device(x.device):
        st = load_library().softmax_fwd_masked(x.data_ptr(), out.data_ptr(), rows, cols, code,
                                               float(scale), mask_ptr, mask_rows, int(causal_q),
                                               _stream_handle(x.device, stream),
                                               KERNEL_IDS[kernel])
    if st != RWS_OK:
        raise SoftmaxError(st, softmax_last_error())
    return out


def softmax_backward(y: torch.Tensor, dy: torch.Tensor, out: torch.Tensor | None = None,
                     kernel: str = "auto", stream=None) -> torch.Tensor:
    """Gradient with respect to the softmax input, from its output ``y`` and
    the upstream gradient ``dy`` (both contiguous, same shape and dtype)."""
    for t, name in ((y, "y"), (dy, "dy")):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    if dy.shape != y.shape or dy.dtype != y.dtype:
        raise ValueError("y and dy must have the same shape and dtype")
    code = dtype_code(y.dtype)
    if out is None:
        out = torch.empty_like(y)
    if out.shape != y.shape or out.dtype != y.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor of y's shape and dtype")
    cols = y.shape[-1] if y.dim() > 0 else 1
    rows = y.numel() // cols if cols > 0 else 0
    if dy.device != y.device or out.device != y.device:
        raise ValueError("y, dy and out must be on the same device")
    with torch.cuda.device(y.device):
        st = load_library().softmax_bwd_kernel(y.data_ptr(), dy.data_ptr(), out.data_ptr(), rows,
                                               cols, code, _stream_handle(y.device, stream),
                                               KERNEL_IDS[kernel])
    if st != RWS_OK:
        raise SoftmaxError(st, softmax_last_error())
    return out


def _norm_operands(x, out, weight, bias):
    if not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous GPU tensor")
    code = dtype_code(x.dtype)
    if out is None:
        out = torch.empty_like(x)
    if out.shape != x.shape or out.dtype != x.dtype or not out.is_contiguous() or \
            out.device != x.device:
        raise ValueError("out must be a contiguous tensor of x's shape, dtype and device")
    cols = x.shape[-1] if x.dim() > 0 else 1
    rows = x.numel() // cols if cols > 0 else 0
    ptrs = []
    for t, name in ((weight, "weight"), (bias, "bias")):
        if t is None:
            ptrs.append(None)
            continue
        if t.dtype != x.dtype or not t.is_contiguous() or t.numel() != cols or \
                t.device != x.device:
            raise ValueError(f"{name} must be a contiguous vector of x's dtype with one entry "
                             "per column, on x's device")
        ptrs.append(t.data_ptr())
    return code, out, rows, cols, ptrs[0], ptrs[1]


def _stats_out(t, rows, device, name):
    if t is None:
        return None
    if t.dtype != torch.float32 or not t.is_contiguous() or t.numel() != rows or \
            t.device != device:
        raise ValueError(f"{name} must be a contiguous float32 tensor with one entry per row")
    return t.data_ptr()


def layer_norm(x: torch.Tensor, eps: float = 1e-5, weight: torch.Tensor | None = None,
               bias: torch.Tensor | None = None, out: torch.Tensor | None = None,
               mean: torch.Tensor | None = None, rstd: torch.Tensor | None = None,
               kernel: str = "auto", stream=None) -> torch.Tensor:
    """LayerNorm of ``x`` along its last dimension: (x - mean) / sqrt(var + eps)
    * weight + bias with the biased variance.  ``weight``/``bias`` (optional)
    have x's dtype and one entry per column; ``mean``/``rstd`` (optional,
    float32, one entry per row) receive the row statistics."""
    code, out, rows, cols, wp, bp = _norm_operands(x, out, weight, bias)
    mp = _stats_out(mean, rows, x.device, "mean")
    rp = _stats_out(rstd, rows, x.device, "rstd")
    with torch.cuda.device(x.device):
        st = load_library().layernorm_fwd_kernel(x.data_ptr(), out.data_ptr(), rows, cols, code,
                                                 float(eps), wp, bp, mp, rp,
                                                 _stream_handle(x.device, stream),
                                                 KERNEL_IDS[kernel])
    if st != RWS_OK:
        raise SoftmaxError(st, softmax_last_error())
    return out


def rms_norm(x: torch.Tensor, eps: float = 1e-5, weight: torch.Tensor | None = None,
             out: torch.Tensor | None = None, rstd: torch.Tensor | None = None,
             kernel: str = "auto", stream=None) -> torch.Tensor:
    """RMSNorm of ``x`` along its last dimension: x / sqrt(mean(x^2) + eps) * weight."""
    code, out, rows, cols, wp, _ = _norm_operands(x, out, weight, None)
    rp = _stats_out(rstd, rows, x.device, "rstd")
    with torch.cuda.device(x.device):
        st = load_library().rmsnorm_fwd_kernel(x.data_ptr(), out.data_ptr(), rows, cols, code,
                                               float(eps), wp, rp,
                                               _stream_handle(x.device, stream),
                                               KERNEL_IDS[kernel])
    if st != RWS_OK:
        raise SoftmaxError(st, softmax_last_error())
    return out


def copy_bytes(src: torch.Tensor, dst: torch.Tensor, stream=None) -> torch.Tensor:
    """16-byte-vector device copy of src's bytes into dst (bandwidth reference)."""
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nbytes:
        raise ValueError("dst is smaller than src")
    with torch.cuda.device(src.device):
        st = load_library().softmax_copy_bytes(src.data_ptr(), dst.data_ptr(), nbytes,
                                               _stream_handle(src.device, stream))
    if st != RWS_OK:
        raise SoftmaxError(st, softmax_last_error())
    return dst


def stream_status(device=None, stream=None) -> None:
    """Raise SoftmaxError if a single-launch split-k call on ``stream``
    (default: the current stream of ``device``) gave up waiting since the
    last check (its outputs are NaN); synchronises that stream."""
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None \
        else torch.device(device)
    with torch.cuda.device(dev):
        st = load_library().softmax_stream_status(_stream_handle(dev, stream))
    if st != RWS_OK:
        raise SoftmaxError(st, softmax_last_error())
