"""Helpers for the GPU tests: put seeded float64 inputs into device tensors of
a dtype (optionally at an element offset inside a larger buffer, so that the
base pointer is not 16-byte aligned), run the library through its C ABI and
read results back."""
from __future__ import annotations

import numpy as np
import torch

import row_wise_safe_amd as rws

TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def have_gpu() -> bool:
    return torch.cuda.is_available()


def to_device(x64: np.ndarray, dtype: str, offset: int = 0, device="cuda"):
    """Round to `dtype` on the host, copy to the GPU at `offset` elements into a
    fresh buffer.  Returns (device view [rows, cols], stored values as float64)."""
    t = torch.from_numpy(np.ascontiguousarray(x64)).to(TORCH_DTYPE[dtype])
    stored = t.to(torch.float64).numpy()
    buf = torch.empty(t.numel() + offset, dtype=t.dtype, device=device)
    view = buf[offset:offset + t.numel()].view(t.shape)
    view.copy_(t.to(device))
    return view, stored


def empty_like_at(x: torch.Tensor, offset: int = 0):
    buf = torch.empty(x.numel() + offset, dtype=x.dtype, device=x.device)
    return buf[offset:offset + x.numel()].view(x.shape)


class NotCoResident(Exception):
    """The fused split-k cannot hold one row's workgroups on the device at once."""


def run(x: torch.Tensor, out: torch.Tensor, kernel: str = "auto") -> np.ndarray:
    try:
        rws.softmax(x, out=out, kernel=kernel)
    except rws.SoftmaxError as e:
        if kernel == "splitk_fused" and e.status == rws.RWS_ERR_UNSUPPORTED_SHAPE:
            raise NotCoResident(str(e))
        raise
    torch.cuda.synchronize()
    return out.to(torch.float64).cpu().numpy()


def window_granules(cols: int, dtype: str, aligned: bool) -> int:
    """Granules of a row window that starts on a 128-byte line (upper bound)."""
    es = 4 if dtype == "f32" else 2
    b = cols * es
    return b // 16 if aligned else (b + 143) // 16


def tile_supports(cols: int, dtype: str) -> bool:
    """tile_rows takes the row (16-byte aligned tensors): at least one
    granule, and a tile of max(4, phase period) rows within 4096 bytes."""
    es = 4 if dtype == "f32" else 2
    g = 16
    while (cols * es) % g:
        g //= 2
    return cols >= 16 // es and max(4, 16 // g) * cols * es <= 4096


def supports(kernel: str, cols: int, dtype: str, aligned: bool) -> bool:
    es = 4 if dtype == "f32" else 2
    line = aligned and (cols * es) % 128 == 0
    w = window_granules(cols, dtype, line)
    if kernel == "wave_row":
        return w <= 512
    if kernel == "block_onepass":
        # rows that are not line-aligned: no LDS parking
        return w <= (16384 if line else 8192)
    return True


class FreshStream:
    """A HIP stream that no earlier call used (torch's own streams come from a
    pool that earlier tests used, so the library may already hold a workspace
    for them), made with the HIP runtime the library is linked against.  The
    library keys its workspaces by stream handle, and a destroyed stream's
    handle can come back from the next create, so these streams are kept
    until the process ends.  Use as `with FreshStream() as s:` (s is a torch
    ExternalStream); the exit synchronises the device."""

    def __enter__(self):
        import ctypes
        handle = ctypes.c_void_p()
        assert rws.load_library().hipStreamCreate(ctypes.byref(handle)) == 0
        return torch.cuda.ExternalStream(handle.value)

    def __exit__(self, *exc):
        torch.cuda.synchronize()
        return False
