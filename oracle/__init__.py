"""CPU oracle for row-wise safe softmax -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline
leg may import this package.  The product path (the HIP library and its Python
binding) never imports it; the two share no code.

Thin ctypes wrappers over ``softmax_oracle.c`` (plain C, IEEE double, libm
``exp``).  Each routine follows one passage of the pages:

* :func:`safe_softmax`  -- the definition y_i = e^(x_i - max x) / sum_j
  e^(x_j - max x) (HIP softmax tutorial, section 1; numpy ``safe_softmax`` on
  the CUDA safe-online-softmax page, section 1).
* :func:`row_stats`     -- the row's (max, sum of exp(x - max)).
* :func:`online_softmax` -- the blockwise running (m, d) of the CUDA
  safe-online-softmax page, section 1 (``safe_online_softmax``, block 256).
* :func:`online_stats_elementwise` -- the element-wise online update of the
  DCU case-study page, section 4.3.
* :func:`splitk_softmax` -- per-chunk partial (m, d) merged with the (m, d)
  rule, CUDA safe-online-softmax page, section 3.2.
* :func:`md_merge`      -- the (m, d) merge rule itself.
* :func:`masked_softmax` -- softmax of scale*x + mask (+ causal limit), the
  attention-score fusion the DCU case-study page proposes (section 9).
* :func:`softmax_backward` -- dx = y * (dy - sum(dy * y)) per row, the
  backward pass the same page (section 5.4) says needs its own check.
* :func:`layernorm`, :func:`rmsnorm` -- the row normalisations the same page
  (section 9) names as having softmax's structure, and the Pangu-Weather
  profile page (section 3) runs as a wave-per-row kernel (``norm_oracle.c``).

Inputs are float64 arrays holding the values as stored in the tensor's dtype.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_lib = None

_D = ctypes.POINTER(ctypes.c_double)
_I64 = ctypes.c_int64


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_build.LIBRARY) or any(
            os.path.getmtime(src) > os.path.getmtime(_build.LIBRARY) for src in _build.SOURCES):
        _build.build()
    lib = ctypes.CDLL(_build.LIBRARY)
    lib.oracle_safe_softmax.argtypes = [_D, _D, _I64, _I64]
    lib.oracle_safe_softmax.restype = None
    lib.oracle_row_stats.argtypes = [_D, _D, _D, _I64, _I64]
    lib.oracle_row_stats.restype = None
    lib.oracle_online_softmax.argtypes = [_D, _D, _I64, _I64, _I64]
    lib.oracle_online_softmax.restype = None
    lib.oracle_online_stats_elementwise.argtypes = [_D, _D, _D, _I64, _I64]
    lib.oracle_online_stats_elementwise.restype = None
    lib.oracle_splitk_softmax.argtypes = [_D, _D, _I64, _I64, _I64]
    lib.oracle_splitk_softmax.restype = None
    lib.oracle_md_merge.argtypes = [ctypes.c_double] * 4 + [_D, _D]
    lib.oracle_md_merge.restype = None
    lib.oracle_masked_softmax.argtypes = [_D, _D, _I64, _I64, ctypes.c_double, _D, _I64, _I64]
    lib.oracle_masked_softmax.restype = None
    lib.oracle_softmax_backward.argtypes = [_D, _D, _D, _I64, _I64]
    lib.oracle_softmax_backward.restype = None
    lib.oracle_layernorm.argtypes = [_D, _D, _I64, _I64, ctypes.c_double, _D, _D, _D, _D]
    lib.oracle_layernorm.restype = None
    lib.oracle_rmsnorm.argtypes = [_D, _D, _I64, _I64, ctypes.c_double, _D, _D]
    lib.oracle_rmsnorm.restype = None
    lib.oracle_safe_softmax_threads.argtypes = [_D, _D, _I64, _I64, ctypes.c_int]
    lib.oracle_safe_softmax_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _as_2d(x) -> np.ndarray:
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    if a.ndim == 1:
        a = a.reshape(1, -1)
    if a.ndim != 2:
        a = a.reshape(-1, a.shape[-1])
    return a


def _p(a: np.ndarray):
    return a.ctypes.data_as(_D)


def safe_softmax(x) -> np.ndarray:
    """Safe softmax along the last axis by its definition, in float64."""
    a = _as_2d(x)
    y = np.empty_like(a)
    _load().oracle_safe_softmax(_p(a), _p(y), a.shape[0], a.shape[1])
    return y.reshape(np.shape(x)) if np.ndim(x) >= 1 else y


def safe_softmax_threads(x, nthreads: int):
    """The definition over row ranges on ``nthreads`` host threads.

    Returns ``(y, threads_used)``.
    """
    a = _as_2d(x)
    y = np.empty_like(a)
    used = _load().oracle_safe_softmax_threads(_p(a), _p(y), a.shape[0], a.shape[1],
                                               int(nthreads))
    return y, int(used)


def row_stats(x):
    """Per-row (m, d): m = max x, d = sum exp(x - m)."""
    a = _as_2d(x)
    m = np.empty(a.shape[0])
    d = np.empty(a.shape[0])
    _load().oracle_row_stats(_p(a), _p(m), _p(d), a.shape[0], a.shape[1])
    return m, d


def online_softmax(x, block: int = 256) -> np.ndarray:
    """Blockwise online (m, d) then e^(x - m)/d; chunks of ``block`` columns."""
    a = _as_2d(x)
    y = np.empty_like(a)
    _load().oracle_online_softmax(_p(a), _p(y), a.shape[0], a.shape[1], int(block))
    return y


def online_stats_elementwise(x):
    """Per-row (m, d) by the one-element-at-a-time online update."""
    a = _as_2d(x)
    m = np.empty(a.shape[0])
    d = np.empty(a.shape[0])
    _load().oracle_online_stats_elementwise(_p(a), _p(m), _p(d), a.shape[0], a.shape[1])
    return m, d


def splitk_softmax(x, chunk: int) -> np.ndarray:
    """Split-k: per-chunk (m, d), merged in chunk order, then e^(x - M)/D."""
    a = _as_2d(x)
    y = np.empty_like(a)
    _load().oracle_splitk_softmax(_p(a), _p(y), a.shape[0], a.shape[1], int(chunk))
    return y


def md_merge(a, b):
    """(m_a, d_a) (+) (m_b, d_b) with the guarded (-inf, 0) identity."""
    m = ctypes.c_double()
    d = ctypes.c_double()
    _load().oracle_md_merge(float(a[0]), float(a[1]), float(b[0]), float(b[1]),
                            ctypes.byref(m), ctypes.byref(d))
    return m.value, d.value


def masked_softmax(x, scale: float = 1.0, mask=None, causal_q: int = 0) -> np.ndarray:
    """Softmax of scale*x + mask[r % mask_rows] with an optional causal limit:
    column j of row r is excluded when j > (r % causal_q) + cols - causal_q."""
    a = _as_2d(x)
    y = np.empty_like(a)
    if mask is None:
        mp, mrows = None, 1
    else:
        m = _as_2d(mask)
        if m.shape[1] != a.shape[1]:
            raise ValueError("mask must have the same number of columns")
        mp, mrows = _p(m), m.shape[0]
    _load().oracle_masked_softmax(_p(a), _p(y), a.shape[0], a.shape[1], float(scale), mp,
                                  mrows, int(causal_q))
    return y


def softmax_backward(y, dy) -> np.ndarray:
    """Gradient with respect to the softmax input: y * (dy - sum_j dy_j y_j)."""
    a = _as_2d(y)
    g = _as_2d(dy)
    if a.shape != g.shape:
        raise ValueError("y and dy must have the same shape")
    dx = np.empty_like(a)
    _load().oracle_softmax_backward(_p(a), _p(g), _p(dx), a.shape[0], a.shape[1])
    return dx


def _vec(v, cols):
    if v is None:
        return None, None
    a = np.ascontiguousarray(np.asarray(v, dtype=np.float64)).reshape(-1)
    if a.shape[0] != cols:
        raise ValueError("weight/bias must have one entry per column")
    return a, _p(a)


def layernorm(x, eps: float = 1e-5, weight=None, bias=None, return_stats: bool = False):
    """LayerNorm along the last axis: (x - mean) / sqrt(var + eps) * w + b with
    the biased variance.  With ``return_stats`` also returns per-row
    ``(mean, rstd)``."""
    a = _as_2d(x)
    y = np.empty_like(a)
    w, wp = _vec(weight, a.shape[1])
    b, bp = _vec(bias, a.shape[1])
    mean = np.empty(a.shape[0])
    rstd = np.empty(a.shape[0])
    _load().oracle_layernorm(_p(a), _p(y), a.shape[0], a.shape[1], float(eps), wp, bp,
                             _p(mean), _p(rstd))
    return (y, mean, rstd) if return_stats else y


def rmsnorm(x, eps: float = 1e-5, weight=None, return_stats: bool = False):
    """RMSNorm along the last axis: x / sqrt(mean(x^2) + eps) * w.  With
    ``return_stats`` also returns per-row ``rstd``."""
    a = _as_2d(x)
    y = np.empty_like(a)
    w, wp = _vec(weight, a.shape[1])
    rstd = np.empty(a.shape[0])
    _load().oracle_rmsnorm(_p(a), _p(y), a.shape[0], a.shape[1], float(eps), wp, _p(rstd))
    return (y, rstd) if return_stats else y
