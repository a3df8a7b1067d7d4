"""fp64 CPU oracle for the fused LoRA linear layer and the pristine merge.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` import this package.  It shares no code
with the GPU library and never imports it.

What it computes (page titles as published):

* "fastaf: Minimal LoRA fine-tuning with hand-written Triton kernels",
  section "FWD kernel speedup": ``Y = X W^T + ((X A^T) B^T) * scale`` with
  ``scale = alpha / r``; the fused kernel changes where the intermediate lives,
  not the mathematics, so the oracle is this definition in fp64.
* unsloth commit log for ``scripts/benchmarks/qwen3_flex_inference.py``, entry
  replacing the copy+merge_adapter pair: ``W_inf = pristine + scaling * (B A)``
  with fp32 accumulation, the pristine copy left untouched.  The oracle gives
  the exact value in fp64 and its bf16 rounding (nearest, ties to even).
* the same fastaf page, section "BWD kernel speedup": the backward of the
  layer with W frozen, ``dX = dY W + scale (dY B) A``,
  ``dA = scale (dY B)^T X``, ``dB = scale dY^T (X A^T)``, in fp64.

Arrays: fp32 data as ``numpy.float32``; bf16 data as ``numpy.uint16`` bit
patterns.  All pins live in ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

from . import build as _build

_F32, _BF16 = 0, 1
_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_build.LIB):
        _build.build()
    lib = ctypes.CDLL(_build.LIB)
    i64, vp, f, dp = ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_void_p
    lib.oracle_fwd_rows.argtypes = [ctypes.c_int, i64, i64, i64, i64, i64, vp, vp, vp, vp, f, dp]
    lib.oracle_fwd_rows.restype = ctypes.c_int
    lib.oracle_fwd_entries.argtypes = [ctypes.c_int, i64, i64, i64, vp, vp, vp, vp, f, i64,
                                       vp, vp, dp]
    lib.oracle_fwd_entries.restype = ctypes.c_int
    lib.oracle_merge_rows.argtypes = [ctypes.c_int, i64, i64, i64, i64, vp, vp, vp, f, vp, vp]
    lib.oracle_merge_rows.restype = ctypes.c_int
    lib.oracle_bwd.argtypes = [ctypes.c_int, i64, i64, i64, i64, vp, vp, vp, vp, vp, f, i64, i64,
                               dp, dp, dp]
    lib.oracle_bwd.restype = ctypes.c_int
    lib.oracle_round_bf16.argtypes = [ctypes.c_double]
    lib.oracle_round_bf16.restype = ctypes.c_uint16
    lib.oracle_round_bf16_n.argtypes = [vp, vp, i64]
    lib.oracle_round_bf16_n.restype = None
    lib.oracle_set_threads.argtypes = [ctypes.c_int]
    lib.oracle_get_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _dt(*arrs: np.ndarray) -> int:
    kinds = {a.dtype for a in arrs}
    if kinds == {np.dtype(np.float32)}:
        return _F32
    if kinds == {np.dtype(np.uint16)}:
        return _BF16
    raise TypeError(f"oracle inputs must all be float32 or all bf16 bits (uint16), got {kinds}")


def _c(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a)


def set_threads(n: int) -> None:
    """Threads the oracle uses (0 = OpenMP default)."""
    _load().oracle_set_threads(int(n))


def get_threads() -> int:
    return int(_load().oracle_get_threads())


def fwd(X: np.ndarray, W: np.ndarray, A: np.ndarray, B: np.ndarray, scale: float,
        rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Exact-input fp64 forward ``X W^T + scale * (X A^T) B^T``.

    ``rows=(m0, m1)`` restricts the result to output rows [m0, m1).
    Returns float64 of shape [m1 - m0, N].
    """
    lib = _load()
    X, W, A, B = _c(X), _c(W), _c(A), _c(B)
    dt = _dt(X, W, A, B)
    M, K = X.shape
    N, K2 = W.shape
    r = A.shape[0]
    if K2 != K or A.shape[1] != K or B.shape != (N, r):
        raise ValueError(f"shape mismatch X{X.shape} W{W.shape} A{A.shape} B{B.shape}")
    m0, m1 = (0, M) if rows is None else (int(rows[0]), int(rows[1]))
    if not (0 <= m0 <= m1 <= M):
        raise ValueError("row range out of bounds")
    Y = np.zeros((m1 - m0, N), dtype=np.float64)
    rc = lib.oracle_fwd_rows(dt, m0, m1, N, K, r, X.ctypes.data, W.ctypes.data, A.ctypes.data,
                             B.ctypes.data, float(np.float32(scale)), Y.ctypes.data)
    if rc != 0:
        raise MemoryError("oracle_fwd_rows could not allocate its work buffers")
    return Y


def fwd_entries(X: np.ndarray, W: np.ndarray, A: np.ndarray, B: np.ndarray, scale: float,
                ms: np.ndarray, ns: np.ndarray) -> np.ndarray:
    """fp64 forward at positions (ms[i], ns[i]); returns float64 [len(ms)]."""
    lib = _load()
    X, W, A, B = _c(X), _c(W), _c(A), _c(B)
    dt = _dt(X, W, A, B)
    M, K = X.shape
    N = W.shape[0]
    r = A.shape[0]
    ms = np.ascontiguousarray(ms, dtype=np.int64)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    if ms.shape != ns.shape or ms.ndim != 1:
        raise ValueError("ms and ns must be 1-D of equal length")
    if ms.size and (ms.min() < 0 or ms.max() >= M or ns.min() < 0 or ns.max() >= N):
        raise ValueError("entry index out of bounds")
    Y = np.zeros(ms.shape, dtype=np.float64)
    lib.oracle_fwd_entries(dt, N, K, r, X.ctypes.data, W.ctypes.data, A.ctypes.data,
                           B.ctypes.data, float(np.float32(scale)), ms.size, ms.ctypes.data,
                           ns.ctypes.data, Y.ctypes.data)
    return Y


def merge(W0: np.ndarray, B: np.ndarray, A: np.ndarray, scale: float,
          rows: Optional[Sequence[int]] = None, want_double: bool = True,
          want_bf16: bool = True):
    """Merge from pristine ``W0 + scale * B A`` in fp64.

    Returns ``(Wd, Wb)``: the exact float64 values and their bf16 rounding
    (uint16 bits), either of them None when not asked for.
    """
    lib = _load()
    W0, B, A = _c(W0), _c(B), _c(A)
    dt = _dt(W0, B, A)
    N, K = W0.shape
    r = A.shape[0]
    if A.shape[1] != K or B.shape != (N, r):
        raise ValueError(f"shape mismatch W0{W0.shape} B{B.shape} A{A.shape}")
    n0, n1 = (0, N) if rows is None else (int(rows[0]), int(rows[1]))
    if not (0 <= n0 <= n1 <= N):
        raise ValueError("row range out of bounds")
    Wd = np.zeros((n1 - n0, K), dtype=np.float64) if want_double else None
    Wb = np.zeros((n1 - n0, K), dtype=np.uint16) if want_bf16 else None
    rc = lib.oracle_merge_rows(dt, n0, n1, K, r, W0.ctypes.data, B.ctypes.data, A.ctypes.data,
                               float(np.float32(scale)),
                               None if Wd is None else Wd.ctypes.data,
                               None if Wb is None else Wb.ctypes.data)
    if rc != 0:
        raise MemoryError("oracle_merge_rows could not allocate its work buffer")
    return Wd, Wb


def bwd(X: np.ndarray, W: np.ndarray, A: np.ndarray, B: np.ndarray, dY: np.ndarray,
        scale: float, dx_rows: Optional[Sequence[int]] = None):
    """Backward of the layer with W frozen, in fp64:
    ``dX = dY W + scale (dY B) A``, ``dA = scale (dY B)^T X``,
    ``dB = scale dY^T (X A^T)``.

    Returns ``(dX, dA, dB)``; dX holds rows ``dx_rows = (m0, m1)`` only (all
    rows when None; ``(0, 0)`` skips it).
    """
    lib = _load()
    X, W, A, B, dY = _c(X), _c(W), _c(A), _c(B), _c(dY)
    dt = _dt(X, W, A, B, dY)
    M, K = X.shape
    N = W.shape[0]
    r = A.shape[0]
    if W.shape != (N, K) or A.shape != (r, K) or B.shape != (N, r) or dY.shape != (M, N):
        raise ValueError(f"shape mismatch X{X.shape} W{W.shape} A{A.shape} B{B.shape} dY{dY.shape}")
    m0, m1 = (0, M) if dx_rows is None else (int(dx_rows[0]), int(dx_rows[1]))
    if not (0 <= m0 <= m1 <= M):
        raise ValueError("row range out of bounds")
    dX = np.zeros((m1 - m0, K), dtype=np.float64)
    dA = np.zeros((r, K), dtype=np.float64)
    dB = np.zeros((N, r), dtype=np.float64)
    rc = lib.oracle_bwd(dt, M, N, K, r, X.ctypes.data, W.ctypes.data, A.ctypes.data,
                        B.ctypes.data, dY.ctypes.data, float(np.float32(scale)), m0, m1,
                        dX.ctypes.data if m1 > m0 else None, dA.ctypes.data, dB.ctypes.data)
    if rc != 0:
        raise MemoryError("oracle_bwd could not allocate its work buffers")
    return dX, dA, dB


def round_bf16(x) -> np.ndarray:
    """Correctly rounded (nearest, ties to even) fp64 -> bf16, as uint16 bits."""
    lib = _load()
    flat = np.ascontiguousarray(np.asarray(x, dtype=np.float64).ravel())
    out = np.empty(flat.size, dtype=np.uint16)
    lib.oracle_round_bf16_n(flat.ctypes.data, out.ctypes.data, flat.size)
    return out.reshape(np.shape(x))


def round_bf16_scalar(x: float) -> int:
    """oracle_round_bf16 on one value (the array form calls it per element)."""
    return int(_load().oracle_round_bf16(float(x)))
