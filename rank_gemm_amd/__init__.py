"""rank_gemm_amd -- Python binding of liblora.so, the MI355X (gfx950) fused
LoRA linear forward and backward and the pristine merge.

The binding only marshals arguments: every step of the computation runs in
the library's HIP kernels.  There is no CPU fallback; if the library cannot be
loaded, the first call raises.

    Y = fwd(X, W, A, B, scale)          # X W^T + scale * (X A^T) B^T
    merge(W0, B, A, scale, out=W_inf)   # W_inf = W0 + scale * B A, W0 untouched
    merge_batch([(W0, B, A, scale, W_inf), ...])   # many targets, few launches
    fwd_batch([(X, W, A, B, scale, Y), ...])       # independent forwards, few launches
    merge_inplace(W, B, A, scale)       # W += scale * B A in place (not bit-reversible)
    dX, dA, dB = bwd(X, W, A, B, dY, scale)   # gradients with W frozen (bf16)
    Y = fwd(X, W, A, B, scale, tile=4)   # one tile configuration (see tune.py)
    Y = fwd_tuned(X, W, A, B, scale)     # the configuration cached for this shape

Tensors are torch tensors on the current HIP device, all bfloat16 or all
float32, 2-D with unit inner stride (rows may be padded: the leading
dimension is passed through).  Work is enqueued on torch's current stream.
The C entry points of the same names are declared in include/lora.h.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

from . import build as _build

LIB_PATH = _build.LIB

LORA_OK = 0
LORA_ERR_NULL = 1
LORA_ERR_SHAPE = 2
LORA_ERR_STRIDE = 3
LORA_ERR_ALIGN = 4
LORA_ERR_DTYPE = 5
LORA_ERR_ALIAS = 6
LORA_ERR_UNSUPPORTED = 7
LORA_ERR_HIP = 8
LORA_ERR_WORKSPACE = 9
LORA_ERR_SCRATCH = 10
NOALLOC_MAX_FORWARDS = 64
LORA_F32 = 0
LORA_BF16 = 1
VARIANTS = {"auto": 0, "tiled": 1, "decode": 2}
MAX_RANK = 256
DECODE_MAX_M = 64

TILE_COUNT = 20

EXPORTS = ("lora_fwd", "lora_fwd_variant", "lora_merge", "lora_merge_batch",
           "lora_merge_inplace", "lora_status_str", "lora_abi_version", "lora_fwd_pick",
           "lora_bwd", "lora_bwd_workspace_size", "lora_tile_get_info", "lora_tile_get_usage",
           "lora_get_device_limits", "lora_fwd_tile", "lora_fwd_batch",
           "lora_fwd_batch_workspace_size", "lora_fwd_batch_noalloc")


class MergeDesc(ctypes.Structure):
    """lora_merge_desc of include/lora.h."""
    _fields_ = [("N", ctypes.c_int64), ("K", ctypes.c_int64), ("r", ctypes.c_int64),
                ("W0", ctypes.c_void_p), ("ldw0", ctypes.c_int64),
                ("B", ctypes.c_void_p), ("ldb", ctypes.c_int64),
                ("A", ctypes.c_void_p), ("lda", ctypes.c_int64),
                ("scale", ctypes.c_float),
                ("W_inf", ctypes.c_void_p), ("ldwi", ctypes.c_int64)]



class FwdDesc(ctypes.Structure):
    """lora_fwd_desc of include/lora.h."""
    _fields_ = [("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
                ("r", ctypes.c_int64), ("X", ctypes.c_void_p), ("ldx", ctypes.c_int64),
                ("W", ctypes.c_void_p), ("ldw", ctypes.c_int64),
                ("A", ctypes.c_void_p), ("lda", ctypes.c_int64),
                ("B", ctypes.c_void_p), ("ldb", ctypes.c_int64),
                ("scale", ctypes.c_float), ("Y", ctypes.c_void_p), ("ldy", ctypes.c_int64)]


class TileInfo(ctypes.Structure):
    """lora_tile_info of include/lora.h."""
    _fields_ = [(n, ctypes.c_int32) for n in ("tile", "bm", "bn", "waves", "stages", "bk",
                                              "group", "rank_pad", "lds_bytes", "k_split")]


class TileUsage(ctypes.Structure):
    """lora_tile_usage of include/lora.h."""
    _fields_ = [(n, ctypes.c_int32) for n in ("vgprs", "scratch_bytes", "blocks_per_cu")]


class DeviceLimits(ctypes.Structure):
    """lora_device_limits of include/lora.h."""
    _fields_ = [(n, ctypes.c_int32) for n in ("compute_units", "lds_per_block", "lds_per_cu",
                                              "regs_per_block", "max_threads_per_block",
                                              "wave_size")]


_lib = None


class LoraError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded liblora.so (built in place first if it is not there)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        _build.build()
    # One HIP runtime per process: torch ships its own libamdhip64 (the same
    # soname liblora.so needs).  Loaded first, it satisfies liblora.so's
    # dependency; loaded after liblora.so, the system runtime would already
    # be in the process and torch would add a second one beside it.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    L = ctypes.CDLL(LIB_PATH)
    i32, i64, vp, f32 = ctypes.c_int, ctypes.c_int64, ctypes.c_void_p, ctypes.c_float
    L.lora_fwd.argtypes = [i32, i64, i64, i64, i64, vp, i64, vp, i64, vp, i64, vp, i64, f32, vp,
                           i64, vp]
    L.lora_fwd.restype = i32
    L.lora_fwd_variant.argtypes = [i32] + L.lora_fwd.argtypes
    L.lora_fwd_variant.restype = i32
    L.lora_merge.argtypes = [i32, i64, i64, i64, vp, i64, vp, i64, vp, i64, f32, vp, i64, vp]
    L.lora_merge.restype = i32
    L.lora_merge_inplace.argtypes = [i32, i64, i64, i64, vp, i64, vp, i64, vp, i64, f32, vp]
    L.lora_merge_inplace.restype = i32
    L.lora_merge_batch.argtypes = [i32, i32, ctypes.POINTER(MergeDesc), vp]
    L.lora_merge_batch.restype = i32
    L.lora_status_str.argtypes = [i32]
    L.lora_status_str.restype = ctypes.c_char_p
    L.lora_abi_version.argtypes = []
    L.lora_abi_version.restype = i32
    L.lora_fwd_pick.argtypes = [i32, i64, i64, i64, i64]
    L.lora_fwd_pick.restype = i32
    L.lora_bwd.argtypes = [i32, i64, i64, i64, i64, vp, i64, vp, i64, vp, i64, vp, i64, vp, i64,
                           f32, vp, i64, vp, i64, vp, i64, vp, i64, vp]
    L.lora_bwd.restype = i32
    L.lora_bwd_workspace_size.argtypes = [i32, i64, i64, i64, i64]
    L.lora_bwd_workspace_size.restype = i64
    L.lora_tile_get_info.argtypes = [i32, i64, ctypes.POINTER(TileInfo)]
    L.lora_tile_get_info.restype = i32
    L.lora_tile_get_usage.argtypes = [i32, i64, ctypes.POINTER(TileUsage)]
    L.lora_tile_get_usage.restype = i32
    L.lora_get_device_limits.argtypes = [ctypes.POINTER(DeviceLimits)]
    L.lora_get_device_limits.restype = i32
    L.lora_fwd_tile.argtypes = [i32] + L.lora_fwd.argtypes
    L.lora_fwd_tile.restype = i32
    L.lora_fwd_batch.argtypes = [i32, i32, ctypes.POINTER(FwdDesc), vp, i64, vp]
    L.lora_fwd_batch.restype = i32
    L.lora_fwd_batch_workspace_size.argtypes = [i32]
    L.lora_fwd_batch_workspace_size.restype = i64
    L.lora_fwd_batch_noalloc.argtypes = [i32, i32, ctypes.POINTER(FwdDesc), vp]
    L.lora_fwd_batch_noalloc.restype = i32
    _lib = L
    return L


def status_str(status: int) -> str:
    return lib().lora_status_str(int(status)).decode()


def abi_version() -> int:
    return int(lib().lora_abi_version())


def fwd_pick(dtype: int, M: int, N: int, K: int, r: int) -> int:
    return int(lib().lora_fwd_pick(dtype, M, N, K, r))


def _check(status: int, what: str) -> None:
    if status != LORA_OK:
        raise LoraError(status, f"{what}: {status_str(status)}")


# ---------------------------------------------------------------- raw ABI

def fwd_auto_raw(dtype: int, M: int, N: int, K: int, r: int, X: int, ldx: int, W: int, ldw: int,
                 A: int, lda: int, B: int, ldb: int, scale: float, Y: int, ldy: int,
                 stream: int = 0) -> int:
    """lora_fwd (the library's own kernel choice) with integer addresses;
    returns the lora_status."""
    return int(lib().lora_fwd(dtype, M, N, K, r, X, ldx, W, ldw, A, lda, B, ldb, scale, Y, ldy,
                              stream or None))


def fwd_raw(variant: int, dtype: int, M: int, N: int, K: int, r: int, X: int, ldx: int, W: int,
            ldw: int, A: int, lda: int, B: int, ldb: int, scale: float, Y: int, ldy: int,
            stream: int = 0) -> int:
    """lora_fwd_variant with integer addresses; returns the lora_status."""
    return int(lib().lora_fwd_variant(variant, dtype, M, N, K, r, X, ldx, W, ldw, A, lda, B, ldb,
                                      scale, Y, ldy, stream or None))


def merge_raw(dtype: int, N: int, K: int, r: int, W0: int, ldw0: int, B: int, ldb: int, A: int,
              lda: int, scale: float, Wi: int, ldwi: int, stream: int = 0) -> int:
    """lora_merge with integer addresses; returns the lora_status."""
    return int(lib().lora_merge(dtype, N, K, r, W0, ldw0, B, ldb, A, lda, scale, Wi, ldwi,
                                stream or None))


def merge_inplace_raw(dtype: int, N: int, K: int, r: int, W: int, ldw: int, B: int, ldb: int,
                      A: int, lda: int, scale: float, stream: int = 0) -> int:
    """lora_merge_inplace with integer addresses; returns the lora_status."""
    return int(lib().lora_merge_inplace(dtype, N, K, r, W, ldw, B, ldb, A, lda, scale,
                                        stream or None))


def fwd_batch_raw(dtype: int, descs, stream: int = 0, ws: int = 0, ws_bytes: int = 0) -> int:
    """lora_fwd_batch over a sequence of FwdDesc (or an array of them)."""
    if not isinstance(descs, ctypes.Array):
        descs = (FwdDesc * len(descs))(*descs)
    return int(lib().lora_fwd_batch(dtype, len(descs), descs, ws or None, ws_bytes, stream or None))


def fwd_batch_noalloc_raw(dtype: int, descs, stream: int = 0) -> int:
    """lora_fwd_batch_noalloc over a sequence of FwdDesc (or an array of them)."""
    if not isinstance(descs, ctypes.Array):
        descs = (FwdDesc * len(descs))(*descs)
    return int(lib().lora_fwd_batch_noalloc(dtype, len(descs), descs, stream or None))


def fwd_batch_workspace_size(count: int) -> int:
    return int(lib().lora_fwd_batch_workspace_size(count))


def merge_batch_raw(dtype: int, descs, stream: int = 0) -> int:
    """lora_merge_batch over a sequence of MergeDesc (or an array of them)."""
    if not isinstance(descs, ctypes.Array):
        descs = (MergeDesc * len(descs))(*descs)
    return int(lib().lora_merge_batch(dtype, len(descs), descs, stream or None))


def tile_info(tile: int, r: int) -> Optional[TileInfo]:
    """Static description of tile configuration `tile` at rank r, or None when
    it is not instantiated for that rank (lora_tile_get_info; no HIP call)."""
    out = TileInfo()
    st = int(lib().lora_tile_get_info(tile, r, ctypes.byref(out)))
    if st == LORA_ERR_UNSUPPORTED:
        return None
    _check(st, "lora_tile_get_info")
    return out


def tile_usage(tile: int, r: int) -> TileUsage:
    """Registers, spill bytes and resident workgroups per CU on the current
    device (lora_tile_get_usage)."""
    out = TileUsage()
    _check(int(lib().lora_tile_get_usage(tile, r, ctypes.byref(out))), "lora_tile_get_usage")
    return out


def device_limits() -> DeviceLimits:
    out = DeviceLimits()
    _check(int(lib().lora_get_device_limits(ctypes.byref(out))), "lora_get_device_limits")
    return out


def fwd_tile_raw(tile: int, dtype: int, M: int, N: int, K: int, r: int, X: int, ldx: int, W: int,
                 ldw: int, A: int, lda: int, B: int, ldb: int, scale: float, Y: int, ldy: int,
                 stream: int = 0) -> int:
    """lora_fwd_tile with integer addresses; returns the lora_status."""
    return int(lib().lora_fwd_tile(tile, dtype, M, N, K, r, X, ldx, W, ldw, A, lda, B, ldb, scale,
                                   Y, ldy, stream or None))


def bwd_workspace_size(dtype: int, M: int, N: int, K: int, r: int) -> int:
    """lora_bwd_workspace_size: bytes, or -1 when not supported."""
    return int(lib().lora_bwd_workspace_size(dtype, M, N, K, r))


def bwd_raw(dtype: int, M: int, N: int, K: int, r: int, X: int, ldx: int, W: int, ldw: int,
            A: int, lda: int, B: int, ldb: int, dY: int, lddy: int, scale: float, dX: int,
            lddx: int, dA: int, ldda: int, dB: int, lddb: int, ws: int, ws_bytes: int,
            stream: int = 0) -> int:
    """lora_bwd with integer addresses (0 for NULL); returns the lora_status."""
    return int(lib().lora_bwd(dtype, M, N, K, r, X or None, ldx, W or None, ldw, A or None, lda,
                              B or None, ldb, dY or None, lddy, scale, dX or None, lddx,
                              dA or None, ldda, dB or None, lddb, ws or None, ws_bytes,
                              stream or None))


# ------------------------------------------------------------ torch-facing

def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return LORA_BF16
    if t.dtype == torch.float32:
        return LORA_F32
    raise TypeError(f"unsupported dtype {t.dtype}; expected bfloat16 or float32")


def _mat(t, name: str):
    """(address, leading dimension) of a row-major 2-D tensor.  Rows must
    not overlap: a row stride shorter than the row (an expand()ed or
    overlapping view) is rejected, since the kernels would read or write
    rows' worth of memory the tensor does not hold."""
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D, got shape {tuple(t.shape)}")
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must have unit inner stride")
    if t.shape[0] > 1 and t.shape[1] > 0 and t.stride(0) < t.shape[1]:
        raise ValueError(f"{name} has row stride {t.stride(0)} < row length {t.shape[1]}: "
                         f"overlapping rows are not supported")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a HIP device")
    return t.data_ptr(), max(t.stride(0), t.shape[1], 1)


def _stream(device) -> int:
    import torch
    return torch.cuda.current_stream(device).cuda_stream


def fwd(X, W, A, B, scale: float, out=None, variant: str = "auto", tile: Optional[int] = None):
    """Fused LoRA forward ``Y = X W^T + scale * (X A^T) B^T`` on the GPU.

    X[M,K], W[N,K], A[r,K], B[N,r]; returns Y[M,N] (``out`` if given).
    ``tile``: run that tiled configuration (lora_fwd_tile, bf16) instead of
    the library's choice; ``variant`` forces tiled/decode otherwise.
    """
    import torch
    M, K = X.shape
    N = W.shape[0]
    r = A.shape[0]
    if W.shape[1] != K or A.shape[1] != K or tuple(B.shape) != (N, r):
        raise ValueError(f"shape mismatch X{tuple(X.shape)} W{tuple(W.shape)} "
                         f"A{tuple(A.shape)} B{tuple(B.shape)}")
    dt = _dtype_code(X)
    for t, nm in ((W, "W"), (A, "A"), (B, "B")):
        if t.dtype != X.dtype or t.device != X.device:
            raise ValueError(f"{nm} must match X in dtype and device")
    if out is None:
        out = torch.empty((M, N), dtype=X.dtype, device=X.device)
    elif tuple(out.shape) != (M, N) or out.dtype != X.dtype or out.device != X.device:
        raise ValueError("out must be [M, N] with X's dtype and device")
    px, ldx = _mat(X, "X")
    pw, ldw = _mat(W, "W")
    pa, lda = _mat(A, "A")
    pb, ldb = _mat(B, "B")
    py, ldy = _mat(out, "out")
    if tile is not None:
        st = fwd_tile_raw(int(tile), dt, M, N, K, r, px, ldx, pw, ldw, pa, lda, pb, ldb,
                          float(scale), py, ldy, _stream(X.device))
        _check(st, "lora_fwd_tile")
        return out
    if variant == "auto":
        st = fwd_auto_raw(dt, M, N, K, r, px, ldx, pw, ldw, pa, lda, pb, ldb, float(scale), py,
                          ldy, _stream(X.device))
        _check(st, "lora_fwd")
        return out
    st = fwd_raw(VARIANTS[variant], dt, M, N, K, r, px, ldx, pw, ldw, pa, lda, pb, ldb,
                 float(scale), py, ldy, _stream(X.device))
    _check(st, "lora_fwd_variant")
    return out


def fwd_batch(items, workspace=None):
    """Several independent forwards in few launches: ``items`` is a sequence of
    ``(X, W, A, B, scale, Y)``; each ``Y`` is written as ``fwd`` would write
    it.  All tensors share one dtype and device.  ``workspace``: an optional
    uint8 device tensor of ``fwd_batch_workspace_size(len(items))`` bytes
    (T computed once per forward: fewer loads for the decode kernel; for
    16 < r <= 32 the outputs then differ from ``fwd``'s by rounding order)."""
    if not items:
        return
    dt = _dtype_code(items[0][0])
    dev = items[0][0].device
    descs = (FwdDesc * len(items))()
    for i, (X, W, A, B, scale, Y) in enumerate(items):
        M, K = X.shape
        N, r = W.shape[0], A.shape[0]
        if (W.shape[1] != K or A.shape[1] != K or tuple(B.shape) != (N, r)
                or tuple(Y.shape) != (M, N)):
            raise ValueError(f"forward {i}: shape mismatch X{tuple(X.shape)} W{tuple(W.shape)} "
                             f"A{tuple(A.shape)} B{tuple(B.shape)} Y{tuple(Y.shape)}")
        for t, nm in ((X, "X"), (W, "W"), (A, "A"), (B, "B"), (Y, "Y")):
            if _dtype_code(t) != dt or t.device != dev:
                raise ValueError(f"forward {i}: {nm} must match the first X in dtype and device")
        px, ldx = _mat(X, "X")
        pw, ldw = _mat(W, "W")
        pa, lda = _mat(A, "A")
        pb, ldb = _mat(B, "B")
        py, ldy = _mat(Y, "Y")
        descs[i] = FwdDesc(M, N, K, r, px, ldx, pw, ldw, pa, lda, pb, ldb, float(scale), py, ldy)
    ws, nb = (workspace.data_ptr(), workspace.numel()) if workspace is not None else (0, 0)
    _check(fwd_batch_raw(dt, descs, _stream(dev), ws, nb), "lora_fwd_batch")


_tile_cache = None


def fwd_tuned(X, W, A, B, scale: float, out=None, cache=None):
    """``fwd`` with the tile configuration a tuner cached for this shape (or
    the nearest cached shape), else the library's own choice.  ``cache``: a
    ``tune.TileCache``; by default the file ``tune.default_cache_path()``,
    loaded once."""
    from . import tune
    global _tile_cache
    if cache is None:
        if _tile_cache is None:
            _tile_cache = tune.TileCache.load()
        cache = _tile_cache
    dt = "bf16" if _dtype_code(X) == LORA_BF16 else "f32"
    choice = cache.lookup(dt, X.shape[0], W.shape[0], X.shape[1], A.shape[0])
    if choice is None:
        return fwd(X, W, A, B, scale, out=out)
    if choice == tune.DECODE:
        return fwd(X, W, A, B, scale, out=out, variant="decode")
    return fwd(X, W, A, B, scale, out=out, tile=int(choice.split(":")[1]))


def merge(W0, B, A, scale: float, out=None):
    """Merge from pristine ``W_inf = W0 + scale * B A`` (W0 is never written).

    W0[N,K], B[N,r], A[r,K]; returns W_inf[N,K] (``out`` if given).
    """
    import torch
    N, K = W0.shape
    r = A.shape[0]
    if A.shape[1] != K or tuple(B.shape) != (N, r):
        raise ValueError(f"shape mismatch W0{tuple(W0.shape)} B{tuple(B.shape)} A{tuple(A.shape)}")
    dt = _dtype_code(W0)
    for t, nm in ((B, "B"), (A, "A")):
        if t.dtype != W0.dtype or t.device != W0.device:
            raise ValueError(f"{nm} must match W0 in dtype and device")
    if out is None:
        out = torch.empty_like(W0)
    elif tuple(out.shape) != (N, K) or out.dtype != W0.dtype or out.device != W0.device:
        raise ValueError("out must be [N, K] with W0's dtype and device")
    p0, ld0 = _mat(W0, "W0")
    pb, ldb = _mat(B, "B")
    pa, lda = _mat(A, "A")
    po, ldo = _mat(out, "out")
    st = merge_raw(dt, N, K, r, p0, ld0, pb, ldb, pa, lda, float(scale), po, ldo,
                   _stream(W0.device))
    _check(st, "lora_merge")
    return out


def merge_batch(targets):
    """Merge from pristine for many targets: ``targets`` is a sequence of
    ``(W0, B, A, scale, W_inf)``; each ``W_inf`` is written as ``merge`` would
    write it.  All tensors share one dtype and device."""
    if not targets:
        return
    dt = _dtype_code(targets[0][0])
    dev = targets[0][0].device
    descs = (MergeDesc * len(targets))()
    for i, (W0, B, A, scale, out) in enumerate(targets):
        N, K = W0.shape
        r = A.shape[0]
        if A.shape[1] != K or tuple(B.shape) != (N, r) or tuple(out.shape) != (N, K):
            raise ValueError(f"target {i}: shape mismatch W0{tuple(W0.shape)} B{tuple(B.shape)} "
                             f"A{tuple(A.shape)} out{tuple(out.shape)}")
        for t, nm in ((W0, "W0"), (B, "B"), (A, "A"), (out, "out")):
            if _dtype_code(t) != dt or t.device != dev:
                raise ValueError(f"target {i}: {nm} must match the first W0 in dtype and device")
        p0, ld0 = _mat(W0, "W0")
        pb, ldb = _mat(B, "B")
        pa, lda = _mat(A, "A")
        po, ldo = _mat(out, "out")
        descs[i] = MergeDesc(N, K, r, p0, ld0, pb, ldb, pa, lda, float(scale), po, ldo)
    _check(merge_batch_raw(dt, descs, _stream(dev)), "lora_merge_batch")


def merge_inplace(W, B, A, scale: float):
    """In-place merge ``W = W + scale * B A`` (a negative scale unmerges).
    Not bit-reversible in bf16; ``merge`` from a pristine copy is."""
    N, K = W.shape
    r = A.shape[0]
    if A.shape[1] != K or tuple(B.shape) != (N, r):
        raise ValueError(f"shape mismatch W{tuple(W.shape)} B{tuple(B.shape)} A{tuple(A.shape)}")
    dt = _dtype_code(W)
    for t, nm in ((B, "B"), (A, "A")):
        if t.dtype != W.dtype or t.device != W.device:
            raise ValueError(f"{nm} must match W in dtype and device")
    pw, ldw = _mat(W, "W")
    pb, ldb = _mat(B, "B")
    pa, lda = _mat(A, "A")
    _check(merge_inplace_raw(dt, N, K, r, pw, ldw, pb, ldb, pa, lda, float(scale), _stream(W.device)),
           "lora_merge_inplace")
    return W


def bwd(X, W, A, B, dY, scale: float, want_dx: bool = True, workspace=None):
    """Backward of the layer with W frozen (bf16 only): returns ``(dX, dA, dB)``

    ``dX = dY W + scale (dY B) A``, ``dA = scale (dY B)^T X``,
    ``dB = scale dY^T (X A^T)``; ``dX`` is None when ``want_dx`` is false (W may
    then be None).  ``workspace``: a uint8 device tensor of at least
    ``bwd_workspace_size`` bytes, allocated here when not given.
    """
    import torch
    M, K = X.shape
    N = dY.shape[1]
    r = A.shape[0]
    if (dY.shape[0] != M or A.shape[1] != K or tuple(B.shape) != (N, r)
            or (want_dx and tuple(W.shape) != (N, K))):
        raise ValueError(f"shape mismatch X{tuple(X.shape)} A{tuple(A.shape)} B{tuple(B.shape)} "
                         f"dY{tuple(dY.shape)}" + (f" W{tuple(W.shape)}" if want_dx else ""))
    dt = _dtype_code(X)
    for t, nm in ((A, "A"), (B, "B"), (dY, "dY")) + (((W, "W"),) if want_dx else ()):
        if t.dtype != X.dtype or t.device != X.device:
            raise ValueError(f"{nm} must match X in dtype and device")
    dev = X.device
    need = bwd_workspace_size(dt, M, N, K, r)
    if need < 0:
        _check(LORA_ERR_UNSUPPORTED if dt == LORA_F32 else LORA_ERR_SHAPE, "lora_bwd")
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    dA = torch.empty((r, K), dtype=X.dtype, device=dev)
    dB = torch.empty((N, r), dtype=X.dtype, device=dev)
    dX = torch.empty((M, K), dtype=X.dtype, device=dev) if want_dx else None
    px, ldx = _mat(X, "X")
    pa, lda = _mat(A, "A")
    pb, ldb = _mat(B, "B")
    pdy, lddy = _mat(dY, "dY")
    pw, ldw = _mat(W, "W") if want_dx else (0, K)
    pdx, lddx = _mat(dX, "dX") if want_dx else (0, K)
    pda, ldda = _mat(dA, "dA")
    pdb, lddb = _mat(dB, "dB")
    st = bwd_raw(dt, M, N, K, r, px, ldx, pw, ldw, pa, lda, pb, ldb, pdy, lddy, float(scale),
                 pdx, lddx, pda, ldda, pdb, lddb, workspace.data_ptr(), workspace.numel(),
                 _stream(dev))
    _check(st, "lora_bwd")
    return dX, dA, dB
