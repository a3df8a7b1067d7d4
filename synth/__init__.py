"""Seeded synthetic inputs for the fused LoRA linear and the pristine merge.

This module is shared by the oracle side and the HIP side of every test and of
the benchmark.  It holds no step of the method's arithmetic: it only draws
normal samples, narrows them to the storage precision and names the workloads.

Recipe (stated once, used everywhere):
  * ``rng = numpy.random.Generator(PCG64(SeedSequence([group, case, tensor])))``
  * ``rng.standard_normal(shape, float64) * std`` where ``std = sqrt(var)``:
    the pages' ``N(0, v)`` is read as mean 0, *variance* v.
  * narrowed to float32 with round-to-nearest-even (numpy ``astype``), then,
    for bf16 workloads, to bf16 with round-to-nearest-even on the fp32 bits.
  * tensor ids: X=0, W/W0=1, A=2, B=3, dY (the output gradient of a
    backward case, N(0, 1)) = 4; merge cycle c draws A with id 10c+2 and B
    with id 10c+3 (cycle 0 therefore uses 2 and 3).

bf16 tensors are returned as ``numpy.uint16`` bit patterns; fp32 tensors as
``numpy.float32``.  Both sides consume exactly these values.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np

TX, TW, TA, TB, TDY = 0, 1, 2, 3, 4


def _rng(group: int, case: int, tensor: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([group, case, tensor])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns uint16 bits.

    Storage narrowing for generated inputs only.  NaN maps to a quiet NaN.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def normal(group: int, case: int, tensor: int, shape: Tuple[int, ...], var: float,
           dtype: str) -> np.ndarray:
    """One seeded tensor: N(0, var) in fp64 -> fp32 (RNE) -> bf16 (RNE) if asked."""
    g = _rng(group, case, tensor)
    x = (g.standard_normal(shape, dtype=np.float64) * math.sqrt(var)).astype(np.float32)
    if dtype == "f32":
        return x
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def to_f64(x: np.ndarray) -> np.ndarray:
    """Exact widening of a generated tensor (fp32 array or bf16 bits) to float64."""
    if x.dtype == np.uint16:
        return bf16_bits_to_f32(x).astype(np.float64)
    return x.astype(np.float64)


# ---------------------------------------------------------------------------
# Workloads.  Shapes: M tokens, N = d_out, K = d_in, r = rank, s = alpha / r.
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class FwdCase:
    name: str
    group: int      # seed group (first SeedSequence word)
    case: int
    M: int
    N: int
    K: int
    r: int
    alpha: float
    dtype: str
    var_x: float = 1.0
    var_w: Optional[float] = None      # default 1/K
    var_a: Optional[float] = None      # default 1/K
    var_b: float = 0.02
    x_from: Optional[Tuple[int, int]] = None   # (group, case) whose X this case shares

    @property
    def scale(self) -> float:
        return self.alpha / self.r

    def flops(self) -> float:
        M, N, K, r = self.M, self.N, self.K, self.r
        return 2.0 * M * N * K + 2.0 * M * K * r + 2.0 * M * N * r

    def bytes(self) -> float:
        e = 4 if self.dtype == "f32" else 2
        M, N, K, r = self.M, self.N, self.K, self.r
        return float(e * (M * K + N * K + r * K + N * r + M * N))

    def make(self, parts: str = "XWAB") -> Dict[str, np.ndarray]:
        vw = self.var_w if self.var_w is not None else 1.0 / self.K
        va = self.var_a if self.var_a is not None else 1.0 / self.K
        out: Dict[str, np.ndarray] = {}
        xc = self.x_from if self.x_from is not None else (self.group, self.case)
        if "X" in parts:
            out["X"] = normal(xc[0], xc[1], TX, (self.M, self.K), self.var_x, self.dtype)
        if "W" in parts:
            out["W"] = normal(self.group, self.case, TW, (self.N, self.K), vw, self.dtype)
        if "A" in parts:
            out["A"] = normal(self.group, self.case, TA, (self.r, self.K), va, self.dtype)
        if "B" in parts:
            out["B"] = normal(self.group, self.case, TB, (self.N, self.r), self.var_b, self.dtype)
        if "D" in parts:
            out["dY"] = normal(self.group, self.case, TDY, (self.M, self.N), 1.0, self.dtype)
        return out


@dataclass(frozen=True)
class MergeTarget:
    name: str
    group: int      # seed group (first SeedSequence word)
    case: int
    N: int        # out features
    K: int        # in features
    r: int
    alpha: float
    dtype: str = "bf16"
    var_w0: float = 0.02
    var_b: float = 0.02

    @property
    def scale(self) -> float:
        return self.alpha / self.r

    def bytes(self) -> float:
        e = 2 if self.dtype == "bf16" else 4
        return float(2 * e * self.N * self.K + e * self.r * (self.N + self.K))

    def flops(self) -> float:
        return 2.0 * self.r * self.N * self.K

    def make_w0(self) -> np.ndarray:
        return normal(self.group, self.case, TW, (self.N, self.K), self.var_w0, self.dtype)

    def make_ab(self, cycle: int = 0) -> Tuple[np.ndarray, np.ndarray]:
        A = normal(self.group, self.case, 10 * cycle + TA, (self.r, self.K), 1.0 / self.K, self.dtype)
        B = normal(self.group, self.case, 10 * cycle + TB, (self.N, self.r), self.var_b, self.dtype)
        return A, B


# Tiny fp32 LoRA linear (seed group 1).
TINY = FwdCase("tiny_f32_x128x512_w512x512_r16", 1, 0, 128, 512, 512, 16, 32.0, "f32")
# bf16 mid-size, 4 x 1024 tokens (seed group 2).
MID = FwdCase("bf16_mid_x4096x1024_w1024x1024_r16", 2, 0, 4096, 1024, 1024, 16, 32.0, "bf16")
# Transformer projection shapes (hidden 2560, 8192 tokens) and a large square
# sweep (seed group 3).
QPROJ = FwdCase("bf16_qproj_x8192x2560_w4096x2560_r32", 3, 0, 8192, 4096, 2560, 32, 64.0, "bf16")
VPROJ = FwdCase("bf16_vproj_x8192x2560_w1024x2560_r32", 3, 1, 8192, 1024, 2560, 32, 64.0, "bf16",
                 x_from=(3, 0))
SQUARE = tuple(
    FwdCase(f"bf16_square_x16384x8192_w8192x8192_r{r}", 3, 2 + i, 16384, 8192, 8192, r, 2.0 * r, "bf16")
    for i, r in enumerate((8, 16, 64, 128)))
# Decode-shaped, bandwidth-bound (seed group 4).
DECODE = tuple(
    FwdCase(f"bf16_decode_m{m}_w4096x4096_r16", 4, i, m, 4096, 4096, 16, 32.0, "bf16")
    for i, m in enumerate((1, 8, 64)))

# Merge from pristine over 36 layers x 7 targets of a hidden-2560 model, rank 32
# (seed group 5).
MERGE_LAYERS = 36
MERGE_TARGET_SHAPES: List[Tuple[str, int, int]] = [
    ("q", 4096, 2560), ("k", 1024, 2560), ("v", 1024, 2560), ("o", 2560, 4096),
    ("gate", 9728, 2560), ("up", 9728, 2560), ("down", 2560, 9728),
]


def merge_targets(layers: int = MERGE_LAYERS) -> List[MergeTarget]:
    out = []
    for layer in range(layers):
        for t, (nm, n, k) in enumerate(MERGE_TARGET_SHAPES):
            out.append(MergeTarget(f"l{layer}.{nm}", 5, layer * 7 + t, n, k, 32, 64.0))
    return out


FWD_CASES: List[FwdCase] = [TINY, MID, QPROJ, VPROJ, *SQUARE, *DECODE]


# ---------------------------------------------------------------------------
# Device-side generation for throughput runs whose inputs are too large to
# draw on the host in reasonable time (the 7.3 GB merge set, the square sweep).
# Same distributions, a different generator: torch's Philox stream on the
# device, seeded from (group, case, tensor).  Parity tests use the numpy recipe.
# ---------------------------------------------------------------------------

def device_seed(group: int, case: int, tensor: int) -> int:
    return int(np.random.SeedSequence([group, case, tensor]).generate_state(1, np.uint64)[0]
               & 0x7FFFFFFFFFFFFFFF)


def device_normal(group: int, case: int, tensor: int, shape, var: float, dtype: str,
                  device="cuda"):
    """N(0, var) drawn on the device, fp32 then narrowed (bf16: nearest-even)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(device_seed(group, case, tensor))
    x = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    x.mul_(math.sqrt(var))
    return x.to(torch.bfloat16) if dtype == "bf16" else x


def dy_on_device(c: FwdCase, device="cuda"):
    """The output gradient of a backward case, drawn on the device."""
    return device_normal(c.group, c.case, TDY, (c.M, c.N), 1.0, c.dtype, device)


def fwd_case_on_device(c: FwdCase, device="cuda"):
    vw = c.var_w if c.var_w is not None else 1.0 / c.K
    va = c.var_a if c.var_a is not None else 1.0 / c.K
    xc = c.x_from if c.x_from is not None else (c.group, c.case)
    return {
        "X": device_normal(xc[0], xc[1], TX, (c.M, c.K), c.var_x, c.dtype, device),
        "W": device_normal(c.group, c.case, TW, (c.N, c.K), vw, c.dtype, device),
        "A": device_normal(c.group, c.case, TA, (c.r, c.K), va, c.dtype, device),
        "B": device_normal(c.group, c.case, TB, (c.N, c.r), c.var_b, c.dtype, device),
    }
