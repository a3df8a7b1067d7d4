"""Shared test helpers: host <-> device transfer of generated inputs and the
error measures the parity bar is written in.

Error measures:
  * relative Frobenius error ||got - ref||_F / ||ref||_F in fp64; when
    ||ref||_F == 0 the result must be exactly zero (the error is ||got||_F);
  * bf16 ULP distance on the ordered integer line of bf16 bit patterns.
"""
from __future__ import annotations

import numpy as np

TOL = {"f32": 1e-5, "bf16": 1e-2}


def rel_fro(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(got - ref)
    return float(num / den) if den > 0 else float(num)


def bf16_ordered(bits: np.ndarray) -> np.ndarray:
    """Map bf16 bit patterns to integers whose order matches the values'."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int32)
    return np.where(b & 0x8000, 0x8000 - b, b)  # -0 and +0 both map to 0


def ulp_distance_bf16(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    return np.abs(bf16_ordered(a) - bf16_ordered(b))


def to_dev(a: np.ndarray, device="cuda"):
    """Generated array (float32, or uint16 bf16 bits) -> torch tensor on device."""
    import torch
    if a.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(device)


def to_host(t) -> np.ndarray:
    """torch tensor -> numpy (bf16 as uint16 bits, fp32 as float32)."""
    import torch
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def as_f64(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def sample_rows(M: int, n: int = 48, seed: int = 0) -> np.ndarray:
    """Row indices covering the first and last tiles and a seeded spread."""
    rng = np.random.default_rng(seed)
    head = np.arange(min(M, 8))
    tail = np.arange(max(0, M - 8), M)
    mid = rng.choice(M, size=min(M, n), replace=False)
    return np.unique(np.concatenate([head, tail, mid]))


def ulp_bf16_of(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values at |x| (2^(e-7) for |x| in [2^e, 2^(e+1)),
    2^-133 in the subnormal range)."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    e = np.where(ax > 0, np.maximum(e, -126.0), -126.0)
    return np.ldexp(1.0, (e - 7).astype(np.int64))


def merge_within_fp32_bound(got_bits, exact, W0, B, A, scale, r):
    """Per-element bar for a merge accumulated in fp32 and rounded once to bf16:
    |got - exact| <= ulp_bf16(exact) / 2 + delta, with
    delta = (r + 2) * 2^-24 * (|W0| + |scale| * sum_j |B[n,j]| |A[j,k]|),
    the worst-case error of fp32 accumulation of the r products and the add.
    Returns (ok_mask, delta)."""
    got = as_f64(got_bits)
    mag = np.abs(as_f64(W0)) + abs(float(np.float32(scale))) * (np.abs(as_f64(B)) @ np.abs(as_f64(A)))
    delta = (r + 2) * 2.0 ** -24 * mag
    ok = np.abs(got - exact) <= 0.5 * ulp_bf16_of(exact) + delta
    return ok, delta
