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


# ------------------------------------------------------- per-element bound
#
# The relative Frobenius bar above is a norm over a whole output: on a large
# output one wrong 16 x 16 block moves it by about 16 * 16 / (M N) of its
# size and can pass.  Every forward and backward parity check therefore also
# bounds each element by the worst case of the arithmetic the kernels do:
#
#   * products of bf16 (or fp32) operands summed in fp32 in any order:
#     a sum of n terms is within gamma_n = n u32 (1 + o(1)) of the exact
#     sum, relative to the sum of the terms' magnitudes (u32 = 2^-24);
#     the bound below doubles it, so that it also holds if the matrix
#     cores' internal additions truncate instead of rounding to nearest;
#   * a rank intermediate (s T in the forward, s G or s T in the backward)
#     rounded once to bf16 before it is an operand again: relative error
#     u_mid = 2^-8 of its own value (bf16 has an 8-bit significand); fp32
#     intermediates: u_mid = 0;
#   * one rounding of the result to the output type: half a unit in the
#     last place of the computed value.
#
# For an output  y = sum_i p_i + sum_j round(s t_j) q_j,  t_j = sum_k u_jk,
# with the exact magnitudes
#   mag_f = sum_i |p_i|                       (products summed directly)
#   mag_t = |s| sum_j |q_j| |t_j|             (through the intermediate)
#   mag_r = |s| sum_j |q_j| sum_k |u_jk|      (the intermediate's own sum)
# the fp32 value c computed before the final rounding satisfies
#   |c - y| <= acc = 2 (n_acc + 4) u32 (mag_f + 1.01 mag_t)
#                    + (2 + 1.01 u_mid) (n_mid + 4) u32 mag_r + 1.01 u_mid mag_t
# (n_acc: terms of the output's fp32 sum, n_mid: terms of t_j's), and the
# stored result differs from y by at most acc + ulp(|y| + acc) / 2.  For the
# forward: p = X[m,:] W[n,:], q = B[n,:], u_jk = X[m,k] A[j,k], n_acc = K + r,
# n_mid = K.

U32 = 2.0 ** -24


def ulp_f32_of(x: np.ndarray) -> np.ndarray:
    """Spacing of fp32 values at |x| (2^(e-23); 2^-149 in the subnormal range)."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    e = np.where(ax > 0, np.maximum(e, -126.0), -126.0)
    return np.ldexp(1.0, (e - 23).astype(np.int64))


def elem_bound(ref, mag_f, mag_t, mag_r, n_acc: int, n_mid: int, dtype: str,
               mid_rounded: bool = True):
    """Per-element error bound of the reasoning above (float64 array)."""
    u_mid = 2.0 ** -8 if (dtype == "bf16" and mid_rounded) else 0.0
    acc = (2.0 * (n_acc + 4) * U32 * (mag_f + 1.01 * mag_t)
           + (2.0 + 1.01 * u_mid) * (n_mid + 4) * U32 * mag_r + 1.01 * u_mid * mag_t)
    big = np.abs(ref) + acc
    half_ulp = 0.5 * (ulp_bf16_of(big) if dtype == "bf16" else ulp_f32_of(big))
    return acc + half_ulp


def within_bound(got, ref, bound):
    """(ok mask, worst |got - ref| / bound) for a result against its bound.
    A NaN in got never passes."""
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - ref)
    ok = err <= bound
    ratio = float(np.nanmax(err / bound)) if err.size else 0.0
    return ok, ratio


def fwd_magnitudes(X, W, A, B, scale):
    """(mag_f, mag_t, mag_r) of the forward for the given rows of X, in
    float64 (magnitudes only scale the bound): |X||W|^T, |s| |X A^T| |B|^T
    and |s| (|X||A|^T) |B|^T."""
    x, w, a, b = (as_f64(t) for t in (X, W, A, B))
    s = abs(float(np.float32(scale)))
    ax, ab = np.abs(x), np.abs(b)
    mag_f = ax @ np.abs(w).T
    mag_t = s * (np.abs(x @ a.T) @ ab.T)
    mag_r = s * ((ax @ np.abs(a).T) @ ab.T)
    return mag_f, mag_t, mag_r


def fwd_bound(ref, X, W, A, B, scale, dtype: str):
    K, r = W.shape[1], A.shape[0]
    return elem_bound(ref, *fwd_magnitudes(X, W, A, B, scale), K + r, K, dtype)


def check_fwd_elements(got_bits, ref, X, W, A, B, scale, dtype: str, name: str = ""):
    """Assert every forward output element is within the bound; X holds the
    rows of the checked output rows only.  Returns the worst ratio."""
    bound = fwd_bound(ref, X, W, A, B, scale, dtype)
    got = as_f64(got_bits)
    ok, ratio = within_bound(got, ref, bound)
    if not ok.all():
        bad = np.argwhere(~ok)
        i = tuple(bad[0])
        raise AssertionError(f"{name}: {len(bad)} elements outside the per-element bound, "
                             f"first at {i}: got {got[i]!r} ref {ref[i]!r} bound {bound[i]:.3e}")
    return ratio


def bwd_bounds(X, W, A, B, dY, scale, dX_ref, dA_ref, dB_ref, dx_rows=None):
    """Per-element bounds of dX, dA, dB (bf16 path: s G and s T rounded once
    to bf16 before they are operands again).  dx_rows: the rows of X / dY
    that dX_ref holds (all when None)."""
    s = abs(float(np.float32(scale)))
    x, a, b, dy = (as_f64(t) for t in (X, A, B, dY))
    ax, aa, ab, ady = np.abs(x), np.abs(a), np.abs(b), np.abs(dy)
    M, K = X.shape
    N, r = B.shape
    G = dy @ b                               # exact G = dY B   [M, r]
    Gm = ady @ ab                            # its sum of magnitudes
    out = []
    if dX_ref is not None and dX_ref.size:
        rows = slice(None) if dx_rows is None else dx_rows
        out.append(elem_bound(dX_ref, ady[rows] @ np.abs(as_f64(W)), s * (np.abs(G[rows]) @ aa),
                              s * (Gm[rows] @ aa), N + r, N, "bf16"))
    else:
        out.append(None)
    zA = np.zeros_like(dA_ref)
    out.append(elem_bound(dA_ref, zA, s * (np.abs(G).T @ ax), s * (Gm.T @ ax), M, N, "bf16"))
    T = x @ a.T
    zB = np.zeros_like(dB_ref)
    out.append(elem_bound(dB_ref, zB, s * (ady.T @ np.abs(T)), s * (ady.T @ (ax @ aa.T)), M, K,
                          "bf16"))
    return out


def check_bwd_elements(got, ref, bounds, name: str = ""):
    """Assert each gradient (bf16 bits) is within its bound; entries of got
    and ref that are None are skipped.  Returns the worst ratios."""
    ratios = []
    for g, rf, bd, nm in zip(got, ref, bounds, ("dX", "dA", "dB")):
        if g is None or bd is None:
            ratios.append(0.0)
            continue
        v = as_f64(g)
        ok, ratio = within_bound(v, rf, bd)
        if not ok.all():
            bad = np.argwhere(~ok)
            i = tuple(bad[0])
            raise AssertionError(f"{name} {nm}: {len(bad)} elements outside the bound, first at "
                                 f"{i}: got {v[i]!r} ref {rf[i]!r} bound {bd[i]:.3e}")
        ratios.append(ratio)
    return ratios


def block_rows(M: int, block: int = 16, seed: int = 0) -> np.ndarray:
    """One row from every `block`-row block (seeded offset within the block),
    plus the first and last row: every M tile of every tile shape is checked."""
    rng = np.random.default_rng(seed)
    nb = (M + block - 1) // block
    off = rng.integers(0, block, size=nb)
    rows = np.minimum(np.arange(nb) * block + off, M - 1)
    return np.unique(np.concatenate([rows, [0, M - 1]]))
