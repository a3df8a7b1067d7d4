"""The test-side error measures, checked against independent computations."""
import numpy as np
import pytest

import oracle
import synth
from helpers import (as_f64, merge_within_fp32_bound, rel_fro, ulp_bf16_of,
                     ulp_distance_bf16)


def test_ulp_spacing():
    assert ulp_bf16_of(np.array([1.0]))[0] == 2.0 ** -7
    assert ulp_bf16_of(np.array([1.99]))[0] == 2.0 ** -7
    assert ulp_bf16_of(np.array([-3.0]))[0] == 2.0 ** -6
    assert ulp_bf16_of(np.array([0.0]))[0] == 2.0 ** -133
    assert ulp_bf16_of(np.array([1e-40]))[0] == 2.0 ** -133


def test_ulp_distance_orders_bit_patterns():
    one, next_up, minus_zero, plus_zero = 0x3F80, 0x3F81, 0x8000, 0x0000
    a = np.array([one, minus_zero, 0x0001, 0x8001], np.uint16)
    b = np.array([next_up, plus_zero, 0x8001, 0x0001], np.uint16)
    np.testing.assert_array_equal(ulp_distance_bf16(a, b), [1, 0, 2, 2])


def test_rel_fro_zero_reference():
    assert rel_fro(np.zeros(3), np.zeros(3)) == 0.0
    assert rel_fro(np.ones(3), np.zeros(3)) > 0


def test_fp32_merge_satisfies_the_merge_bar():
    """An independent fp32 merge (numpy float32 matmul and add, then bf16
    rounding) meets the per-element bound used for the GPU merge."""
    tgt = synth.MergeTarget("probe", 93, 0, 384, 512, 32, 64.0)
    W0 = tgt.make_w0()
    A, B = tgt.make_ab(0)
    Wd, _ = oracle.merge(W0, B, A, tgt.scale, want_bf16=False)
    w32 = (synth.bf16_bits_to_f32(W0)
           + np.float32(tgt.scale) * (synth.bf16_bits_to_f32(B) @ synth.bf16_bits_to_f32(A)))
    got = synth.f32_to_bf16_bits(w32.astype(np.float32))
    ok, _ = merge_within_fp32_bound(got, Wd, W0, B, A, tgt.scale, tgt.r)
    assert ok.all()
    # and a value off by a whole bf16 step in a calm region fails it
    bad = got.copy()
    i = int(np.argmax(np.abs(as_f64(got))))
    bad.flat[i] += 1
    ok_bad, _ = merge_within_fp32_bound(bad, Wd, W0, B, A, tgt.scale, tgt.r)
    assert not ok_bad.flat[i]


# ------------------------------------------------------- per-element bound

from helpers import (block_rows, bwd_bounds, check_fwd_elements, fwd_bound,  # noqa: E402
                     within_bound)


def _f32(a):
    return synth.bf16_bits_to_f32(a) if a.dtype == np.uint16 else a


def _emulate_bf16_fwd(t, s):
    """The tiled kernel's arithmetic emulated independently in numpy float32
    (BLAS sgemm order): fp32 sums, s T rounded once to bf16, one rounding
    of the result."""
    X, W, A, B = (_f32(t[k]) for k in "XWAB")
    T = X @ A.T
    sT = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits((np.float32(s) * T).astype(np.float32)))
    acc = X @ W.T + sT @ B.T
    return synth.f32_to_bf16_bits(acc.astype(np.float32))


@pytest.fixture(scope="module")
def mid_case():
    c = synth.MID
    t = c.make()
    ref = oracle.fwd(t["X"], t["W"], t["A"], t["B"], c.scale)
    return c, t, ref


def test_bound_accepts_fp32_emulation_of_the_kernel(mid_case):
    c, t, ref = mid_case
    got = _emulate_bf16_fwd(t, c.scale)
    ratio = check_fwd_elements(got, ref, t["X"], t["W"], t["A"], t["B"], c.scale, "bf16", "emul")
    assert ratio < 1.0


def test_bound_rejects_one_zeroed_block_that_rel_fro_accepts(mid_case):
    """One 16 x 16 MFMA block of the output left at zero: the relative
    Frobenius bar still passes on this 4096 x 1024 output, the per-element
    bound does not."""
    c, t, ref = mid_case
    got = _emulate_bf16_fwd(t, c.scale)
    bad = got.copy()
    bad[1024:1040, 512:528] = 0
    assert rel_fro(as_f64(bad), ref) <= 1e-2          # the norm alone misses it
    bound = fwd_bound(ref, t["X"], t["W"], t["A"], t["B"], c.scale, "bf16")
    ok, _ = within_bound(as_f64(bad), ref, bound)
    assert not ok[1024:1040, 512:528].all()
    assert ok[:1024].all() and ok[1040:].all()


@pytest.mark.parametrize("mistake", ["minus_scale", "no_lora", "unscaled_T", "A_rows_swapped",
                                     "one_row_shifted"])
def test_bound_rejects_plausible_mistakes(mid_case, mistake):
    c, t, ref = mid_case
    t2 = dict(t)
    s = c.scale
    if mistake == "minus_scale":
        s = -s
    elif mistake == "no_lora":
        s = 0.0
    elif mistake == "unscaled_T":
        s = 1.0
    elif mistake == "A_rows_swapped":
        t2["A"] = t["A"][::-1].copy()
    got = _emulate_bf16_fwd(t2, s)
    if mistake == "one_row_shifted":
        got = got.copy()
        got[17] = got[18]
    bound = fwd_bound(ref, t["X"], t["W"], t["A"], t["B"], c.scale, "bf16")
    ok, _ = within_bound(as_f64(got), ref, bound)
    assert (~ok).sum() > 0.5 * (1 if mistake == "one_row_shifted" else c.M) * c.N


def test_bound_fp32_path():
    """fp32 operands (cfg 1 shape): float32 emulation passes; the largest
    element moved by 1 % fails (a worst-case bound on 528-term fp32 sums is
    about 0.3 % of a typical element here, so finer errors are left to the
    1e-5 relative Frobenius bar)."""
    c = synth.TINY
    t = c.make()
    ref = oracle.fwd(t["X"], t["W"], t["A"], t["B"], c.scale)
    X, W, A, B = (t[k] for k in "XWAB")
    got = (X @ W.T + np.float32(c.scale) * ((X @ A.T) @ B.T)).astype(np.float32)
    check_fwd_elements(got, ref, X, W, A, B, c.scale, "f32", "tiny")
    bad = got.copy()
    i = np.unravel_index(np.argmax(np.abs(ref)), ref.shape)
    bad[i] *= np.float32(1.01)
    ok, _ = within_bound(bad.astype(np.float64), ref, fwd_bound(ref, X, W, A, B, c.scale, "f32"))
    assert not ok[i] and ok.sum() == ok.size - 1


def test_bwd_bound_accepts_emulation_and_rejects_a_zeroed_row():
    c = synth.FwdCase("bwd_bound", 6, 77, 600, 264, 328, 16, 32.0, "bf16")
    t = c.make("XWABD")
    s = np.float32(c.scale)
    X, W, A, B, dY = (_f32(t[k]) for k in ("X", "W", "A", "B", "dY"))
    bf = lambda a: synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(a.astype(np.float32)))  # noqa
    sG = bf(s * (dY @ B))
    sT = bf(s * (X @ A.T))
    got = [synth.f32_to_bf16_bits((dY @ W + sG @ A).astype(np.float32)),
           synth.f32_to_bf16_bits((sG.T @ X).astype(np.float32)),
           synth.f32_to_bf16_bits((dY.T @ sT).astype(np.float32))]
    ref = oracle.bwd(t["X"], t["W"], t["A"], t["B"], t["dY"], c.scale)
    bounds = bwd_bounds(t["X"], t["W"], t["A"], t["B"], t["dY"], c.scale, *ref)
    for g, r, b in zip(got, ref, bounds):
        ok, ratio = within_bound(as_f64(g), r, b)
        assert ok.all() and ratio < 1.0
    bad = got[1].copy()
    bad[3] = 0
    ok, _ = within_bound(as_f64(bad), ref[1], bounds[1])
    assert not ok[3].all() and ok[:3].all()


def test_block_rows_cover_every_block():
    rows = block_rows(16384, 16, seed=3)
    assert rows[0] == 0 and rows[-1] == 16383
    assert set(rows // 16) == set(range(1024))
    assert len(block_rows(37, 16)) >= 3
