"""The test-side error measures, checked against independent computations."""
import numpy as np

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
