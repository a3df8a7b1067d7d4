"""The seeded input generators: determinism, distributions, bf16 narrowing."""
import numpy as np
import pytest

import synth


def test_same_seed_same_bytes():
    a = synth.MID.make()
    b = synth.MID.make()
    for k in "XWAB":
        assert a[k].tobytes() == b[k].tobytes()
    c = synth.TINY.make()
    assert c["X"].dtype == np.float32 and a["X"].dtype == np.uint16


def test_distinct_tensors_and_shared_hidden_states():
    q = synth.QPROJ.make("XA")
    v = synth.VPROJ.make("XA")
    assert q["X"].tobytes() == v["X"].tobytes()          # q and v read the same X
    assert q["A"].tobytes() != v["A"].tobytes()


def test_variance_reading():
    # N(0, v) is read as variance v: std of B ~ sqrt(0.02), of W ~ sqrt(1/K)
    t = synth.MID.make()
    w = synth.to_f64(t["W"])
    b = synth.to_f64(t["B"])
    assert abs(w.std() - (1 / 1024) ** 0.5) / (1 / 1024) ** 0.5 < 0.01
    assert abs(b.std() - 0.02 ** 0.5) / 0.02 ** 0.5 < 0.03


def test_bf16_narrowing_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-30, 30, 100000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(synth.f32_to_bf16_bits(x), ref)
    np.testing.assert_array_equal(synth.bf16_bits_to_f32(ref),
                                  torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16)
                                  .float().numpy())


def test_workload_sizes():
    assert round(synth.MID.flops() / 1e9, 3) == 8.858
    assert round(synth.QPROJ.flops() / 1e9, 2) == 175.29
    assert round(synth.DECODE[0].bytes() / 1e6, 3) == 33.833
    tg = synth.merge_targets()
    assert len(tg) == 252
    assert round(sum(t.bytes() for t in tg) / 1e9, 3) == 14.665
