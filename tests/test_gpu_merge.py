"""Parity and invariants of the HIP merge from pristine against the fp64
oracle, through the C ABI, on seeded inputs.

Bar (bf16): relative Frobenius error <= 1e-2, and every element equal to the
bf16 rounding of a value within the fp32-accumulation error bound of the
exact result (|got - exact| <= ulp/2 + (r+2) 2^-24 (|W0| + |s| sum|B||A|)).
That is the meaning of "within 1 bf16 ULP of an fp32-accumulating path" at
weight magnitude; where W0 + s B A nearly cancels, the result is tiny and the
same absolute error spans more ULPs of it, so the ULP distance to the
correctly rounded value is reported (max, exact-match fraction) and bounded
by 1 only away from such cancellation.  W0 bit-identical after 10
perturb+merge cycles; re-merging the cycle-0 adapter reproduces the cycle-0
W_inf bitwise; B = 0 or scale = 0 reproduce W0 bitwise.  fp32: relative
Frobenius error <= 1e-5.
"""
import numpy as np
import pytest

import oracle
import synth
from helpers import (TOL, as_f64, merge_within_fp32_bound, rel_fro, to_dev, to_host,
                     ulp_bf16_of, ulp_distance_bf16)

pytestmark = pytest.mark.gpu

LAYER0 = synth.merge_targets(1)


def _merge(rg, W0, A, B, s, out=None):
    import torch
    Wi = rg.merge(W0, B, A, s, out=out)
    torch.cuda.synchronize()
    return Wi


@pytest.mark.parametrize("tgt", LAYER0, ids=lambda t: t.name)
def test_layer0_targets_parity(gpu_lib, tgt):
    W0 = tgt.make_w0()
    A, B = tgt.make_ab(0)
    got = to_host(_merge(gpu_lib, to_dev(W0), to_dev(A), to_dev(B), tgt.scale))
    Wd, Wb = oracle.merge(W0, B, A, tgt.scale)
    _check_bf16_merge(got, Wd, Wb, W0, B, A, tgt.scale, tgt.r, tgt.name)


def _check_bf16_merge(got, Wd, Wb, W0, B, A, s, r, name):
    err = rel_fro(as_f64(got), Wd)
    ulp = ulp_distance_bf16(got, Wb)
    ok, delta = merge_within_fp32_bound(got, Wd, W0, B, A, s, r)
    # away from cancellation (fp32 error below a quarter ulp) at most 1 ulp
    calm = delta < 0.25 * ulp_bf16_of(Wd)
    print(f"{name}: rel_fro={err:.3e} max_ulp={int(ulp.max())} "
          f"max_ulp_away_from_cancellation={int(ulp[calm].max())} "
          f"exact={float((ulp == 0).mean()):.6f} bound_ok={bool(ok.all())}")
    assert err <= TOL["bf16"]
    assert ok.all()
    assert int(ulp[calm].max()) <= 1


def test_ten_cycles_pristine_and_remerge(gpu_lib):
    """Perturb+merge cycles with fresh adapters: W0 stays bit-identical, and
    merging the cycle-0 adapter again reproduces cycle 0's W_inf bitwise."""
    import torch
    tg = LAYER0
    w0_host = [t.make_w0() for t in tg]
    w0_dev = [to_dev(w) for w in w0_host]
    wi_dev = [torch.empty_like(w) for w in w0_dev]
    first = None
    for cycle in range(10):
        for t, w0, wi in zip(tg, w0_dev, wi_dev):
            A, B = t.make_ab(cycle)
            gpu_lib.merge(w0, to_dev(B), to_dev(A), t.scale, out=wi)
        torch.cuda.synchronize()
        if cycle == 0:
            first = [to_host(w) for w in wi_dev]
    for w_host, w in zip(w0_host, w0_dev):
        assert to_host(w).tobytes() == w_host.tobytes()
    for t, w0, wi, ref in zip(tg, w0_dev, wi_dev, first):
        A, B = t.make_ab(0)
        gpu_lib.merge(w0, to_dev(B), to_dev(A), t.scale, out=wi)
        torch.cuda.synchronize()
        assert to_host(wi).tobytes() == ref.tobytes(), t.name


@pytest.mark.parametrize("which", ["B0", "s0"])
def test_zero_adapter_reproduces_pristine(gpu_lib, which):
    t = LAYER0[1]
    W0 = t.make_w0()
    A, B = t.make_ab(0)
    if which == "B0":
        B = np.zeros_like(B)
    s = 0.0 if which == "s0" else t.scale
    got = to_host(_merge(gpu_lib, to_dev(W0), to_dev(A), to_dev(B), s))
    assert got.tobytes() == W0.tobytes()


RAGGED = [
    # N, K, r, dtype
    (1, 8, 1, "bf16"),
    (37, 264, 7, "bf16"),
    (100, 520, 32, "bf16"),
    (33, 1000, 33, "bf16"),
    (300, 256, 64, "bf16"),
    (64, 776, 100, "bf16"),
    (17, 272, 128, "bf16"),
    (70, 520, 200, "bf16"),
    (40, 264, 256, "bf16"),
    (1024, 4096, 32, "bf16"),
    (33, 100, 5, "f32"),
    (64, 1028, 32, "f32"),
]


@pytest.mark.parametrize("N,K,r,dtype", RAGGED)
def test_ragged_shapes(gpu_lib, N, K, r, dtype):
    t = synth.MergeTarget(f"m{N}x{K}r{r}", 91, N * 3 + r, N, K, r, 2.0 * r, dtype)
    W0 = t.make_w0()
    A, B = t.make_ab(0)
    got = to_host(_merge(gpu_lib, to_dev(W0), to_dev(A), to_dev(B), t.scale))
    Wd, Wb = oracle.merge(W0, B, A, t.scale, want_bf16=(dtype == "bf16"))
    if dtype == "bf16":
        _check_bf16_merge(got, Wd, Wb, W0, B, A, t.scale, r, f"N{N} K{K} r{r}")
    else:
        err = rel_fro(as_f64(got), Wd)
        print(f"N{N} K{K} r{r} {dtype}: rel_fro={err:.3e}")
        assert err <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_padded_leading_dimensions(gpu_lib, dtype):
    import torch
    N, K, r = 48, 264, 20
    t = synth.MergeTarget("pad", 92, 0, N, K, r, 40.0, dtype)
    W0 = t.make_w0()
    A, B = t.make_ab(0)

    def padded(a, p):
        d = to_dev(a)
        big = torch.zeros((d.shape[0], d.shape[1] + p), dtype=d.dtype, device=d.device)
        big[:, : d.shape[1]] = d
        return big[:, : d.shape[1]]

    w0, a, b = padded(W0, 16), padded(A, 8), padded(B, 5)
    big = torch.full((N, K + 8), float("nan"), dtype=w0.dtype, device=w0.device)
    _merge(gpu_lib, w0, a, b, t.scale, out=big[:, :K])
    got = to_host(big)
    Wd, _ = oracle.merge(W0, B, A, t.scale, want_bf16=False)
    assert rel_fro(as_f64(got[:, :K]), Wd) <= TOL[dtype]
    assert np.isnan(as_f64(got[:, K:])).all()


def test_deterministic(gpu_lib):
    t = LAYER0[4]
    W0 = t.make_w0()
    A, B = t.make_ab(3)
    w0, a, b = to_dev(W0), to_dev(A), to_dev(B)
    x = to_host(_merge(gpu_lib, w0, a, b, t.scale))
    y = to_host(_merge(gpu_lib, w0, a, b, t.scale))
    assert x.tobytes() == y.tobytes()


def test_rslora_scale_passed_through(gpu_lib):
    """rsLoRA folds alpha / sqrt(r) into the scaling; the merge uses it as given."""
    t = LAYER0[0]
    W0 = t.make_w0()
    A, B = t.make_ab(0)
    s = 64.0 / np.sqrt(32.0)
    got = to_host(_merge(gpu_lib, to_dev(W0), to_dev(A), to_dev(B), s))
    Wd, Wb = oracle.merge(W0, B, A, s)
    _check_bf16_merge(got, Wd, Wb, W0, B, A, s, t.r, "rslora")


def _batch_targets(dtype):
    """Layer-0 targets plus ragged ones with mixed ranks, 31 in all (more
    than one launch's worth, rank changes forcing separate launches)."""
    tg = list(LAYER0) if dtype == "bf16" else []
    shapes = [(37, 264, 7), (100, 520, 32), (33, 1000, 33), (300, 256, 64), (17, 272, 128),
              (70, 520, 200), (1, 8, 1), (64, 776, 100)]
    i = 0
    while len(tg) < 31:
        N, K, r = shapes[i % len(shapes)]
        tg.append(synth.MergeTarget(f"b{i}", 93, i, N + i, K, r, 2.0 * r, dtype))
        i += 1
    return tg


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_batch_equals_per_target_merges(gpu_lib, dtype):
    import torch
    tg = _batch_targets(dtype)
    ins, w0_host = [], []
    for t in tg:
        W0 = t.make_w0()
        A, B = t.make_ab(0)
        w0_host.append(W0)
        ins.append((to_dev(W0), to_dev(B), to_dev(A), t.scale))
    one = [_merge(gpu_lib, w0, a, b, s) for (w0, b, a, s) in ins]
    outs = [torch.full_like(o, float("nan")) for o in one]
    gpu_lib.merge_batch([(w0, b, a, s, o) for (w0, b, a, s), o in zip(ins, outs)])
    torch.cuda.synchronize()
    for t, o, ref, (w0, _, _, _), h in zip(tg, outs, one, ins, w0_host):
        assert to_host(o).tobytes() == to_host(ref).tobytes(), t.name
        assert to_host(w0).tobytes() == h.tobytes(), t.name  # pristine untouched
    # one ragged target against the oracle directly
    t = tg[-1]
    A, B = t.make_ab(0)
    Wd, Wb = oracle.merge(w0_host[-1], B, A, t.scale, want_bf16=(dtype == "bf16"))
    got = to_host(outs[-1])
    if dtype == "bf16":
        _check_bf16_merge(got, Wd, Wb, w0_host[-1], B, A, t.scale, t.r, "batch " + t.name)
    else:
        assert rel_fro(as_f64(got), Wd) <= TOL[dtype]


def test_batch_full_model_pass_matches_per_target(gpu_lib):
    """All 36 x 7 targets in one call, bitwise equal to one call per target."""
    import torch
    tg = synth.merge_targets(36)
    w0, a, b, one, outs = [], [], [], [], []
    for t in tg:
        w0.append(synth.device_normal(t.group, t.case, synth.TW, (t.N, t.K), t.var_w0, "bf16"))
        a.append(synth.device_normal(t.group, t.case, synth.TA, (t.r, t.K), 1.0 / t.K, "bf16"))
        b.append(synth.device_normal(t.group, t.case, synth.TB, (t.N, t.r), t.var_b, "bf16"))
    for i, t in enumerate(tg):
        one.append(gpu_lib.merge(w0[i], b[i], a[i], t.scale))
        outs.append(torch.empty_like(w0[i]))
    gpu_lib.merge_batch([(w0[i], b[i], a[i], t.scale, outs[i]) for i, t in enumerate(tg)])
    torch.cuda.synchronize()
    for i in range(len(tg)):
        assert torch.equal(outs[i].view(torch.int16), one[i].view(torch.int16)), tg[i].name


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_inplace_merge_equals_pristine_merge(gpu_lib, dtype):
    """One in-place merge writes exactly what the merge from pristine writes."""
    t = synth.MergeTarget("inplace", 95, 0, 300, 520, 32, 64.0, dtype)
    W0 = t.make_w0()
    A, B = t.make_ab(0)
    a, b = to_dev(A), to_dev(B)
    ref = to_host(_merge(gpu_lib, to_dev(W0), a, b, t.scale))
    w = to_dev(W0)
    gpu_lib.merge_inplace(w, b, a, t.scale)
    import torch
    torch.cuda.synchronize()
    assert to_host(w).tobytes() == ref.tobytes()


def test_merge_unmerge_cycles_drift_but_pristine_does_not(gpu_lib):
    """Negative control for the pristine invariant: ten in-place merge +
    unmerge cycles (scale, then -scale) leave the bf16 base changed, while ten
    merges from pristine leave W0 bit-identical.  Reports the drift."""
    import torch
    t = LAYER0[0]
    W0 = t.make_w0()
    w = to_dev(W0)
    w0 = to_dev(W0)
    wi = torch.empty_like(w0)
    for cycle in range(10):
        A, B = t.make_ab(cycle)
        a, b = to_dev(A), to_dev(B)
        gpu_lib.merge_inplace(w, b, a, t.scale)
        gpu_lib.merge_inplace(w, b, a, -t.scale)
        gpu_lib.merge(w0, b, a, t.scale, out=wi)
    torch.cuda.synchronize()
    drifted = to_host(w)
    ulp = ulp_distance_bf16(drifted, W0)
    diff = np.abs(as_f64(drifted) - as_f64(W0))
    print(f"after 10 merge/unmerge cycles: {float((ulp > 0).mean()):.4f} of elements moved, "
          f"max {int(ulp.max())} ulp, max abs {diff.max():.3e}")
    assert (ulp > 0).any()                                  # the in-place path drifts
    assert to_host(w0).tobytes() == W0.tobytes()            # the pristine path does not


@pytest.mark.slow
def test_full_model_ten_cycles_through_merge_batch(gpu_lib):
    """The merge configuration at its own scale (unsloth commit log: base
    bit-identical across 10 perturb+refresh cycles): 36 layers x 7 targets,
    rank 32, ten cycles, each drawing a fresh adapter for every target (seed
    ids 10c+2, 10c+3) and merging all 252 targets in one lora_merge_batch
    call, the path the benchmark times.  Afterwards every W0 equals its
    device clone byte for byte, re-merging the cycle-0 adapters reproduces
    cycle 0's W_inf byte for byte, and cycle 0 of one target of each shape
    (layer 0) meets the oracle's per-element merge bar."""
    import torch
    rg = gpu_lib
    tg = synth.merge_targets(36)
    w0 = [synth.device_normal(t.group, t.case, synth.TW, (t.N, t.K), t.var_w0, "bf16") for t in tg]
    w0_clone = [w.clone() for w in w0]
    wi = [torch.empty_like(w) for w in w0]

    def adapters(cycle):
        a = [synth.device_normal(t.group, t.case, 10 * cycle + synth.TA, (t.r, t.K), 1.0 / t.K,
                                 "bf16") for t in tg]
        b = [synth.device_normal(t.group, t.case, 10 * cycle + synth.TB, (t.N, t.r), t.var_b,
                                 "bf16") for t in tg]
        return a, b

    first, ab0 = None, None
    for cycle in range(10):
        a, b = adapters(cycle)
        rg.merge_batch([(w0[i], b[i], a[i], t.scale, wi[i]) for i, t in enumerate(tg)])
        torch.cuda.synchronize()
        if cycle == 0:
            first = [w.clone() for w in wi]
            ab0 = (a, b)
        print(f"cycle {cycle}: 252 targets merged", flush=True)
    for i, t in enumerate(tg):
        assert torch.equal(w0[i].view(torch.int16), w0_clone[i].view(torch.int16)), t.name
    a, b = ab0
    rg.merge_batch([(w0[i], b[i], a[i], t.scale, wi[i]) for i, t in enumerate(tg)])
    torch.cuda.synchronize()
    for i, t in enumerate(tg):
        assert torch.equal(wi[i].view(torch.int16), first[i].view(torch.int16)), t.name
    for i in range(7):                                    # one target of each shape
        t = tg[i]
        W0h, Ah, Bh = to_host(w0[i]), to_host(a[i]), to_host(b[i])
        Wd, Wb = oracle.merge(W0h, Bh, Ah, t.scale)
        _check_bf16_merge(to_host(first[i]), Wd, Wb, W0h, Bh, Ah, t.scale, t.r, "cycle0 " + t.name)


def test_merge_unmerge_cycles_against_oracle_model(gpu_lib):
    """The in-place merge / unmerge negative control (unsloth commit log: the
    merge_adapter / unmerge path leaks about one bf16 ULP per cycle, the
    pristine restore none) against an oracle model of the same cycles.

    Each of the 20 in-place steps (W <- round(W + s B A), then
    W <- round(W - s B A), ten adapters) is checked element by element
    against the oracle applied to the GPU's own previous state: every
    element within the fp32-accumulation merge bound, at most 1 ULP from
    the correctly rounded value away from cancellation.  The whole chain is
    also run in the oracle alone (fp64 arithmetic, one bf16 rounding per
    step) from the same W0: the GPU's drift after each cycle is reported
    beside the model's and must match it up to the elements where an fp32
    rounding landed on the other side of a bf16 rounding boundary (about
    1e-4 of the elements per step, carried forward by later steps)."""
    import torch
    t = LAYER0[0]                                   # q: 4096 x 2560, rank 32
    W0 = t.make_w0()
    w = to_dev(W0)
    model = W0.copy()
    for cycle in range(10):
        A, B = t.make_ab(cycle)
        a, b = to_dev(A), to_dev(B)
        for step, s in (("merge", t.scale), ("unmerge", -t.scale)):
            prev = to_host(w)
            gpu_lib.merge_inplace(w, b, a, s)
            torch.cuda.synchronize()
            got = to_host(w)
            Wd, Wb = oracle.merge(prev, B, A, s)
            ok, delta = merge_within_fp32_bound(got, Wd, prev, B, A, s, t.r)
            ulp = ulp_distance_bf16(got, Wb)
            calm = delta < 0.25 * ulp_bf16_of(Wd)
            assert ok.all(), (cycle, step)
            assert int(ulp[calm].max()) <= 1, (cycle, step)
            model = oracle.merge(model, B, A, s, want_double=False)[1]
        drift_gpu = ulp_distance_bf16(got, W0)
        drift_model = ulp_distance_bf16(model, W0)
        diff = int((got != model).sum())
        print(f"cycle {cycle + 1}: moved gpu {float((drift_gpu > 0).mean()):.4f} "
              f"model {float((drift_model > 0).mean()):.4f}; mean ulp gpu "
              f"{float(drift_gpu.mean()):.3f} model {float(drift_model.mean()):.3f}; "
              f"max ulp gpu {int(drift_gpu.max())} model {int(drift_model.max())}; "
              f"elements differing from the model {diff}")
        assert abs(float((drift_gpu > 0).mean()) - float((drift_model > 0).mean())) < 1e-2
        assert diff <= 1e-2 * W0.size
    assert (drift_model > 0).any()                  # the model drifts too: the page's effect
