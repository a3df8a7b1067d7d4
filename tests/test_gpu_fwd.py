"""Parity of the HIP fused LoRA forward (tiled and decode kernels) against the
fp64 oracle, through the C ABI, on seeded inputs.

Bar: relative Frobenius error <= 1e-5 for fp32 inputs and <= 1e-2 for bf16
inputs (fp32 accumulate, bf16 output), per case; bitwise equality where the
exact result is representable (integer inputs) and where two calls must agree
(determinism, B = 0 versus scale = 0).
"""
import numpy as np
import pytest

import oracle
import synth
from helpers import TOL, as_f64, rel_fro, sample_rows, to_dev, to_host

pytestmark = pytest.mark.gpu


def _run(rg, t, scale, variant="auto"):
    import torch
    X, W, A, B = (to_dev(t[k]) for k in "XWAB")
    Y = rg.fwd(X, W, A, B, scale, variant=variant)
    torch.cuda.synchronize()
    return to_host(Y)


def _oracle_rows(t, scale, rows):
    """Oracle on selected output rows: row m of Y depends only on row m of X."""
    Xs = np.ascontiguousarray(t["X"][rows])
    return oracle.fwd(Xs, t["W"], t["A"], t["B"], scale)


def _case_name(c):
    return c.name


# ------------------------------------------------------------ the workloads

def test_tiny_fp32_full(gpu_lib):
    c = synth.TINY
    t = c.make()
    got = _run(gpu_lib, t, c.scale)
    ref = oracle.fwd(t["X"], t["W"], t["A"], t["B"], c.scale)
    err = rel_fro(got, ref)
    print(f"{c.name}: rel_fro={err:.3e}")
    assert err <= TOL["f32"]


def test_mid_bf16_full(gpu_lib):
    c = synth.MID
    t = c.make()
    got = _run(gpu_lib, t, c.scale)
    ref = oracle.fwd(t["X"], t["W"], t["A"], t["B"], c.scale)
    err = rel_fro(as_f64(got), ref)
    print(f"{c.name}: rel_fro={err:.3e}")
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("c", synth.DECODE, ids=_case_name)
@pytest.mark.parametrize("variant", ["decode", "tiled"])
def test_decode_shapes_full(gpu_lib, c, variant):
    t = c.make()
    got = _run(gpu_lib, t, c.scale, variant)
    ref = oracle.fwd(t["X"], t["W"], t["A"], t["B"], c.scale)
    err = rel_fro(as_f64(got), ref)
    print(f"{c.name} [{variant}]: rel_fro={err:.3e}")
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("c", [synth.QPROJ, synth.VPROJ], ids=_case_name)
def test_projection_sampled_rows(gpu_lib, c):
    t = c.make()
    got = _run(gpu_lib, t, c.scale)
    rows = sample_rows(c.M, 64, seed=c.case)
    ref = _oracle_rows(t, c.scale, rows)
    err = rel_fro(as_f64(got[rows]), ref)
    print(f"{c.name}: rows={len(rows)} rel_fro={err:.3e}")
    assert err <= TOL["bf16"]
    assert np.isfinite(as_f64(got)).all()


@pytest.mark.slow
@pytest.mark.parametrize("c", synth.SQUARE, ids=_case_name)
def test_square_rank_sweep_sampled_rows(gpu_lib, c):
    t = c.make()
    got = _run(gpu_lib, t, c.scale)
    rows = sample_rows(c.M, 24, seed=c.case)
    ref = _oracle_rows(t, c.scale, rows)
    err = rel_fro(as_f64(got[rows]), ref)
    print(f"{c.name}: rows={len(rows)} rel_fro={err:.3e}")
    assert err <= TOL["bf16"]
    assert np.isfinite(as_f64(got)).all()


@pytest.mark.parametrize("M,N,K,r", [(4097, 4100, 264, 100), (4096, 4096, 136, 128)])
def test_large_rank_groups_sampled_rows(gpu_lib, M, N, K, r):
    """Large ranks on 128 x 128 tiles where a workgroup computes T once for a
    group of N tiles: ragged M and N (the last group runs past N), ranks below
    the padded rank, checked on sampled rows against the oracle."""
    c = synth.FwdCase(f"grp{M}x{N}r{r}", 94, r, M, N, K, r, 2.0 * r, "bf16")
    t = c.make()
    got = _run(gpu_lib, t, c.scale)
    rows = sample_rows(M, 32, seed=r)
    ref = _oracle_rows(t, c.scale, rows)
    err = rel_fro(as_f64(got[rows]), ref)
    print(f"{c.name}: rows={len(rows)} rel_fro={err:.3e}")
    assert err <= TOL["bf16"]
    assert np.isfinite(as_f64(got)).all()


@pytest.mark.parametrize("M,N,K,r", [(256, 4096, 4096, 16), (1000, 1024, 2056, 40),
                                     (512, 1032, 1024, 32), (64, 4096, 4096, 64),
                                     (40, 2048, 2048, 24)])
def test_small_grid_loader_tiles_sampled_rows(gpu_lib, M, N, K, r):
    """Grids with few 128 x 128 tiles run on the 64 x 64, 64 x 32 and 32 x 32
    tiles with loader waves (W streamed by many workgroups): full size,
    ragged N and K, ranks below the padded rank, sampled rows against the
    oracle, and the same result on a second call."""
    c = synth.FwdCase(f"small{M}x{N}x{K}r{r}", 95, r, M, N, K, r, 2.0 * r, "bf16")
    t = c.make()
    got = _run(gpu_lib, t, c.scale)
    again = _run(gpu_lib, t, c.scale)
    rows = sample_rows(M, 32, seed=r)
    ref = _oracle_rows(t, c.scale, rows)
    err = rel_fro(as_f64(got[rows]), ref)
    print(f"{c.name}: rows={len(rows)} rel_fro={err:.3e}")
    assert err <= TOL["bf16"]
    assert np.isfinite(as_f64(got)).all()
    assert np.array_equal(got, again)


# ------------------------------------------------------ shapes and edges

def _rand_case(seed, M, N, K, r, dtype, var_b=0.02):
    return synth.FwdCase(f"edge{seed}", 90, seed, M, N, K, r, 2.0 * r, dtype, var_b=var_b).make()


EDGE = [
    # M, N, K, r, dtype, variant
    (1, 1, 8, 1, "bf16", "tiled"),
    (1, 1, 8, 1, "bf16", "decode"),
    (3, 17, 24, 5, "bf16", "tiled"),
    (3, 17, 24, 5, "bf16", "decode"),
    (200, 300, 520, 7, "bf16", "tiled"),
    (129, 130, 136, 17, "bf16", "tiled"),
    (64, 100, 1000, 33, "bf16", "tiled"),
    (77, 64, 64, 100, "bf16", "tiled"),
    (130, 260, 72, 256, "bf16", "tiled"),
    (257, 129, 200, 128, "bf16", "tiled"),
    (40, 97, 264, 20, "bf16", "tiled"),         # tall tiles: ragged N, rank 20
    (64, 4100, 2056, 32, "bf16", "tiled"),
    (33, 4100, 2056, 16, "bf16", "decode"),
    (64, 513, 4104, 32, "bf16", "decode"),
    (17, 513, 4104, 20, "bf16", "decode"),
    (5, 7, 12, 3, "f32", "tiled"),
    (65, 70, 516, 20, "f32", "tiled"),
    (130, 129, 64, 256, "f32", "tiled"),
]


@pytest.mark.parametrize("M,N,K,r,dtype,variant", EDGE)
def test_ragged_shapes(gpu_lib, M, N, K, r, dtype, variant):
    t = _rand_case(M * 7 + N, M, N, K, r, dtype)
    s = 2.0
    got = _run(gpu_lib, t, s, variant)
    ref = oracle.fwd(t["X"], t["W"], t["A"], t["B"], s)
    err = rel_fro(as_f64(got), ref)
    print(f"M{M} N{N} K{K} r{r} {dtype} {variant}: rel_fro={err:.3e}")
    assert err <= TOL[dtype]


@pytest.mark.parametrize("dtype,variant", [("bf16", "tiled"), ("bf16", "decode"), ("f32", "tiled")])
def test_padded_leading_dimensions(gpu_lib, dtype, variant):
    import torch
    M, N, K, r = 40, 72, 200, 12
    t = _rand_case(5, M, N, K, r, dtype)
    pad = {"X": 24, "W": 8, "A": 16, "B": 3}
    dev = {}
    for k, p in pad.items():
        a = to_dev(t[k])
        big = torch.zeros((a.shape[0], a.shape[1] + p), dtype=a.dtype, device=a.device)
        big[:, : a.shape[1]] = a
        dev[k] = big[:, : a.shape[1]]
        assert dev[k].stride(0) == a.shape[1] + p
    Ybig = torch.full((M, N + 5), float("nan"), dtype=dev["X"].dtype, device=dev["X"].device)
    Y = Ybig[:, :N]
    gpu_lib.fwd(dev["X"], dev["W"], dev["A"], dev["B"], 1.5, out=Y, variant=variant)
    torch.cuda.synchronize()
    got = to_host(Ybig)
    ref = oracle.fwd(t["X"], t["W"], t["A"], t["B"], 1.5)
    assert rel_fro(as_f64(got[:, :N]), ref) <= TOL[dtype]
    assert np.isnan(as_f64(got[:, N:])).all()          # padding columns untouched


@pytest.mark.parametrize("dtype,variant", [("bf16", "tiled"), ("bf16", "decode"), ("f32", "tiled")])
def test_k_zero_gives_zero(gpu_lib, dtype, variant):
    import torch
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    M, N, r = 9, 33, 4
    X = torch.empty((M, 0), dtype=tdt, device="cuda")
    W = torch.empty((N, 0), dtype=tdt, device="cuda")
    A = torch.empty((r, 0), dtype=tdt, device="cuda")
    B = torch.randn((N, r), device="cuda").to(tdt)
    Y = torch.full((M, N), 7.0, dtype=tdt, device="cuda")
    gpu_lib.fwd(X, W, A, B, 2.0, out=Y, variant=variant)
    torch.cuda.synchronize()
    assert (Y == 0).all().item()


@pytest.mark.parametrize("dtype,variant", [("bf16", "tiled"), ("bf16", "decode"), ("f32", "tiled")])
def test_b_zero_equals_scale_zero_and_base(gpu_lib, dtype, variant):
    """B = 0 and scale = 0 both leave exactly the base product (bitwise the
    same output), which matches the oracle's X W^T."""
    M, N, K, r = 48, 96, 320, 16
    t = _rand_case(11, M, N, K, r, dtype)
    tz = dict(t)
    tz["B"] = np.zeros_like(t["B"])
    y_b0 = _run(gpu_lib, tz, 2.0, variant)
    y_s0 = _run(gpu_lib, t, 0.0, variant)
    np.testing.assert_array_equal(y_b0, y_s0)
    base = oracle.fwd(t["X"], t["W"], t["A"][:0], t["B"][:, :0], 1.0)
    assert rel_fro(as_f64(y_b0), base) <= TOL[dtype]


@pytest.mark.parametrize("dtype,variant", [("bf16", "tiled"), ("bf16", "decode"), ("f32", "tiled")])
def test_w_zero_isolates_lora_path(gpu_lib, dtype, variant):
    M, N, K, r = 40, 80, 264, 16
    t = _rand_case(12, M, N, K, r, dtype, var_b=1.0)
    t["W"] = np.zeros_like(t["W"])
    got = _run(gpu_lib, t, 2.0, variant)
    ref = oracle.fwd(t["X"], t["W"], t["A"], t["B"], 2.0)
    err = rel_fro(as_f64(got), ref)
    print(f"W=0 {dtype} {variant}: rel_fro={err:.3e}")
    assert err <= TOL[dtype]


INT_CASES = [
    # M, N, K, r, scale, dtype, variant
    (67, 130, 200, 2, 2.0, "bf16", "tiled"),
    (130, 67, 256, 5, 0.5, "bf16", "tiled"),
    (64, 70, 136, 1, 1.0, "bf16", "decode"),
    (61, 70, 136, 2, 2.0, "bf16", "tiled"),
    (9, 33, 256, 3, 2.0, "bf16", "decode"),
    (67, 130, 200, 2, 2.0, "f32", "tiled"),
]


@pytest.mark.parametrize("M,N,K,r,s,dtype,variant", INT_CASES)
def test_integer_inputs_bitwise(gpu_lib, M, N, K, r, s, dtype, variant):
    """Inputs in {-1, 0, 1}, K <= 256: every partial sum and s*T is exact, so
    the GPU result must be the exact value rounded once (bitwise)."""
    rng = np.random.default_rng(M * 1000 + N)
    ints = {k: rng.integers(-1, 2, shp).astype(np.float32)
            for k, shp in (("X", (M, K)), ("W", (N, K)), ("A", (r, K)), ("B", (N, r)))}
    if dtype == "bf16":
        t = {k: synth.f32_to_bf16_bits(v) for k, v in ints.items()}
    else:
        t = ints
    got = _run(gpu_lib, t, s, variant)
    ref = oracle.fwd(t["X"], t["W"], t["A"], t["B"], s)
    if dtype == "bf16":
        np.testing.assert_array_equal(got, oracle.round_bf16(ref))
    else:
        np.testing.assert_array_equal(got.astype(np.float64), ref)


@pytest.mark.parametrize("c", [synth.MID, synth.DECODE[2], synth.TINY], ids=_case_name)
def test_deterministic(gpu_lib, c):
    t = c.make()
    a = _run(gpu_lib, t, c.scale)
    b = _run(gpu_lib, t, c.scale)
    np.testing.assert_array_equal(a, b)


def test_fwd_matches_merged_weight_forward(gpu_lib):
    """X (W + s B A)^T on the merged weight gives the same layer output as the
    fused forward (two GPU results compared with each other; each of the two
    exports is checked against the oracle elsewhere)."""
    import torch
    M, N, K, r = 256, 512, 512, 32
    t = _rand_case(13, M, N, K, r, "bf16")
    X, W, A, B = (to_dev(t[k]) for k in "XWAB")
    y_fused = gpu_lib.fwd(X, W, A, B, 2.0)
    W_inf = gpu_lib.merge(W, B, A, 2.0)
    y_merged = gpu_lib.fwd(X, W_inf, A, B, 0.0)
    torch.cuda.synchronize()
    assert rel_fro(as_f64(to_host(y_fused)), as_f64(to_host(y_merged))) <= 1e-2
