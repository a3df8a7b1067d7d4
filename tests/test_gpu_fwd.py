"""Parity of the HIP fused LoRA forward (tiled and decode kernels) against the
fp64 oracle, through the C ABI, on seeded inputs.

Bar: relative Frobenius error <= 1e-5 for fp32 inputs and <= 1e-2 for bf16
inputs (fp32 accumulate, bf16 output), per case, AND every checked element
within the worst-case bound of the kernels' arithmetic (tests/helpers.py:
fp32 sums, s T rounded once to bf16, one output rounding), so that one wrong
MFMA block cannot hide in a norm; bitwise equality where the exact result is
representable (integer inputs) and where two calls must agree (determinism,
B = 0 versus scale = 0).  Full outputs up to the projection shapes; on the
16384-token square one row of every 16-row block (the oracle computes rows
one by one).  The default path goes through the lora_fwd entry point.
"""
import numpy as np
import pytest

import oracle
import synth
from helpers import (TOL, as_f64, block_rows, check_fwd_elements, rel_fro, to_dev,
                     to_host)

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


def _check(name, got, ref, t, scale, dtype, rows=None):
    """rel_fro and the per-element bound on output rows `rows` (all if None)."""
    X = t["X"] if rows is None else np.ascontiguousarray(t["X"][rows])
    g = got if rows is None else got[rows]
    err = rel_fro(as_f64(g), ref)
    ratio = check_fwd_elements(g, ref, X, t["W"], t["A"], t["B"], scale, dtype, name)
    print(f"{name}: rows={g.shape[0]} rel_fro={err:.3e} worst/bound={ratio:.3f}")
    assert err <= TOL[dtype]
    return err


# ------------------------------------------------------------ the workloads

def test_tiny_fp32_full(gpu_lib):
    c = synth.TINY
    t = c.make()
    got = _run(gpu_lib, t, c.scale)
    ref = oracle.fwd(t["X"], t["W"], t["A"], t["B"], c.scale)
    _check(c.name, got, ref, t, c.scale, "f32")


def test_mid_bf16_full(gpu_lib):
    c = synth.MID
    t = c.make()
    got = _run(gpu_lib, t, c.scale)
    ref = oracle.fwd(t["X"], t["W"], t["A"], t["B"], c.scale)
    _check(c.name, got, ref, t, c.scale, "bf16")


@pytest.mark.parametrize("c", synth.DECODE, ids=_case_name)
@pytest.mark.parametrize("variant", ["decode", "tiled"])
def test_decode_shapes_full(gpu_lib, c, variant):
    t = c.make()
    got = _run(gpu_lib, t, c.scale, variant)
    ref = oracle.fwd(t["X"], t["W"], t["A"], t["B"], c.scale)
    _check(f"{c.name} [{variant}]", got, ref, t, c.scale, "bf16")


@pytest.mark.parametrize("c", [synth.QPROJ, synth.VPROJ], ids=_case_name)
def test_projection_full(gpu_lib, c):
    """The q_proj and v_proj workloads (8192 tokens, hidden 2560, r 32),
    every output element."""
    t = c.make()
    got = _run(gpu_lib, t, c.scale)
    ref = oracle.fwd(t["X"], t["W"], t["A"], t["B"], c.scale)
    _check(c.name, got, ref, t, c.scale, "bf16")


@pytest.mark.slow
@pytest.mark.parametrize("c", synth.SQUARE, ids=_case_name)
def test_square_rank_sweep_block_rows(gpu_lib, c):
    """The 16384 x 8192 x 8192 square at each rank, in the launch
    configuration the benchmark times: one row of every 16-row block (every
    M tile and every MFMA row block of every tile), all 8192 columns."""
    t = c.make()
    got = _run(gpu_lib, t, c.scale)
    rows = block_rows(c.M, 16, seed=c.case)
    ref = _oracle_rows(t, c.scale, rows)
    _check(c.name, got, ref, t, c.scale, "bf16", rows)
    assert np.isfinite(as_f64(got)).all()


@pytest.mark.parametrize("M,N,K,r", [(4097, 4100, 264, 100), (4096, 4096, 136, 128)])
def test_large_rank_groups_full(gpu_lib, M, N, K, r):
    """Large ranks on 128 x 128 tiles where a workgroup computes T once for a
    group of N tiles: ragged M and N (the last group runs past N), ranks below
    the padded rank, every output element against the oracle."""
    c = synth.FwdCase(f"grp{M}x{N}r{r}", 94, r, M, N, K, r, 2.0 * r, "bf16")
    t = c.make()
    got = _run(gpu_lib, t, c.scale)
    ref = oracle.fwd(t["X"], t["W"], t["A"], t["B"], c.scale)
    _check(c.name, got, ref, t, c.scale, "bf16")


@pytest.mark.parametrize("M,N,K,r", [(256, 4096, 4096, 16), (1000, 1024, 2056, 40),
                                     (512, 1032, 1024, 32), (64, 4096, 4096, 64),
                                     (40, 2048, 2048, 24)])
def test_small_grid_loader_tiles_full(gpu_lib, M, N, K, r):
    """Grids with few 128 x 128 tiles run on the 64 x 64, 64 x 32 and 32 x 32
    tiles with loader waves (W streamed by many workgroups): ragged N and K,
    ranks below the padded rank, every element against the oracle, and the
    same result on a second call."""
    c = synth.FwdCase(f"small{M}x{N}x{K}r{r}", 95, r, M, N, K, r, 2.0 * r, "bf16")
    t = c.make()
    got = _run(gpu_lib, t, c.scale)
    again = _run(gpu_lib, t, c.scale)
    ref = oracle.fwd(t["X"], t["W"], t["A"], t["B"], c.scale)
    _check(c.name, got, ref, t, c.scale, "bf16")
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
    (1, 4100, 2056, 32, "bf16", "decode"),      # one token: ragged N, K not a multiple of 64
    (1, 33, 520, 17, "bf16", "decode"),
    (1, 17, 8, 9, "bf16", "decode"),
    (5, 7, 12, 3, "f32", "tiled"),
    (65, 70, 516, 20, "f32", "tiled"),
    (130, 129, 64, 256, "f32", "tiled"),
    (1030, 1030, 72, 20, "f32", "tiled"),       # 64 x 64 fp32 tiles (>= 128 of them), ragged
]


@pytest.mark.parametrize("M,N,K,r,dtype,variant", EDGE)
def test_ragged_shapes(gpu_lib, M, N, K, r, dtype, variant):
    t = _rand_case(M * 7 + N, M, N, K, r, dtype)
    s = 2.0
    got = _run(gpu_lib, t, s, variant)
    ref = oracle.fwd(t["X"], t["W"], t["A"], t["B"], s)
    _check(f"M{M} N{N} K{K} r{r} {dtype} {variant}", got, ref, t, s, dtype)


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
    _check(f"padded {dtype} {variant}", np.ascontiguousarray(got[:, :N]), ref, t, 1.5, dtype)
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
    assert np.array_equal(base, oracle.fwd(tz["X"], tz["W"], tz["A"], tz["B"], 2.0))
    _check(f"B=0 {dtype} {variant}", y_b0, base, tz, 2.0, dtype)


@pytest.mark.parametrize("dtype,variant", [("bf16", "tiled"), ("bf16", "decode"), ("f32", "tiled")])
def test_w_zero_isolates_lora_path(gpu_lib, dtype, variant):
    M, N, K, r = 40, 80, 264, 16
    t = _rand_case(12, M, N, K, r, dtype, var_b=1.0)
    t["W"] = np.zeros_like(t["W"])
    got = _run(gpu_lib, t, 2.0, variant)
    ref = oracle.fwd(t["X"], t["W"], t["A"], t["B"], 2.0)
    _check(f"W=0 {dtype} {variant}", got, ref, t, 2.0, dtype)


INT_CASES = [
    # M, N, K, r, scale, dtype, variant
    (67, 130, 200, 2, 2.0, "bf16", "tiled"),
    (130, 67, 256, 5, 0.5, "bf16", "tiled"),
    (64, 70, 136, 1, 1.0, "bf16", "decode"),
    (61, 70, 136, 2, 2.0, "bf16", "tiled"),
    (9, 33, 256, 3, 2.0, "bf16", "decode"),
    (1, 70, 200, 3, 2.0, "bf16", "decode"),
    (1, 33, 256, 20, 0.5, "bf16", "decode"),
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


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_fwd_matches_fp64_gemm_on_gpu_merged_weight(gpu_lib, dtype):
    """The merged-form identity tying the two exports together: the fused
    lora_fwd agrees with a plain fp64 GEMM of X against the W_inf that
    lora_merge wrote on the GPU (Y = X (W + s B A)^T), within the
    configuration's bar (1e-5 fp32, 1e-2 bf16)."""
    import torch
    M, N, K, r = 512, 1024, 1024, 32
    t = _rand_case(13, M, N, K, r, dtype)
    X, W, A, B = (to_dev(t[k]) for k in "XWAB")
    y_fused = to_host(gpu_lib.fwd(X, W, A, B, 2.0))
    W_inf = to_host(gpu_lib.merge(W, B, A, 2.0))
    torch.cuda.synchronize()
    ref = as_f64(t["X"]) @ as_f64(W_inf).T          # numpy float64 GEMM
    err = rel_fro(as_f64(y_fused), ref)
    print(f"fused vs X W_inf^T ({dtype}): rel_fro={err:.3e}")
    assert err <= TOL[dtype]


@pytest.mark.parametrize("M,r", [(1, 20), (8, 12), (16, 28)])
def test_decode_b_ending_at_its_last_element(gpu_lib, M, r):
    """Ragged rank with 16-B aligned B rows (ldb % 8 == 0): B is a view whose
    storage ends exactly at element (N - 1) ldb + r, so no 16-B read of a
    row may reach past column r.  Every element within the bound."""
    import torch
    N, K = 1000, 1024
    ldb = (r + 7) // 8 * 8                     # 16-B aligned rows, r % 8 != 0
    c = synth.FwdCase(f"bend_m{M}_r{r}", 97, M * 100 + r, M, N, K, r, 2.0 * r, "bf16")
    t = c.make()
    flat = torch.zeros((N - 1) * ldb + r, dtype=torch.bfloat16, device="cuda")
    B = flat.as_strided((N, r), (ldb, 1))
    B.copy_(to_dev(t["B"]))
    X, W, A = (to_dev(t[k]) for k in "XWA")
    assert gpu_lib.fwd_pick(gpu_lib.LORA_BF16, M, N, K, r) == 2      # the decode kernel
    got = to_host(gpu_lib.fwd(X, W, A, B, c.scale))
    torch.cuda.synchronize()
    ref = oracle.fwd(t["X"], t["W"], t["A"], t["B"], c.scale)
    _check(c.name, got, ref, t, c.scale, "bf16")


@pytest.mark.parametrize("c", [synth.MID, synth.DECODE[0], synth.TINY], ids=_case_name)
def test_lora_fwd_entry_point_raw(gpu_lib, c):
    """The lora_fwd symbol called with raw device pointers and the stream
    handle, as a C caller would, against the oracle."""
    import torch
    rg = gpu_lib
    t = c.make()
    X, W, A, B = (to_dev(t[k]) for k in "XWAB")
    Y = torch.full((c.M, c.N), float("nan"), dtype=X.dtype, device="cuda")
    dt = rg.LORA_BF16 if c.dtype == "bf16" else rg.LORA_F32
    st = rg.lib().lora_fwd(dt, c.M, c.N, c.K, c.r, X.data_ptr(), c.K, W.data_ptr(), c.K,
                           A.data_ptr(), c.K, B.data_ptr(), c.r, c.scale, Y.data_ptr(), c.N,
                           torch.cuda.current_stream().cuda_stream)
    assert st == rg.LORA_OK, rg.status_str(st)
    torch.cuda.synchronize()
    ref = oracle.fwd(t["X"], t["W"], t["A"], t["B"], c.scale)
    _check("lora_fwd raw " + c.name, to_host(Y), ref, t, c.scale, c.dtype)


LORA_MAX_LD = (1 << 22) - 8   # include/lora.h


@pytest.mark.parametrize("dtype,r,tile", [("bf16", 8, None), ("bf16", 8, 4), ("bf16", 8, 18),
                                          ("bf16", 256, None), ("f32", 128, None)])
def test_largest_leading_dimensions(gpu_lib, dtype, r, tile):
    """ldx = ldw = lda = LORA_MAX_LD, the largest the C ABI accepts, where a
    256-row tile of X or W (bf16) and r rows of A (bf16 at r 256, fp32 at r
    128) each span 2^31 - 4096 or 2^31 - 16384 bytes: just inside the
    kernels' signed 32-bit buffer ranges.  Ragged 300 x 300 output (two row
    and two column tiles of 256), every element against the oracle; tiles 4
    and 18 are the 256 x 256 configurations, forced through lora_fwd_tile."""
    import torch
    M, N, K = 300, 300, 64
    t = _rand_case(8, M, N, K, r, dtype)
    ld = LORA_MAX_LD
    big = {}
    for k in "XWA":
        a = to_dev(t[k])
        b = torch.zeros((a.shape[0], ld), dtype=a.dtype, device=a.device)
        b[:, :K] = a
        big[k] = b
    B = to_dev(t["B"])
    Y = torch.full((M, N), float("nan"), dtype=B.dtype, device=B.device)
    scale = 2.0
    if tile is None:
        gpu_lib.fwd(big["X"][:, :K], big["W"][:, :K], big["A"][:, :K], B, scale, out=Y)
    else:
        st = gpu_lib.fwd_tile_raw(tile, gpu_lib.LORA_BF16, M, N, K, r, big["X"].data_ptr(), ld,
                                  big["W"].data_ptr(), ld, big["A"].data_ptr(), ld, B.data_ptr(),
                                  r, scale, Y.data_ptr(), N,
                                  torch.cuda.current_stream().cuda_stream)
        assert st == 0, st
    torch.cuda.synchronize()
    del big
    got = to_host(Y)
    ref = oracle.fwd(t["X"], t["W"], t["A"], t["B"], scale)
    _check(f"max ld {dtype} r{r} tile {tile}", got, ref, t, scale, dtype)


@pytest.mark.parametrize("M,N,K,r,dtype,variant", [(130, 200, 264, 20, "bf16", "tiled"),
                                                   (4, 300, 136, 16, "bf16", "decode"),
                                                   (1, 300, 136, 32, "bf16", "decode"),
                                                   (70, 90, 100, 12, "f32", "tiled")])
def test_nan_and_inf_propagate(gpu_lib, M, N, K, r, dtype, variant):
    """A NaN in X[m0, k0], +Inf in W[n1, k1] and a NaN in B[n2, j2] (j2 < r)
    give what the fp64 oracle gives: row m0 and column n2 NaN, column n1 +-Inf
    with the oracle's signs (NaN at m0), and every other element within the
    per-element bound of the arithmetic (those touch no special value)."""
    import torch
    t = _rand_case(9, M, N, K, r, dtype)
    X, W, B = t["X"].copy(), t["W"].copy(), t["B"].copy()
    m0, k0, n1, k1, n2, j2 = M // 2, K // 3, N // 4, K - 1, N - 2, r - 1
    if dtype == "bf16":          # bf16 operands are held as their bit patterns
        nan, inf = np.uint16(0x7FC0), np.uint16(0x7F80)
    else:
        nan, inf = np.float32(np.nan), np.float32(np.inf)
    X[m0, k0] = nan
    W[n1, k1] = inf
    B[n2, j2] = nan
    scale = 2.0
    Xd, Wd, Ad, Bd = to_dev(X), to_dev(W), to_dev(t["A"]), to_dev(B)
    Y = gpu_lib.fwd(Xd, Wd, Ad, Bd, scale, variant=variant)
    torch.cuda.synchronize()
    got = as_f64(to_host(Y))
    ref = oracle.fwd(X, W, t["A"], B, scale)
    assert np.isnan(ref[m0]).all() and np.isnan(ref[:, n2]).all()
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(np.isinf(got), np.isinf(ref))
    inf = np.isinf(ref)
    assert inf[:, n1].sum() == M - 1
    assert np.array_equal(np.sign(got[inf]), np.sign(ref[inf]))
    rows = [m for m in range(M) if m != m0]
    cols = [n for n in range(N) if n not in (n1, n2)]
    g = np.ascontiguousarray(to_host(Y)[np.ix_(rows, cols)])
    rs = np.ascontiguousarray(ref[np.ix_(rows, cols)])
    ratio = check_fwd_elements(g, rs, np.ascontiguousarray(X[rows]), np.ascontiguousarray(W[cols]),
                               t["A"], np.ascontiguousarray(B[cols]), scale, dtype,
                               f"special {dtype} {variant}")
    assert rel_fro(as_f64(g), rs) <= TOL[dtype]
    print(f"special values {dtype} {variant}: worst/bound={ratio:.3f}")
