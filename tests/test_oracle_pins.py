"""Pins for the fp64 oracle, independent of the oracle's own code.

Each test ties the oracle to something it does not compute itself: hand-worked
examples, closed forms of the definition, a literal brute-force transcription
of the definition, numpy's float64 products, integer arithmetic, and torch's
float32 -> bf16 conversion.  A dropped term, a wrong sign, a transposed
operand or a misplaced scale fails at least one of them:

* dropped LoRA term / misplaced scale: W=0 case, scale-linearity, golden;
* wrong sign or index: golden, brute force, integer exactness;
* transposed operand (A vs A^T, B vs B^T): non-square shapes everywhere;
* double rounding in the merge's bf16 step: explicit tie cases.

Definitions pinned (page titles as published): "fastaf: Minimal LoRA
fine-tuning with hand-written Triton kernels", section "FWD kernel speedup";
unsloth commit log for scripts/benchmarks/qwen3_flex_inference.py, the entry
that replaces copy+merge_adapter by one addmm from the pristine copy.
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f32(a):
    return np.asarray(a, dtype=np.float32)


def _rel_fro(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / nb if nb else np.linalg.norm(a)


def _rand_case(rng, M, N, K, r, dtype="f32", scale=None):
    X = rng.standard_normal((M, K)).astype(np.float32)
    W = (rng.standard_normal((N, K)) / np.sqrt(max(K, 1))).astype(np.float32)
    A = (rng.standard_normal((r, K)) / np.sqrt(max(K, 1))).astype(np.float32)
    B = (rng.standard_normal((N, r)) * 0.15).astype(np.float32)
    if dtype == "bf16":
        X, W, A, B = (synth.f32_to_bf16_bits(t) for t in (X, W, A, B))
    s = np.float32(rng.uniform(0.25, 3.0) if scale is None else scale)
    return X, W, A, B, s


# ---------------------------------------------------------------- golden

def test_golden_hand_worked_forward_and_merge():
    with open(os.path.join(GOLDEN, "fwd_worked_examples.json")) as f:
        data = json.load(f)
    for c in data["cases"]:
        X, W, A, B = (_f32(c[k]) for k in "XWAB")
        Y = oracle.fwd(X, W, A, B, c["scale"])
        np.testing.assert_array_equal(Y, np.asarray(c["Y"], np.float64), err_msg=c["name"])
        Wd, _ = oracle.merge(W, B, A, c["scale"], want_bf16=False)
        np.testing.assert_array_equal(Wd, np.asarray(c["W_inf"], np.float64), err_msg=c["name"])
        # the same case in bf16 storage (every value is exact in bf16)
        Yb = oracle.fwd(*(synth.f32_to_bf16_bits(t) for t in (X, W, A, B)), c["scale"])
        np.testing.assert_array_equal(Yb, Y)


# ---------------------------------------------------------- brute force

def _brute_force_fwd(X, W, A, B, s):
    """Literal transcription of out = X W^T + ((X A^T) B^T) * s, one element at a
    time in pure Python floats (IEEE double), sums in ascending index order."""
    M, K = len(X), len(X[0]) if len(X) else 0
    N, r = len(W), len(A)
    T = [[sum((X[m][k] * A[j][k] for k in range(K)), 0.0) for j in range(r)] for m in range(M)]
    out = []
    for m in range(M):
        row = []
        for n in range(N):
            base = 0.0
            for k in range(K):
                base += X[m][k] * W[n][k]
            low = 0.0
            for j in range(r):
                low += T[m][j] * B[n][j]
            row.append(base + float(s) * low)
        out.append(row)
    return out


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_brute_force_tiny_shapes_bitwise(dtype):
    rng = np.random.default_rng(1234)
    sizes = (1, 2, 3, 5, 8, 17)
    for M, N, K in itertools.product(sizes, sizes, sizes):
        r = int(rng.choice([1, 2, 3, 8, 16]))
        X, W, A, B, s = _rand_case(rng, M, N, K, r, dtype)
        Xd, Wd, Ad, Bd = (synth.to_f64(t).tolist() for t in (X, W, A, B))
        ref = np.asarray(_brute_force_fwd(Xd, Wd, Ad, Bd, s))
        got = oracle.fwd(X, W, A, B, s)
        # same operations in the same order, no contraction: bitwise equal
        np.testing.assert_array_equal(got, ref, err_msg=f"M{M} N{N} K{K} r{r}")


def test_entries_match_rows_bitwise():
    rng = np.random.default_rng(7)
    X, W, A, B, s = _rand_case(rng, 37, 29, 41, 5, "bf16")
    full = oracle.fwd(X, W, A, B, s)
    ms = rng.integers(0, 37, 200)
    ns = rng.integers(0, 29, 200)
    np.testing.assert_array_equal(oracle.fwd_entries(X, W, A, B, s, ms, ns), full[ms, ns])
    part = oracle.fwd(X, W, A, B, s, rows=(5, 19))
    np.testing.assert_array_equal(part, full[5:19])


# ------------------------------------------------------------ closed forms

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_b_zero_and_s_zero_give_base_exactly(dtype):
    """B = 0 (or s = 0): the LoRA term is exactly 0.0, Y == X W^T bitwise."""
    rng = np.random.default_rng(3)
    X, W, A, B, s = _rand_case(rng, 19, 23, 70, 4, dtype)
    Bz = np.zeros_like(B)
    base = oracle.fwd(X, W, A[:0], B[:, :0], 1.0)          # r = 0: plain X W^T
    np.testing.assert_array_equal(oracle.fwd(X, W, A, Bz, s), base)
    np.testing.assert_array_equal(oracle.fwd(X, W, A, B, 0.0), base)
    # and the plain product agrees with numpy's float64 matmul
    ref = synth.to_f64(X) @ synth.to_f64(W).T
    assert _rel_fro(base, ref) < 1e-13


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_w_zero_isolates_lora_path(dtype):
    """W = 0: Y = s (X A^T) B^T, so the base cannot mask a LoRA-path error."""
    rng = np.random.default_rng(4)
    X, W, A, B, s = _rand_case(rng, 21, 13, 50, 6, dtype)
    Wz = np.zeros_like(W)
    got = oracle.fwd(X, Wz, A, B, s)
    x, a, b = (synth.to_f64(t) for t in (X, A, B))
    ref = float(s) * ((x @ a.T) @ b.T)
    assert _rel_fro(got, ref) < 1e-13


def test_scale_enters_linearly():
    """Y(s) - Y(0) = s * L for two different s (a scale applied twice, or to
    the base, breaks this)."""
    rng = np.random.default_rng(5)
    X, W, A, B, _ = _rand_case(rng, 9, 11, 33, 3, "f32")
    y0 = oracle.fwd(X, W, A, B, 0.0)
    y1 = oracle.fwd(X, W, A, B, 1.0)
    y3 = oracle.fwd(X, W, A, B, 3.0)
    np.testing.assert_allclose(y3 - y0, 3.0 * (y1 - y0), rtol=1e-12, atol=1e-12)


def test_merged_form_identity():
    """X (W + s B A)^T equals the fused forward (the merged layer computes the
    same function; the commit log's merged short-circuit relies on it)."""
    rng = np.random.default_rng(6)
    for dtype in ("f32", "bf16"):
        X, W, A, B, s = _rand_case(rng, 31, 45, 64, 8, dtype)
        Wd, _ = oracle.merge(W, B, A, s, want_bf16=False)
        merged = synth.to_f64(X) @ Wd.T
        assert _rel_fro(oracle.fwd(X, W, A, B, s), merged) < 1e-12


def test_integer_inputs_exact():
    """Inputs in {-1, 0, 1} and an integer scale: every value is an integer,
    so the oracle must equal int64 arithmetic exactly (non-square shapes)."""
    rng = np.random.default_rng(8)
    for (M, N, K, r) in [(7, 5, 32, 2), (3, 17, 9, 1), (16, 16, 31, 3)]:
        Xi = rng.integers(-1, 2, (M, K))
        Wi = rng.integers(-1, 2, (N, K))
        Ai = rng.integers(-1, 2, (r, K))
        Bi = rng.integers(-1, 2, (N, r))
        s = 2
        ref = Xi @ Wi.T + s * ((Xi @ Ai.T) @ Bi.T)
        got = oracle.fwd(*(t.astype(np.float32) for t in (Xi, Wi, Ai, Bi)), float(s))
        np.testing.assert_array_equal(got, ref.astype(np.float64))
        Wd, Wb = oracle.merge(Wi.astype(np.float32), Bi.astype(np.float32),
                              Ai.astype(np.float32), float(s))
        np.testing.assert_array_equal(Wd, (Wi + s * (Bi @ Ai)).astype(np.float64))


# --------------------------------------------------- library cross-checks

@pytest.mark.parametrize("case", [synth.TINY, synth.MID], ids=lambda c: c.name)
def test_numpy_cross_check_on_workloads(case):
    t = case.make()
    rows = (0, case.M) if case.M <= 256 else (1000, 1096)
    got = oracle.fwd(t["X"], t["W"], t["A"], t["B"], case.scale, rows=rows)
    x, w, a, b = (synth.to_f64(t[k]) for k in "XWAB")
    x = x[rows[0]:rows[1]]
    ref = x @ w.T + case.scale * ((x @ a.T) @ b.T)
    assert _rel_fro(got, ref) < 1e-12


def test_numpy_cross_check_merge_target():
    tgt = synth.MergeTarget("k_small", 5, 1, 256, 640, 32, 64.0)
    W0 = tgt.make_w0()
    A, B = tgt.make_ab(0)
    Wd, Wb = oracle.merge(W0, B, A, tgt.scale)
    ref = synth.to_f64(W0) + tgt.scale * (synth.to_f64(B) @ synth.to_f64(A))
    assert _rel_fro(Wd, ref) < 1e-13
    # bf16 rounding of the exact value is within half a bf16 ulp of it
    wb = synth.to_f64(Wb)
    assert np.all(np.abs(wb - ref) <= np.abs(ref) * 2.0 ** -8 + 2.0 ** -134)


def test_merge_special_cases():
    rng = np.random.default_rng(9)
    W0 = synth.f32_to_bf16_bits(rng.standard_normal((40, 24)).astype(np.float32) * 0.1)
    A = synth.f32_to_bf16_bits(rng.standard_normal((4, 24)).astype(np.float32))
    B = synth.f32_to_bf16_bits(rng.standard_normal((40, 4)).astype(np.float32))
    keep = W0.copy()
    _, Wb = oracle.merge(W0, np.zeros_like(B), A, 2.0)
    np.testing.assert_array_equal(Wb, W0)              # B = 0: W_inf == W0 bitwise
    _, Wb = oracle.merge(W0, B, A, 0.0)
    np.testing.assert_array_equal(Wb, W0)              # s = 0: W_inf == W0 bitwise
    np.testing.assert_array_equal(W0, keep)            # pristine untouched
    _, part = oracle.merge(W0, B, A, 2.0, rows=(10, 30))
    _, full = oracle.merge(W0, B, A, 2.0)
    np.testing.assert_array_equal(part, full[10:30])


# ---------------------------------------------------------- bf16 rounding

def test_round_bf16_matches_torch_on_float32_values():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(10)
    vals = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-38).astype(np.float32),     # subnormal range
        (rng.standard_normal(2000) * 1e37).astype(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38, -3.4e38, np.inf, -np.inf], np.float32),
    ])
    # exact midpoints between neighbouring bf16 values (tie cases)
    b = rng.integers(0x0001, 0x7F7F, 3000).astype(np.uint32)
    mids = ((b << 16) | 0x8000).view(np.float32)
    vals = np.concatenate([vals, mids, -mids])
    ref = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.round_bf16(vals.astype(np.float64))
    np.testing.assert_array_equal(got, ref)


def test_round_bf16_single_rounding_from_double():
    # 1 + 2^-8 + 2^-30 lies just above the midpoint of 1 and 1 + 2^-7: the
    # correctly rounded bf16 value is 1 + 2^-7 (0x3F81).  Rounding through
    # float first would land on the midpoint and then tie to even, 1.0.
    assert oracle.round_bf16(1.0 + 2.0 ** -8 + 2.0 ** -30) == 0x3F81
    assert oracle.round_bf16(1.0 + 2.0 ** -8) == 0x3F80              # tie -> even
    assert oracle.round_bf16(1.0 + 3 * 2.0 ** -8) == 0x3F82          # tie -> even (up)
    assert oracle.round_bf16(-(1.0 + 2.0 ** -8 + 2.0 ** -30)) == 0xBF81
    big = (2.0 - 2.0 ** -7) * 2.0 ** 127                             # largest finite bf16
    assert oracle.round_bf16(big) == 0x7F7F
    assert oracle.round_bf16((2.0 - 2.0 ** -8) * 2.0 ** 127) == 0x7F80   # tie -> inf
    assert oracle.round_bf16(2.0 ** -133) == 0x0001                   # smallest subnormal
    assert oracle.round_bf16(2.0 ** -134) == 0x0000                   # tie -> even (0)
    assert oracle.round_bf16(1.5 * 2.0 ** -134) == 0x0001
    assert oracle.round_bf16(float("nan")) == 0x7FC0


def test_round_bf16_array_equals_scalar_entry_point():
    """The array form rounds each value exactly as the scalar entry point."""
    rng = np.random.default_rng(11)
    vals = np.concatenate([rng.standard_normal(500) * 10.0 ** rng.integers(-40, 39, 500),
                           [0.0, -0.0, np.inf, -np.inf, np.nan, 1.0 + 2.0 ** -8 + 2.0 ** -30]])
    got = oracle.round_bf16(vals)
    want = np.array([oracle.round_bf16_scalar(v) for v in vals], dtype=np.uint16)
    np.testing.assert_array_equal(got, want)
    assert oracle.round_bf16(vals.reshape(2, -1)).shape == (2, vals.size // 2)


# ---------------------------------------------------------------- backward

def _bwd_inputs(seed, M, N, K, r, dtype="f32"):
    c = synth.FwdCase(f"bwd{seed}", 96, seed, M, N, K, r, 2.0 * r, dtype)
    t = c.make()
    dY = synth.normal(96, seed, 4, (M, N), 1.0, dtype)
    return t["X"], t["W"], t["A"], t["B"], dY, c.scale


@pytest.mark.parametrize("shape", [(7, 9, 12, 3), (33, 40, 24, 16), (64, 17, 80, 5)])
def test_bwd_adjoint_identities_against_forward(shape):
    """The layer is linear in X, in A and in B separately, so its gradients
    are pinned by <dY, Y(X)> = <dX, X>, <dY, Y(A) - Y(0)> = <dA, A> and
    <dY, Y(B) - Y(0)> = <dB, B>, with Y from the forward oracle."""
    M, N, K, r = shape
    X, W, A, B, dY, s = _bwd_inputs(1, M, N, K, r)
    dX, dA, dB = oracle.bwd(X, W, A, B, dY, s)
    f64 = synth.to_f64
    Y = oracle.fwd(X, W, A, B, s)
    Y0A = oracle.fwd(X, W, np.zeros_like(A), B, s)
    Y0B = oracle.fwd(X, W, A, np.zeros_like(B), s)
    dy = f64(dY)

    def close(a, b):
        assert abs(a - b) <= 1e-11 * max(1.0, abs(a), abs(b)), (a, b)

    close(float((dy * Y).sum()), float((dX * f64(X)).sum()))
    close(float((dy * (Y - Y0A)).sum()), float((dA * f64(A)).sum()))
    close(float((dy * (Y - Y0B)).sum()), float((dB * f64(B)).sum()))


def test_bwd_brute_force_tiny_bitwise():
    """A literal loop transcription (same summation order) on tiny shapes."""
    for (M, N, K, r) in [(1, 1, 1, 1), (2, 3, 5, 2), (5, 3, 2, 3)]:
        X, W, A, B, dY, s = _bwd_inputs(2, M, N, K, r)
        x, w, a, b, dy = (synth.to_f64(v).tolist() for v in (X, W, A, B, dY))
        sd = float(np.float32(s))
        T = [[sum(x[m][k] * a[j][k] for k in range(K)) for j in range(r)] for m in range(M)]
        G = [[sum(dy[m][n] * b[n][j] for n in range(N)) for j in range(r)] for m in range(M)]
        dX = [[sum(dy[m][n] * w[n][k] for n in range(N)) + sd * sum(G[m][j] * a[j][k] for j in range(r))
               for k in range(K)] for m in range(M)]
        dA = [[sd * sum(G[m][j] * x[m][k] for m in range(M)) for k in range(K)] for j in range(r)]
        dB = [[sd * sum(dy[m][n] * T[m][j] for m in range(M)) for j in range(r)] for n in range(N)]
        gX, gA, gB = oracle.bwd(X, W, A, B, dY, s)
        assert gX.tolist() == dX and gA.tolist() == dA and gB.tolist() == dB


def test_bwd_zero_adapter_cases():
    M, N, K, r = 20, 24, 32, 4
    X, W, A, B, dY, s = _bwd_inputs(3, M, N, K, r)
    base = synth.to_f64(dY) @ synth.to_f64(W)
    dX, dA, dB = oracle.bwd(X, W, A, np.zeros_like(B), dY, s)   # B = 0: G = 0
    assert (dA == 0).all() and np.array_equal(dX, oracle.bwd(X, W, A, B, dY, 0.0)[0])
    assert np.abs(dX - base).max() < 1e-12
    dX, dA, dB = oracle.bwd(X, W, np.zeros_like(A), B, dY, s)   # A = 0: T = 0
    assert (dB == 0).all()
    dX, dA, dB = oracle.bwd(X, W, A, B, dY, 0.0)                # scale = 0
    assert (dA == 0).all() and (dB == 0).all()


def test_bwd_numpy_cross_check_bf16():
    M, N, K, r = 96, 80, 136, 16
    X, W, A, B, dY, s = _bwd_inputs(4, M, N, K, r, "bf16")
    dX, dA, dB = oracle.bwd(X, W, A, B, dY, s)
    x, w, a, b, dy = (synth.to_f64(v) for v in (X, W, A, B, dY))
    G, T = dy @ b, x @ a.T
    assert _rel_fro(dX, dy @ w + s * G @ a) < 1e-12
    assert _rel_fro(dA, s * G.T @ x) < 1e-12
    assert _rel_fro(dB, s * dy.T @ T) < 1e-12
    dXr, _, _ = oracle.bwd(X, W, A, B, dY, s, dx_rows=(10, 30))
    assert np.array_equal(dXr, dX[10:30])
