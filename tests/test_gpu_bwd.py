"""Parity of the HIP backward (lora_bwd) against the fp64 oracle, through the
C ABI, on seeded inputs.

Bar: the forward's bf16 bar applied to each gradient, relative Frobenius error
<= 1e-2 for dX, dA and dB (bf16 inputs, fp32 accumulation, bf16 outputs),
and every element of each gradient within the worst-case bound of the
kernels' arithmetic (tests/helpers.py: fp32 sums, s G and s T rounded once
to bf16, one rounding per gradient); bitwise equality with the oracle's
rounding where every intermediate is exactly representable (small-integer
inputs), and between repeated calls (the token ranges are added in a fixed
order, no atomics).  Every gradient element is checked, full-size workloads
included.
"""
import numpy as np
import pytest

import oracle
import synth
from helpers import TOL, as_f64, bwd_bounds, check_bwd_elements, rel_fro, to_dev, to_host

pytestmark = pytest.mark.gpu


def _case(name, case, M, N, K, r, dtype="bf16"):
    return synth.FwdCase(name, 6, case, M, N, K, r, 2.0 * r, dtype)


def _run(rg, t, scale, want_dx=True):
    import torch
    X, W, A, B, dY = (to_dev(t[k]) for k in ("X", "W", "A", "B", "dY"))
    dX, dA, dB = rg.bwd(X, W if want_dx else None, A, B, dY, scale, want_dx=want_dx)
    torch.cuda.synchronize()
    return (to_host(dX) if dX is not None else None), to_host(dA), to_host(dB)


def _check(name, got, ref, t, scale):
    errs = [rel_fro(as_f64(g), r) for g, r in zip(got, ref)]
    bounds = bwd_bounds(t["X"], t["W"], t["A"], t["B"], t["dY"], scale, *ref)
    ratios = check_bwd_elements(got, ref, bounds, name)
    print(f"{name}: rel_fro dX={errs[0]:.3e} dA={errs[1]:.3e} dB={errs[2]:.3e} "
          f"worst/bound dX={ratios[0]:.3f} dA={ratios[1]:.3f} dB={ratios[2]:.3f}")
    assert max(errs) <= TOL["bf16"], errs


# Ragged shapes spanning several tiles, token ranges and every padded rank
# (16, 32, 64, 128, 256), and token counts for each projection wave split
# (4, 2 and 1 waves per 16 tokens); N and K multiples of 8 as the ABI requires.
SHAPES = [
    ("b_m64_n64_k64_r16", 64, 64, 64, 16),
    ("b_m300_n136_k264_r5", 300, 136, 264, 5),
    ("b_m1000_n512_k768_r16", 1000, 512, 768, 16),
    ("b_m513_n256_k384_r33", 513, 256, 384, 33),
    ("b_m200_n392_k200_r100", 200, 392, 200, 100),
    ("b_m130_n256_k520_r130", 130, 256, 520, 130),
    ("b_m1_n512_k256_r16", 1, 512, 256, 16),
    ("b_m63_n8_k8_r3", 63, 8, 8, 3),
    ("b_m2049_n128_k96_r24", 2049, 128, 96, 24),
    ("b_m4500_n72_k136_r40", 4500, 72, 136, 40),
    ("b_m8200_n64_k72_r200", 8200, 64, 72, 200),
]


@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
def test_bwd_ragged_full(gpu_lib, shape):
    name, M, N, K, r = shape
    c = _case(name, SHAPES.index(shape), M, N, K, r)
    t = c.make("XWABD")
    got = _run(gpu_lib, t, c.scale)
    ref = oracle.bwd(t["X"], t["W"], t["A"], t["B"], t["dY"], c.scale)
    _check(name, got, ref, t, c.scale)


def test_bwd_mid_full(gpu_lib):
    """The mid-size workload (X[4096,1024], W[1024,1024], r 16) in full."""
    c = synth.MID
    t = c.make("XWABD")
    got = _run(gpu_lib, t, c.scale)
    ref = oracle.bwd(t["X"], t["W"], t["A"], t["B"], t["dY"], c.scale)
    _check(c.name, got, ref, t, c.scale)


@pytest.mark.parametrize("c", [synth.QPROJ, _case("b_m4096_n512_k4096_r16", 20, 4096, 512, 4096, 16),
                               _case("b_m4096_n256_k4096_r128", 21, 4096, 256, 4096, 128),
                               _case("b_m8192_n256_k8192_r128", 22, 8192, 256, 8192, 128)],
                         ids=lambda c: c.name)
def test_bwd_large_full(gpu_lib, c):
    """256 x 160 (rank <= 32) and grouped rank-128 dX tiles at full size
    (the q_proj shape, two 4096-token shapes, and an 8192 x 8192 dX product
    on the 128 x 256 tile that keeps s G after its ring): every element of
    dX, dA and dB."""
    t = c.make("XWABD")
    got = _run(gpu_lib, t, c.scale)
    ref = oracle.bwd(t["X"], t["W"], t["A"], t["B"], t["dY"], c.scale)
    _check(c.name, got, ref, t, c.scale)


def test_bwd_integer_inputs_bitwise(gpu_lib):
    """Entries in {-1, 0, 1} and scale 2: T (|T| <= K = 192) and G
    (|G| <= N = 128) are integers exact in bf16, every fp32 sum is exact, so
    each gradient is the oracle's exact value rounded once to bf16."""
    M, N, K, r = 200, 128, 192, 16
    rng = np.random.default_rng(5)

    def ints(shape):
        return synth.f32_to_bf16_bits(rng.integers(-1, 2, size=shape).astype(np.float32))

    t = {"X": ints((M, K)), "W": ints((N, K)), "A": ints((r, K)), "B": ints((N, r)),
         "dY": ints((M, N))}
    got = _run(gpu_lib, t, 2.0)
    ref = oracle.bwd(t["X"], t["W"], t["A"], t["B"], t["dY"], 2.0)
    for g, e in zip(got, ref):
        assert np.array_equal(g, oracle.round_bf16(e))


@pytest.mark.parametrize("M", [700, 4100, 9000], ids=lambda m: f"m{m}")
def test_bwd_without_dx_and_repeatable(gpu_lib, M):
    """Repeated calls are bitwise equal.  Without dX, s T is projected the
    same way (the wave split depends on the tokens only), so dB is bitwise
    the same; s G comes from the projection kernel instead of the dX kernel,
    summed in another order, so dA agrees to the bf16 bar.  M spans the 4-,
    2- and 1-wave projection splits."""
    c = _case(f"b_m{M}_n264_k328_r16", 30, M, 264, 328, 16)
    t = c.make("XWABD")
    full = _run(gpu_lib, t, c.scale)
    again = _run(gpu_lib, t, c.scale)
    part = _run(gpu_lib, t, c.scale, want_dx=False)
    assert part[0] is None
    for a, b in zip(full, again):
        assert np.array_equal(a, b)
    assert np.array_equal(part[2], full[2])
    assert rel_fro(as_f64(part[1]), as_f64(full[1])) <= TOL["bf16"]
    _, dA, dB = oracle.bwd(t["X"], t["W"], t["A"], t["B"], t["dY"], c.scale, dx_rows=(0, 0))
    errs = [rel_fro(as_f64(part[1]), dA), rel_fro(as_f64(part[2]), dB)]
    bounds = bwd_bounds(t["X"], t["W"], t["A"], t["B"], t["dY"], c.scale, None, dA, dB)
    check_bwd_elements((None, part[1], part[2]), (None, dA, dB), bounds, c.name + " no dX")
    print(f"{c.name} without dX: rel_fro dA={errs[0]:.3e} dB={errs[1]:.3e}")
    assert max(errs) <= TOL["bf16"], errs


def test_bwd_no_tokens_writes_zero_gradients(gpu_lib):
    import torch
    dev = "cuda"
    K, N, r = 64, 48, 8
    X = torch.empty((0, K), dtype=torch.bfloat16, device=dev)
    dY = torch.empty((0, N), dtype=torch.bfloat16, device=dev)
    W = torch.randn((N, K), device=dev).to(torch.bfloat16)
    A = torch.randn((r, K), device=dev).to(torch.bfloat16)
    B = torch.randn((N, r), device=dev).to(torch.bfloat16)
    dX, dA, dB = gpu_lib.bwd(X, W, A, B, dY, 1.5)
    torch.cuda.synchronize()
    assert dX.shape == (0, K)
    assert (dA.float() == 0).all() and (dB.float() == 0).all()


def test_bwd_strided_operands(gpu_lib):
    """Every operand a row-padded view; padding never read or written."""
    import torch
    M, N, K, r = 257, 136, 200, 12
    c = _case("b_strided", 31, M, N, K, r)
    t = c.make("XWABD")

    def padded(a, extra, fill=float("nan")):
        d = to_dev(a)
        big = torch.full((d.shape[0], d.shape[1] + extra), fill, dtype=d.dtype, device=d.device)
        big[:, : d.shape[1]] = d
        return big[:, : d.shape[1]]

    X, W, A, dY = (padded(t[k], 24) for k in ("X", "W", "A", "dY"))
    B = padded(t["B"], 5)
    dXb = torch.full((M, K + 16), 7.0, dtype=torch.bfloat16, device="cuda")
    dAb = torch.full((r, K + 8), 7.0, dtype=torch.bfloat16, device="cuda")
    dBb = torch.full((N, r + 3), 7.0, dtype=torch.bfloat16, device="cuda")
    need = gpu_lib.bwd_workspace_size(gpu_lib.LORA_BF16, M, N, K, r)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    p = gpu_lib._mat
    st = gpu_lib.bwd_raw(gpu_lib.LORA_BF16, M, N, K, r, *p(X, "X"), *p(W, "W"), *p(A, "A"),
                         *p(B, "B"), *p(dY, "dY"), c.scale, *p(dXb[:, :K], "dX"),
                         *p(dAb[:, :K], "dA"), *p(dBb[:, :r], "dB"), ws.data_ptr(), need,
                         gpu_lib._stream(X.device))
    assert st == gpu_lib.LORA_OK
    torch.cuda.synchronize()
    got = (to_host(dXb[:, :K]), to_host(dAb[:, :K]), to_host(dBb[:, :r]))
    ref = oracle.bwd(t["X"], t["W"], t["A"], t["B"], t["dY"], c.scale)
    _check("b_strided", got, ref, t, c.scale)
    assert (dXb[:, K:].float() == 7).all() and (dAb[:, K:].float() == 7).all()
    assert (dBb[:, r:].float() == 7).all()


@pytest.mark.parametrize("N,K,want_dx", [(0, 64, True), (0, 64, False), (48, 0, False),
                                         (48, 0, True)],
                         ids=["n0_dx", "n0_nodx", "k0_nodx", "k0_dx"])
def test_bwd_empty_feature_dims(gpu_lib, N, K, want_dx):
    """N = 0: G = 0, so dX = 0 and dA = 0 (dB is empty); K = 0: T = 0, so
    dB = 0 (dX and dA are empty)."""
    import torch
    rg = gpu_lib
    M, r = 130, 8
    dev = "cuda"
    X = torch.randn((M, K), device=dev).to(torch.bfloat16)
    W = torch.randn((N, K), device=dev).to(torch.bfloat16)
    A = torch.randn((r, K), device=dev).to(torch.bfloat16)
    B = torch.randn((N, r), device=dev).to(torch.bfloat16)
    dY = torch.randn((M, N), device=dev).to(torch.bfloat16)
    dX, dA, dB = rg.bwd(X, W, A, B, dY, 2.0, want_dx=want_dx)
    torch.cuda.synchronize()
    for g in (dX, dA, dB):
        if g is not None and g.numel():
            assert (g.float() == 0).all()
