"""Every tiled configuration, bitwise, over whole outputs, in each of the
three orders in which workgroups walk the tiles.

Inputs in {-1, 0, 1} with K <= 256 and scale in {0.5, 1, 2}: every product,
every fp32 partial sum and s T are exact integers (|T| <= K <= 256 is exact in
bf16), so the output must be the oracle's exact value rounded once to bf16,
bit for bit, at every position.  A wrong tile index, a skipped or repeated
MFMA block, a mis-ordered XCD mapping or a ragged-edge error shows up as a
mismatch at an exact position.

Shapes per tile (its BM x BN and its group of G N tiles), with ragged M, N
and K tails: 8 x 16 tile groups (the mapping where each XCD owns N tiles and
all XCDs sweep the same M tiles), 16 x 2 (each XCD owns M tiles) and 3 x 5
(neither divides: XCD-contiguous ids grouped along M).
"""
import numpy as np
import pytest

import oracle
import synth
from helpers import to_dev, to_host

pytestmark = pytest.mark.gpu


def _tiles():
    import rank_gemm_amd as rg
    out = []
    for tid in range(rg.TILE_COUNT):
        for r in (5, 40, 100, 200):
            info = rg.tile_info(tid, r)
            if info is None:
                continue
            # rank 200 only where the tile reaches it; 100 where 128 is the
            # cap; 40 (padded to 64) only where it is the tile's lowest rank
            # class (the T-keeping tiles, whose rank-64 form differs)
            if r == 200 and info.rank_pad != 256:
                continue
            if r == 40 and rg.tile_info(tid, 5) is not None:
                continue
            out.append((tid, r, info.bm, info.bn, info.group))
    return out


CASES = []
for tid, r, bm, bn, g in _tiles():
    for mode, (tm, tn) in (("xcd_n", (8, 16)), ("xcd_m", (16, 2)), ("grouped", (3, 5))):
        M = tm * bm - 3
        N = tn * bn * g - 5
        CASES.append((tid, r, mode, M, N))


@pytest.mark.parametrize("tid,r,mode,M,N", CASES,
                         ids=[f"tile{c[0]}_r{c[1]}_{c[2]}_m{c[3]}_n{c[4]}" for c in CASES])
def test_tile_integer_inputs_bitwise(gpu_lib, tid, r, mode, M, N):
    import torch
    K = 200                                   # three full 64-deep stages and a tail of 8
    s = (0.5, 1.0, 2.0)[(tid + r) % 3]
    rng = np.random.default_rng(tid * 1000 + r * 7 + M)
    ints = {k: rng.integers(-1, 2, shp).astype(np.float32)
            for k, shp in (("X", (M, K)), ("W", (N, K)), ("A", (r, K)), ("B", (N, r)))}
    t = {k: synth.f32_to_bf16_bits(v) for k, v in ints.items()}
    X, W, A, B = (to_dev(t[k]) for k in "XWAB")
    print(f"tile {tid} r {r} {mode}: M {M} N {N} K {K} s {s}", flush=True)
    Y = to_host(gpu_lib.fwd(X, W, A, B, s, tile=tid))
    torch.cuda.synchronize()
    want = oracle.round_bf16(oracle.fwd(t["X"], t["W"], t["A"], t["B"], s))
    bad = np.argwhere(Y != want)
    assert bad.size == 0, f"{len(bad)} mismatches, first at {tuple(bad[0])}"


_FIRST_RANK = {}
for _tid, _r, *_ in _tiles():
    _FIRST_RANK.setdefault(_tid, _r)
SHORT_K = [(tid, r, k) for tid, r in _FIRST_RANK.items() for k in (8, 0)]


@pytest.mark.parametrize("tid,r,K", SHORT_K, ids=[f"tile{c[0]}_r{c[1]}_k{c[2]}" for c in SHORT_K])
def test_tile_short_k(gpu_lib, tid, r, K):
    """K = 8 (one 16-B chunk per row, every stage but the first past K) and
    K = 0 (no stage in range: the output is exactly zero) on every tile, at
    its first rank class, on a grid that neither mapping divides."""
    import torch
    info = gpu_lib.tile_info(tid, r)
    M, N = 3 * info.bm - 3, 5 * info.bn * info.group - 5
    rng = np.random.default_rng(tid * 31 + K)
    ints = {k: rng.integers(-1, 2, shp).astype(np.float32)
            for k, shp in (("X", (M, K)), ("W", (N, K)), ("A", (r, K)), ("B", (N, r)))}
    t = {k: synth.f32_to_bf16_bits(v) for k, v in ints.items()}
    X, W, A, B = (to_dev(t[k]) for k in "XWAB")
    Yt = torch.full((M, N), 7.0, dtype=torch.bfloat16, device="cuda")  # must be overwritten
    print(f"tile {tid} r {r}: M {M} N {N} K {K}", flush=True)
    gpu_lib.fwd(X, W, A, B, 2.0, out=Yt, tile=tid)
    torch.cuda.synchronize()
    if K == 0:
        assert (Yt == 0).all().item()
        return
    Y = to_host(Yt)
    want = oracle.round_bf16(oracle.fwd(t["X"], t["W"], t["A"], t["B"], 2.0))
    bad = np.argwhere(Y != want)
    assert bad.size == 0, f"{len(bad)} mismatches, first at {tuple(bad[0])}"
