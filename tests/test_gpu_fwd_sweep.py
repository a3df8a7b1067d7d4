"""The forward's built-in tile choice across its boundaries: shapes picked so
that every default configuration (decode kernel; 32 x 32, 64 x 32, 64 x 64,
128 x 128 and 128 x 256 tiles with loader waves; 128 x 128 two-stage; 256 x
256; 128 x 128, 128 x 256 and 256 x 256 tiles keeping T over several N
tiles) runs with ragged M, N and K tails and ranks below their padded rank.

Bar: relative Frobenius error <= 1e-2 (bf16) against the fp64 oracle and
every element within the per-element bound of the kernels' arithmetic
(tests/helpers.py), on the whole output, and the same bits on a second call.
"""
import numpy as np
import pytest

import oracle
import synth
from helpers import TOL, as_f64, check_fwd_elements, rel_fro, to_dev, to_host

pytestmark = pytest.mark.gpu

# (M, N, K, r): the default tile each lands on, by the selection rule.
SHAPES = [
    (16, 1000, 2056, 32),    # decode kernel (M <= 16, r <= 32)
    (17, 1000, 2056, 32),    # 32 x 32 loader tile
    (90, 2100, 512, 12),     # 32 x 32 loader tile
    (40, 4096, 72, 64),      # 32 x 32 loader tile, rank 64
    (200, 1500, 1024, 30),   # 64 x 32 loader tile
    (1000, 2040, 200, 16),   # 64 x 64 loader tile
    (300, 3000, 1000, 64),   # 64 x 64 loader tile, rank 64
    (1288, 2048, 72, 5),     # 128 x 128 loader tile (176 tiles)
    (2600, 1400, 520, 40),   # 128 x 128 loader tile, rank 64
    (3000, 900, 2056, 128),  # 128 x 128 loader tile, rank 128
    (64, 520, 1000, 128),    # 128 x 128 loader tile, rank 128, one row tile
    (4100, 1032, 264, 24),   # 128 x 256 loader tile
    (4000, 2504, 264, 24),   # 256 x 160 loader tile (ragged M and N)
    (8192, 2560, 136, 32),   # 256 x 160 loader tile (512 tiles, two full rounds)
    (4100, 1032, 264, 100),  # 128 x 128, two stages, rank 128
    (8190, 8188, 136, 120),  # 128 x 256 keeping T over 8 N tiles (256 workgroups), rank 128
    (4100, 4100, 136, 128),  # 128 x 128 sharing T over 2 N tiles (too few 128 x 256 groups)
    (5000, 3000, 136, 200),  # 128 x 128, two stages, rank 256
    (4000, 4096, 96, 20),    # 256 x 256 (256 tiles, ragged M)
    (16380, 8190, 136, 120), # 256 x 256 keeping T over 8 N tiles, T from a prologue, rank 128
    (16380, 8190, 136, 40),  # the same tile, rank 64 (two 64-deep stages)
]


@pytest.mark.parametrize("shape", SHAPES, ids=[f"m{s[0]}_n{s[1]}_k{s[2]}_r{s[3]}" for s in SHAPES])
def test_default_tile_boundaries(gpu_lib, shape):
    import torch
    M, N, K, r = shape
    c = synth.FwdCase(f"sweep{M}x{N}x{K}r{r}", 96, SHAPES.index(shape), M, N, K, r, 2.0 * r, "bf16")
    t = c.make()
    X, W, A, B = (to_dev(t[k]) for k in "XWAB")
    Y1 = to_host(gpu_lib.fwd(X, W, A, B, c.scale))
    Y2 = to_host(gpu_lib.fwd(X, W, A, B, c.scale))
    torch.cuda.synchronize()
    ref = oracle.fwd(t["X"], t["W"], t["A"], t["B"], c.scale)
    err = rel_fro(as_f64(Y1), ref)
    ratio = check_fwd_elements(Y1, ref, t["X"], t["W"], t["A"], t["B"], c.scale, "bf16", c.name)
    print(f"{c.name}: rel_fro={err:.3e} worst/bound={ratio:.3f}")
    assert err <= TOL["bf16"]
    assert np.array_equal(Y1, Y2)
