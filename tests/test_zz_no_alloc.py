"""lora_fwd_batch_noalloc: the batch forward with its workspace in the
library's static device scratch (for callers that cannot allocate), through
the C ABI, against lora_fwd_batch with a caller workspace (bitwise: the same
kernels on the same partition) and against the oracle (per-element bound), on
two calls in a row, the second with fewer and smaller forwards than the
first; and its size limit."""
import numpy as np
import pytest

import oracle
import synth
from helpers import check_fwd_elements, to_dev, to_host

pytestmark = pytest.mark.gpu

# (M, N, K, r): decode-shaped forwards of both rank classes, a change of M,
# and one tiled forward in between.
FIRST = [(1, 1024, 2560, 32), (1, 264, 2560, 32), (1, 4100, 2560, 24), (1, 520, 2560, 16),
         (8, 2048, 512, 16), (8, 136, 512, 32), (100, 512, 512, 16), (16, 1040, 256, 32),
         (1, 200, 512, 8), (1, 4096, 4096, 16)]
SECOND = [(1, 300, 1024, 16), (4, 96, 264, 20), (1, 64, 128, 32)]


def _descs(rg, shapes, group):
    import torch
    items, descs = [], []
    for i, (M, N, K, r) in enumerate(shapes):
        c = synth.FwdCase(f"noalloc{group}_{i}", 88, group * 100 + i, M, N, K, r, 2.0 * r, "bf16")
        t = c.make()
        X, W, A, B = (to_dev(t[k]) for k in "XWAB")
        Y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
        Yref = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
        items.append((c, t, X, W, A, B, Y, Yref))
        descs.append((rg.FwdDesc(M, N, K, r, X.data_ptr(), K, W.data_ptr(), K, A.data_ptr(), K,
                                 B.data_ptr(), r, c.scale, Y.data_ptr(), N),
                      rg.FwdDesc(M, N, K, r, X.data_ptr(), K, W.data_ptr(), K, A.data_ptr(), K,
                                 B.data_ptr(), r, c.scale, Yref.data_ptr(), N)))
    return items, descs


def test_noalloc_batch_equals_workspace_batch_two_calls(gpu_lib):
    import torch
    rg = gpu_lib
    stream = torch.cuda.current_stream().cuda_stream
    for group, shapes in ((1, FIRST), (2, SECOND)):
        items, descs = _descs(rg, shapes, group)
        print(f"call {group}: {len(shapes)} forwards", flush=True)
        st = rg.fwd_batch_noalloc_raw(rg.LORA_BF16, [d[0] for d in descs], stream)
        assert st == rg.LORA_OK, rg.status_str(st)
        ws = torch.empty((rg.fwd_batch_workspace_size(len(descs)),), dtype=torch.uint8,
                         device="cuda")
        st = rg.fwd_batch_raw(rg.LORA_BF16, [d[1] for d in descs], stream, ws.data_ptr(),
                              ws.numel())
        assert st == rg.LORA_OK, rg.status_str(st)
        torch.cuda.synchronize()
        for c, t, X, W, A, B, Y, Yref in items:
            got, want = to_host(Y), to_host(Yref)
            assert np.array_equal(got, want), c.name
            ref = oracle.fwd(t["X"], t["W"], t["A"], t["B"], c.scale)
            check_fwd_elements(got, ref, t["X"], t["W"], t["A"], t["B"], c.scale, "bf16", c.name)


def test_noalloc_limit_and_empty(gpu_lib):
    rg = gpu_lib
    d = rg.FwdDesc(1, 64, 64, 16, 0x10000000, 64, 0x20000000, 64, 0x30000000, 64, 0x40000000,
                   16, 2.0, 0x50000000, 64)
    too_many = [d] * (rg.NOALLOC_MAX_FORWARDS + 1)
    assert rg.fwd_batch_noalloc_raw(rg.LORA_BF16, too_many) == rg.LORA_ERR_SCRATCH
    assert rg.fwd_batch_noalloc_raw(rg.LORA_BF16, []) == rg.LORA_OK
    empty = rg.FwdDesc(0, 64, 64, 16, 0, 64, 0, 64, 0, 64, 0, 16, 2.0, 0, 64)
    assert rg.fwd_batch_noalloc_raw(rg.LORA_BF16, [empty]) == rg.LORA_OK
