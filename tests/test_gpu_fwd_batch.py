"""lora_fwd_batch on the GPU: each output bitwise equal to lora_fwd's for the
same forward (the batched decode launch runs the same kernel code per
forward; one-token forwards with a workspace take T from workgroups that
reproduce the one-token kernel's own partial sums, in the same launch or,
for very wide forwards, in a launch of their own; with a workspace, 2 <= M
<= 16 and 16 < r <= 32, equal up to fp32 rounding order),
over a mix that exercises the grouping: several decode-shaped
forwards sharing X (different N and K), a change of rank class, a change of
M, a tiled forward in between, and a ragged last column block; plus parity
with the oracle and bitwise equal HIP graph replays."""
import numpy as np
import pytest

import oracle
import synth
from helpers import TOL, as_f64, check_fwd_elements, rel_fro, to_dev, to_host

pytestmark = pytest.mark.gpu

# (M, N, K, r, shares X with the previous forward)
MIX = [(1, 1024, 2560, 32, False), (1, 264, 2560, 32, True), (1, 4100, 2560, 24, True),
       (1, 520, 2560, 16, True), (1, 1032, 1024, 16, False), (8, 2048, 512, 16, False),
       (8, 136, 512, 32, True), (100, 512, 512, 16, False), (1, 200, 512, 8, False),
       (16, 1040, 256, 32, False),
       # one-token forwards whose K ends inside a 64-deep segment
       (1, 72, 1000, 20, False), (1, 48, 136, 8, False),
       # more 16-row blocks than a workspace slot has flags: T by a launch
       # of its own
       (1, 30736, 64, 16, False)]


def _make(i, M, N, K, r):
    c = synth.FwdCase(f"batch{i}", 8, i, M, N, K, r, 2.0 * r, "bf16")
    return c, c.make()


@pytest.mark.parametrize("with_ws", [False, True], ids=["no_workspace", "workspace"])
def test_fwd_batch_equals_fwd(gpu_lib, with_ws):
    import torch
    rg = gpu_lib
    cases, X = [], None
    for i, (M, N, K, r, share) in enumerate(MIX):
        c, t = _make(i, M, N, K, r)
        if not share or X is None or X.shape != (M, K):
            X = to_dev(t["X"])
            Xh = t["X"]
        cases.append((c, Xh, X, to_dev(t["W"]), to_dev(t["A"]), to_dev(t["B"]), t))
    outs = [torch.empty((c.M, c.N), dtype=torch.bfloat16, device="cuda") for c, *_ in cases]
    ws = None
    if with_ws:  # garbage content: the kernels must not depend on it
        ws = torch.full((rg.fwd_batch_workspace_size(len(cases)),), 0xFF, dtype=torch.uint8,
                        device="cuda")
    rg.fwd_batch([(X, W, A, B, c.scale, Y) for (c, _, X, W, A, B, _), Y in zip(cases, outs)],
                 workspace=ws)
    torch.cuda.synchronize()
    for (c, Xh, X, W, A, B, t), Y in zip(cases, outs):
        single = to_host(rg.fwd(X, W, A, B, c.scale))
        got = to_host(Y)
        if with_ws and 1 < c.M <= 16 and c.r > 16:
            # the weight stream runs four K blocks per wave here (two in
            # lora_fwd at this rank): same values up to fp32 rounding order
            assert rel_fro(as_f64(got), as_f64(single)) <= 1e-3, c.name
        else:
            assert np.array_equal(got, single), c.name
        ref = oracle.fwd(Xh, t["W"], t["A"], t["B"], c.scale)
        err = rel_fro(as_f64(got), ref)
        ratio = check_fwd_elements(got, ref, Xh, t["W"], t["A"], t["B"], c.scale, "bf16", c.name)
        print(f"{c.name} M{c.M} N{c.N} K{c.K} r{c.r}: rel_fro={err:.3e} worst/bound={ratio:.3f}")
        assert err <= TOL["bf16"]


@pytest.mark.parametrize("with_ws", [False, True], ids=["no_workspace", "workspace"])
def test_fwd_batch_graph_replays(gpu_lib, with_ws):
    import torch
    rg = gpu_lib
    items, outs = [], []
    for i, (M, N, K, r, _) in enumerate(MIX[:5]):
        c, t = _make(20 + i, M, N, K, r)
        Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        items.append((to_dev(t["X"]), to_dev(t["W"]), to_dev(t["A"]), to_dev(t["B"]), c.scale, Y))
        outs.append(Y)
    ws = (torch.empty((rg.fwd_batch_workspace_size(len(items)),), dtype=torch.uint8, device="cuda")
          if with_ws else None)
    rg.fwd_batch(items, workspace=ws)
    torch.cuda.synchronize()
    eager = [to_host(Y) for Y in outs]
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            rg.fwd_batch(items, workspace=ws)
    torch.cuda.synchronize()
    for rep in range(3):
        for Y in outs:
            Y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for e, Y in zip(eager, outs):
            assert np.array_equal(to_host(Y), e), rep


def test_fwd_batch_graph_new_tokens(gpu_lib):
    """One-token forwards with a workspace, captured once and replayed with a
    new X before each replay (as a decode loop does): every replay equals
    lora_fwd on that replay's X, so no replay reads the T partial sums or
    flags a previous one left in the workspace."""
    import torch
    rg = gpu_lib
    # two launches, each with more weight workgroups than CUs (T computed in
    # the weight stream's launch)
    shapes = [(1, 4096, 2560, 32), (1, 1024, 2560, 32), (1, 4100, 1024, 16), (1, 200, 1024, 8)]
    items, outs, xs, ops = [], [], [], []
    for i, (M, N, K, r) in enumerate(shapes):
        c, t = _make(40 + i, M, N, K, r)
        X, W, A, B = (to_dev(t[k]) for k in ("X", "W", "A", "B"))
        Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        items.append((X, W, A, B, c.scale, Y))
        outs.append(Y)
        xs.append(X)
        ops.append((W, A, B, c.scale))
    ws = torch.full((rg.fwd_batch_workspace_size(len(items)),), 0xFF, dtype=torch.uint8,
                    device="cuda")
    rg.fwd_batch(items, workspace=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            rg.fwd_batch(items, workspace=ws)
    torch.cuda.synchronize()
    for rep in range(4):
        fresh = []
        for i, (X, (M, N, K, r)) in enumerate(zip(xs, shapes)):
            new = synth.FwdCase(f"tok{rep}_{i}", 9, 100 * rep + i, M, N, K, r, 2.0 * r,
                                "bf16").make("X")["X"]
            X.copy_(to_dev(new))
            fresh.append(X.clone())
        for Y in outs:
            Y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for X, (W, A, B, scale), Y in zip(fresh, ops, outs):
            single = to_host(rg.fwd(X, W, A, B, scale))
            assert np.array_equal(to_host(Y), single), rep
