"""The C-ABI launches replayed from a HIP graph give the eager results
bitwise, replay after replay, with eager work and synchronisations between
the replays (the library records only kernel launches, no memsets)."""
import numpy as np
import pytest

import synth
from helpers import to_dev, to_host

pytestmark = pytest.mark.gpu


def _replays_match_eager(launch, outs, replays=3):
    import torch
    launch()
    torch.cuda.synchronize()
    eager = [to_host(o).copy() for o in outs]
    for o in outs:
        o.fill_(float("nan"))
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            launch()
    torch.cuda.synchronize()
    for k in range(replays):
        for o in outs:
            o.fill_(float("nan"))  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert to_host(o).tobytes() == e.tobytes(), f"replay {k}"


# M = 1: decode kernel; 64: 32 x 32 loader tile; 300: 64 x 32 loader tile;
# 4096: 128 x 128 loader tile; 8192: 128 x 256 loader tile.
@pytest.mark.parametrize("M", [1, 64, 300, 4096, 8192])
def test_fwd_graph_replay(gpu_lib, M):
    import torch
    c = synth.FwdCase(f"g{M}", 97, M, M, 1024, 768, 16, 32.0, "bf16")
    t = c.make()
    X, W, A, B = (to_dev(t[k]) for k in "XWAB")
    Y = torch.empty((M, c.N), dtype=torch.bfloat16, device="cuda")
    _replays_match_eager(lambda: gpu_lib.fwd(X, W, A, B, c.scale, out=Y), [Y])


def test_merge_graph_replay(gpu_lib):
    import torch
    tg = synth.merge_targets(1)[:3]
    ins, outs = [], []
    for t in tg:
        A, B = t.make_ab(0)
        ins.append((to_dev(t.make_w0()), to_dev(B), to_dev(A), t.scale))
        outs.append(torch.empty((t.N, t.K), dtype=torch.bfloat16, device="cuda"))

    def launch():
        for (w0, b, a, s), o in zip(ins, outs):
            gpu_lib.merge(w0, b, a, s, out=o)

    _replays_match_eager(launch, outs)


def test_merge_batch_graph_replay(gpu_lib):
    import torch
    tg = synth.merge_targets(2)
    ins, outs = [], []
    for t in tg:
        A, B = t.make_ab(1)
        ins.append((to_dev(t.make_w0()), to_dev(B), to_dev(A), t.scale))
        outs.append(torch.empty((t.N, t.K), dtype=torch.bfloat16, device="cuda"))

    def launch():
        gpu_lib.merge_batch([(w0, b, a, s, o) for (w0, b, a, s), o in zip(ins, outs)])

    _replays_match_eager(launch, outs)


@pytest.mark.parametrize("want_dx", [True, False], ids=["with_dx", "no_dx"])
def test_bwd_graph_replay(gpu_lib, want_dx):
    """The backward's launches (transposes + projection, dX, token contraction,
    reduce) replayed from a graph, the workspace reused across replays with
    NaN written over it in between."""
    import torch
    rg = gpu_lib
    M, N, K, r = 700, 264, 328, 24
    c = synth.FwdCase("gbwd", 97, 900, M, N, K, r, 48.0, "bf16")
    t = c.make("XWABD")
    X, W, A, B, dY = (to_dev(t[k]) for k in ("X", "W", "A", "B", "dY"))
    dX = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    dA = torch.empty((r, K), dtype=torch.bfloat16, device="cuda")
    dB = torch.empty((N, r), dtype=torch.bfloat16, device="cuda")
    need = rg.bwd_workspace_size(rg.LORA_BF16, M, N, K, r)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    p = rg._mat

    def launch():
        ws.fill_(0xFF)  # a torch fill kernel, recorded too: garbage the kernels must not read
        st = rg.bwd_raw(rg.LORA_BF16, M, N, K, r, *p(X, "X"), *p(W, "W"), *p(A, "A"),
                        *p(B, "B"), *p(dY, "dY"), c.scale,
                        *(p(dX, "dX") if want_dx else (0, K)), *p(dA, "dA"), *p(dB, "dB"),
                        ws.data_ptr(), need, torch.cuda.current_stream().cuda_stream)
        assert st == rg.LORA_OK

    _replays_match_eager(launch, [dX, dA, dB] if want_dx else [dA, dB])
