"""Throughput of the fused LoRA linear forward and the pristine merge on one
MI355X, with roofline fractions and the fp64 oracle timed on the host.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick] [--only NAME]

One step = one fused forward (tiled MFMA kernel) on the headline workload,
bf16 X[4096,1024] (4 x 1024 tokens), W[1024,1024], A[16,1024], B[1024,16],
r = 16, alpha = 32, fp32 accumulate, bf16 output; inputs resident in HBM.
Printed: one JSON line (rank 0).  Besides the headline, "workloads" reports
the other shapes of the same path measured in the same run: transformer
projections (8192 tokens, hidden 2560, r = 32), the 16384 x 8192 x 8192
square at r in {8, 16, 64, 128}, decode-shaped forwards (M in {1, 8, 64},
W[4096,4096], rotated over 16 operand sets so the 256 MB last-level cache
cannot hold them), a decode step through 36 layers' q/k/v and gate/up
projections (batched against one launch per projection), the merge of 36
layers x 7 targets at r = 32, and the backward (dX, dA, dB with W frozen)
on the mid-size and q_proj shapes.

--only NAME runs just one kernel a few times (for rocprofv3); NAME is one of
tiny, mid, q, v, sq8, sq16, sq64, sq128, dec1, dec8, dec64, decstep, merge,
copy, bwd_mid, bwd_q.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6      # 256 CU x 4096 flop/clk x 2.4 GHz, dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")


def _kernel_source_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "rank_gemm_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _traffic(name, src_files, per_launch_units=1.0):
    """HBM bytes per launch from the committed counter runs, if they were taken
    on the kernel source as it is now; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    e = data.get(name)
    if not e or e.get("source_hash") != _kernel_source_hash(src_files):
        return None
    return e.get("hbm_bytes_per_launch")


def timed_region(fn, steps, warmup):
    """fn(i) for i < warmup untimed, then `steps` calls back to back between
    two events on the launch stream; returns the region time in ms.  For
    kernels longer than the host's per-call cost the stream stays busy, so
    region / steps is the average launch duration."""
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    r0 = torch.cuda.Event(enable_timing=True)
    r1 = torch.cuda.Event(enable_timing=True)
    r0.record()
    for i in range(steps):
        fn(i)
    r1.record()
    torch.cuda.synchronize()
    return r0.elapsed_time(r1)


def graph_region(fn, count, replays, warmup=1):
    """Capture fn(0) .. fn(count - 1) into one HIP graph and time `replays`
    replays between two events; returns ms per replay.  Used where one launch
    is shorter than the host's per-call cost, so the device time is measured
    rather than the Python dispatch rate."""
    import torch
    fn(0)  # first call outside capture (one-time kernel attribute set-up)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for i in range(count):
                fn(i)
    torch.cuda.synchronize()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    r0 = torch.cuda.Event(enable_timing=True)
    r1 = torch.cuda.Event(enable_timing=True)
    r0.record()
    for _ in range(replays):
        g.replay()
    r1.record()
    torch.cuda.synchronize()
    return r0.elapsed_time(r1) / replays


def median(xs):
    xs = sorted(xs)
    n = len(xs)
    return xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])


# ------------------------------------------------------------------ workloads

def run_fwd_case(rg, c, steps, warmup, rotate=1, variant="auto", graph=False):
    """One forward workload.  graph=True times `steps` launches (rotating over
    `rotate` operand sets) captured in a HIP graph; else back-to-back eager
    launches between region events."""
    import torch
    import synth
    sets = [synth.fwd_case_on_device(
        synth.FwdCase(c.name, c.group, c.case + 100 * i, c.M, c.N, c.K, c.r, c.alpha, c.dtype,
                      var_b=c.var_b) if i else c) for i in range(rotate)]
    outs = [torch.empty((c.M, c.N), dtype=sets[0]["X"].dtype, device="cuda") for _ in sets]

    def fn(i):
        s = sets[i % rotate]
        rg.fwd(s["X"], s["W"], s["A"], s["B"], c.scale, out=outs[i % rotate], variant=variant)

    if graph:
        k_ms = graph_region(fn, steps, 3) / steps
        eager_ms = timed_region(fn, steps, warmup) / steps
    else:
        k_ms = timed_region(fn, steps, warmup) / steps
        eager_ms = k_ms
    return {
        "workload": c.name,
        "variant": variant if variant != "auto" else ("decode" if rg.fwd_pick(
            rg.LORA_BF16, c.M, c.N, c.K, c.r) == 2 else "tiled"),
        "timing": "hip graph of back-to-back launches" if graph else "back-to-back launches",
        "kernel_us_mean": round(k_ms * 1e3, 3),
        "eager_us_per_call": round(eager_ms * 1e3, 3),
        "tflops": round(c.flops() / (k_ms * 1e-3) / 1e12, 2),
        "pct_bf16_peak": round(100 * c.flops() / (k_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
        "gbs": round(c.bytes() / (k_ms * 1e-3) / 1e9, 1),
        "pct_hbm_peak": round(100 * c.bytes() / (k_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 2),
        "operand_sets": rotate,
    }


def run_merge_pass(rg, steps, warmup, layers=36):
    """All 36 x 7 targets on one stream: one pass = one lora_merge_batch call
    (timed as a HIP graph replay and eagerly), and for comparison one
    lora_merge launch per target (a HIP graph of the 252 launches: a launch of
    a small target is shorter than the host's per-call cost)."""
    import torch
    import synth
    tg = synth.merge_targets(layers)
    w0, a, b, wi = [], [], [], []
    for t in tg:
        w0.append(synth.device_normal(t.group, t.case, synth.TW, (t.N, t.K), t.var_w0, "bf16"))
        a.append(synth.device_normal(t.group, t.case, synth.TA, (t.r, t.K), 1.0 / t.K, "bf16"))
        b.append(synth.device_normal(t.group, t.case, synth.TB, (t.N, t.r), t.var_b, "bf16"))
        wi.append(torch.empty_like(w0[-1]))

    def launch(i):
        t = tg[i]
        rg.merge(w0[i], b[i], a[i], t.scale, out=wi[i])

    # The pass as one lora_merge_batch call (descriptors built once, as a
    # caller refreshing the same buffers every cycle would), and as one
    # lora_merge call per target.
    descs = (rg.MergeDesc * len(tg))(*[
        rg.MergeDesc(t.N, t.K, t.r, w0[i].data_ptr(), t.K, b[i].data_ptr(), t.r, a[i].data_ptr(),
                     t.K, t.scale, wi[i].data_ptr(), t.K) for i, t in enumerate(tg)])

    def batch(_):
        st = rg.merge_batch_raw(rg.LORA_BF16, descs, torch.cuda.current_stream().cuda_stream)
        assert st == rg.LORA_OK, rg.status_str(st)

    pass_ms = graph_region(batch, 1, steps, warmup)
    eager_ms = timed_region(batch, steps, warmup) / steps
    per_target_ms = graph_region(launch, len(tg), steps, warmup)
    total_bytes = sum(t.bytes() for t in tg)
    # per-target-shape kernel times: one graph of that target in all layers
    shape_ms = {}
    for i, t in enumerate(tg[:7]):
        ms = graph_region(lambda j, i=i: launch(i + 7 * j), layers, 5) / layers
        shape_ms[t.name.split(".")[1]] = {
            "shape": [t.N, t.K], "kernel_us_mean": round(ms * 1e3, 2),
            "gbs": round(t.bytes() / (ms * 1e-3) / 1e9, 1)}
    return {
        "workload": f"merge_from_pristine_{layers}x7_targets_r32",
        "timing": "hip graph of one lora_merge_batch call over the 252 targets",
        "pass_ms_mean": round(pass_ms, 4),
        "eager_pass_ms": round(eager_ms, 4),
        "one_launch_per_target_pass_ms": round(per_target_ms, 4),
        "gbs": round(total_bytes / (pass_ms * 1e-3) / 1e9, 1),
        "pct_hbm_peak": round(100 * total_bytes / (pass_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 2),
        "bytes_per_pass": int(total_bytes),
        "per_target_shape": shape_ms,
    }


def run_decode_step(rg, steps, warmup, layers=36):
    """One decode token (M = 1) through the projections of 36 layers that read
    the same input: q, k, v (hidden 2560 -> 4096, 1024, 1024) and gate, up
    (2560 -> 9728, 9728), rank 32.  Per layer: two lora_fwd_batch calls (one
    per shared input) against five lora_fwd calls; both captured in HIP graphs
    (one launch is shorter than the host's per-call cost).  The batched
    calls run with and without a workspace (with one, T is computed once per
    forward in a launch of its own).  The weights of 36 layers (4.7 GB) do
    not fit the last-level cache."""
    import torch
    import synth
    groups = [("q", "k", "v"), ("gate", "up")]
    shapes = {n: (o, i) for n, o, i in synth.MERGE_TARGET_SHAPES}
    r, scale = 32, 2.0
    layer_items, total_bytes = [], 0
    for layer in range(layers):
        items = []
        for gi, grp in enumerate(groups):
            K = shapes[grp[0]][1]
            X = synth.device_normal(9, layer * 2 + gi, synth.TX, (1, K), 1.0, "bf16")
            for t, name in enumerate(grp):
                N = shapes[name][0]
                case = layer * 7 + t + 3 * gi
                W = synth.device_normal(9, case, synth.TW, (N, K), 1.0 / K, "bf16")
                A = synth.device_normal(9, case, synth.TA, (r, K), 1.0 / K, "bf16")
                B = synth.device_normal(9, case, synth.TB, (N, r), 0.02, "bf16")
                Y = torch.empty((1, N), dtype=torch.bfloat16, device="cuda")
                items.append((gi, (X, W, A, B, scale, Y)))
                total_bytes += 2 * (K + N * K + r * K + N * r + N)
        layer_items.append(items)

    group_items = [[[it for g, it in items if g == gi] for gi in range(len(groups))]
                   for items in layer_items]
    ws = torch.empty((rg.fwd_batch_workspace_size(3),), dtype=torch.uint8, device="cuda")

    def batched(_):
        for per_layer in group_items:
            for its in per_layer:
                rg.fwd_batch(its)

    def batched_ws(_):
        for per_layer in group_items:
            for its in per_layer:
                rg.fwd_batch(its, workspace=ws)

    def single(_):
        for items in layer_items:
            for _, (X, W, A, B, sc, Y) in items:
                rg.fwd(X, W, A, B, sc, out=Y)

    w_ms = graph_region(batched_ws, 1, steps, warmup)
    b_ms = graph_region(batched, 1, steps, warmup)
    s_ms = graph_region(single, 1, steps, warmup)
    return {
        "workload": f"decode_step_{layers}_layers_qkv_gateup_m1_r32",
        "timing": "hip graph of one decode step (all layers), replayed",
        "step_us_batched_with_workspace": round(w_ms * 1e3, 2),
        "step_us_batched": round(b_ms * 1e3, 2),
        "step_us_one_launch_per_projection": round(s_ms * 1e3, 2),
        "launches_per_layer": {"batched_with_workspace": 2 * len(groups),
                               "batched": len(groups), "one_per_projection": 5},
        "gbs": round(total_bytes / (w_ms * 1e-3) / 1e9, 1),
        "pct_hbm_peak": round(100 * total_bytes / (w_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 2),
        "bytes_per_step": int(total_bytes),
    }


def bwd_flops(c):
    """Algorithmic flops of one backward: dY W (2 M N K), G = dY B and
    dB = s dY^T T (2 M N r each), T = X A^T, s G A and dA = s G^T X
    (2 M K r each)."""
    M, N, K, r = c.M, c.N, c.K, c.r
    return 2.0 * M * N * K + 4.0 * M * N * r + 6.0 * M * K * r


def run_bwd_case(rg, c, steps, warmup):
    """One backward workload (lora_bwd: four launches): `steps` back-to-back
    eager passes between region events, and a HIP graph of `steps` passes."""
    import torch
    import synth
    t = synth.fwd_case_on_device(c)
    dY = synth.dy_on_device(c)
    M, N, K, r = c.M, c.N, c.K, c.r
    dX = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    dA = torch.empty((r, K), dtype=torch.bfloat16, device="cuda")
    dB = torch.empty((N, r), dtype=torch.bfloat16, device="cuda")
    need = rg.bwd_workspace_size(rg.LORA_BF16, M, N, K, r)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    args = (rg.LORA_BF16, M, N, K, r, t["X"].data_ptr(), K, t["W"].data_ptr(), K,
            t["A"].data_ptr(), K, t["B"].data_ptr(), r, dY.data_ptr(), N, c.scale,
            dX.data_ptr(), K, dA.data_ptr(), K, dB.data_ptr(), r, ws.data_ptr(), need)

    def fn(_):
        st = rg.bwd_raw(*args, torch.cuda.current_stream().cuda_stream)
        assert st == rg.LORA_OK, rg.status_str(st)

    graph_ms = graph_region(fn, steps, 3) / steps
    ms = timed_region(fn, steps, warmup) / steps
    f = bwd_flops(c)
    return {
        "workload": "bwd_" + c.name,
        "timing": "back-to-back eager backward passes (4 launches each; a pass outlasts "
                  "the host's per-call cost)",
        "pass_us_mean": round(ms * 1e3, 3),
        "graph_replay_us_per_pass": round(graph_ms * 1e3, 3),
        "tflops": round(f / (ms * 1e-3) / 1e12, 2),
        "pct_bf16_peak": round(100 * f / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
        "algorithmic_flop_per_pass": f,
        "workspace_bytes": need,
    }


def cpu_baseline(c, budget_s=10.0):
    """The fp64 oracle, as it is, on the host cores: full passes of the
    headline workload until the budget is spent."""
    import oracle
    t = c.make()
    threads = len(os.sched_getaffinity(0))
    oracle.set_threads(threads)
    n, t0 = 0, time.time()
    while True:
        oracle.fwd(t["X"], t["W"], t["A"], t["B"], c.scale)
        n += 1
        if time.time() - t0 >= budget_s:
            break
    dt = time.time() - t0
    return {"value": round(n * c.flops() / dt / 1e12, 5), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{n} full fp64 oracle pass(es) of {c.name} ({c.flops() / 1e9:.3f} GFLOP "
                      f"each) in {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--quick", action="store_true", help="headline workload only")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle timing")
    ap.add_argument("--only", default=None)
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    import rank_gemm_amd as rg
    import synth

    torch.cuda.set_device(0)
    rg.lib()

    if args.only:
        return only(rg, args.only, args.steps, args.warmup)

    head = synth.MID
    t = head.make()

    def dev(a):
        import numpy as np
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()

    X, W, A, B = (dev(t[k]) for k in "XWAB")
    Y = torch.empty((head.M, head.N), dtype=torch.bfloat16, device="cuda")

    def step(_):
        rg.fwd(X, W, A, B, head.scale, out=Y)

    # One step is one launch and the kernel outlasts the host's per-call cost,
    # so region / steps is the kernel's average launch duration.
    region_ms = timed_region(step, args.steps, args.warmup)
    ms_per_step = region_ms / args.steps
    value = head.flops() / (ms_per_step * 1e-3) / 1e12
    achieved = value
    traffic = _traffic("fwd_tiled_mid_x4096x1024_w1024_r16", ["fwd_tiled.hip", "common.h"])

    line = {
        "metric": "fused LoRA fwd TFLOP/s (% bf16 MFMA peak); merge/decode GB/s (% HBM peak)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded normal inputs)",
        "config": {"workload": head.name, "M": head.M, "N": head.N, "K": head.K, "r": head.r,
                   "alpha": head.alpha, "accumulate": "fp32", "output": "bf16"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic, "kernel_us_mean": round(ms_per_step * 1e3, 3),
                     "algorithmic_flop_per_launch": head.flops()},
    }

    if not args.quick:
        work = []
        for c in (synth.QPROJ, synth.VPROJ):
            work.append(run_fwd_case(rg, c, 30, 5))
        for c in synth.SQUARE:
            work.append(run_fwd_case(rg, c, 10, 2))
        for c in synth.DECODE:
            work.append(run_fwd_case(rg, c, 256, 32, rotate=16, graph=True))
        work.append(run_decode_step(rg, 10, 2))
        work.append(run_merge_pass(rg, 5, 1))
        for c in (synth.MID, synth.QPROJ):
            work.append(run_bwd_case(rg, c, 20, 3))
        line["workloads"] = work

    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(head)
    print(json.dumps(line), flush=True)


def only(rg, name, steps, warmup):
    """One kernel, a few launches, for profiler runs."""
    import torch
    import synth
    table = {"tiny": synth.TINY, "mid": synth.MID, "q": synth.QPROJ, "v": synth.VPROJ,
             "sq8": synth.SQUARE[0], "sq16": synth.SQUARE[1], "sq64": synth.SQUARE[2],
             "sq128": synth.SQUARE[3], "dec1": synth.DECODE[0], "dec8": synth.DECODE[1],
             "dec64": synth.DECODE[2]}
    if name in table:
        c = table[name]
        dec = name.startswith("dec")
        res = run_fwd_case(rg, c, steps, warmup, rotate=16 if dec else 1, graph=dec)
    elif name == "merge":
        res = run_merge_pass(rg, steps, warmup)
    elif name == "decstep":
        res = run_decode_step(rg, steps, warmup)
    elif name in ("bwd_mid", "bwd_q"):
        res = run_bwd_case(rg, synth.MID if name == "bwd_mid" else synth.QPROJ, steps, warmup)
    elif name == "copy":
        # Plain device copy of a known size: the reference for counter scaling.
        n = 256 << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        ms = timed_region(lambda _: dst.copy_(src), steps, warmup) / steps
        res = {"workload": f"copy_{n}_bytes", "kernel_us_mean": ms * 1e3,
               "gbs": 2 * n / (ms * 1e-3) / 1e9}
    else:
        raise SystemExit(f"unknown --only {name}")
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
