"""Throughput of the fused LoRA linear forward and the pristine merge on one
MI355X, with roofline fractions, measured machine ceilings and the fp64
oracle timed on the host.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick] [--no-cpu]
                  [--only NAME]

One step = one fused forward (tiled MFMA kernel) on the large square
workload: bf16 X[16384,8192] (16384 tokens), W[8192,8192], A[16,8192],
B[8192,16], r = 16, alpha = 32, fp32 accumulate, bf16 output (2207.6 GFLOP),
inputs resident in HBM.  `value` is algorithmic TFLOP/s over the K timed
steps; the per-launch median / p10 / p90 come from HIP events around every
launch on the launch stream.

Printed: one JSON line.  Besides the headline it carries
  * "roofline": the headline kernel against the dense bf16 MFMA peak, with
    the HBM traffic per launch from the committed FETCH_SIZE / WRITE_SIZE
    counter runs when they were taken on the current kernel source;
  * "ceilings": what this GPU sustains in the same run for the same kind of
    work (a pure-MFMA loop with its clock, a streaming copy, a streaming
    read at 1 GiB and at the decode weight's size);
  * "gpu_clock": the driver's shader-clock level (sysfs) sampled over a
    sustained ~0.5-s run of the headline kernel after the timed region;
  * "workloads": the other shapes of the path in the same run (projection
    shapes, the other ranks of the square, decode M in {1, 8, 64} over 16
    rotating operand sets, a 36-layer decode step, the 36 x 7 target merge,
    the backward), each as % of the nominal peak and of the measured ceiling;
  * "oracle_timing" and "cpu_baseline": the fp64 oracle on the host cores
    (all of them, and one core for the small configurations), per config,
    on full passes or labelled row samples.

--only NAME runs just one kernel a few times (for rocprofv3); NAME is one of
tiny, mid, q, v, sq8, sq16, sq64, sq128, dec1, dec8, dec64, decstep, merge,
copy, bwd_mid, bwd_q, ceil_mfma (all ceilings), and clock (the shader clock
under sustained loads: the fused square, the MFMA loop, the library GEMM).
"""
from __future__ import annotations

import argparse
import ctypes
import glob
import hashlib
import json
import os
import re
import subprocess
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6      # 256 CU x 4096 flop/clk x 2.4 GHz, dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
METRIC = "fused LoRA fwd TFLOP/s (% bf16 MFMA peak); merge/decode GB/s (% HBM peak)"


def _kernel_source_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "rank_gemm_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _traffic(name, src_files):
    """HBM bytes per launch (read, write, total) from the committed counter
    runs, if they were taken on the kernel source as it is now; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    e = data.get(name)
    if not e or e.get("source_hash") != _kernel_source_hash(src_files):
        return None
    return e


def pct(x):
    """Percentiles (p10, median, p90) of a list."""
    xs = sorted(x)
    n = len(xs)

    def q(p):
        i = min(n - 1, max(0, int(round(p * (n - 1)))))
        return xs[i]
    return q(0.1), q(0.5), q(0.9)


def per_launch(fn, steps, warmup):
    """fn(i) for i < warmup untimed, then `steps` calls with a HIP event on
    the launch stream before each and after the last.  Returns
    (per-launch ms list, region ms, host wall seconds of the region)."""
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i].record()
        fn(i)
    ev[steps].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    times = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    return times, ev[0].elapsed_time(ev[steps]), wall


def graph_replays(fn, count, replays, warmup=1):
    """Capture fn(0) .. fn(count - 1) into one HIP graph and time each of
    `replays` replays with events; returns the per-replay ms list.  Used where
    one launch is shorter than the host's per-call cost, so the device time
    is measured rather than the Python dispatch rate."""
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
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(replays + 1)]
    for i in range(replays):
        ev[i].record()
        g.replay()
    ev[replays].record()
    torch.cuda.synchronize()
    return [ev[i].elapsed_time(ev[i + 1]) for i in range(replays)]


def stats_us(ms_list, per=1):
    """{mean, median, p10, p90} in us of a list of ms, divided by `per`."""
    p10, med, p90 = pct(ms_list)
    mean = sum(ms_list) / len(ms_list)
    return {"mean_us": round(mean * 1e3 / per, 3), "median_us": round(med * 1e3 / per, 3),
            "p10_us": round(p10 * 1e3 / per, 3), "p90_us": round(p90 * 1e3 / per, 3)}


# ------------------------------------------------------------- GPU clock

class ClockSampler:
    """Samples the GPU's shader clock on a host thread while a region runs:
    the current level of the driver's sclk table (sysfs pp_dpm_sclk), else
    `amd-smi metric --clock`.  Reports what it could read, or why not."""

    def __init__(self, period_s=0.02):
        self.period = period_s
        self.samples = []
        self.source = None
        self.error = None
        self._stop = threading.Event()
        self._path = None
        for p in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
            try:
                if "*" in open(p).read():
                    self._path = p
                    break
            except OSError:
                continue

    def _read(self):
        if self._path:
            txt = open(self._path).read()
            for line in txt.splitlines():
                if line.strip().endswith("*"):
                    m = re.search(r"(\d+)\s*[Mm][Hh]z", line)
                    if m:
                        return float(m.group(1))
            return None
        r = subprocess.run(["amd-smi", "metric", "--clock", "-g", "0"], capture_output=True,
                           text=True, timeout=5)
        m = re.search(r"GFX_0:\s*\n\s*CLK:\s*(\d+)", r.stdout) or re.search(
            r"CLK:\s*(\d+)\s*MHz", r.stdout)
        return float(m.group(1)) if m else None

    def _loop(self):
        while not self._stop.is_set():
            try:
                v = self._read()
                if v is not None:
                    self.samples.append(v)
            except Exception as e:  # noqa: BLE001 -- a clock reading is optional
                self.error = str(e)[:200]
                return
            self._stop.wait(self.period)

    def __enter__(self):
        self.source = ("sysfs " + self._path) if self._path else "amd-smi metric --clock"
        self._t = threading.Thread(target=self._loop, daemon=True)
        self._t.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        self._t.join(timeout=10)

    def report(self):
        if not self.samples:
            return {"source": self.source, "samples": 0, "error": self.error or "no reading"}
        p10, med, p90 = pct(self.samples)
        late = self.samples[len(self.samples) // 4:]
        return {"source": self.source, "samples": len(self.samples), "median_mhz": med,
                "p10_mhz": p10, "p90_mhz": p90, "min_mhz": min(self.samples),
                "max_mhz": max(self.samples),
                "median_mhz_after_first_quarter": pct(late)[1] if late else None,
                "note": "the driver's current shader-clock level, read by a host thread; "
                        "the first samples lag the ramp from idle"}


# ------------------------------------------------------------- ceilings

def ceil_lib():
    import torch  # noqa: F401 -- torch's HIP runtime first (one runtime per process)
    from rank_gemm_amd import build as b
    if not os.path.exists(b.CEIL_LIB):
        b.build()
    L = ctypes.CDLL(b.CEIL_LIB)
    i32, i64, vp = ctypes.c_int, ctypes.c_int64, ctypes.c_void_p
    L.ceil_mfma.argtypes = [i32, i32, i32, vp, vp, vp]
    L.ceil_mfma_flops.argtypes = [i32, i32, i32]
    L.ceil_mfma_flops.restype = ctypes.c_double
    L.ceil_copy.argtypes = [vp, vp, i64, i32, i32, vp]
    L.ceil_read.argtypes = [vp, i64, vp, i32, i32, vp]
    return L


def run_ceilings(steps=20):
    """Pure-MFMA loop (with its clock), streaming copy and streaming read."""
    import torch
    L = ceil_lib()
    st = lambda: torch.cuda.current_stream().cuda_stream  # noqa: E731
    out = {}
    # MFMA: 512 workgroups of 8 waves (4 waves per SIMD), ~2 ms per launch.
    wg, waves, iters = 512, 8, 5000
    buf = torch.empty(wg * waves * 64, dtype=torch.float32, device="cuda")
    clk = torch.zeros(wg * 4, dtype=torch.int64, device="cuda")
    clocks = []

    def mf(_):
        assert L.ceil_mfma(wg, waves, iters, buf.data_ptr(), clk.data_ptr(), st()) == 0

    def mf_clock(i):
        mf(i)
        c = clk.view(-1, 4).cpu().double()
        span_t, span_r = c[:, 1] - c[:, 0], c[:, 3] - c[:, 2]
        ok = span_r > 0
        if ok.any():
            clocks.append(float((span_t[ok] / span_r[ok]).median()) * 100.0)  # MHz

    times, _, _ = per_launch(mf, steps, 3)
    for i in range(3):
        mf_clock(i)
    flops = L.ceil_mfma_flops(wg, waves, iters)
    p10, med, p90 = pct(times)
    out["mfma_bf16"] = {"tflops_median": round(flops / (med * 1e-3) / 1e12, 1),
                        "tflops_p10": round(flops / (p90 * 1e-3) / 1e12, 1),
                        "tflops_p90": round(flops / (p10 * 1e-3) / 1e12, 1),
                        "pct_nominal": round(100 * flops / (med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
                        "shader_clock_mhz": round(sorted(clocks)[len(clocks) // 2], 0) if clocks else None,
                        "what": f"{wg} workgroups x {waves} waves x {iters} x 8 "
                                "v_mfma_f32_16x16x32_bf16 on register operands; clock = "
                                "s_memtime span / s_memrealtime span x 100 MHz"}
    # Streaming copy and read of 1 GiB (far past the 256 MB last-level cache):
    # the best of three access patterns and three grid sizes.
    n = 1 << 30
    src = torch.zeros(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    sink = torch.zeros(8192, dtype=torch.int32, device="cuda")
    L.ceil_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                            ctypes.c_int, ctypes.c_void_p]
    L.ceil_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
                            ctypes.c_int, ctypes.c_void_p]
    names = {0: "grid-stride", 1: "contiguous block per workgroup", 2: "block, non-temporal"}
    for kind in ("copy", "read"):
        best = None
        for var in (0, 1, 2):
            for wg in (1024, 2048, 4096):
                if kind == "copy":
                    fn = lambda _, v=var, w=wg: L.ceil_copy(src.data_ptr(), dst.data_ptr(), n, w,  # noqa
                                                            v, st())
                else:
                    fn = lambda _, v=var, w=wg: L.ceil_read(src.data_ptr(), n, sink.data_ptr(),  # noqa
                                                            w, v, st())
                times, _, _ = per_launch(fn, steps, 3)
                med = pct(times)[1]
                gbs = (2 if kind == "copy" else 1) * n / (med * 1e-3) / 1e9
                if best is None or gbs > best[0]:
                    best = (gbs, var, wg)
        out[kind + "_1gib"] = {"gbs_median": round(best[0], 1),
                               "pct_nominal": round(100 * best[0] / PEAK_HBM_GBS, 2),
                               "what": f"{'read + write' if kind == 'copy' else 'read'} of 1 GiB, "
                                       f"16 B per lane; best of 3 patterns x 3 grids: "
                                       f"{names[best[1]]}, {best[2]} workgroups"}
    del dst
    # Read at the decode weight's size (32 MiB), 16 rotating buffers, graph.
    nd = 4096 * 4096 * 2
    bufs = [torch.zeros(nd, dtype=torch.uint8, device="cuda") for _ in range(16)]
    best = None
    for var in (1, 2):
        reps = graph_replays(lambda i, v=var: L.ceil_read(bufs[i % 16].data_ptr(), nd,  # noqa
                                                          sink.data_ptr(), 1024, v, st()), 256, 20)
        per = pct(reps)[1] / 256
        if best is None or per < best[0]:
            best = (per, var)
    per = best[0]
    out["read_32mib_rotating"] = {"us_per_launch": round(per * 1e3, 3),
                                  "gbs": round(nd / (per * 1e-3) / 1e9, 1),
                                  "pct_nominal": round(100 * nd / (per * 1e-3) / 1e9 / PEAK_HBM_GBS, 2),
                                  "what": "read of one of 16 rotating 32 MiB buffers per launch "
                                          f"(1024 workgroups, {names[best[1]]}), 256 launches per "
                                          "HIP graph; includes the launch-to-launch gap"}
    return out


def run_clock_phases(seconds=0.6):
    """The shader clock under sustained loads, sampled every 5 ms: the fused
    forward on the square (headline) workload, the dense MFMA loop, and the
    library's plain bf16 GEMM (hipBLASLt via torch.matmul, no LoRA term) on
    the same X and W, for reference.  Each phase runs about `seconds`."""
    import torch
    import rank_gemm_amd as rg
    import synth
    c = synth.SQUARE[1]
    t = synth.fwd_case_on_device(c)
    Y = torch.empty((c.M, c.N), dtype=torch.bfloat16, device="cuda")
    L = ceil_lib()
    wg, waves, iters = 512, 8, 5000
    buf = torch.empty(wg * waves * 64, dtype=torch.float32, device="cuda")
    clk = torch.zeros(wg * 4, dtype=torch.int64, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    phases = [
        ("fused_forward_square_r16", lambda i: rg.fwd(t["X"], t["W"], t["A"], t["B"], c.scale, out=Y),
         c.flops()),
        ("mfma_loop", lambda i: L.ceil_mfma(wg, waves, iters, buf.data_ptr(), clk.data_ptr(), st),
         L.ceil_mfma_flops(wg, waves, iters)),
        ("hipblaslt_plain_gemm_same_x_w", lambda i: torch.matmul(t["X"], t["W"].t(), out=Y),
         2.0 * c.M * c.N * c.K)]
    out = []
    for rep in range(2):
        for name, fn, flops in phases:
            fn(0)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn(0)
            e1.record()
            torch.cuda.synchronize()
            n = max(5, int(seconds / (e0.elapsed_time(e1) * 1e-3)))
            sampler = ClockSampler(period_s=0.005)
            with sampler:
                e0.record()
                for i in range(n):
                    fn(i)
                e1.record()
                torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / n
            smp = sampler.samples[len(sampler.samples) // 4:]   # after the ramp
            p10, med, p90 = pct(smp) if smp else (None, None, None)
            out.append({"phase": name, "repeat": rep, "launches": n, "ms_per_launch": round(ms, 4),
                        "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
                        "clock_mhz_p10_median_p90": [p10, med, p90], "samples": len(smp),
                        "source": sampler.source})
    return out


# ------------------------------------------------------------------ workloads

def _fwd_line(c, ms_list, per=1, timing="", variant="tiled", ceil=None, bound="mfma"):
    s = stats_us(ms_list, per)
    med_s = s["median_us"] * 1e-6
    tf = c.flops() / med_s / 1e12
    gbs = c.bytes() / med_s / 1e9
    d = {"workload": c.name, "variant": variant, "timing": timing, **s,
         "tflops": round(tf, 2), "pct_bf16_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2),
         "gbs": round(gbs, 1), "pct_hbm_peak": round(100 * gbs / PEAK_HBM_GBS, 2)}
    if ceil:
        if bound == "mfma" and ceil.get("mfma_bf16"):
            d["pct_measured_mfma_ceiling"] = round(100 * tf / ceil["mfma_bf16"]["tflops_median"], 2)
        if bound == "hbm" and ceil.get("read_32mib_rotating"):
            d["pct_measured_read_ceiling"] = round(100 * gbs / ceil["read_32mib_rotating"]["gbs"], 2)
    return d


def run_fwd_case(rg, c, steps, warmup, rotate=1, variant="auto", graph=False, ceil=None,
                 bound=None):
    """One forward workload.  graph=True: `steps` launches (rotating over
    `rotate` operand sets) captured in one HIP graph, replays timed; else
    back-to-back eager launches, each timed."""
    import torch
    import synth
    sets = [synth.fwd_case_on_device(
        synth.FwdCase(c.name, c.group, c.case + 100 * i, c.M, c.N, c.K, c.r, c.alpha, c.dtype,
                      var_b=c.var_b) if i else c) for i in range(rotate)]
    outs = [torch.empty((c.M, c.N), dtype=sets[0]["X"].dtype, device="cuda") for _ in sets]

    def fn(i):
        s = sets[i % rotate]
        rg.fwd(s["X"], s["W"], s["A"], s["B"], c.scale, out=outs[i % rotate], variant=variant)

    vname = variant if variant != "auto" else (
        "decode" if rg.fwd_pick(rg.LORA_BF16, c.M, c.N, c.K, c.r) == 2 else "tiled")
    if bound is None:
        bound = "hbm" if c.M <= 64 else "mfma"
    if graph:
        reps = graph_replays(fn, steps, 10)
        d = _fwd_line(c, reps, per=steps, variant=vname, ceil=ceil, bound=bound,
                      timing=f"HIP graph of {steps} launches over {rotate} operand sets; "
                             "statistics over replays, per launch")
        key = {1: ("fwd_decode_m1_w4096_r16", "fwd_decode.hip"),
               8: ("fwd_decode_m8_w4096_r16", "fwd_decode.hip"),
               64: ("fwd_tiled_decode_m64_w4096_r16", "fwd_tiled.hip")}.get(c.M)
        if key and c.N == 4096 and c.K == 4096 and c.r == 16:
            tr = _traffic(key[0], [key[1], "common.h"])
            d["traffic_bytes_per_launch"] = tr["hbm_bytes_per_launch"] if tr else None
        return d
    times, _, _ = per_launch(fn, steps, warmup)
    return _fwd_line(c, times, variant=vname, ceil=ceil, bound=bound,
                     timing="back-to-back launches, HIP events around each")


def run_merge_pass(rg, steps, warmup, layers=36, ceil=None):
    """All 36 x 7 targets on one stream: one pass = one lora_merge_batch call
    (HIP graph replays, and eagerly), and for comparison one lora_merge launch
    per target (a HIP graph of the 252 launches)."""
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

    descs = (rg.MergeDesc * len(tg))(*[
        rg.MergeDesc(t.N, t.K, t.r, w0[i].data_ptr(), t.K, b[i].data_ptr(), t.r, a[i].data_ptr(),
                     t.K, t.scale, wi[i].data_ptr(), t.K) for i, t in enumerate(tg)])

    def batch(_):
        st = rg.merge_batch_raw(rg.LORA_BF16, descs, torch.cuda.current_stream().cuda_stream)
        assert st == rg.LORA_OK, rg.status_str(st)

    reps = graph_replays(batch, 1, steps, warmup)
    eager, _, _ = per_launch(batch, steps, warmup)
    per_target = graph_replays(launch, len(tg), max(3, steps // 4), warmup)
    total_bytes = sum(t.bytes() for t in tg)
    s = stats_us(reps)
    med = s["median_us"] * 1e-6
    shape_ms = {}
    for i, t in enumerate(tg[:7]):
        r_ = graph_replays(lambda j, i=i: launch(i + 7 * j), layers, 5)
        ms = pct(r_)[1] / layers
        shape_ms[t.name.split(".")[1]] = {
            "shape": [t.N, t.K], "median_us": round(ms * 1e3, 2),
            "gbs": round(t.bytes() / (ms * 1e-3) / 1e9, 1)}
    gbs = total_bytes / med / 1e9
    d = {"workload": f"merge_from_pristine_{layers}x7_targets_r32",
         "timing": "HIP graph of one lora_merge_batch call over the 252 targets; statistics "
                   "over replays",
         **{"pass_" + k: v for k, v in s.items()},
         "eager_pass_median_us": stats_us(eager)["median_us"],
         "one_launch_per_target_pass_median_us": stats_us(per_target)["median_us"],
         "gbs": round(gbs, 1), "pct_hbm_peak": round(100 * gbs / PEAK_HBM_GBS, 2),
         "bytes_per_pass": int(total_bytes), "per_target_shape": shape_ms}
    if ceil and ceil.get("copy_1gib"):
        d["pct_measured_copy_ceiling"] = round(100 * gbs / ceil["copy_1gib"]["gbs_median"], 2)
    tr = _traffic("merge_batch_36x7_r32_pass", ["merge.hip", "common.h"])
    d["traffic_bytes_per_pass"] = tr["hbm_bytes_per_launch"] if tr else None
    return d


def run_decode_step(rg, steps, warmup, layers=36):
    """One decode token (M = 1) through the projections of 36 layers that read
    the same input: q, k, v (hidden 2560 -> 4096, 1024, 1024) and gate, up
    (2560 -> 9728, 9728), rank 32.  Per layer: two lora_fwd_batch calls (one
    per shared input) against five lora_fwd calls; both captured in HIP graphs
    (one launch is shorter than the host's per-call cost).  The batched
    calls run with and without a workspace (with one, T is computed once per
    forward, by the first workgroups of the same launch).  The weights of 36 layers (4.7 GB) do
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

    w_ms = pct(graph_replays(batched_ws, 1, steps, warmup))[1]
    b_ms = pct(graph_replays(batched, 1, steps, warmup))[1]
    s_ms = pct(graph_replays(single, 1, steps, warmup))[1]
    return {
        "workload": f"decode_step_{layers}_layers_qkv_gateup_m1_r32",
        "timing": "HIP graph of one decode step (all layers), median over replays",
        "step_us_batched_with_workspace": round(w_ms * 1e3, 2),
        "step_us_batched": round(b_ms * 1e3, 2),
        "step_us_one_launch_per_projection": round(s_ms * 1e3, 2),
        "launches_per_layer": {"batched_with_workspace": len(groups),
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
    """One backward workload (lora_bwd: four launches), back-to-back eager
    passes with events around each, and a HIP graph of passes."""
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

    graph_ms = pct(graph_replays(fn, steps, 3))[1] / steps
    times, _, _ = per_launch(fn, steps, warmup)
    s = stats_us(times)
    f = bwd_flops(c)
    med = s["median_us"] * 1e-6
    return {"workload": "bwd_" + c.name,
            "timing": "back-to-back eager backward passes (4 launches each), events around each",
            **{"pass_" + k: v for k, v in s.items()},
            "graph_replay_us_per_pass": round(graph_ms * 1e3, 3),
            "tflops": round(f / med / 1e12, 2),
            "pct_bf16_peak": round(100 * f / med / 1e12 / PEAK_BF16_TFLOPS, 2),
            "algorithmic_flop_per_pass": f, "workspace_bytes": need}


# ------------------------------------------------------------- the oracle

def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _time_oracle(fn, budget_s, min_runs=1):
    n, t0 = 0, time.perf_counter()
    while True:
        fn()
        n += 1
        dt = time.perf_counter() - t0
        if n >= min_runs and dt >= budget_s:
            return dt / n, n


def _sample_rows(M, n, seed):
    """n seeded rows spread over [0, M): one from each of n equal blocks."""
    import numpy as np
    rng = np.random.default_rng(seed)
    edges = np.linspace(0, M, n + 1).astype(np.int64)
    return np.array([rng.integers(edges[i], max(edges[i] + 1, edges[i + 1])) for i in range(n)])


def oracle_timing(gpu_us, head_baseline=None, head_name=None, quick=False):
    """The fp64 oracle as it is, on the host cores: per config wall time and
    achieved GFLOP/s on all cores (full passes, or labelled row samples of
    the large shapes: an output row costs the same whichever row it is), the
    GPU speed-up, and one-core times for the tiny, mid, decode and one merge
    configuration."""
    import numpy as np
    import oracle
    import synth
    threads = len(os.sched_getaffinity(0))
    out = {"cores": threads, "cpu_model": _cpu_model(), "configs": []}
    cases = [(synth.TINY, None), (synth.MID, None), (synth.QPROJ, 512), (synth.VPROJ, 512)]
    cases += [(c, 256) for c in synth.SQUARE if c.name != head_name]
    cases += [(c, None) for c in synth.DECODE]
    if head_baseline is not None:
        # the headline's own timing is the cpu_baseline leg (1024-row sample)
        hb = head_baseline
        e = {"config": head_name, "rows": hb["rows"], "seconds_all_cores": hb["seconds"],
             "gflops_all_cores": round(hb["value"] * 1e3, 2),
             "full_pass_seconds_all_cores": hb["full_pass_seconds"]}
        if head_name in gpu_us:
            e["gpu_speedup"] = round(hb["full_pass_seconds"] / (gpu_us[head_name] * 1e-6), 1)
        out["configs"].append(e)
    single = {synth.TINY.name, synth.MID.name, *(c.name for c in synth.DECODE)}
    for c, rows in cases:
        if quick and c.M > 4096:
            continue
        t = c.make()
        X = t["X"] if rows is None else np.ascontiguousarray(t["X"][_sample_rows(c.M, rows, 1)])
        m = X.shape[0]
        flops = c.flops() * m / c.M
        e = {"config": c.name, "rows": m if rows else "all"}
        oracle.set_threads(threads)
        sec, n = _time_oracle(lambda: oracle.fwd(X, t["W"], t["A"], t["B"], c.scale), 1.0)
        e["seconds_all_cores"] = round(sec, 5)
        e["gflops_all_cores"] = round(flops / sec / 1e9, 2)
        full = sec * c.M / m
        e["full_pass_seconds_all_cores"] = round(full, 4)
        if c.name in gpu_us:
            e["gpu_speedup"] = round(full / (gpu_us[c.name] * 1e-6), 1)
        if c.name in single:
            oracle.set_threads(1)
            sec1, _ = _time_oracle(lambda: oracle.fwd(X, t["W"], t["A"], t["B"], c.scale), 0.5)
            e["seconds_one_core"] = round(sec1, 5)
            e["gflops_one_core"] = round(flops / sec1 / 1e9, 3)
        out["configs"].append(e)
    tgt = synth.merge_targets(1)[4]  # gate: 9728 x 2560
    W0 = tgt.make_w0()
    A, B = tgt.make_ab(0)
    e = {"config": "merge_target_" + tgt.name, "rows": "all"}
    for nt, key in ((threads, "all_cores"), (1, "one_core")):
        oracle.set_threads(nt)
        sec, _ = _time_oracle(lambda: oracle.merge(W0, B, A, tgt.scale), 0.5)
        e["seconds_" + key] = round(sec, 5)
        e["gbs_" + key] = round(tgt.bytes() / sec / 1e9, 3)
    if tgt.name in gpu_us:
        e["gpu_speedup"] = round(e["seconds_all_cores"] / (gpu_us[tgt.name] * 1e-6), 1)
    out["configs"].append(e)
    oracle.set_threads(threads)
    return out


def cpu_baseline(c, rows=1024, budget_s=10.0):
    """The fp64 oracle, as it is, on all host cores, over a seeded sample of
    `rows` output rows of the headline workload (every column), repeated
    until the budget is spent; scaled to TFLOP/s of the algorithmic work."""
    import numpy as np
    import oracle
    t = c.make()
    X = np.ascontiguousarray(t["X"][_sample_rows(c.M, rows, 0)])
    threads = len(os.sched_getaffinity(0))
    oracle.set_threads(threads)
    sec, n = _time_oracle(lambda: oracle.fwd(X, t["W"], t["A"], t["B"], c.scale), budget_s)
    flops = c.flops() * rows / c.M
    return {"value": round(flops / sec / 1e12, 5), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle", "cpu_model": _cpu_model(), "rows": rows,
            "seconds": round(sec, 4), "full_pass_seconds": round(sec * c.M / rows, 2),
            "sample": f"{rows} seeded rows (one per {c.M // rows}-row block) x all {c.N} columns "
                      f"of {c.name}: {flops / 1e9:.1f} GFLOP per pass, {n} pass(es) in "
                      f"{sec * n:.1f} s (a full pass would take {sec * c.M / rows:.0f} s)"}


# ------------------------------------------------------------------ main

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

    head = synth.SQUARE[1]                      # X[16384,8192] W[8192^2] r16
    t = synth.fwd_case_on_device(head)
    Y = torch.empty((head.M, head.N), dtype=torch.bfloat16, device="cuda")

    def step(_):
        rg.fwd(t["X"], t["W"], t["A"], t["B"], head.scale, out=Y)

    times, region_ms, wall = per_launch(step, args.steps, args.warmup)
    ms_per_step = region_ms / args.steps
    # The shader clock under the headline: the driver's current sclk level,
    # sampled every 5 ms over a sustained run of its own (~0.5 s, outside the
    # timed region), the first quarter (the ramp from idle) dropped.
    clk = ClockSampler(period_s=0.005)
    n_clk = max(20, int(0.5 / max(ms_per_step * 1e-3, 1e-6)))
    with clk:
        for i in range(n_clk):
            step(i)
        torch.cuda.synchronize()
    value = head.flops() / (ms_per_step * 1e-3) / 1e12
    s = stats_us(times)
    tr = _traffic("fwd_tiled_square_x16384x8192_w8192_r16", ["fwd_tiled.hip", "common.h"])
    print(f"headline {head.name}: {ms_per_step * 1e3:.1f} us/launch, {value:.1f} TFLOP/s",
          file=sys.stderr, flush=True)

    line = {
        "metric": METRIC,
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
        "data": "synthetic (seeded normal inputs drawn on the device)",
        "config": {"workload": head.name, "M": head.M, "N": head.N, "K": head.K, "r": head.r,
                   "alpha": head.alpha, "accumulate": "fp32", "output": "bf16",
                   "kernel": "fwd_tiled_bf16_kernel 256x256 tile (lora_fwd's choice)"},
        "timing": {**s, "region_ms": round(region_ms, 4), "host_wall_s": round(wall, 4),
                   "method": "HIP events on the launch stream before each launch and after "
                             "the last; value = algorithmic flops x steps / region"},
        "roofline": {"bound": "mfma", "achieved": round(value, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(value / PEAK_BF16_TFLOPS, 4),
                     "traffic": tr["hbm_bytes_per_launch"] if tr else None,
                     "kernel_us_mean": round(ms_per_step * 1e3, 3),
                     "kernel_us_median": s["median_us"],
                     "algorithmic_flop_per_launch": head.flops(),
                     "algorithmic_bytes_per_launch": head.bytes(),
                     "traffic_read_bytes": tr["read_bytes_per_launch"] if tr else None,
                     "traffic_write_bytes": tr["write_bytes_per_launch"] if tr else None},
        "gpu_clock": {**clk.report(), "window": f"{n_clk} back-to-back headline launches "
                                                 "after the timed region"},
    }
    med_clk = line["gpu_clock"].get("median_mhz_after_first_quarter")
    if med_clk:
        # 4096 dense bf16 flops per CU and clock, 256 CUs: the peak at the
        # clock the headline ran at.
        at_clock = 256 * 4096 * med_clk * 1e6 / 1e12
        line["roofline"]["peak_at_sampled_clock"] = round(at_clock, 1)
        line["roofline"]["frac_at_sampled_clock"] = round(value / at_clock, 4)
    del t, Y
    torch.cuda.empty_cache()

    gpu_us = {head.name: s["median_us"]}
    if not args.quick:
        ceil = run_ceilings()
        line["ceilings"] = ceil
        mf = ceil["mfma_bf16"]["tflops_median"]
        line["roofline"]["pct_measured_mfma_ceiling"] = round(100 * value / mf, 2)
        work = []
        for c in (synth.QPROJ, synth.VPROJ):
            work.append(run_fwd_case(rg, c, 30, 5, ceil=ceil))
        for c in synth.SQUARE:
            if c is not head:
                work.append(run_fwd_case(rg, c, 10, 2, ceil=ceil))
        for c in synth.DECODE:
            work.append(run_fwd_case(rg, c, 256, 32, rotate=16, graph=True, ceil=ceil))
        work.append(run_decode_step(rg, 10, 2))
        work.append(run_merge_pass(rg, 8, 2, ceil=ceil))
        for c in (synth.MID, synth.QPROJ):
            work.append(run_bwd_case(rg, c, 20, 3))
        # short kernels: timed in HIP graphs (a launch is shorter than the host's
        # per-call cost)
        work.append(run_fwd_case(rg, synth.MID, 50, 10, graph=True, ceil=ceil))
        work.append(run_fwd_case(rg, synth.TINY, 50, 10, graph=True))
        line["workloads"] = work
        for w in work:
            if "median_us" in w:
                gpu_us[w["workload"]] = w["median_us"]
        mp = [w for w in work if w["workload"].startswith("merge_from_pristine")]
        if mp:
            gate = mp[0]["per_target_shape"].get("gate")
            if gate:
                gpu_us["l0.gate"] = gate["median_us"]

    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(head)
        if not args.quick:
            line["oracle_timing"] = oracle_timing(gpu_us, line["cpu_baseline"], head.name)
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
        times, _, _ = per_launch(lambda _: dst.copy_(src), steps, warmup)
        ms = pct(times)[1]
        res = {"workload": f"copy_{n}_bytes", "median_us": ms * 1e3,
               "gbs": 2 * n / (ms * 1e-3) / 1e9}
    elif name.startswith("ceil_"):
        res = run_ceilings(steps)
    elif name == "clock":
        res = run_clock_phases()
    else:
        raise SystemExit(f"unknown --only {name}")
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
