"""Shape-keyed tile-configuration tuner for the fused LoRA forward.

After "fastaf: Minimal LoRA fine-tuning with hand-written Triton kernels",
section "Block size tuning": candidate configurations are pruned with the
device's limits (threads per workgroup, LDS per workgroup, the register
budget, a minimum occupancy), the survivors are timed on the GPU, and the
fastest is cached per shape in a JSON file.  A shape missing from the cache
takes the choice of the nearest cached shape; with no usable entry the
library's own choice (lora_fwd) is used.

Candidates are the tiled configurations of lora_fwd_tile (ids 0-19 except
the retired id 5, each at the ranks it is instantiated for; see
include/lora.h) and, for bf16 with M <= 64 and r <= 32, the weight-streaming
decode kernel ("decode").  Pruning rules, in order:
  * threads per workgroup above the device's limit;
  * dynamic LDS above the per-workgroup limit;
  * register budget: a configuration that spills (scratch bytes > 0), or that
    the occupancy calculator cannot place on a CU (0 workgroups per CU);
  * minimum occupancy: a grid of fewer workgroups than min_grid_frac x CUs
    (unless every candidate falls below it: then those with the largest grid
    stay).

    python -m rank_gemm_amd.tune --shapes 4096x1024x1024x16,8192x4096x2560x32
    python -m rank_gemm_amd.tune --preset bench          # the benchmark's shapes

Cache file: $RANK_GEMM_AMD_TILE_CACHE, else ~/.cache/rank_gemm_amd/tiles.json.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import time
from dataclasses import dataclass
from typing import Dict, Iterable, List, Optional, Sequence, Tuple

DECODE = "decode"
CACHE_VERSION = 1


def default_cache_path() -> str:
    env = os.environ.get("RANK_GEMM_AMD_TILE_CACHE")
    if env:
        return env
    return os.path.join(os.path.expanduser("~"), ".cache", "rank_gemm_amd", "tiles.json")


def pad_rank(r: int) -> int:
    for p in (16, 32, 64, 128):
        if r <= p:
            return p
    return 256


def shape_key(dtype: str, M: int, N: int, K: int, r: int) -> str:
    return f"{dtype}:{M}:{N}:{K}:{r}"


def parse_key(key: str) -> Tuple[str, int, int, int, int]:
    dt, M, N, K, r = key.split(":")
    return dt, int(M), int(N), int(K), int(r)


@dataclass
class Candidate:
    name: str              # "tile:<id>" or "decode"
    threads: int
    lds_bytes: int
    scratch_bytes: int
    blocks_per_cu: int
    grid: int              # workgroups this shape launches


@dataclass
class Limits:
    compute_units: int
    lds_per_block: int
    max_threads_per_block: int


def tile_grid(bm: int, bn: int, group: int, M: int, N: int) -> int:
    return -(-M // bm) * -(-N // (bn * group))


def prune(cands: Sequence[Candidate], lim: Limits,
          min_grid_frac: float = 0.5) -> Tuple[List[Candidate], Dict[str, str]]:
    """The survivors, and for each pruned candidate the rule that removed it."""
    why: Dict[str, str] = {}
    keep: List[Candidate] = []
    for c in cands:
        if c.threads > lim.max_threads_per_block:
            why[c.name] = f"threads {c.threads} > {lim.max_threads_per_block}"
        elif c.lds_bytes > lim.lds_per_block:
            why[c.name] = f"LDS {c.lds_bytes} > {lim.lds_per_block}"
        elif c.scratch_bytes > 0:
            why[c.name] = f"register spill ({c.scratch_bytes} B scratch per lane)"
        elif c.blocks_per_cu < 1:
            why[c.name] = "no workgroup fits on a CU"
        else:
            keep.append(c)
    need = min_grid_frac * lim.compute_units
    full = [c for c in keep if c.grid >= need]
    if full:
        for c in keep:
            if c.grid < need:
                why[c.name] = f"grid {c.grid} workgroups < {need:g}"
        return full, why
    if keep:
        top = max(c.grid for c in keep)
        for c in keep:
            if c.grid < top:
                why[c.name] = f"grid {c.grid} workgroups (largest is {top})"
        return [c for c in keep if c.grid == top], why
    return [], why


class TileCache:
    """Per-shape choices: {key: {"choice": name, "us": {name: time}, ...}}."""

    def __init__(self, entries: Optional[Dict[str, dict]] = None, device: str = ""):
        self.entries: Dict[str, dict] = dict(entries or {})
        self.device = device

    @classmethod
    def load(cls, path: Optional[str] = None) -> "TileCache":
        path = path or default_cache_path()
        try:
            with open(path) as f:
                data = json.load(f)
        except (OSError, ValueError):
            return cls()
        if data.get("version") != CACHE_VERSION:
            return cls()
        return cls(data.get("entries", {}), data.get("device", ""))

    def save(self, path: Optional[str] = None) -> str:
        path = path or default_cache_path()
        os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
        tmp = path + ".tmp"
        with open(tmp, "w") as f:
            json.dump({"version": CACHE_VERSION, "device": self.device, "entries": self.entries},
                      f, indent=1, sort_keys=True)
        os.replace(tmp, path)
        return path

    def lookup(self, dtype: str, M: int, N: int, K: int, r: int) -> Optional[str]:
        """The cached choice for this shape, else the nearest cached shape's
        (same dtype and padded rank; distance = sum of |log2| ratios of M, N,
        K) when that choice can run this shape, else None."""
        e = self.entries.get(shape_key(dtype, M, N, K, r))
        if e is not None and valid_for(e["choice"], dtype, M, r):
            return e["choice"]
        best: Optional[Tuple[float, str]] = None
        for key, e in self.entries.items():
            dt, m, n, k, rr = parse_key(key)
            if dt != dtype or pad_rank(rr) != pad_rank(r) or not valid_for(e["choice"], dtype, M, r):
                continue
            d = sum(abs(math.log2(max(a, 1) / max(b, 1))) for a, b in ((M, m), (N, n), (K, k)))
            if best is None or d < best[0]:
                best = (d, e["choice"])
        return best[1] if best else None


def valid_for(choice: str, dtype: str, M: int, r: int) -> bool:
    """Whether a cached choice can run a shape (the decode kernel needs bf16,
    M <= 64 and r <= 32; a tile id must be instantiated for the rank)."""
    if dtype != "bf16":
        return False
    if choice == DECODE:
        return M <= 64 and r <= 32
    if not choice.startswith("tile:"):
        return False
    tid = int(choice.split(":")[1])
    return _tile_ranks(tid, r)


def _tile_ranks(tid: int, r: int) -> bool:
    # Same table as include/lora.h (checked against lora_tile_get_info by the
    # tests); id 5 is retired (never instantiated); ids 14 and 19 start at
    # rank 64.
    limit = {0: 32, 1: 256, 2: 128, 3: 128, 4: 64, 6: 128, 7: 64, 8: 128, 9: 32,
             10: 64, 11: 64, 12: 64, 13: 32, 14: 128, 15: 64, 16: 64, 17: 64, 18: 64,
             19: 128}.get(tid)
    low = {14: 64, 19: 64}.get(tid, 16)
    return limit is not None and low <= pad_rank(r) <= limit


# ---------------------------------------------------------------- on the GPU

def candidates(rg, M: int, N: int, K: int, r: int) -> List[Candidate]:
    out = []
    for tid in range(rg.TILE_COUNT):
        info = rg.tile_info(tid, r)
        if info is None:
            continue
        use = rg.tile_usage(tid, r)
        out.append(Candidate(f"tile:{tid}", info.waves * 64, info.lds_bytes, use.scratch_bytes,
                             use.blocks_per_cu,
                             tile_grid(info.bm, info.bn, info.group, M, N)))
    if M <= rg.DECODE_MAX_M and r <= 32:
        # 8 waves, one workgroup per 16 rows of W; its LDS is small.
        out.append(Candidate(DECODE, 512, 0, 0, 1, -(-N // 16)))
    return out


def _time_us(fn, count: int = 20, replays: int = 5) -> float:
    """Per-launch time of `fn` from HIP graph replays (min over replays)."""
    import torch
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for _ in range(count):
                fn()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    best = float("inf")
    for _ in range(replays):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1) * 1e3 / count)
    return best


def tune_shape(rg, M: int, N: int, K: int, r: int, min_grid_frac: float = 0.5,
               count: int = 20, replays: int = 5) -> dict:
    """Prune, time every survivor (and lora_fwd's own choice), return the entry."""
    import torch
    lim_c = rg.device_limits()
    lim = Limits(lim_c.compute_units, lim_c.lds_per_block, lim_c.max_threads_per_block)
    keep, why = prune(candidates(rg, M, N, K, r), lim, min_grid_frac)
    dev = "cuda"
    g = torch.Generator(device=dev)
    g.manual_seed(1234)
    X = torch.randn((M, K), generator=g, device=dev).to(torch.bfloat16)
    W = (torch.randn((N, K), generator=g, device=dev) / math.sqrt(K)).to(torch.bfloat16)
    A = (torch.randn((r, K), generator=g, device=dev) / math.sqrt(K)).to(torch.bfloat16)
    B = (torch.randn((N, r), generator=g, device=dev) * math.sqrt(0.02)).to(torch.bfloat16)
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    us: Dict[str, float] = {}
    fns = {}
    default_fn = lambda: rg.fwd(X, W, A, B, 2.0, out=Y)  # noqa: E731
    # lora_fwd's own choice first, and again with the winner at the end: a
    # figure taken right after a slow candidate can be several percent off
    # (the clock settles with the load), so each keeps its best.
    default_us = _time_us(default_fn, count, replays)
    for c in keep:
        if c.name == DECODE:
            fn = lambda: rg.fwd(X, W, A, B, 2.0, out=Y, variant="decode")  # noqa: E731
        else:
            tid = int(c.name.split(":")[1])
            fn = lambda tid=tid: rg.fwd(X, W, A, B, 2.0, out=Y, tile=tid)  # noqa: E731
        fns[c.name] = fn
        us[c.name] = round(_time_us(fn, count, replays), 3)
    choice = min(us, key=us.get) if us else None
    if choice is not None:
        us[choice] = round(min(us[choice], _time_us(fns[choice], count, replays)), 3)
    default_us = round(min(default_us, _time_us(default_fn, count, replays)), 3)
    choice = min(us, key=us.get) if us else None
    return {"choice": choice, "us": us, "default_us": default_us, "pruned": why}


def tune(rg, shapes: Iterable[Tuple[int, int, int, int]], cache: TileCache,
         log=print, **kw) -> TileCache:
    import torch
    cache.device = torch.cuda.get_device_properties(0).name
    for (M, N, K, r) in shapes:
        t0 = time.time()
        e = tune_shape(rg, M, N, K, r, **kw)
        if e["choice"] is not None:
            cache.entries[shape_key("bf16", M, N, K, r)] = e
        log(f"{M}x{N}x{K} r{r}: choice {e['choice']} "
            f"({e['us'].get(e['choice'], float('nan')):.2f} us; lora_fwd {e['default_us']:.2f} us); "
            f"timed {sorted(e['us'].items(), key=lambda kv: kv[1])}; pruned {e['pruned']} "
            f"[{time.time() - t0:.1f} s]")
    return cache


BENCH_SHAPES = [
    (4096, 1024, 1024, 16),      # mid-size forward (the headline)
    (8192, 4096, 2560, 32),      # q_proj
    (8192, 1024, 2560, 32),      # v_proj
    (16384, 8192, 8192, 16),     # square, r 16
    (16384, 8192, 8192, 128),    # square, r 128
    (1, 4096, 4096, 16), (8, 4096, 4096, 16), (64, 4096, 4096, 16),   # decode-shaped
    (8192, 2560, 4096, 32),      # the q_proj backward's dX product
    (2048, 2048, 2048, 16),      # a square that fills 256 128 x 128 tiles
    (1024, 1024, 2048, 16),      # 64 128 x 128 tiles: a smaller tile fills the CUs
    (256, 4096, 4096, 16),       # few tokens, W streamed by many workgroups
]


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--shapes", default="", help="comma list of MxNxKxR")
    ap.add_argument("--preset", choices=["bench"], default=None)
    ap.add_argument("--cache", default=None, help="cache file (default: %(default)s)")
    ap.add_argument("--min-grid-frac", type=float, default=0.5)
    args = ap.parse_args(argv)
    shapes: List[Tuple[int, int, int, int]] = []
    if args.preset == "bench":
        shapes += list(dict.fromkeys(BENCH_SHAPES))
    for s in filter(None, args.shapes.split(",")):
        M, N, K, r = (int(v) for v in s.lower().split("x"))
        shapes.append((M, N, K, r))
    if not shapes:
        ap.error("no shapes (--shapes or --preset)")
    import rank_gemm_amd as rg
    cache = TileCache.load(args.cache)
    tune(rg, shapes, cache, log=lambda m: print(m, flush=True), min_grid_frac=args.min_grid_frac)
    print("cache:", cache.save(args.cache), flush=True)
    return 0


if __name__ == "__main__":
    raise SystemExit(main())
