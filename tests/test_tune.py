"""The tile tuner's host logic: pruning rules, cache lookup (exact, nearest,
fallback), the JSON file, and the tile table it assumes against the
library's own (lora_tile_get_info, no HIP call)."""
import pytest

import rank_gemm_amd as rg
from rank_gemm_amd import tune

LIM = tune.Limits(compute_units=256, lds_per_block=160 * 1024, max_threads_per_block=1024)


def C(name, threads=512, lds=64 * 1024, scratch=0, blocks=1, grid=1024):
    return tune.Candidate(name, threads, lds, scratch, blocks, grid)


def test_prune_rules_in_order():
    cands = [C("tile:a", threads=2048), C("tile:b", lds=200 * 1024), C("tile:c", scratch=20),
             C("tile:d", blocks=0), C("tile:e", grid=64), C("tile:f"), C("tile:g", grid=128)]
    keep, why = tune.prune(cands, LIM)
    assert [c.name for c in keep] == ["tile:f", "tile:g"]
    assert "threads" in why["tile:a"] and "LDS" in why["tile:b"]
    assert "spill" in why["tile:c"] and "fits" in why["tile:d"]
    assert "grid" in why["tile:e"]


def test_prune_keeps_largest_grid_when_all_small():
    keep, why = tune.prune([C("tile:a", grid=8), C("tile:b", grid=32), C("tile:c", grid=32)], LIM)
    assert sorted(c.name for c in keep) == ["tile:b", "tile:c"]
    assert "largest" in why["tile:a"]


def test_prune_everything_infeasible():
    keep, why = tune.prune([C("tile:a", scratch=4)], LIM)
    assert keep == [] and "tile:a" in why


def test_tile_grid():
    assert tune.tile_grid(128, 128, 1, 4096, 1024) == 256
    assert tune.tile_grid(128, 128, 4, 4096, 1024) == 64
    assert tune.tile_grid(256, 256, 1, 300, 257) == 4


def test_lookup_exact_nearest_and_fallback(tmp_path):
    cache = tune.TileCache({
        tune.shape_key("bf16", 4096, 1024, 1024, 16): {"choice": "tile:1"},
        tune.shape_key("bf16", 16384, 8192, 8192, 16): {"choice": "tile:4"},
        tune.shape_key("bf16", 8, 4096, 4096, 16): {"choice": "decode"},
        tune.shape_key("bf16", 16384, 8192, 8192, 128): {"choice": "tile:3"},
    })
    assert cache.lookup("bf16", 4096, 1024, 1024, 16) == "tile:1"
    assert cache.lookup("bf16", 4096, 1024, 1024, 12) == "tile:1"          # same padded rank
    assert cache.lookup("bf16", 12000, 8192, 8192, 16) == "tile:4"          # nearest
    assert cache.lookup("bf16", 3000, 1536, 1024, 16) == "tile:1"
    assert cache.lookup("bf16", 4, 4096, 4096, 16) == "decode"
    # the nearest shape's choice cannot run here: decode needs M <= 64
    assert cache.lookup("bf16", 128, 4096, 4096, 16) in ("tile:1", "tile:4")
    # rank 128 has only the rank-128 entry; rank 64 none of its class
    assert cache.lookup("bf16", 1000, 1000, 1000, 100) == "tile:3"
    assert cache.lookup("bf16", 1000, 1000, 1000, 64) is None
    assert cache.lookup("f32", 4096, 1024, 1024, 16) is None
    assert tune.TileCache().lookup("bf16", 4096, 1024, 1024, 16) is None
    # JSON round trip
    p = cache.save(str(tmp_path / "sub" / "tiles.json"))
    again = tune.TileCache.load(p)
    assert again.entries == cache.entries
    assert tune.TileCache.load(str(tmp_path / "missing.json")).entries == {}


def test_cache_version_mismatch_is_ignored(tmp_path):
    p = tmp_path / "t.json"
    p.write_text('{"version": 999, "entries": {"bf16:1:1:1:1": {"choice": "tile:1"}}}')
    assert tune.TileCache.load(str(p)).entries == {}


def test_tile_table_matches_library():
    """The rank limits tune.py assumes are the library's instantiations."""
    for tid in range(rg.TILE_COUNT):
        for r in (1, 16, 17, 32, 33, 64, 65, 128, 129, 256):
            info = rg.tile_info(tid, r)
            assert (info is not None) == tune.valid_for(f"tile:{tid}", "bf16", 100, r), (tid, r)
            if info is not None:
                assert info.tile == tid and info.rank_pad == tune.pad_rank(r)
                assert info.lds_bytes <= 160 * 1024
                assert info.waves * 64 <= 1024
                assert info.k_split == (2 if tid == 7 else 1)
    assert rg.tile_info(rg.TILE_COUNT, 16) is None
    assert rg.tile_info(-1, 16) is None
    assert int(rg.lib().lora_tile_get_info(0, 0, None)) in (rg.LORA_ERR_NULL, rg.LORA_ERR_SHAPE)
