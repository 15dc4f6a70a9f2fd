"""The planning rule of the local-window attention, on the CPU: for every
256-query block it must list each 64-key tile that holds a key inside some
query's box (checked by brute force over all query-key pairs on small
grids), ascending and without repeats. The rule is the one bench.py uses to
count FLOPs; a GPU test checks that the planning kernel writes the same
lists."""
import importlib.util
import os

import numpy as np
import pytest

import workloads as wlmod

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
_spec = importlib.util.spec_from_file_location("bench_module", os.path.join(ROOT, "bench.py"))
bench = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(bench)

CASES = [
    ((3, 11, 17), (1, 2, 3)),
    ((5, 13, 17), (2, 0, 5)),
    ((2, 9, 11), (0, 0, 0)),
    ((6, 5, 7), (1, 4, 2)),     # frames of 35 tokens: blocks span many frames
    ((4, 8, 8), (3, 1, 0)),
    ((3, 20, 30), (1, 3, 4)),   # blocks straddling frame boundaries
    ((4, 16, 40), (1, 2, 6)),   # rows inside a block far apart across the boundary
    ((2, 3, 129), (1, 1, 200)),
    ((4, 6, 100), (1, 1, 3)),   # rows of 100 tokens, blocks straddling frames
    ((5, 4, 70), (1, 0, 2)),
    ((3, 9, 64), (2, 1, 5)),
    ((4, 3, 40), (0, 0, 2)),    # blocks covering three frames
    ((5, 3, 40), (1, 0, 1)),
    ((6, 5, 20), (0, 0, 1)),
]


def visible_tiles(grid, radius):
    F, H, W = grid
    N = F * H * W
    n = np.arange(N)
    f, y, x = n // (H * W), (n // W) % H, n % W
    out = []
    for i in range(-(-N // 256)):
        q = n[256 * i:256 * i + 256]
        vis = ((np.abs(f[q][:, None] - f[None, :]) <= radius[0]) & (np.abs(y[q][:, None] - y[None, :]) <= radius[1])
               & (np.abs(x[q][:, None] - x[None, :]) <= radius[2]))
        out.append(set(np.unique(np.nonzero(vis.any(axis=0))[0] // 64).tolist()))
    return out


def whole_row_tiles(grid, radius):
    """The rule by brute force: for each block, every row (f, y) with some
    query of the block at (fq, yq) where |f - fq| <= r_f and |y - yq| <= r_h;
    the tiles holding any token of those rows."""
    F, H, W = grid
    N = F * H * W
    n = np.arange(N)
    out = []
    for i in range(-(-N // 256)):
        q = n[256 * i:256 * i + 256]
        occ = set(zip((q // (H * W)).tolist(), ((q // W) % H).tolist()))
        rows = {(f, y) for (fq, yq) in occ for f in range(F) for y in range(H)
                if abs(f - fq) <= radius[0] and abs(y - yq) <= radius[1]}
        tiles = set()
        for (f, y) in rows:
            tiles.update(range(((f * H + y) * W) // 64, ((f * H + y) * W + W - 1) // 64 + 1))
        out.append(sorted(tiles))
    return out


@pytest.mark.parametrize("grid,radius", CASES, ids=lambda c: "x".join(map(str, c)))
def test_plan_lists_are_the_whole_row_rule(grid, radius):
    wl = wlmod.custom(1, 1, grid, 64, (16, 24, 24))
    assert bench.window_plan_lists(wl, radius) == whole_row_tiles(grid, radius)


@pytest.mark.parametrize("grid,radius", CASES, ids=lambda c: "x".join(map(str, c)))
def test_plan_lists_cover_every_visible_tile(grid, radius):
    wl = wlmod.custom(1, 1, grid, 64, (16, 24, 24))
    lists = bench.window_plan_lists(wl, radius)
    need = visible_tiles(grid, radius)
    nkt = -(-wl.N // 64)
    assert len(lists) == len(need)
    for i, (got, want) in enumerate(zip(lists, need)):
        assert got == sorted(set(got)) and all(0 <= t < nkt for t in got), i
        assert want <= set(got), (i, sorted(want - set(got)))


def test_plan_on_the_benchmark_grid_is_tighter_than_whole_frames():
    wl = wlmod.WORKLOADS[5]
    counts = bench.window_plan_counts(wl, (1, 7, 7))
    assert max(counts) <= 70 and sum(counts) / len(counts) < 63
