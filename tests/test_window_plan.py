"""The planning rules of the local-window attention, on the CPU. Row layout:
for every 256-query block the list must hold each 64-key tile that holds a
key inside some query's box (checked by brute force over all query-key pairs
on small grids), ascending and without repeats. Patch layout: for every
16 x 16 query patch the list must be exactly the 8 x 8 key patches that
hold such a key. The rules are the ones bench.py uses to count FLOPs; a GPU
test checks that the planning kernels write the same lists, and the layout
the library picks is the one these rules say lists fewer tiles."""
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


PATCH_CASES = CASES + [
    ((2, 16, 32), (1, 7, 7)),
    ((2, 24, 40), (0, 8, 8)),
    ((3, 33, 18), (1, 9, 2)),
    ((1, 7, 5), (0, 2, 2)),      # smaller than one patch
    ((2, 17, 17), (1, 0, 0)),
]


def patch_tiles_brute(grid, radius):
    """Per query patch (frame-major), the key patches (tile index
    (tf*ceil(H/8) + ty)*ceil(W/8) + tx) holding a key inside some query's
    box, by brute force over all query-key pairs."""
    F, H, W = grid
    n = np.arange(F * H * W)
    f, y, x = n // (H * W), (n // W) % H, n % W
    tile = (f * -(-H // 8) + y // 8) * -(-W // 8) + x // 8
    out = []
    for pf in range(F):
        for py in range(-(-H // 16)):
            for px in range(-(-W // 16)):
                q = n[(f == pf) & (y // 16 == py) & (x // 16 == px)]
                vis = ((np.abs(f[q][:, None] - f[None, :]) <= radius[0])
                       & (np.abs(y[q][:, None] - y[None, :]) <= radius[1])
                       & (np.abs(x[q][:, None] - x[None, :]) <= radius[2]))
                out.append(sorted(set(tile[np.nonzero(vis.any(axis=0))[0]].tolist())))
    return out


@pytest.mark.parametrize("grid,radius", PATCH_CASES, ids=lambda c: "x".join(map(str, c)))
def test_patch_plan_lists_are_exactly_the_visible_patches(grid, radius):
    wl = wlmod.custom(1, 1, grid, 64, (16, 24, 24))
    assert bench.window_patch_lists(wl, radius) == patch_tiles_brute(grid, radius)


def test_library_picks_the_layout_that_lists_fewer_tiles():
    """The window workspace size reveals the layout the library resolved
    for VIDATTN_WINDOW_AUTO (the key/value image has ceil(N/64) tiles per
    (b, head) in rows, F*ceil(H/8)*ceil(W/8) in patches); it must be the
    one the restated rules say lists fewer key tiles, and a forced layout
    must give that layout's size."""
    import video_diffusion_transformer_rope3d_amd as va

    def size(nqb, nkt, cap, d=64):  # the image, the counts, lists of cap entries per block
        return 256 * d * nkt + (4 * nqb + 255) // 256 * 256 + 4 * nqb * cap

    cases = PATCH_CASES + [((21, 45, 80), r) for r in ((1, 7, 7), (1, 3, 3), (0, 0, 80), (2, 1, 1), (21, 45, 80))]
    picked = set()
    for grid, radius in cases:
        wl = wlmod.custom(1, 1, grid, 64, (16, 24, 24))
        F, H, W = grid
        rows = size(-(-wl.N // 256), -(-wl.N // 64), max(bench.window_plan_counts(wl, radius, "rows")))
        patches = size(F * -(-H // 16) * -(-W // 16), F * -(-H // 8) * -(-W // 8),
                       max(bench.window_plan_counts(wl, radius, "patches")))
        want = bench.window_layout(wl, radius)
        picked.add(want)
        got = {lay: va.vidattn_fwd_window_workspace_size(va.BF16, 1, 1, wl.N, 64, True,
                                                         va.WindowDesc.make(grid, radius, lay))
               for lay in ("auto", "rows", "patches")}
        assert got["rows"] == rows and got["patches"] == patches, (grid, radius)
        assert got["auto"] == (patches if want == "patches" else rows), (grid, radius, want)
    assert picked == {"rows", "patches"}


def test_window_size_query_rejects_a_bad_window():
    import video_diffusion_transformer_rope3d_amd as va
    ok = va.WindowDesc.make((2, 3, 4), (1, 1, 1))
    assert va.vidattn_fwd_window_workspace_size(va.BF16, 1, 1, 24, 64, True, ok) > 0
    for bad in (None, va.WindowDesc.make((2, 3, 5), (1, 1, 1)), va.WindowDesc.make((2, 3, 4), (1, -1, 1)),
                va.WindowDesc.make((2, 3, 4), (1, 1, 1), 3)):
        assert va.vidattn_fwd_window_workspace_size(va.BF16, 1, 1, 24, 64, True, bad) == 0


def test_auto_layout_falls_back_to_rows_past_the_patch_limit():
    """A grid of 2^22 or more key patches cannot take the patch layout: the
    automatic choice gives the row layout's workspace there, and a forced
    patch layout is refused (size 0). Lists hold as many entries per block
    as the most any block lists, so even these 2^24-token grids need lists
    of a few MB, not of N^2/4096 entries."""
    import video_diffusion_transformer_rope3d_amd as va
    N = 1 << 24
    grid = (1 << 16, 1, 256)  # 2^16 * 1 * 32 = 2^21 key patches: still allowed
    ok = va.vidattn_fwd_window_workspace_size(va.BF16, 1, 1, N, 64, False, va.WindowDesc.make(grid, (0, 0, 1), "patches"))
    # one frame, one tile row, and columns 16p-1 .. 16p+16: tiles 2p-1 .. 2p+2, 4 at most
    nqb, cap = (1 << 16) * 16, 4
    assert ok == 256 * 64 * (1 << 16) * 32 + (4 * nqb + 255) // 256 * 256 + 4 * nqb * cap
    grid = (1 << 24, 1, 1)  # 2^24 key patches
    # rows: a block's 256 one-token frames, radius 0 in frames: the block's own 4 tiles
    rows = 256 * 64 * (N // 64) + (4 * (N // 256) + 255) // 256 * 256 + 4 * (N // 256) * 4
    assert va.vidattn_fwd_window_workspace_size(va.BF16, 1, 1, N, 64, False,
                                                va.WindowDesc.make(grid, (0, 0, 1), "auto")) == rows
    assert va.vidattn_fwd_window_workspace_size(va.BF16, 1, 1, N, 64, False,
                                                va.WindowDesc.make(grid, (0, 0, 1), "patches")) == 0


@pytest.mark.parametrize("grid", [(2, 16, 32), (3, 33, 18), (1, 7, 5), (21, 45, 80)], ids=lambda g: "x".join(map(str, g)))
def test_block_rows_cover_every_token_once(grid):
    """The query rows bench.py counts per block (for the visited-pair FLOPs)
    add up to N in both layouts, and a patch never counts more than 256."""
    wl = wlmod.custom(1, 1, grid, 64, (16, 24, 24))
    for layout in ("rows", "patches"):
        rows = bench.window_block_rows(wl, layout)
        assert sum(rows) == wl.N and max(rows) <= 256 and min(rows) >= 1
