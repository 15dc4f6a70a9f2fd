"""Parity of the query-subset, block-sparse and local-window attention (HIP path through
the C ABI) with the fp64 CPU oracle on the same seeded inputs, plus the
identities that tie them to the dense attention. Needs an MI355X."""
import numpy as np
import pytest

import oracle
import workloads as wlmod
from tests import parity

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

QB, KB = 256, 64  # query / key block sizes of the block-sparse entry point


@pytest.fixture(scope="module")
def va():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import video_diffusion_transformer_rope3d_amd as m
    assert (m.SPARSE_Q_BLOCK, m.SPARSE_K_BLOCK) == (QB, KB)
    return m


def _log(msg):
    print(msg, flush=True)


def _prepare(va, wl, host, rope=True):
    q, k, v = (parity.to_torch(host[n]) for n in ("q", "k", "v"))
    kw = dict(grid=wl.grid, split=wl.split, theta=wl.theta) if rope else {}
    ws = va.prepare(k, v, **kw)
    return q, k, v, ws, kw


def _stats(got, ref):
    e = np.abs(got - ref)
    sr = float(np.abs(ref).sum())
    return dict(max_abs=float(e.max()) if e.size else 0.0, mean_rel=float(e.sum()) / sr if sr > 0 else 0.0,
                finite=bool(np.all(np.isfinite(got))))


def _within(st):
    t = parity.TOL["bf16"]
    return st["finite"] and st["max_abs"] <= t["max_abs"] and st["mean_rel"] <= t["mean_rel"]


def _merge(parts):
    return dict(max_abs=max(p["max_abs"] for p in parts), mean_rel=max(p["mean_rel"] for p in parts),
                finite=all(p["finite"] for p in parts))


# ------------------------------------------------------------------ query subset

SUBSET_CASES = [
    # grid, d, split, B, H, how the Nq query tokens are chosen
    ((3, 11, 17), 128, (44, 42, 42), 2, 2, "random-with-repeats", 300),
    ((3, 11, 17), 64, (16, 24, 24), 1, 3, "random-with-repeats", 257),
    ((5, 13, 17), 128, (44, 42, 42), 1, 2, "distinct-ascending", 700),
    ((2, 4, 8), 128, (44, 42, 42), 1, 1, "single", 1),
    ((2, 9, 11), 128, (44, 42, 42), 2, 1, "more-rows-than-keys", 500),
]


def _subset_index(wl, how, nq, seed):
    g = np.random.default_rng(seed)
    if how == "distinct-ascending":
        return np.sort(g.choice(wl.N, size=nq, replace=False)).astype(np.int32)
    if how == "single":
        return np.array([wl.N - 1], dtype=np.int32)
    return g.integers(0, wl.N, size=nq).astype(np.int32)


@pytest.mark.parametrize("case", SUBSET_CASES, ids=lambda c: f"{c[5]}-{c[0][0]}x{c[0][1]}x{c[0][2]}-d{c[1]}-nq{c[6]}")
@pytest.mark.parametrize("rope", [True, False], ids=["rope", "norope"])
def test_subset_small(va, case, rope):
    grid, d, split, B, H, how, nq = case
    wl = wlmod.custom(B, H, grid, d, split, seed_id=600 + d + nq)
    host = parity.host_inputs(wl)
    idx = _subset_index(wl, how, nq, seed=nq)
    _log(f"subset {wl.name} nq={nq} {how} rope={rope}")
    _, _, _, ws, kw = _prepare(va, wl, host, rope)
    q_sub = np.ascontiguousarray(host["q"][:, :, idx])
    o = va.attend_subset(parity.to_torch(q_sub), torch.from_numpy(idx).cuda(), ws, wl.N, scale=wl.scale, **kw)
    torch.cuda.synchronize()
    got = parity.from_torch(o)
    parts = []
    for b in range(B):
        for h in range(H):
            qd, kd, vd = (parity.decode(wl, a) for a in (q_sub[b, h], host["k"][b, h], host["v"][b, h]))
            if rope:
                ref = oracle.rope_attention_subset(qd, idx, kd, vd, wl.grid, wl.split, wl.theta, wl.scale)
            else:
                ref = oracle.attention(qd, kd, vd, wl.scale)
            parts.append(_stats(got[b, h], ref))
    st = _merge(parts)
    _log(f"  {st}")
    assert _within(st), st


def test_subset_identity_is_the_dense_attention_bitwise(va):
    wl = wlmod.custom(2, 2, (3, 11, 17), 128, (44, 42, 42), seed_id=620)
    host = parity.host_inputs(wl)
    q, k, v, ws, kw = _prepare(va, wl, host)
    idx = torch.arange(wl.N, dtype=torch.int32, device="cuda")
    a = va.attend_subset(q, idx, ws, wl.N, scale=wl.scale, **kw)
    b = va.attend(q, k, v, ws, scale=wl.scale, **kw)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_subset_rows_equal_gathered_dense_rows_bitwise(va):
    """Each output row depends only on its query and its token index, so a
    gathered subset reproduces the dense rows of those tokens bit for bit."""
    wl = wlmod.custom(1, 2, (5, 13, 17), 128, (44, 42, 42), seed_id=621)
    host = parity.host_inputs(wl)
    q, k, v, ws, kw = _prepare(va, wl, host)
    idx = wlmod.subset_index(wl, 333)
    it = torch.from_numpy(idx).long().cuda()
    a = va.attend_subset(q[:, :, it].contiguous(), it.int(), ws, wl.N, scale=wl.scale, **kw)
    dense = va.attend(q, k, v, ws, scale=wl.scale, **kw)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), dense[:, :, it].contiguous().view(torch.int16))


def test_subset_large(va):
    """The 32760-token grid with a quarter of the tokens active; every active
    row of two (b, head) slices is checked against the oracle."""
    wl = wlmod.WORKLOADS[2]
    host = parity.host_inputs(wl)
    idx = wlmod.subset_index(wl, 8190)
    _log(f"subset {wl.name} nq={len(idx)}")
    _, _, _, ws, kw = _prepare(va, wl, host)
    q_sub = np.ascontiguousarray(host["q"][:, :, idx])
    o = va.attend_subset(parity.to_torch(q_sub), torch.from_numpy(idx).cuda(), ws, wl.N, scale=wl.scale, **kw)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(5).choice(len(idx), size=256, replace=False))
    parts = []
    for (b, h) in [(0, 0), (wl.B - 1, wl.heads - 1)]:
        got = parity.from_torch(o[b, h, torch.from_numpy(rows).cuda()])
        qd, kd, vd = (parity.decode(wl, a) for a in (q_sub[b, h], host["k"][b, h], host["v"][b, h]))
        ref = oracle.rope_attention_subset(qd, idx, kd, vd, wl.grid, wl.split, wl.theta, wl.scale, rows=rows)
        parts.append(_stats(got, ref))
    st = _merge(parts)
    _log(f"  {st}")
    assert _within(st), st


# ------------------------------------------------------------------ block sparse

def _random_lists(wl, seed, max_blocks, empty_every=0):
    """Ascending lists of random length (0 .. max_blocks), the last key block
    (the ragged one) always among the candidates."""
    g = np.random.default_rng(seed)
    nqb, nkb = -(-wl.N // QB), -(-wl.N // KB)
    blocks = np.full((wl.B, wl.heads, nqb, max_blocks), -1, dtype=np.int32)
    count = np.zeros((wl.B, wl.heads, nqb), dtype=np.int32)
    for b in range(wl.B):
        for h in range(wl.heads):
            for i in range(nqb):
                c = int(g.integers(1, max_blocks + 1))
                if empty_every and (b * wl.heads + h + i) % empty_every == 0:
                    c = 0
                sel = np.sort(g.choice(nkb, size=min(c, nkb), replace=False))
                blocks[b, h, i, :len(sel)] = sel
                count[b, h, i] = len(sel)
    return blocks, count


def _check_sparse(va, wl, host, blocks, count, rope=True, rows=None, slices=None):
    q, _, _, ws, kw = _prepare(va, wl, host, rope)
    o = va.attend_block_sparse(q, ws, torch.from_numpy(blocks).cuda(), torch.from_numpy(count).cuda(),
                               scale=wl.scale, **kw)
    torch.cuda.synchronize()
    parts = []
    for (b, h) in (slices or [(b, h) for b in range(wl.B) for h in range(wl.heads)]):
        r = np.arange(wl.N) if rows is None else rows
        got = parity.from_torch(o[b, h, torch.from_numpy(r).cuda()])
        qd, kd, vd = (parity.decode(wl, host[n][b, h]) for n in ("q", "k", "v"))
        ref = oracle.block_sparse_attention(qd, kd, vd, wl.grid if rope else None, wl.split, wl.theta, wl.scale,
                                            blocks[b, h], count[b, h], QB, KB, rows=r)
        # query blocks without keys must be exactly zero
        empty = count[b, h][r // QB] == 0
        assert np.all(got[empty] == 0.0)
        parts.append(_stats(got, ref))
    return o, _merge(parts)


SPARSE_CASES = [
    # grid, d, split, B, H, max listed key blocks, every n-th query block empty (0: none)
    ((3, 11, 17), 128, (44, 42, 42), 2, 2, 4, 0),
    ((3, 11, 17), 64, (16, 24, 24), 1, 3, 9, 3),
    ((5, 13, 17), 128, (44, 42, 42), 1, 2, 6, 4),
    ((2, 9, 11), 128, (44, 42, 42), 2, 1, 1, 0),
    ((4, 8, 8), 128, (44, 42, 42), 1, 2, 3, 0),
]


@pytest.mark.parametrize("case", SPARSE_CASES, ids=lambda c: f"{c[0][0]}x{c[0][1]}x{c[0][2]}-d{c[1]}-max{c[5]}")
@pytest.mark.parametrize("rope", [True, False], ids=["rope", "norope"])
def test_sparse_small(va, case, rope):
    grid, d, split, B, H, maxb, empty_every = case
    wl = wlmod.custom(B, H, grid, d, split, seed_id=640 + d + maxb)
    host = parity.host_inputs(wl)
    blocks, count = _random_lists(wl, seed=maxb + d, max_blocks=min(maxb, -(-wl.N // KB)), empty_every=empty_every)
    _log(f"sparse {wl.name} max_blocks={blocks.shape[-1]} rope={rope}")
    _, st = _check_sparse(va, wl, host, blocks, count, rope)
    _log(f"  {st}")
    assert _within(st), st


# ------------------------------------------------------------------ block sparse from a bit mask

def _random_mask(wl, seed, density, empty_every=0):
    g = np.random.default_rng(seed)
    nqb, nkb = -(-wl.N // QB), -(-wl.N // KB)
    m = g.random((wl.B, wl.heads, nqb, nkb)) < density
    m[..., nkb - 1] |= g.random((wl.B, wl.heads, nqb)) < 0.5  # the ragged last key block often set
    if empty_every:
        flat = m.reshape(-1, nkb)
        flat[::empty_every] = False
    return m


def _check_mask(va, wl, host, mask, rope=True, rows=None, slices=None):
    q, k, v = (parity.to_torch(host[n]) for n in ("q", "k", "v"))
    kw = dict(grid=wl.grid, split=wl.split, theta=wl.theta) if rope else {}
    ws = va.block_mask_workspace_for(q, rope)
    va.prepare(k, v, workspace=ws, **kw)
    words = torch.from_numpy(wlmod.block_mask_words(mask).view(np.int32)).cuda()
    o = va.attend_block_mask(q, ws, words, scale=wl.scale, **kw)
    torch.cuda.synchronize()
    parts = []
    for (b, h) in (slices or [(b, h) for b in range(wl.B) for h in range(wl.heads)]):
        r = np.arange(wl.N) if rows is None else rows
        got = parity.from_torch(o[b, h, torch.from_numpy(r).cuda()])
        qd, kd, vd = (parity.decode(wl, host[n][b, h]) for n in ("q", "k", "v"))
        ref = oracle.block_mask_attention(qd, kd, vd, wl.grid if rope else None, wl.split, wl.theta, wl.scale,
                                          mask[b, h], QB, KB, rows=r)
        empty = ~mask[b, h].any(axis=1)[r // QB]
        assert np.all(got[empty] == 0.0)
        parts.append(_stats(got, ref))
    return o, ws, _merge(parts)


MASK_CASES = [
    # grid, d, split, B, H, bit density, every n-th mask row empty (0: none)
    ((3, 11, 17), 128, (44, 42, 42), 2, 2, 0.3, 0),
    ((3, 11, 17), 64, (16, 24, 24), 1, 3, 0.6, 3),
    ((5, 13, 17), 128, (44, 42, 42), 1, 2, 0.15, 4),
    ((2, 45, 80), 128, (44, 42, 42), 1, 1, 0.1, 5),  # 113 key blocks: four mask words per row
]


@pytest.mark.parametrize("case", MASK_CASES, ids=lambda c: f"{c[0][0]}x{c[0][1]}x{c[0][2]}-d{c[1]}-p{c[5]}")
@pytest.mark.parametrize("rope", [True, False], ids=["rope", "norope"])
def test_block_mask_small(va, case, rope):
    grid, d, split, B, H, density, empty_every = case
    wl = wlmod.custom(B, H, grid, d, split, seed_id=760 + d)
    host = parity.host_inputs(wl)
    mask = _random_mask(wl, seed=int(density * 100) + d, density=density, empty_every=empty_every)
    _log(f"block mask {wl.name} density={density} rope={rope}")
    _, _, st = _check_mask(va, wl, host, mask, rope)
    _log(f"  {st}")
    assert _within(st), st


def test_block_mask_equals_the_lists_bitwise(va):
    """The mask path and the list path on the same blocks give the same bits;
    a full mask gives the dense attention's bits."""
    wl = wlmod.custom(2, 2, (4, 15, 29), 128, (44, 42, 42), seed_id=770)
    host = parity.host_inputs(wl)
    mask = _random_mask(wl, seed=771, density=0.35, empty_every=4)
    o_mask, ws, st = _check_mask(va, wl, host, mask)
    assert _within(st), st
    nkb = mask.shape[-1]
    blocks = np.full(mask.shape, -1, dtype=np.int32)
    count = mask.sum(axis=-1).astype(np.int32)
    for idx in np.ndindex(mask.shape[:-1]):
        sel = np.nonzero(mask[idx])[0]
        blocks[idx][:len(sel)] = sel
    q = parity.to_torch(host["q"])
    kw = dict(grid=wl.grid, split=wl.split, theta=wl.theta)
    o_list = va.attend_block_sparse(q, ws, torch.from_numpy(blocks).cuda(), torch.from_numpy(count).cuda(),
                                    scale=wl.scale, **kw)
    full = torch.from_numpy(wlmod.block_mask_words(np.ones_like(mask)).view(np.int32)).cuda()
    o_full = va.attend_block_mask(q, ws, full, scale=wl.scale, **kw)
    o_dense = va.attend(q, parity.to_torch(host["k"]), parity.to_torch(host["v"]), ws, scale=wl.scale, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o_mask.view(torch.int16), o_list.view(torch.int16))
    assert torch.equal(o_full.view(torch.int16), o_dense.view(torch.int16))
    assert nkb == -(-wl.N // KB)


def test_block_mask_large(va):
    """The 32760-token grid (21 x 30 x 52), a 25 % mask, 256 sampled rows of
    two slices."""
    wl = wlmod.WORKLOADS[2]
    host = parity.host_inputs(wl)
    mask = _random_mask(wl, seed=780, density=0.25)
    rows = wlmod.sample_rows(wl, 0, 0)
    _log(f"block mask {wl.name} density=0.25")
    _, _, st = _check_mask(va, wl, host, mask, rows=rows, slices=[(0, 0), (wl.B - 1, wl.heads - 1)])
    _log(f"  {st}")
    assert _within(st), st


def test_sparse_window_and_global_blocks(va):
    """Lists of the kind the pages describe (a local band around the query
    block plus a persistent global set), on a grid of 7 query blocks."""
    wl = wlmod.custom(2, 2, (4, 15, 29), 128, (44, 42, 42), seed_id=660)
    host = parity.host_inputs(wl)
    blocks, count = wlmod.block_lists(wl, QB, KB, window=2, n_global=3)
    _log(f"sparse {wl.name} window lists max={blocks.shape[-1]}")
    _, st = _check_sparse(va, wl, host, blocks, count)
    _log(f"  {st}")
    assert _within(st), st


def test_sparse_all_blocks_is_the_dense_attention_bitwise(va):
    wl = wlmod.custom(2, 2, (3, 11, 17), 128, (44, 42, 42), seed_id=661)
    host = parity.host_inputs(wl)
    q, k, v, ws, kw = _prepare(va, wl, host)
    nqb, nkb = -(-wl.N // QB), -(-wl.N // KB)
    blocks = torch.arange(nkb, dtype=torch.int32, device="cuda").repeat(wl.B, wl.heads, nqb, 1).contiguous()
    count = torch.full((wl.B, wl.heads, nqb), nkb, dtype=torch.int32, device="cuda")
    a = va.attend_block_sparse(q, ws, blocks, count, scale=wl.scale, **kw)
    b = va.attend(q, k, v, ws, scale=wl.scale, **kw)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_sparse_out_of_range_counts_and_indices_are_clamped(va):
    """Counts above max_blocks act as max_blocks and an index past the last
    key block acts as the last key block: same bits as the clamped lists."""
    wl = wlmod.custom(1, 2, (3, 11, 17), 128, (44, 42, 42), seed_id=662)
    host = parity.host_inputs(wl)
    q, _, _, ws, kw = _prepare(va, wl, host)
    nqb, nkb = -(-wl.N // QB), -(-wl.N // KB)
    clean = np.tile(np.array([0, 3, nkb - 1], dtype=np.int32), (wl.B, wl.heads, nqb, 1))
    dirty = clean.copy()
    dirty[..., 2] = 1 << 20
    cnt = np.full((wl.B, wl.heads, nqb), 3, dtype=np.int32)
    over = np.full((wl.B, wl.heads, nqb), 1 << 30, dtype=np.int32)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    a = va.attend_block_sparse(q, ws, t(clean), t(cnt), scale=wl.scale, **kw)
    b = va.attend_block_sparse(q, ws, t(dirty), t(over), scale=wl.scale, **kw)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_sparse_large(va):
    """The 32760-token grid (128 query blocks, 512 key blocks) with local
    band + global lists; 256 sampled rows of two slices."""
    wl = wlmod.WORKLOADS[2]
    host = parity.host_inputs(wl)
    blocks, count = wlmod.block_lists(wl, QB, KB, window=16, n_global=32)
    rows = wlmod.sample_rows(wl, 0, 0)
    _log(f"sparse {wl.name} window=16 global=32 max={blocks.shape[-1]}")
    _, st = _check_sparse(va, wl, host, blocks, count, rows=rows, slices=[(0, 0), (wl.B - 1, wl.heads - 1)])
    _log(f"  {st}")
    assert _within(st), st


# ------------------------------------------------------------------ local window

WINDOW_CASES = [
    # grid, d, split, B, H, radius (frame, row, column)
    ((3, 11, 17), 128, (44, 42, 42), 2, 2, (1, 2, 3)),
    ((3, 11, 17), 64, (16, 24, 24), 1, 3, (0, 1, 1)),
    ((5, 13, 17), 128, (44, 42, 42), 1, 2, (2, 0, 5)),
    ((2, 9, 11), 128, (44, 42, 42), 2, 1, (0, 0, 0)),
    ((6, 5, 7), 128, (44, 42, 42), 1, 2, (1, 4, 2)),
    ((4, 8, 8), 64, (16, 24, 24), 1, 1, (3, 1, 0)),
    # rows of >= 64 tokens: whole-tile test (a tile spans at most two rows)
    ((2, 3, 63), 128, (44, 42, 42), 1, 2, (1, 1, 5)),
    ((2, 3, 64), 128, (44, 42, 42), 1, 2, (1, 1, 5)),
    ((2, 4, 70), 64, (16, 24, 24), 2, 1, (0, 2, 9)),
    ((3, 2, 100), 128, (44, 42, 42), 1, 2, (1, 0, 30)),
    ((2, 3, 129), 128, (44, 42, 42), 1, 1, (1, 1, 200)),
    # per-workgroup cos/sin table: too large for a ring stage (each lane
    # evaluates its angles), for d = 128 and d = 64, and a split with empty
    # frame and column chunks
    ((1, 2, 400), 128, (44, 42, 42), 1, 1, (0, 1, 20)),
    ((1, 2, 200), 64, (16, 24, 24), 1, 2, (0, 1, 9)),
    ((3, 11, 17), 128, (0, 128, 0), 1, 2, (1, 2, 3)),
    # patch layout: whole and ragged 16 x 16 query patches and 8 x 8 key
    # patches, a grid smaller than one patch
    ((2, 16, 32), 128, (44, 42, 42), 1, 2, (1, 7, 7)),
    ((2, 24, 40), 64, (16, 24, 24), 1, 2, (0, 8, 8)),
    ((3, 33, 18), 128, (44, 42, 42), 2, 1, (1, 9, 2)),
    ((1, 7, 5), 128, (44, 42, 42), 1, 1, (0, 2, 2)),
]


def _check_window(va, wl, host, radius, rope=True, rows=None, slices=None, layout="auto"):
    q, k, v = (parity.to_torch(host[n]) for n in ("q", "k", "v"))
    o = va.window_attention(q, k, v, radius, grid=wl.grid, split=wl.split, theta=wl.theta, scale=wl.scale, rope=rope,
                            layout=layout)
    torch.cuda.synchronize()
    parts = []
    for (b, h) in (slices or [(b, h) for b in range(wl.B) for h in range(wl.heads)]):
        r = np.arange(wl.N) if rows is None else rows
        got = parity.from_torch(o[b, h, torch.from_numpy(r).cuda()])
        qd, kd, vd = (parity.decode(wl, host[n][b, h]) for n in ("q", "k", "v"))
        ref = oracle.window_attention(qd, kd, vd, wl.grid, wl.split, wl.theta, wl.scale, radius, rows=r, rope=rope)
        parts.append(_stats(got, ref))
    return o, _merge(parts)


@pytest.mark.parametrize("case", WINDOW_CASES,
                         ids=lambda c: f"{c[0][0]}x{c[0][1]}x{c[0][2]}-d{c[1]}-r{c[5][0]}{c[5][1]}{c[5][2]}")
@pytest.mark.parametrize("rope", [True, False], ids=["rope", "norope"])
@pytest.mark.parametrize("layout", ["rows", "patches"])
def test_window_small(va, case, rope, layout):
    grid, d, split, B, H, radius = case
    wl = wlmod.custom(B, H, grid, d, split, seed_id=680 + d + sum(radius))
    host = parity.host_inputs(wl)
    _log(f"window {wl.name} radius={radius} rope={rope} layout={layout}")
    _, st = _check_window(va, wl, host, radius, rope, layout=layout)
    _log(f"  {st}")
    assert _within(st), st


def test_window_unbounded_is_the_dense_attention_bitwise(va):
    wl = wlmod.custom(2, 2, (3, 11, 17), 128, (44, 42, 42), seed_id=690)
    host = parity.host_inputs(wl)
    q, k, v = (parity.to_torch(host[n]) for n in ("q", "k", "v"))
    kw = dict(grid=wl.grid, split=wl.split, theta=wl.theta, scale=wl.scale)
    a = va.window_attention(q, k, v, (1 << 30, 1 << 30, 1 << 30), **kw)
    b = va.attention(q, k, v, **kw)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("layout", ["rows", "patches"])
def test_window_plan_kernel_writes_the_rule(va, layout):
    """The planning kernels' tile lists (in the workspace tail after a call)
    equal the rules that bench.py counts FLOPs with, on the grids of the CPU
    rule tests."""
    import importlib.util
    import os
    from tests import test_window_plan as rule_tests
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    spec = importlib.util.spec_from_file_location("bench_module", os.path.join(root, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    for grid, radius in (rule_tests.PATCH_CASES if layout == "patches" else rule_tests.CASES):
        wl = wlmod.custom(1, 1, grid, 64, (16, 24, 24), seed_id=700)
        q, k, v = (parity.to_torch(wlmod.full(wl, n)) for n in ("q", "k", "v"))
        desc = va.WindowDesc.make(grid, radius, layout)
        n = va.vidattn_fwd_window_workspace_size(va.BF16, 1, 1, wl.N, wl.d, True, desc)
        ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
        va.window_attention(q, k, v, radius, grid=grid, split=wl.split, layout=layout, workspace=ws)
        torch.cuda.synchronize()
        F, H, W = grid
        if layout == "rows":
            nqb, nkt = -(-wl.N // 256), -(-wl.N // 64)
            want = bench.window_plan_lists(wl, radius)
        else:
            nqb, nkt = F * -(-H // 16) * -(-W // 16), F * -(-H // 8) * -(-W // 8)
            want = bench.window_patch_lists(wl, radius)
        base = 256 * wl.d * nkt  # the key/value image of one (b, head)
        cap = max(len(t) for t in want)  # list rows are as wide as the longest list
        assert n == base + (4 * nqb + 255) // 256 * 256 + 4 * nqb * cap, (grid, radius)
        counts = ws[base:base + 4 * nqb].view(torch.int32).cpu().tolist()
        off = base + (4 * nqb + 255) // 256 * 256
        lists = ws[off:off + 4 * nqb * cap].view(torch.int32).view(nqb, cap).cpu().tolist()
        got = [row[:c] for row, c in zip(lists, counts)]
        assert got == want, (grid, radius)


@pytest.mark.parametrize("layout", ["patches", "rows"])
def test_window_large_wide_rows(va, layout):
    """The 75600-token grid (21 x 45 x 80) with radius (1, 7, 7), in the
    patch layout (the one picked for it) and in rows (whole-tile test); 256
    sampled rows of two slices."""
    wl = wlmod.WORKLOADS[3]
    host = parity.host_inputs(wl)
    rows = wlmod.sample_rows(wl, 0, 0)
    _log(f"window {wl.name} radius=(1, 7, 7) layout={layout}")
    _, st = _check_window(va, wl, host, (1, 7, 7), rows=rows, slices=[(0, 0), (wl.B - 1, wl.heads - 1)],
                          layout=layout)
    _log(f"  {st}")
    assert _within(st), st


@pytest.mark.parametrize("layout", ["patches", "rows"])
def test_window_large(va, layout):
    """The 32760-token grid (21 x 30 x 52) with radius (2, 6, 6), in both
    layouts; 256 sampled rows of two slices."""
    wl = wlmod.WORKLOADS[2]
    host = parity.host_inputs(wl)
    rows = wlmod.sample_rows(wl, 0, 0)
    _log(f"window {wl.name} radius=(2, 6, 6) layout={layout}")
    _, st = _check_window(va, wl, host, (2, 6, 6), rows=rows, slices=[(0, 0), (wl.B - 1, wl.heads - 1)],
                          layout=layout)
    _log(f"  {st}")
    assert _within(st), st


def test_window_patches_d64_ragged_grid(va):
    """The patch layout at d = 64 on a grid whose patches are ragged in both
    axes (44 = 2*16 + 12 rows, 70 = 4*16 + 6 columns), 2 x 3 heads, radius
    (1, 5, 9); 256 sampled rows of two slices."""
    wl = wlmod.custom(2, 3, (6, 44, 70), 64, (16, 24, 24), seed_id=705)
    host = parity.host_inputs(wl)
    rows = wlmod.sample_rows(wl, 0, 0)
    _log(f"window {wl.name} radius=(1, 5, 9) layout=patches")
    _, st = _check_window(va, wl, host, (1, 5, 9), rows=rows, slices=[(0, 0), (wl.B - 1, wl.heads - 1)],
                          layout="patches")
    _log(f"  {st}")
    assert _within(st), st
