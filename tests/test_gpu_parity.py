"""Parity of the HIP path (through the C ABI) with the fp64 CPU oracle on
the same seeded inputs, plus structural invariants. Needs an MI355X."""
import math

import numpy as np
import pytest

import oracle
import workloads as wlmod
from tests import parity

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def va():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import video_diffusion_transformer_rope3d_amd as m
    return m


def _log(msg):
    print(msg, flush=True)


# ------------------------------------------------------------------ rotation alone

def _ulp(x, mant_bits):
    ax = np.maximum(np.abs(x), 2.0 ** -14 if mant_bits == 10 else 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(ax)) - mant_bits)


@pytest.mark.parametrize("in_dt,out_dt", [("bf16", "bf16"), ("bf16", "f16"), ("bf16", "f32"), ("f32", "f32"),
                                          ("f32", "bf16")])
@pytest.mark.parametrize("shape", [((4, 8, 8), 64, (16, 24, 24)), ((21, 30, 52), 128, (44, 42, 42)),
                                   ((3, 5, 7), 128, (44, 42, 42))])
def test_rope3d_standalone(va, in_dt, out_dt, shape):
    grid, d, split = shape
    wl = wlmod.custom(2, 3, grid, d, split, dtype=in_dt, seed_id=300, std=(1.0, 1.0, 1.0))
    _log(f"rope3d {in_dt}->{out_dt} grid={grid} d={d}")
    x_h = wlmod.full(wl, "q")
    x = parity.to_torch(x_h)
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[out_dt]
    prescale = 0.75
    y = va.rope3d(x, grid, split, wl.theta, out_dtype=tdt, prescale=prescale)
    torch.cuda.synchronize()
    got = parity.from_torch(y) if out_dt != "f16" else y.double().cpu().numpy()
    ref = oracle.rope3d(parity.decode(wl, x_h), grid, split, wl.theta) * prescale
    err = np.abs(got - ref)
    mag = 1.0 + np.abs(ref)
    if out_dt == "f32":
        tol = 2e-6 * mag
    else:
        tol = 0.5 * _ulp(ref, 7 if out_dt == "bf16" else 10) + 2e-6 * mag
    assert np.all(err <= tol), float(np.max(err - tol))


@pytest.mark.parametrize("grid,d,split,shards", [
    ((3, 5, 7), 128, (44, 42, 42), [(0, 105), (0, 1), (17, 40), (104, 1), (60, 45)]),
    ((21, 30, 52), 64, (16, 24, 24), [(0, 8190), (8190, 8190), (24570, 8190), (32000, 760), (12345, 6789)]),
])
@pytest.mark.parametrize("in_dt,out_dt", [("bf16", "bf16"), ("f32", "f32")])
def test_rope3d_token_shards(va, grid, d, split, shards, in_dt, out_dt):
    """A run of tokens rotated with its global positions (a sequence shard):
    against the oracle at those positions, and bit for bit the matching rows
    of the whole-grid rotation."""
    wl = wlmod.custom(2, 3, grid, d, split, dtype=in_dt, seed_id=310, std=(1.0, 1.0, 1.0))
    _log(f"rope3d shards {in_dt}->{out_dt} grid={grid} d={d}")
    x_h = wlmod.full(wl, "q")
    x = parity.to_torch(x_h)
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32}[out_dt]
    whole = va.rope3d(x, grid, split, wl.theta, out_dtype=tdt, prescale=0.75)
    pos = oracle.grid_positions(grid)
    for off, n in shards:
        part = va.rope3d(x[:, :, off:off + n].contiguous(), grid, split, wl.theta, token_offset=off, out_dtype=tdt,
                         prescale=0.75)
        torch.cuda.synchronize()
        assert torch.equal(part.view(torch.int16) if tdt == torch.bfloat16 else part,
                           whole[:, :, off:off + n].view(torch.int16) if tdt == torch.bfloat16
                           else whole[:, :, off:off + n]), (off, n)
        got = parity.from_torch(part)
        ref = oracle.rope3d_at(parity.decode(wl, x_h[:, :, off:off + n]), pos[off:off + n], split, wl.theta) * 0.75
        err = np.abs(got - ref)
        mag = 1.0 + np.abs(ref)
        tol = 2e-6 * mag if out_dt == "f32" else 0.5 * _ulp(ref, 7) + 2e-6 * mag
        assert np.all(err <= tol), (off, n, float(np.max(err - tol)))


def test_rope3d_in_place_matches_out_of_place(va):
    wl = wlmod.custom(1, 2, (5, 6, 7), 128, (44, 42, 42), seed_id=301)
    x = parity.to_torch(wlmod.full(wl, "k"))
    a = va.rope3d(x, wl.grid, wl.split, 1e4)
    va.rope3d(x, wl.grid, wl.split, 1e4, out=x)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), x.view(torch.int16))


# ------------------------------------------------------------------ attention, small shapes (every row)

SMALL = [
    # grid, d, split, dtype, B, heads
    ((1, 1, 1), 128, (44, 42, 42), "bf16", 1, 1),     # N = 1
    ((1, 1, 7), 64, (16, 24, 24), "bf16", 1, 2),      # N = 7 < one tile
    ((2, 4, 8), 128, (44, 42, 42), "bf16", 1, 1),     # N = 64, one full key tile
    ((3, 5, 7), 128, (44, 42, 42), "bf16", 2, 2),     # N = 105, ragged
    ((2, 9, 11), 64, (16, 24, 24), "bf16", 1, 3),     # N = 198, d = 64
    ((3, 11, 17), 128, (44, 42, 42), "bf16", 1, 2),   # N = 561: several tiles + tail
    ((5, 13, 17), 128, (44, 42, 42), "bf16", 1, 1),   # N = 1105
    ((4, 8, 8), 64, (16, 24, 24), "f32", 1, 4),       # the fp32 workload shape
    ((3, 5, 7), 128, (44, 42, 42), "f32", 2, 1),      # fp32 d=128, ragged
    ((1, 1, 1), 64, (16, 24, 24), "f32", 1, 1),       # fp32 N = 1
    ((3, 7, 9), 64, (0, 32, 32), "f32", 1, 2),        # empty frame chunk
    # uneven splits: the axis boundaries fall inside and between the
    # 4-pair groups of the two lane halves in other places
    ((3, 5, 7), 128, (2, 2, 124), "bf16", 1, 1),
    ((3, 5, 7), 128, (124, 2, 2), "bf16", 1, 1),
    ((3, 5, 7), 128, (6, 0, 122), "bf16", 1, 1),      # empty row chunk
    ((2, 9, 11), 64, (0, 64, 0), "bf16", 1, 1),       # rows only
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"{c[3]}-{c[0][0]}x{c[0][1]}x{c[0][2]}-d{c[1]}")
@pytest.mark.parametrize("rope", [True, False], ids=["rope", "norope"])
def test_attention_small(va, case, rope):
    grid, d, split, dt, B, H = case
    wl = wlmod.custom(B, H, grid, d, split, dtype=dt, seed_id=400 + d + len(grid),
                      std=(1.0, 1.0, 1.0) if dt == "f32" else (0.5, 0.5, 0.5))
    _log(f"attention {wl.name} rope={rope}")
    host = parity.host_inputs(wl)
    o = parity.run_gpu(wl, host, rope=rope)
    torch.cuda.synchronize()
    st = parity.compare(wl, host, o, rope=rope)
    _log(f"  {st}")
    assert parity.within(wl, st), st


# ------------------------------------------------------------------ the five workloads (sampled rows)

@pytest.mark.parametrize("wid", [1, 2, 3, 4, 5])
def test_workload_parity(va, wid):
    wl = wlmod.WORKLOADS[wid]
    _log(f"workload {wl.name}: generating inputs")
    host = parity.host_inputs(wl)
    _log("  running HIP path")
    o = parity.run_gpu(wl, host)
    torch.cuda.synchronize()
    _log("  oracle on sampled rows")
    st = parity.compare(wl, host, o)
    _log(f"  {st}")
    assert parity.within(wl, st), st
    del o
    torch.cuda.empty_cache()


def test_tensors_beyond_4_gib(va):
    """3 x 80 heads of the 21x45x80 grid (75600 tokens), d = 128: each of Q,
    K, V, O holds 4.6 GB and the key/value workspace 9.3 GB: (b, head) slice
    i starts at byte i * 19.4 MB of its tensor, beyond 2^31 from i = 111 on
    and beyond 2^32 from i = 222 on. Slices 0, 120 and 239 carry seeded inputs
    and are checked on 256 sampled rows each; every other head is zero
    (heads do not interact), so its output must be exactly zero."""
    import dataclasses
    wl = dataclasses.replace(wlmod.custom(3, 80, (21, 45, 80), 128, (44, 42, 42), seed_id=720), full_rows=False)
    checked = [(0, 0), (1, 40), (2, 79)]
    shape = (wl.B, wl.heads, wl.N, wl.d)
    _log(f"large {wl.name}: {4 * wl.B * wl.heads * wl.N * wl.d * 2 / 1e9:.1f} GB of q, k, v, o")
    dev = {n: torch.zeros(shape, dtype=torch.bfloat16, device="cuda") for n in ("q", "k", "v")}
    host = {}
    for (b, h) in checked:
        for n in ("q", "k", "v"):
            host[(n, b, h)] = wlmod.slice_values(wl, n, b, h)
            dev[n][b, h].copy_(parity.to_torch(host[(n, b, h)]))
    o = va.attention(dev["q"], dev["k"], dev["v"], scale=wl.scale, grid=wl.grid, split=wl.split, theta=wl.theta)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all().item())
    for (b, h) in [(0, 1), (1, 39), (1, 41), (2, 78)]:
        assert o[b, h].abs().max().item() == 0.0, (b, h)
    parts = []
    for (b, h) in checked:
        rows = wlmod.sample_rows(wl, b, h)
        got = parity.from_torch(o[b, h].index_select(0, torch.from_numpy(rows).cuda()))
        q, k, v = (oracle.decode_bf16(host[(n, b, h)]) for n in ("q", "k", "v"))
        ref = oracle.rope_attention(q, k, v, wl.grid, wl.split, wl.theta, wl.scale, rows=rows)
        e = np.abs(got - ref)
        parts.append((float(e.max()), float(e.sum()), float(np.abs(ref).sum())))
        _log(f"  head ({b}, {h}): max_abs {parts[-1][0]:.3g}, mean_rel {parts[-1][1] / parts[-1][2]:.3g}")
    st = dict(max_abs=max(p[0] for p in parts), mean_rel=sum(p[1] for p in parts) / sum(p[2] for p in parts),
              finite=True)
    assert parity.within(wl, st), st
    del o, dev
    torch.cuda.empty_cache()


def test_no_device_memory_beyond_the_buffers(va):
    """A call on the 2 x 10 heads x 75600-token workload, with the output and
    workspace supplied, leaves the device's free memory unchanged: nothing
    of the 75600^2 scores per head (23 GB in fp32) is ever stored."""
    wl = wlmod.WORKLOADS[3]
    shape = (wl.B, wl.heads, wl.N, wl.d)
    q, k, v = (torch.randn(shape, device="cuda").mul_(0.5).to(torch.bfloat16) for _ in range(3))
    o = torch.empty_like(q)
    ws = va.workspace_for(q, True)
    kw = dict(scale=wl.scale, grid=wl.grid, split=wl.split, theta=wl.theta, out=o, workspace=ws)
    va.attention(q, k, v, **kw)
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    peak0 = torch.cuda.max_memory_allocated()
    va.attention(q, k, v, **kw)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert free1 == free0
    assert torch.cuda.max_memory_allocated() == peak0
    assert ws.numel() == 4 * wl.B * wl.heads * (-(-wl.N // 64) * 64) * wl.d


# ------------------------------------------------------------------ invariants (no oracle)

def _rand(shape, dt, seed, std=0.5):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(shape, generator=g) * std
    return x.to(dt).cuda()


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_zero_query_gives_mean_of_v(va, dt):
    grid, split = (3, 6, 9), (44, 42, 42)
    shape = (1, 2, 162, 128)
    q = torch.zeros(shape, dtype=dt, device="cuda")
    k, v = _rand(shape, dt, 1), _rand(shape, dt, 2)
    o = va.attention(q, k, v, grid=grid, split=split)
    ref = v.double().mean(dim=2, keepdim=True).expand_as(o)
    tol = 1e-5 if dt == torch.float32 else 4e-3
    assert (o.double() - ref).abs().max().item() <= tol


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_unit_values_give_one(va, dt):
    shape = (2, 2, 300, 128)
    q, k = _rand(shape, dt, 3, 1.0), _rand(shape, dt, 4, 1.0)
    v = torch.ones(shape, dtype=dt, device="cuda")
    o = va.attention(q, k, v, grid=(3, 10, 10), split=(44, 42, 42))
    tol = 1e-6 if dt == torch.float32 else 4e-3
    assert (o.double() - 1.0).abs().max().item() <= tol


def test_single_token_gives_v(va):
    shape = (2, 3, 1, 128)
    q, k, v = (_rand(shape, torch.bfloat16, s) for s in (5, 6, 7))
    o = va.attention(q, k, v, grid=(1, 1, 1), split=(44, 42, 42))
    assert torch.equal(o.view(torch.int16), v.view(torch.int16))


def test_many_slices_single_token(va):
    """270000 (batch, head) slices of one token each: the pre-pass and the
    rotation spread the slices over the grid's second dimension, which must
    stay within 65535 blocks, and one key gives O = V exactly."""
    B, H, d = 1, 270000, 64
    _log(f"many slices B={B} heads={H} N=1 d={d}")
    q, k, v = (_rand((B, H, 1, d), torch.bfloat16, 70 + i) for i in range(3))
    o = va.attention(q, k, v, grid=(1, 1, 1), split=(16, 24, 24))
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), v.view(torch.int16))
    r = va.rope3d(q, (1, 1, 1), (16, 24, 24), 1e4)
    torch.cuda.synchronize()
    assert torch.equal(r.view(torch.int16), q.view(torch.int16))  # position (0, 0, 0) is the identity


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_bitwise_deterministic_and_overwrites_poison(va, dt):
    shape = (2, 4, 1105, 128)
    q, k, v = (_rand(shape, dt, s) for s in (8, 9, 10))
    o1 = torch.full(shape, float("nan"), dtype=dt, device="cuda")
    o2 = torch.full(shape, float("nan"), dtype=dt, device="cuda")
    va.attention(q, k, v, grid=(5, 13, 17), split=(44, 42, 42), out=o1)
    va.attention(q, k, v, grid=(5, 13, 17), split=(44, 42, 42), out=o2)
    torch.cuda.synchronize()
    assert torch.isfinite(o1).all()
    assert torch.equal(o1.view(torch.int16 if dt == torch.bfloat16 else torch.int32),
                       o2.view(torch.int16 if dt == torch.bfloat16 else torch.int32))


def test_guard_regions_untouched(va):
    """Outputs and workspace are written only inside their extents."""
    shape = (1, 2, 561, 128)
    n = math.prod(shape)
    guard = 4096
    q, k, v = (_rand(shape, torch.bfloat16, s) for s in (11, 12, 13))
    obuf = torch.full((n + 2 * guard,), 7.0, dtype=torch.bfloat16, device="cuda")
    o = obuf[guard:guard + n].view(shape)
    wsn = va.vidattn_fwd_workspace_size(va.BF16, 1, 2, 561, 128, True)
    wbuf = torch.full((wsn + 2 * guard,), 0x5A, dtype=torch.uint8, device="cuda")
    ws = wbuf[guard:guard + wsn]
    va.attention(q, k, v, grid=(3, 11, 17), split=(44, 42, 42), out=o, workspace=ws)
    torch.cuda.synchronize()
    assert (obuf[:guard] == 7.0).all() and (obuf[guard + n:] == 7.0).all()
    assert (wbuf[:guard] == 0x5A).all() and (wbuf[guard + wsn:] == 0x5A).all()


def test_no_rope_matches_prerotated(va):
    """rope=NULL with pre-rotated fp32 inputs equals the fused rotation."""
    wl = wlmod.custom(1, 2, (3, 5, 7), 128, (44, 42, 42), dtype="f32", seed_id=500, std=(1, 1, 1))
    host = parity.host_inputs(wl)
    q, k, v = (parity.to_torch(host[n]) for n in ("q", "k", "v"))
    qr = va.rope3d(q, wl.grid, wl.split, wl.theta)
    kr = va.rope3d(k, wl.grid, wl.split, wl.theta)
    a = va.attention(q, k, v, grid=wl.grid, split=wl.split, theta=wl.theta)
    b = va.attention(qr, kr, v)
    torch.cuda.synchronize()
    assert (a - b).abs().max().item() <= 2e-6


def test_error_status_raises(va):
    q = torch.zeros((1, 1, 10, 96), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(va.VidattnError) as e:
        va.attention(q, q.clone(), q.clone())
    assert e.value.status == 2


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("rope", [True, False], ids=["rope", "norope"])
def test_two_phase_equals_fused_bitwise(va, dt, rope):
    wl = wlmod.custom(2, 3, (3, 11, 17), 128, (44, 42, 42), dtype=dt, seed_id=600)
    host = parity.host_inputs(wl)
    q, k, v = (parity.to_torch(host[n]) for n in ("q", "k", "v"))
    kw = dict(grid=wl.grid, split=wl.split, theta=wl.theta) if rope else {}
    fused = va.attention(q, k, v, **kw)
    ws = va.prepare(k, v, **kw)
    a1 = va.attend(q, k, v, ws, **kw)
    a2 = va.attend(q, k, v, ws, **kw)  # the workspace is only read
    torch.cuda.synchronize()
    iv = torch.int16 if dt == "bf16" else torch.int32
    assert torch.equal(fused.view(iv), a1.view(iv)) and torch.equal(a1.view(iv), a2.view(iv))


# ------------------------------------------------------------------ softmax edge cases
# The kernel keeps the running maximum lazily: it redoes a tile against the
# exact maximum only when some probability exp2(s - m - 20) reaches 2. These
# cases drive each branch of that rule, dense, block-sparse and windowed,
# against the oracle on every row. Flash attention must reproduce the plain
# softmax exactly (vidax summary, "2 System Architecture & Design", heading
# "3D RoPE, 3D VAEs, and flash attention"), so the bound is the usual bf16 one.

EDGE_N, EDGE_D = 1000, 128
EDGE_CASES = {
    # a late key 25-34 log2 units above the running maximum (finite exact step),
    # then a later one 111-167 above it (exp2 overflows to +inf for most rows)
    "late_dominant": [[(330, 2.0), (600, 10.5)], [(700, 2.0), (980, 10.5)]],
    # the first tile holds the maximum of every row: by ~48 and by ~7 log2 units
    "first_tile_dominant": [[(5, 3.75)], [(40, 0.5)]],
    # identical key rows in several tiles (and twice in one tile): exact ties
    "ties": [[(100, 4.0), (101, 4.0), (500, 4.0), (900, 4.0)], [(63, 4.0), (64, 4.0), (999, 4.0)]],
}


def _edge_inputs(case):
    q, k, v = wlmod.planted_keys(EDGE_N, EDGE_D, 2, EDGE_CASES[case])
    return q, k, v


def _edge_compare(got_t, ref_fn, heads=2):
    got = parity.from_torch(got_t)
    err = ref = 0.0
    worst = 0.0
    for h in range(heads):
        r = ref_fn(h)
        e = np.abs(got[0, h] - r)
        worst = max(worst, float(e.max()))
        err += float(e.sum())
        ref += float(np.abs(r).sum())
    assert np.isfinite(got).all()
    assert worst <= 2e-2 and err / ref <= 5e-3, (worst, err / ref)
    return worst, err / ref


@pytest.mark.parametrize("case", sorted(EDGE_CASES))
def test_softmax_edge_dense(va, case):
    _log(f"softmax edge dense {case}")
    qh, kh, vh = _edge_inputs(case)
    q, k, v = (parity.to_torch(x) for x in (qh, kh, vh))
    scale = 1.0 / math.sqrt(EDGE_D)
    o = va.attention(q, k, v, scale=scale)
    torch.cuda.synchronize()
    dec = oracle.decode_bf16
    stats = _edge_compare(o, lambda h: oracle.attention(dec(qh[0, h]), dec(kh[0, h]), dec(vh[0, h]), scale))
    _log(f"  max-abs {stats[0]:.3e} mean-rel {stats[1]:.3e}")


@pytest.mark.parametrize("case", sorted(EDGE_CASES))
def test_softmax_edge_block_sparse(va, case):
    _log(f"softmax edge block-sparse {case}")
    qh, kh, vh = _edge_inputs(case)
    q, k, v = (parity.to_torch(x) for x in (qh, kh, vh))
    scale = 1.0 / math.sqrt(EDGE_D)
    nqb = -(-EDGE_N // va.SPARSE_Q_BLOCK)
    # query block 0: the early and the planted tiles; 1: everything but tiles
    # 9 and 15; 2: tile 9 alone; 3: the ragged last tile alone
    lists = [[0, 1, 5, 7, 9, 10, 14, 15], [t for t in range(16) if t not in (9, 15)], [9], [15]]
    width = max(len(x) for x in lists)
    blocks = np.full((1, 2, nqb, width), -1, dtype=np.int32)
    count = np.zeros((1, 2, nqb), dtype=np.int32)
    for h in range(2):
        for i, x in enumerate(lists):
            blocks[0, h, i, :len(x)] = x
            count[0, h, i] = len(x)
    ws = va.prepare(k, v)
    o = va.attend_block_sparse(q, ws, torch.from_numpy(blocks).cuda(), torch.from_numpy(count).cuda(), scale=scale)
    torch.cuda.synchronize()
    dec = oracle.decode_bf16
    stats = _edge_compare(o, lambda h: oracle.block_sparse_attention(
        dec(qh[0, h]), dec(kh[0, h]), dec(vh[0, h]), None, None, None, scale, blocks[0, h], count[0, h],
        va.SPARSE_Q_BLOCK, va.SPARSE_K_BLOCK))
    _log(f"  max-abs {stats[0]:.3e} mean-rel {stats[1]:.3e}")


@pytest.mark.parametrize("case", sorted(EDGE_CASES))
@pytest.mark.parametrize("grid,radius", [((4, 10, 25), (1, 3, 6)), ((2, 4, 125), (1, 1, 20))])
@pytest.mark.parametrize("layout", ["rows", "patches"])
def test_softmax_edge_window(va, case, grid, radius, layout):
    _log(f"softmax edge window {case} grid={grid} radius={radius} layout={layout}")
    qh, kh, vh = _edge_inputs(case)
    q, k, v = (parity.to_torch(x) for x in (qh, kh, vh))
    scale = 1.0 / math.sqrt(EDGE_D)
    o = va.window_attention(q, k, v, radius, grid=grid, rope=False, scale=scale, layout=layout)
    torch.cuda.synchronize()
    dec = oracle.decode_bf16
    stats = _edge_compare(o, lambda h: oracle.window_attention(
        dec(qh[0, h]), dec(kh[0, h]), dec(vh[0, h]), grid, None, None, scale, radius, rope=False))
    _log(f"  max-abs {stats[0]:.3e} mean-rel {stats[1]:.3e}")


def test_side_stream_buffers_follow_the_stream(va):
    """attention() on a side stream, workspace and output left to the
    binding: both are allocated on that stream, so the caching allocator
    cannot hand the dropped workspace to work queued on the current stream
    while the side stream's kernels still use it. Allocations filled with
    junk on the current stream right after each call must not disturb the
    result (bit for bit against the same call on the current stream)."""
    wl = wlmod.custom(1, 4, (6, 20, 64), 128, (44, 42, 42), seed_id=911)
    _log(f"side stream {wl.name}")
    host = parity.host_inputs(wl)
    q, k, v = (parity.to_torch(host[n]) for n in ("q", "k", "v"))
    kw = dict(scale=wl.scale, grid=wl.grid, split=wl.split, theta=wl.theta)
    ref = va.attention(q, k, v, **kw)
    torch.cuda.synchronize()
    nbytes = va.vidattn_fwd_workspace_size(va.BF16, wl.B, wl.heads, wl.N, wl.d, True)
    side = torch.cuda.Stream()
    for _ in range(3):
        side.wait_stream(torch.cuda.current_stream())
        o = va.attention(q, k, v, stream=side, **kw)
        junk = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
        junk.fill_(0xFF)
        junk_o = torch.empty_like(q)
        junk_o.fill_(float("nan"))
        torch.cuda.current_stream().wait_stream(side)
        assert torch.equal(o.view(torch.int16), ref.view(torch.int16))
        del junk, junk_o
    torch.cuda.synchronize()
