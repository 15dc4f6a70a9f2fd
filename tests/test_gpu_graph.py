"""Capture in a HIP graph (through torch.cuda.CUDAGraph) and replay.

The library allocates nothing, clears nothing with memset and never
synchronises, so a call can be captured on the caller's stream. Each test
captures one call, replays it several times with eager work and
synchronisation between the replays (the output is overwritten with NaN
before every replay), and checks every replay against the eager result bit
for bit."""
import pytest
import torch

import workloads as wlmod

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def va():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import video_diffusion_transformer_rope3d_amd as m
    return m


def _inputs(seed):
    wl = wlmod.custom(1, 2, (3, 11, 17), 128, (44, 42, 42), dtype="bf16", seed_id=seed)
    g = torch.Generator().manual_seed(seed)
    q, k, v = ((torch.randn((wl.B, wl.heads, wl.N, wl.d), generator=g) * 0.5).to(torch.bfloat16).cuda()
               for _ in range(3))
    return wl, q, k, v


def _capture_and_replay(call, out, replays=3):
    call()
    torch.cuda.synchronize()
    ref = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()  # warm-up on the side stream, as torch asks before a capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for _ in range(replays):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


def test_graph_replays_fused_attention(va):
    wl, q, k, v = _inputs(950)
    o = torch.empty_like(q)
    ws = va.workspace_for(q, True)
    _capture_and_replay(lambda: va.attention(q, k, v, scale=wl.scale, grid=wl.grid, split=wl.split,
                                             theta=wl.theta, out=o, workspace=ws), o)


@pytest.mark.parametrize("layout", ["rows", "patches"])
def test_graph_replays_window_attention(va, layout):
    wl, q, k, v = _inputs(951)
    o = torch.empty_like(q)
    B, H, N, d = q.shape
    n = va.vidattn_fwd_window_workspace_size(0, B, H, N, d, True, va.WindowDesc.make(wl.grid, (1, 2, 3), layout))
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    _capture_and_replay(lambda: va.window_attention(q, k, v, (1, 2, 3), grid=wl.grid, split=wl.split,
                                                    theta=wl.theta, layout=layout, out=o, workspace=ws), o)


def _prepared(va, seed):
    wl, q, k, v = _inputs(seed)
    rope = dict(grid=wl.grid, split=wl.split, theta=wl.theta)
    return wl, q, k, v, rope


def test_graph_replays_prepare_then_subset(va):
    """The two-phase path: the key/value pre-pass and a query-subset
    attention, captured together."""
    wl, q, k, v, rope = _prepared(va, 952)
    idx = torch.tensor([0, 5, 200, 560, 333, 5], dtype=torch.int32, device="cuda")
    q_sub = q[:, :, idx.long()].contiguous()
    o = torch.empty_like(q_sub)
    ws = va.workspace_for(q, True)

    def call():
        va.prepare(k, v, workspace=ws, **rope)
        va.attend_subset(q_sub, idx, ws, wl.N, scale=wl.scale, out=o, **rope)

    _capture_and_replay(call, o)


def test_graph_replays_block_sparse_lists_and_mask(va):
    """Block-sparse attention from lists, and from a bit mask (whose list
    building kernel runs inside the captured call)."""
    import numpy as np
    wl, q, k, v, rope = _prepared(va, 953)
    nqb, nkb = -(-wl.N // va.SPARSE_Q_BLOCK), -(-wl.N // va.SPARSE_K_BLOCK)
    blocks = np.full((wl.B, wl.heads, nqb, nkb), -1, dtype=np.int32)
    count = np.zeros((wl.B, wl.heads, nqb), dtype=np.int32)
    mask = np.zeros((wl.B, wl.heads, nqb, nkb), dtype=bool)
    rng = np.random.default_rng(953)
    for ix in np.ndindex(count.shape):
        sel = np.sort(rng.choice(nkb, size=int(rng.integers(1, nkb + 1)), replace=False))
        blocks[ix][:len(sel)] = sel
        count[ix] = len(sel)
        mask[ix][sel] = True
    bt, ct = torch.from_numpy(blocks).cuda(), torch.from_numpy(count).cuda()
    words = torch.from_numpy(wlmod.block_mask_words(mask).view(np.int32)).cuda()
    ws = va.prepare(k, v, **rope)
    o = torch.empty_like(q)
    _capture_and_replay(lambda: va.attend_block_sparse(q, ws, bt, ct, scale=wl.scale, out=o, **rope), o)
    wsm = va.block_mask_workspace_for(q, True)
    va.prepare(k, v, workspace=wsm, **rope)
    om = torch.empty_like(q)
    _capture_and_replay(lambda: va.attend_block_mask(q, wsm, words, scale=wl.scale, out=om, **rope), om)
    assert torch.equal(om.view(torch.int16), o.view(torch.int16))
