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
