"""The Python binding hands the library raw pointers, so it rejects, before any
library call, tensors that are not on the GPU, not contiguous, or (for a
caller-given output or workspace) of the wrong shape, dtype or device. The
CPU tests check the host-tensor case; the GPU tests the others. No test here
reaches a kernel launch."""
import pytest

torch = pytest.importorskip("torch")

GRID, SPLIT = (2, 3, 4), (20, 22, 22)  # 24 tokens, head dim 64


@pytest.fixture(scope="module")
def va():
    import video_diffusion_transformer_rope3d_amd as m
    return m


def _qkv(device, dtype=torch.bfloat16):
    g = torch.Generator().manual_seed(3)
    return [torch.randn(1, 2, 24, 64, generator=g).to(dtype).to(device) for _ in range(3)]


def test_host_tensors_are_rejected(va):
    q, k, v = _qkv("cpu")
    calls = [
        lambda: va.attention(q, k, v, grid=GRID, split=SPLIT),
        lambda: va.prepare(k, v, grid=GRID, split=SPLIT),
        lambda: va.attend(q, k, v, torch.empty(16, dtype=torch.uint8)),
        lambda: va.attend_subset(q, torch.arange(24, dtype=torch.int32), torch.empty(16, dtype=torch.uint8), 24),
        lambda: va.attend_block_sparse(q, torch.empty(16, dtype=torch.uint8), torch.zeros(1, 2, 1, 1, dtype=torch.int32),
                                       torch.zeros(1, 2, 1, dtype=torch.int32)),
        lambda: va.attend_block_mask(q, torch.empty(16, dtype=torch.uint8), torch.zeros(1, 2, 1, 1, dtype=torch.int32)),
        lambda: va.window_attention(q, k, v, (1, 1, 1), grid=GRID, split=SPLIT),
        lambda: va.rope3d(q, GRID, SPLIT),
    ]
    for call in calls:
        with pytest.raises(ValueError, match="GPU"):
            call()


@pytest.mark.gpu
def test_bad_out_workspace_and_layout_are_rejected(va):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q, k, v = _qkv("cuda")
    ws = va.workspace_for(q, True)
    bad = [
        (lambda: va.attention(q, k, v, grid=GRID, split=SPLIT, out=torch.empty(1, 2, 24, 32, dtype=q.dtype,
                                                                                   device="cuda")), "out must"),
        (lambda: va.attention(q, k, v, grid=GRID, split=SPLIT, out=torch.empty_like(q, dtype=torch.float32)),
         "out must"),
        (lambda: va.attention(q, k, v, grid=GRID, split=SPLIT, out=torch.empty_like(q, device="cpu")), "out is on"),
        (lambda: va.attention(q, k, v, grid=GRID, split=SPLIT, workspace=ws.cpu()), "workspace is on"),
        (lambda: va.attention(q, k, v, grid=GRID, split=SPLIT, workspace=ws[::2]), "workspace must be contiguous"),
        (lambda: va.attend_subset(q.transpose(2, 3), torch.arange(64, dtype=torch.int32, device="cuda"), ws, 24),
         "q must be contiguous"),
        (lambda: va.attend_subset(q, torch.arange(24, dtype=torch.int32), ws, 24), "q_index is on"),
        (lambda: va.rope3d(q, GRID, SPLIT, out=torch.empty_like(q), out_dtype=torch.float32), "out must"),
    ]
    for call, msg in bad:
        with pytest.raises(ValueError, match=msg):
            call()
    torch.cuda.synchronize()
