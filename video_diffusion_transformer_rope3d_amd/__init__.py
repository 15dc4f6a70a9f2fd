"""Python binding of libvidattn (3D-RoPE full attention on MI355X).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libvidattn.so``; PyTorch supplies device memory and streams.
The low-level functions carry the C names (``vidattn_fwd`` ...) and take
raw device pointers; ``attention`` and ``rope3d`` accept torch tensors.
Importing this package loads the library and raises if it is missing;
there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = [
    "BF16", "F16", "F32", "VidattnError", "Rope3dDesc", "lib_path", "load",
    "vidattn_rope3d", "vidattn_rope3d_tokens", "vidattn_fwd", "vidattn_fwd_prepare", "vidattn_fwd_attend", "vidattn_fwd_attend_subset",
    "vidattn_fwd_attend_block_sparse", "vidattn_fwd_workspace_size", "vidattn_status_string",
    "vidattn_last_error", "vidattn_abi_version", "attention", "prepare", "attend", "attend_subset",
    "attend_block_sparse", "rope3d", "workspace_for", "SPARSE_Q_BLOCK", "SPARSE_K_BLOCK", "EXPORTED_SYMBOLS",
    "WindowDesc", "vidattn_fwd_window", "vidattn_fwd_window_workspace_size", "window_attention",
    "vidattn_fwd_attend_block_mask", "vidattn_fwd_block_mask_workspace_size", "attend_block_mask",
    "block_mask_workspace_for", "vidattn_fwd_noalloc", "NOALLOC_SCRATCH_BYTES",
]

BF16, F16, F32 = 0, 1, 2
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = 0, 1, 2, 3, 4
ABI_VERSION = 7

SPARSE_Q_BLOCK, SPARSE_K_BLOCK = 256, 64  # VIDATTN_SPARSE_Q_BLOCK, VIDATTN_SPARSE_K_BLOCK
NOALLOC_SCRATCH_BYTES = 64 << 20  # VIDATTN_NOALLOC_SCRATCH_BYTES

EXPORTED_SYMBOLS = ("vidattn_rope3d", "vidattn_rope3d_tokens", "vidattn_fwd", "vidattn_fwd_prepare",
                    "vidattn_fwd_attend",
                    "vidattn_fwd_attend_subset", "vidattn_fwd_attend_block_sparse", "vidattn_fwd_window",
                    "vidattn_fwd_window_workspace_size", "vidattn_fwd_workspace_size", "vidattn_status_string",
                    "vidattn_last_error", "vidattn_abi_version", "vidattn_fwd_attend_block_mask",
                    "vidattn_fwd_block_mask_workspace_size", "vidattn_fwd_noalloc")

_HERE = os.path.dirname(os.path.abspath(__file__))


def lib_path() -> str:
    return os.environ.get("VIDATTN_LIB", os.path.join(_HERE, "libvidattn.so"))


class VidattnError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"vidattn status {status} ({_status_text(status)}): {detail}")
        self.status = status
        self.detail = detail


class Rope3dDesc(ctypes.Structure):
    _fields_ = [("F", ctypes.c_int64), ("H", ctypes.c_int64), ("W", ctypes.c_int64),
                ("d_t", ctypes.c_int32), ("d_h", ctypes.c_int32), ("d_w", ctypes.c_int32),
                ("theta", ctypes.c_double)]

    @classmethod
    def make(cls, grid, split, theta=10000.0) -> "Rope3dDesc":
        F, H, W = (int(g) for g in grid)
        d_t, d_h, d_w = (int(s) for s in split)
        return cls(F, H, W, d_t, d_h, d_w, float(theta))


WINDOW_AUTO, WINDOW_ROWS, WINDOW_PATCHES = 0, 1, 2
_WINDOW_LAYOUTS = {"auto": WINDOW_AUTO, "rows": WINDOW_ROWS, "patches": WINDOW_PATCHES}


class WindowDesc(ctypes.Structure):
    """vidattn_window_desc: the token grid, the window radii (frame, row,
    column) and the tiling layout (auto, rows or patches)."""
    _fields_ = [("F", ctypes.c_int64), ("H", ctypes.c_int64), ("W", ctypes.c_int64),
                ("r_f", ctypes.c_int32), ("r_h", ctypes.c_int32), ("r_w", ctypes.c_int32),
                ("layout", ctypes.c_int32)]

    @classmethod
    def make(cls, grid, radius, layout="auto") -> "WindowDesc":
        F, H, W = (int(g) for g in grid)
        r_f, r_h, r_w = (int(r) for r in radius)
        return cls(F, H, W, r_f, r_h, r_w, _WINDOW_LAYOUTS[layout] if isinstance(layout, str) else int(layout))


_LIB = None


def _loaded_hip_runtimes() -> set:
    """Distinct libamdhip64 files mapped into this process."""
    out = set()
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                parts = line.split()
                if len(parts) >= 6 and "libamdhip64" in parts[-1]:
                    out.add(os.path.realpath(parts[-1]))
    except OSError:
        pass
    return out


def load() -> ctypes.CDLL:
    """Load libvidattn.so once; raises ImportError if it is not built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = lib_path()
    if not os.path.exists(path):
        raise ImportError(f"libvidattn.so not found at {path}; build it with "
                          "`python video_diffusion_transformer_rope3d_amd/build.py`")
    # PyTorch-ROCm bundles its own HIP runtime under the same soname as the
    # system one. Loading torch first makes libvidattn bind to that copy, so
    # the streams and device pointers torch hands over belong to the runtime
    # that launches the kernels.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    runtimes = _loaded_hip_runtimes()
    if len(runtimes) > 1:
        raise ImportError("two HIP runtimes are loaded in this process (" + ", ".join(sorted(runtimes)) +
                          "); import torch before anything that loads /opt/rocm's libamdhip64")
    vp, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    lib.vidattn_rope3d.restype = ctypes.c_int
    lib.vidattn_rope3d.argtypes = [vp, ctypes.c_int, vp, ctypes.c_int, i64, i64, i64,
                                   ctypes.POINTER(Rope3dDesc), ctypes.c_float, vp]
    lib.vidattn_rope3d_tokens.restype = ctypes.c_int
    lib.vidattn_rope3d_tokens.argtypes = [vp, ctypes.c_int, vp, ctypes.c_int, i64, i64, i64, i64, i64,
                                          ctypes.POINTER(Rope3dDesc), ctypes.c_float, vp]
    lib.vidattn_fwd.restype = ctypes.c_int
    lib.vidattn_fwd.argtypes = [vp, vp, vp, vp, ctypes.c_int, i64, i64, i64, i64, ctypes.c_float,
                                ctypes.POINTER(Rope3dDesc), vp, sz, vp]
    lib.vidattn_fwd_noalloc.restype = ctypes.c_int
    lib.vidattn_fwd_noalloc.argtypes = [vp, vp, vp, vp, ctypes.c_int, i64, i64, i64, i64, ctypes.c_float,
                                        ctypes.POINTER(Rope3dDesc), vp]
    lib.vidattn_fwd_prepare.restype = ctypes.c_int
    lib.vidattn_fwd_prepare.argtypes = [vp, vp, ctypes.c_int, i64, i64, i64, i64, ctypes.POINTER(Rope3dDesc), vp,
                                        sz, vp]
    lib.vidattn_fwd_attend.restype = ctypes.c_int
    lib.vidattn_fwd_attend.argtypes = [vp, vp, vp, vp, vp, ctypes.c_int, i64, i64, i64, i64, ctypes.c_float,
                                       ctypes.POINTER(Rope3dDesc), sz, vp]
    lib.vidattn_fwd_attend_subset.restype = ctypes.c_int
    lib.vidattn_fwd_attend_subset.argtypes = [vp, vp, i64, vp, vp, ctypes.c_int, i64, i64, i64, i64, ctypes.c_float,
                                              ctypes.POINTER(Rope3dDesc), sz, vp]
    lib.vidattn_fwd_attend_block_sparse.restype = ctypes.c_int
    lib.vidattn_fwd_attend_block_sparse.argtypes = [vp, vp, vp, ctypes.c_int, i64, i64, i64, i64, ctypes.c_float,
                                                    ctypes.POINTER(Rope3dDesc), vp, vp, i64, sz, vp]
    lib.vidattn_fwd_attend_block_mask.restype = ctypes.c_int
    lib.vidattn_fwd_attend_block_mask.argtypes = [vp, vp, vp, vp, ctypes.c_int, i64, i64, i64, i64, ctypes.c_float,
                                                  ctypes.POINTER(Rope3dDesc), sz, vp]
    lib.vidattn_fwd_block_mask_workspace_size.restype = sz
    lib.vidattn_fwd_block_mask_workspace_size.argtypes = [ctypes.c_int, i64, i64, i64, i64, ctypes.c_int]
    lib.vidattn_fwd_window.restype = ctypes.c_int
    lib.vidattn_fwd_window.argtypes = [vp, vp, vp, vp, ctypes.c_int, i64, i64, i64, i64, ctypes.c_float,
                                       ctypes.POINTER(Rope3dDesc), ctypes.POINTER(WindowDesc), vp, sz, vp]
    lib.vidattn_fwd_window_workspace_size.restype = sz
    lib.vidattn_fwd_window_workspace_size.argtypes = [ctypes.c_int, i64, i64, i64, i64, ctypes.c_int,
                                                      ctypes.POINTER(WindowDesc)]
    lib.vidattn_fwd_workspace_size.restype = sz
    lib.vidattn_fwd_workspace_size.argtypes = [ctypes.c_int, i64, i64, i64, i64, ctypes.c_int]
    lib.vidattn_status_string.restype = ctypes.c_char_p
    lib.vidattn_status_string.argtypes = [ctypes.c_int]
    lib.vidattn_last_error.restype = ctypes.c_char_p
    lib.vidattn_last_error.argtypes = []
    lib.vidattn_abi_version.restype = ctypes.c_int
    lib.vidattn_abi_version.argtypes = []
    if lib.vidattn_abi_version() != ABI_VERSION:
        raise ImportError(f"libvidattn ABI {lib.vidattn_abi_version()} != binding ABI {ABI_VERSION}")
    _LIB = lib
    return lib


def _status_text(s: int) -> str:
    return load().vidattn_status_string(s).decode()


# ------------------------------------------------------------------ C names, raw pointers

def vidattn_rope3d(inp, in_dt, out, out_dt, B, heads, d, rope, prescale=1.0, stream=None) -> int:
    return load().vidattn_rope3d(inp, in_dt, out, out_dt, B, heads, d,
                                 ctypes.byref(rope) if rope is not None else None, prescale, stream)


def vidattn_rope3d_tokens(inp, in_dt, out, out_dt, B, heads, n_tokens, token_offset, d, rope, prescale=1.0,
                          stream=None) -> int:
    return load().vidattn_rope3d_tokens(inp, in_dt, out, out_dt, B, heads, n_tokens, token_offset, d,
                                        ctypes.byref(rope) if rope is not None else None, prescale, stream)


def vidattn_fwd(q, k, v, o, dt, B, heads, N, d, softmax_scale, rope, workspace, workspace_bytes,
                stream=None) -> int:
    return load().vidattn_fwd(q, k, v, o, dt, B, heads, N, d, softmax_scale,
                              ctypes.byref(rope) if rope is not None else None, workspace, workspace_bytes,
                              stream)


def vidattn_fwd_noalloc(q, k, v, o, dt, B, heads, N, d, softmax_scale, rope, stream=None) -> int:
    return load().vidattn_fwd_noalloc(q, k, v, o, dt, B, heads, N, d, softmax_scale,
                                      ctypes.byref(rope) if rope is not None else None, stream)


def vidattn_fwd_prepare(k, v, dt, B, heads, N, d, rope, workspace, workspace_bytes, stream=None) -> int:
    return load().vidattn_fwd_prepare(k, v, dt, B, heads, N, d, ctypes.byref(rope) if rope is not None else None,
                                      workspace, workspace_bytes, stream)


def vidattn_fwd_attend(q, k, v, workspace, o, dt, B, heads, N, d, softmax_scale, rope, workspace_bytes,
                       stream=None) -> int:
    return load().vidattn_fwd_attend(q, k, v, workspace, o, dt, B, heads, N, d, softmax_scale,
                                     ctypes.byref(rope) if rope is not None else None, workspace_bytes, stream)


def vidattn_fwd_attend_subset(q, q_index, Nq, workspace, o, dt, B, heads, N, d, softmax_scale, rope, workspace_bytes,
                              stream=None) -> int:
    return load().vidattn_fwd_attend_subset(q, q_index, Nq, workspace, o, dt, B, heads, N, d, softmax_scale,
                                            ctypes.byref(rope) if rope is not None else None, workspace_bytes,
                                            stream)


def vidattn_fwd_attend_block_sparse(q, workspace, o, dt, B, heads, N, d, softmax_scale, rope, kv_blocks, kv_count,
                                    max_blocks, workspace_bytes, stream=None) -> int:
    return load().vidattn_fwd_attend_block_sparse(q, workspace, o, dt, B, heads, N, d, softmax_scale,
                                                  ctypes.byref(rope) if rope is not None else None, kv_blocks,
                                                  kv_count, max_blocks, workspace_bytes, stream)


def vidattn_fwd_attend_block_mask(q, mask, workspace, o, dt, B, heads, N, d, softmax_scale, rope, workspace_bytes,
                                  stream=None) -> int:
    return load().vidattn_fwd_attend_block_mask(q, mask, workspace, o, dt, B, heads, N, d, softmax_scale,
                                                ctypes.byref(rope) if rope is not None else None, workspace_bytes,
                                                stream)


def vidattn_fwd_block_mask_workspace_size(dt, B, heads, N, d, use_rope) -> int:
    return load().vidattn_fwd_block_mask_workspace_size(dt, B, heads, N, d, int(bool(use_rope)))


def vidattn_fwd_window(q, k, v, o, dt, B, heads, N, d, softmax_scale, rope, window, workspace, workspace_bytes,
                       stream=None) -> int:
    return load().vidattn_fwd_window(q, k, v, o, dt, B, heads, N, d, softmax_scale,
                                     ctypes.byref(rope) if rope is not None else None,
                                     ctypes.byref(window) if window is not None else None, workspace,
                                     workspace_bytes, stream)


def vidattn_fwd_window_workspace_size(dt, B, heads, N, d, use_rope, window) -> int:
    return load().vidattn_fwd_window_workspace_size(dt, B, heads, N, d, int(bool(use_rope)),
                                                    ctypes.byref(window) if window is not None else None)


def vidattn_fwd_workspace_size(dt, B, heads, N, d, use_rope) -> int:
    return load().vidattn_fwd_workspace_size(dt, B, heads, N, d, int(bool(use_rope)))


def vidattn_status_string(s: int) -> str:
    return _status_text(s)


def vidattn_last_error() -> str:
    return load().vidattn_last_error().decode()


def vidattn_abi_version() -> int:
    return load().vidattn_abi_version()


def _raise(status: int):
    if status != OK:
        raise VidattnError(status, vidattn_last_error())


# ------------------------------------------------------------------ torch conveniences

def _torch():
    import torch
    return torch


def _dt(t) -> int:
    torch = _torch()
    m = {torch.bfloat16: BF16, torch.float16: F16, torch.float32: F32}
    if t.dtype not in m:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return m[t.dtype]


def _stream(stream):
    if stream is None:
        return _torch().cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _torch_stream(stream, device):
    """The stream the kernels will run on, as a torch stream object."""
    torch = _torch()
    if stream is None:
        return torch.cuda.current_stream(device)
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(getattr(stream, "cuda_stream", stream)), device=device)


def _empty(shape, dtype, device, stream):
    """A new device tensor owned by the stream the kernels run on: the caching
    allocator then reuses its memory only in that stream's order, so a buffer
    the binding drops on return cannot be handed to work on another stream
    while the kernels still read or write it."""
    torch = _torch()
    with torch.cuda.stream(_torch_stream(stream, device)):
        return torch.empty(shape, dtype=dtype, device=device)


def workspace_for(q, use_rope: bool, stream=None):
    """A torch byte buffer of the size vidattn_fwd needs for q's shape (None if
    0), allocated on ``stream`` (default: the current stream)."""
    torch = _torch()
    B, H, N, d = q.shape
    n = vidattn_fwd_workspace_size(_dt(q), B, H, N, d, use_rope)
    if n == 0:
        return None
    return _empty(n, torch.uint8, q.device, stream)


def attention(q, k, v, *, scale=None, grid=None, split=None, theta=10000.0, out=None, workspace=None,
              stream=None):
    """O = softmax(scale * rot(q) rot(k)^T) v for [B, heads, N, d] tensors.
    With grid/split given, q and k are rotated by 3D RoPE inside the call;
    otherwise they are used as given."""
    B, H, N, d = q.shape
    _check_qkv(q, k, v)
    out = _out(out, q, stream=stream)
    rope = Rope3dDesc.make(grid, split, theta) if grid is not None else None
    if workspace is None:
        workspace = workspace_for(q, rope is not None, stream)
    ws_ptr, ws_bytes = _ws(workspace, q)
    s = 1.0 / math.sqrt(d) if scale is None else float(scale)
    _raise(vidattn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), _dt(q), B, H, N, d, s, rope,
                       ws_ptr, ws_bytes, _stream(stream)))
    return out


def _check_qkv(q, k, v):
    for t in (k, v):
        if t.shape != q.shape or t.dtype != q.dtype or t.device != q.device:
            raise ValueError("q, k, v must share shape, dtype and device")
    for t in (q, k, v):
        if not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous [B, heads, N, d]")
    _on_gpu(q)


def _on_gpu(ref, **tensors):
    """The library takes device pointers: ref and every tensor given (None
    skipped) must be contiguous and on ref's GPU."""
    if not ref.is_cuda:
        raise ValueError(f"tensors must be on a GPU, got {ref.device}")
    for name, t in tensors.items():
        if t is None:
            continue
        if t.device != ref.device:
            raise ValueError(f"{name} is on {t.device}, expected {ref.device}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")


def _out(out, ref, dtype=None, stream=None):
    """The output tensor: a new one shaped like ref (allocated on the stream
    the kernels run on), or the caller's, checked for ref's shape, the dtype
    and ref's device."""
    dtype = ref.dtype if dtype is None else dtype
    if out is None:
        return _empty(ref.shape, dtype, ref.device, stream)
    if tuple(out.shape) != tuple(ref.shape) or out.dtype != dtype:
        raise ValueError(f"out must be a {dtype} tensor of shape {tuple(ref.shape)}, got {out.dtype} "
                         f"{tuple(out.shape)}")
    _on_gpu(ref, out=out)
    return out


def _ws(workspace, ref=None):
    if workspace is None:
        return None, 0
    if ref is not None:
        _on_gpu(ref, workspace=workspace)
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def prepare(k, v, *, grid=None, split=None, theta=10000.0, workspace=None, stream=None):
    """First phase of ``attention``: write the key/value operand image of k,
    v into a workspace (allocated if not given) and return it."""
    _check_qkv(k, k, v)
    B, H, N, d = k.shape
    rope = Rope3dDesc.make(grid, split, theta) if grid is not None else None
    if workspace is None:
        workspace = workspace_for(k, rope is not None, stream)
    ptr, nbytes = _ws(workspace, k)
    _raise(vidattn_fwd_prepare(k.data_ptr(), v.data_ptr(), _dt(k), B, H, N, d, rope, ptr, nbytes,
                               _stream(stream)))
    return workspace


def attend(q, k, v, workspace, *, scale=None, grid=None, split=None, theta=10000.0, out=None, stream=None):
    """Second phase of ``attention``: attention of q against the key/value
    image ``prepare`` wrote for k, v with the same rotary arguments."""
    _check_qkv(q, k, v)
    B, H, N, d = q.shape
    out = _out(out, q, stream=stream)
    rope = Rope3dDesc.make(grid, split, theta) if grid is not None else None
    ptr, nbytes = _ws(workspace, q)
    s = 1.0 / math.sqrt(d) if scale is None else float(scale)
    _raise(vidattn_fwd_attend(q.data_ptr(), k.data_ptr(), v.data_ptr(), ptr, out.data_ptr(), _dt(q), B, H, N, d, s,
                              rope, nbytes, _stream(stream)))
    return out


def attend_subset(q, q_index, workspace, N, *, scale=None, grid=None, split=None, theta=10000.0, out=None,
                  stream=None):
    """Query-subset attention: the Nq rows of q (tokens ``q_index``, an int32
    device tensor of Nq entries in [0, N)) attend to all N keys of the
    key/value image ``prepare`` wrote (BF16)."""
    torch = _torch()
    B, H, Nq, d = q.shape
    _on_gpu(q, q=q, q_index=q_index)
    if q_index.dtype != torch.int32 or q_index.dim() != 1 or q_index.numel() != Nq:
        raise ValueError("q_index must be a contiguous int32 vector with one entry per query row")
    out = _out(out, q, stream=stream)
    rope = Rope3dDesc.make(grid, split, theta) if grid is not None else None
    ptr, nbytes = _ws(workspace, q)
    s = 1.0 / math.sqrt(d) if scale is None else float(scale)
    _raise(vidattn_fwd_attend_subset(q.data_ptr(), q_index.data_ptr(), Nq, ptr, out.data_ptr(), _dt(q), B, H, N, d,
                                     s, rope, nbytes, _stream(stream)))
    return out


def attend_block_sparse(q, workspace, kv_blocks, kv_count, *, scale=None, grid=None, split=None, theta=10000.0,
                        out=None, stream=None):
    """Block-sparse attention: query block i (tokens 256i..256i+255) of each
    (b, head) attends only to the key blocks (64 tokens each) listed in
    ``kv_blocks[b, head, i, :kv_count[b, head, i]]`` (int32 device tensors of
    shapes [B, heads, ceil(N/256), max_blocks] and [B, heads, ceil(N/256)])."""
    torch = _torch()
    B, H, N, d = q.shape
    nqb = -(-N // SPARSE_Q_BLOCK)
    _on_gpu(q, q=q, kv_blocks=kv_blocks, kv_count=kv_count)
    if kv_blocks.dtype != torch.int32 or kv_count.dtype != torch.int32:
        raise ValueError("kv_blocks and kv_count must be int32")
    if kv_blocks.dim() != 4 or tuple(kv_blocks.shape[:3]) != (B, H, nqb) or not kv_blocks.is_contiguous():
        raise ValueError(f"kv_blocks must be a contiguous [{B}, {H}, {nqb}, max_blocks] tensor")
    if tuple(kv_count.shape) != (B, H, nqb) or not kv_count.is_contiguous():
        raise ValueError(f"kv_count must be a contiguous [{B}, {H}, {nqb}] tensor")
    out = _out(out, q, stream=stream)
    rope = Rope3dDesc.make(grid, split, theta) if grid is not None else None
    ptr, nbytes = _ws(workspace, q)
    s = 1.0 / math.sqrt(d) if scale is None else float(scale)
    _raise(vidattn_fwd_attend_block_sparse(q.data_ptr(), ptr, out.data_ptr(), _dt(q), B, H, N, d, s, rope,
                                           kv_blocks.data_ptr(), kv_count.data_ptr(), kv_blocks.shape[3], nbytes,
                                           _stream(stream)))
    return out


def block_mask_workspace_for(q, use_rope: bool):
    """A torch byte buffer large enough for prepare + attend_block_mask."""
    torch = _torch()
    B, H, N, d = q.shape
    n = vidattn_fwd_block_mask_workspace_size(_dt(q), B, H, N, d, use_rope)
    if n == 0:
        raise ValueError("block-mask attention supports bf16 [B, heads, N, d] with d in {64, 128}")
    return torch.empty(n, dtype=torch.uint8, device=q.device)


def attend_block_mask(q, workspace, mask, *, scale=None, grid=None, split=None, theta=10000.0, out=None,
                      stream=None):
    """Block-sparse attention from a bit mask: query block i (tokens
    256i..256i+255) of each (b, head) attends only to the key blocks (64
    tokens each) whose bit is set in ``mask``, an int32 device tensor of
    packed words [B, heads, ceil(N/256), ceil(ceil(N/64)/32)] (bit j%32 of
    word j//32 is key block j). ``workspace`` holds the prepared key/value
    image (``prepare``) and room for the lists (``block_mask_workspace_for``)."""
    torch = _torch()
    B, H, N, d = q.shape
    nqb, nkb = -(-N // SPARSE_Q_BLOCK), -(-N // SPARSE_K_BLOCK)
    _on_gpu(q, q=q, mask=mask)
    if mask.dtype != torch.int32 or tuple(mask.shape) != (B, H, nqb, -(-nkb // 32)) or not mask.is_contiguous():
        raise ValueError(f"mask must be a contiguous int32 [{B}, {H}, {nqb}, {-(-nkb // 32)}] tensor")
    out = _out(out, q, stream=stream)
    rope = Rope3dDesc.make(grid, split, theta) if grid is not None else None
    ptr, nbytes = _ws(workspace, q)
    s = 1.0 / math.sqrt(d) if scale is None else float(scale)
    _raise(vidattn_fwd_attend_block_mask(q.data_ptr(), mask.data_ptr(), ptr, out.data_ptr(), _dt(q), B, H, N, d, s,
                                         rope, nbytes, _stream(stream)))
    return out


def window_attention(q, k, v, radius, *, grid, split=None, theta=10000.0, scale=None, rope=True, layout="auto",
                     workspace=None, out=None, stream=None):
    """Local-window attention (BF16): each query attends to the keys within
    ``radius`` = (r_f, r_h, r_w) of its position on the token ``grid``
    (rotary embedding on ``grid`` with ``split`` unless rope=False).
    ``layout`` ("auto", "rows" or "patches") picks the tiling."""
    torch = _torch()
    _check_qkv(q, k, v)
    B, H, N, d = q.shape
    out = _out(out, q, stream=stream)
    rd = Rope3dDesc.make(grid, split, theta) if rope else None
    wd = WindowDesc.make(grid, radius, layout)
    if workspace is None:
        n = vidattn_fwd_window_workspace_size(_dt(q), B, H, N, d, rope, wd)
        workspace = _empty(n, torch.uint8, q.device, stream) if n else None
    ptr, nbytes = _ws(workspace, q)
    s = 1.0 / math.sqrt(d) if scale is None else float(scale)
    _raise(vidattn_fwd_window(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), _dt(q), B, H, N, d, s, rd, wd,
                              ptr, nbytes, _stream(stream)))
    return out


def rope3d(x, grid, split, theta=10000.0, *, token_offset=None, out=None, out_dtype=None, prescale=1.0,
           stream=None):
    """3D rotary embedding of a [B, heads, n, d] tensor (out may be x). With
    token_offset, row r is grid token token_offset + r (a sequence shard);
    without it, x holds the whole grid."""
    torch = _torch()
    B, H, N, d = x.shape
    _on_gpu(x, x=x)
    n_grid = int(grid[0]) * int(grid[1]) * int(grid[2])
    if token_offset is None and N != n_grid:
        raise ValueError(f"x has {N} tokens, grid {tuple(grid)} has {n_grid}")
    out = _out(out, x, out_dtype or (out.dtype if out is not None else x.dtype), stream=stream)
    desc = Rope3dDesc.make(grid, split, theta)
    if token_offset is None:
        _raise(vidattn_rope3d(x.data_ptr(), _dt(x), out.data_ptr(), _dt(out), B, H, d, desc, prescale,
                              _stream(stream)))
    else:
        _raise(vidattn_rope3d_tokens(x.data_ptr(), _dt(x), out.data_ptr(), _dt(out), B, H, N, int(token_offset), d,
                                     desc, prescale, _stream(stream)))
    return out


load()
