"""The C ABI on the CPU: the library loads, exports every function the
header declares, and rejects malformed calls with the documented status
before touching any device. Only calls that fail validation are made here
(the pointers are fake and never dereferenced)."""
import ctypes
import os
import re

import pytest

import video_diffusion_transformer_rope3d_amd as va
from video_diffusion_transformer_rope3d_amd import Rope3dDesc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vidattn.h")

P = 0x10000  # fake, 16-byte aligned device addresses (never dereferenced)
Q, K, V, O, WS = P, 2 * P, 3 * P, 4 * P, 5 * P
GOOD = Rope3dDesc.make((21, 45, 80), (44, 42, 42), 1e4)
N5 = 75600


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]*?\b(vidattn_\w+)\s*\(", text, re.M)))


def test_header_declares_exactly_the_exported_set():
    assert header_functions() == sorted(va.EXPORTED_SYMBOLS)


def test_library_exports_every_header_symbol():
    lib = ctypes.CDLL(va.lib_path())
    for name in header_functions():
        assert hasattr(lib, name), name


def test_abi_version_and_strings():
    assert va.vidattn_abi_version() == 7 == va.ABI_VERSION
    for s, txt in [(0, "ok"), (1, "invalid argument"), (2, "unsupported"), (3, "workspace too small"),
                   (4, "HIP error")]:
        assert va.vidattn_status_string(s) == txt
    assert va.vidattn_status_string(99) == "unknown status"


def test_workspace_size():
    ws = va.vidattn_fwd_workspace_size
    assert ws(va.BF16, 2, 40, N5, 128, 1) == 4 * 80 * 75648 * 128
    assert ws(va.BF16, 2, 40, N5, 128, 0) == 4 * 80 * 75648 * 128
    assert ws(va.BF16, 1, 1, 1, 64, 1) == 4 * 64 * 64
    assert ws(va.F32, 1, 4, 256, 64, 1) == 4 * 4 * 256 * 64
    assert ws(va.F32, 1, 4, 256, 64, 0) == 0
    assert ws(va.BF16, 1, 4, 256, 96, 1) == 0
    assert ws(va.BF16, 0, 4, 256, 64, 1) == 0


def fwd(q=Q, k=K, v=V, o=O, dt=va.BF16, B=2, H=40, N=N5, d=128, scale=0.088, rope=GOOD, ws=WS, wsb=None):
    if wsb is None:
        wsb = va.vidattn_fwd_workspace_size(dt, max(B, 1), max(H, 1), max(N, 1), d, rope is not None) or 0
    return va.vidattn_fwd(q, k, v, o, dt, B, H, N, d, scale, rope, ws, wsb), va.vidattn_last_error()


@pytest.mark.parametrize("kw,status,needle", [
    (dict(q=None), 1, "non-null"),
    (dict(o=None), 1, "non-null"),
    (dict(k=K + 8), 1, "aligned"),
    (dict(dt=va.F16), 2, "dtype"),
    (dict(dt=7), 1, "dtype"),
    (dict(B=0), 1, ">= 1"),
    (dict(N=0), 1, ">= 1"),
    (dict(d=96), 2, "head dim"),
    (dict(d=63), 1, "even"),
    (dict(scale=0.0), 1, "softmax_scale"),
    (dict(scale=float("nan")), 1, "softmax_scale"),
    (dict(scale=float("inf")), 1, "softmax_scale"),
    (dict(N=N5 - 1), 1, "does not equal N"),
    (dict(rope=Rope3dDesc.make((21, 45, 80), (44, 42, 40))), 1, "sum"),
    (dict(rope=Rope3dDesc.make((21, 45, 80), (43, 43, 42))), 1, "even"),
    (dict(rope=Rope3dDesc.make((21, 45, 80), (44, 42, 42), 0.0)), 1, "theta"),
    (dict(rope=Rope3dDesc.make((21, 45, 80), (44, 42, 42), float("nan"))), 1, "theta"),
    (dict(rope=Rope3dDesc.make((0, 45, 80), (44, 42, 42))), 1, "extents"),
    (dict(ws=None), 3, "workspace"),
    (dict(wsb=1000), 3, "workspace"),
    (dict(ws=WS + 16), 1, "256-byte"),
    (dict(o=Q), 1, "overlap"),
    (dict(o=WS), 1, "overlap"),
    (dict(B=1 << 40), 1, "overflow"),
    (dict(N=(1 << 24) + 1, rope=None), 2, "exceeds"),
    (dict(B=1 << 11, H=1 << 10), 1, "exceeds"),
])
def test_fwd_rejects(kw, status, needle):
    s, msg = fwd(**kw)
    assert s == status, (s, msg)
    assert needle in msg


def test_fwd_f32_without_rope_needs_no_workspace_but_checks_overlap():
    # a valid call shape would launch; make it fail on overlap instead
    s, msg = fwd(dt=va.F32, rope=None, ws=None, wsb=0, o=K)
    assert s == 1 and "overlap" in msg


def rope_call(inp=Q, in_dt=va.BF16, out=O, out_dt=va.F16, B=2, H=40, d=128, rope=GOOD, prescale=1.0):
    return va.vidattn_rope3d(inp, in_dt, out, out_dt, B, H, d, rope, prescale), va.vidattn_last_error()


@pytest.mark.parametrize("kw,status,needle", [
    (dict(inp=None), 1, "non-null"),
    (dict(rope=None), 1, "non-null"),
    (dict(out=O + 4), 1, "aligned"),
    (dict(in_dt=va.F16), 2, "dtype"),
    (dict(out_dt=9), 1, "dtype"),
    (dict(d=127), 1, "even"),
    (dict(d=130), 2, "multiples of 8"),
    (dict(d=264), 2, "multiples of 8"),
    (dict(rope=Rope3dDesc.make((21, 45, 80), (44, 42, 44))), 1, "sum"),
    (dict(prescale=float("inf")), 1, "prescale"),
    (dict(out=Q + 16), 1, "overlap"),
    (dict(out=Q, out_dt=va.F32), 1, "in-place"),
])
def test_rope_rejects(kw, status, needle):
    s, msg = rope_call(**kw)
    assert s == status, (s, msg)
    assert needle in msg


def test_rope3d_tokens_rejects():
    """The token-offset rotation validates the token range against the grid
    (and everything vidattn_rope3d validates) before any HIP call."""
    def rt(n=100, off=0, d=128, rope=GOOD, inp=Q, out=O):
        return va.vidattn_rope3d_tokens(inp, va.BF16, out, va.BF16, 2, 40, n, off, d, rope, 1.0, None)
    for kw in (dict(n=0), dict(n=-1), dict(off=-1), dict(off=N5 - 99), dict(n=N5 + 1), dict(off=1 << 40),
               dict(n=N5, off=1)):
        assert rt(**kw) == 1, kw
        assert "outside" in va.vidattn_last_error(), (kw, va.vidattn_last_error())
    assert rt(inp=None) == 1 and "non-null" in va.vidattn_last_error()
    assert rt(d=100) == 2
    assert rt(rope=Rope3dDesc.make((0, 45, 80), (44, 42, 42))) == 1 and "extents" in va.vidattn_last_error()
    assert rt(out=Q + 16) == 1 and "overlap" in va.vidattn_last_error()


def test_last_error_is_per_call():
    fwd(q=None)
    assert va.vidattn_last_error() != ""


def test_prepare_and_attend_reject():
    wsb = va.vidattn_fwd_workspace_size(va.BF16, 2, 40, N5, 128, 1)
    s = va.vidattn_fwd_prepare(K, V, va.BF16, 2, 40, N5, 128, GOOD, WS, wsb - 1)
    assert s == 3 and "workspace" in va.vidattn_last_error()
    s = va.vidattn_fwd_prepare(K, V, va.BF16, 2, 40, N5, 128, GOOD, K, wsb)
    assert s == 1 and "overlaps" in va.vidattn_last_error()
    s = va.vidattn_fwd_prepare(None, V, va.BF16, 2, 40, N5, 128, GOOD, WS, wsb)
    assert s == 1
    s = va.vidattn_fwd_attend(Q, K, V, WS, O, va.BF16, 2, 40, N5, 128, -1.0, GOOD, wsb)
    assert s == 1 and "softmax_scale" in va.vidattn_last_error()
    s = va.vidattn_fwd_attend(Q, K, V, None, O, va.BF16, 2, 40, N5, 128, 0.1, GOOD, wsb)
    assert s == 3
    s = va.vidattn_fwd_attend(Q, K, V, WS, WS, va.BF16, 2, 40, N5, 128, 0.1, GOOD, wsb)
    assert s == 1 and "overlaps" in va.vidattn_last_error()
    s = va.vidattn_fwd_attend(Q, K, V, WS, O, va.BF16, 2, 40, N5 + 1, 128, 0.1, GOOD, wsb)
    assert s == 1 and "does not equal N" in va.vidattn_last_error()


QI, KB, KC = 6 * P, 7 * P, 8 * P  # fake index arrays
T = 1 << 40  # fake, far-apart tensor addresses for full-size shapes
QF, OF, WSF = T, 2 * T, 3 * T


def test_attend_subset_rejects():
    wsb = va.vidattn_fwd_workspace_size(va.BF16, 2, 40, N5, 128, 1)
    sub = lambda **kw: va.vidattn_fwd_attend_subset(**{**dict(
        q=QF, q_index=QI, Nq=1000, workspace=WSF, o=OF, dt=va.BF16, B=2, heads=40, N=N5, d=128, softmax_scale=0.1,
        rope=GOOD, workspace_bytes=wsb), **kw})
    assert sub(dt=va.F32) == 2
    assert sub(q_index=None) == 1 and "q_index" in va.vidattn_last_error()
    assert sub(q_index=QI + 2) == 1 and "aligned" in va.vidattn_last_error()
    assert sub(Nq=0) == 1
    assert sub(Nq=(1 << 24) + 1) == 2
    assert sub(workspace_bytes=wsb - 1) == 3
    assert sub(softmax_scale=float("nan")) == 1 and "softmax_scale" in va.vidattn_last_error()
    assert sub(N=N5 + 1) == 1 and "does not equal N" in va.vidattn_last_error()
    # o overlaps q only through the Nq rows it has: 2*40*1000*128*2 bytes
    assert sub(o=QF + 2 * 40 * 1000 * 128 * 2 - 16) == 1 and "overlaps q" in va.vidattn_last_error()
    assert sub(o=WSF) == 1 and "overlaps" in va.vidattn_last_error()


def test_attend_block_sparse_rejects():
    wsb = va.vidattn_fwd_workspace_size(va.BF16, 2, 40, N5, 128, 1)
    nkb = -(-N5 // va.SPARSE_K_BLOCK)
    bs = lambda **kw: va.vidattn_fwd_attend_block_sparse(**{**dict(
        q=QF, workspace=WSF, o=OF, dt=va.BF16, B=2, heads=40, N=N5, d=128, softmax_scale=0.1, rope=GOOD,
        kv_blocks=KB, kv_count=KC, max_blocks=16, workspace_bytes=wsb), **kw})
    assert bs(dt=va.F32) == 2
    assert bs(kv_blocks=None) == 1 and "kv_blocks" in va.vidattn_last_error()
    assert bs(kv_count=KC + 1) == 1 and "aligned" in va.vidattn_last_error()
    assert bs(max_blocks=0) == 1 and "max_blocks" in va.vidattn_last_error()
    assert bs(max_blocks=nkb + 1) == 1 and "max_blocks" in va.vidattn_last_error()
    assert bs(workspace_bytes=wsb - 1) == 3
    assert bs(d=96) == 2
    assert bs(o=QF) == 1 and "overlaps q" in va.vidattn_last_error()


def test_attend_block_mask_rejects_and_sizes():
    base = va.vidattn_fwd_workspace_size(va.BF16, 2, 40, N5, 128, True)
    need = va.vidattn_fwd_block_mask_workspace_size(va.BF16, 2, 40, N5, 128, True)
    nqb, nkt = -(-N5 // 256), -(-N5 // 64)
    assert need == base + (80 * nqb * 4 + 255) // 256 * 256 + 80 * nqb * nkt * 4
    assert va.vidattn_fwd_block_mask_workspace_size(va.F32, 2, 40, N5, 128, True) == 0
    assert va.vidattn_fwd_block_mask_workspace_size(va.BF16, 2, 40, N5, 96, True) == 0
    MK = 6 << 40  # fake mask address, far from the other fake buffers

    def bm(mask=MK, dt=va.BF16, wsb=need, o=OF, ws=WSF):
        return va.vidattn_fwd_attend_block_mask(QF, mask, ws, o, dt, 2, 40, N5, 128, 0.088, GOOD, wsb, None)
    assert bm(mask=None) == 1 and "mask" in va.vidattn_last_error()
    assert bm(mask=MK + 2) == 1 and "aligned" in va.vidattn_last_error()
    assert bm(dt=va.F32) == 2
    assert bm(wsb=need - 1) == 3
    assert bm(wsb=base) == 3
    assert bm(mask=WSF + need - 64) == 1 and "overlaps the workspace" in va.vidattn_last_error()
    assert bm(o=WSF + 4096) == 1 and "overlap" in va.vidattn_last_error()


def test_block_mask_words_layout():
    """Bit j % 32 of word j // 32 is key block j; padding bits stay 0."""
    import workloads as wlmod
    import numpy as np
    m = np.zeros((2, 3, 40), dtype=bool)
    m[0, 0, 0] = m[0, 0, 31] = m[0, 0, 32] = m[1, 2, 39] = True
    w = wlmod.block_mask_words(m)
    assert w.shape == (2, 3, 2) and w.dtype == np.uint32
    assert w[0, 0, 0] == (1 | (1 << 31)) and w[0, 0, 1] == 1 and w[1, 2, 1] == 1 << 7
    assert int(w.sum()) - int(w[0, 0].sum()) - int(w[1, 2].sum()) == 0


def test_window_rejects_and_sizes():
    """Sizes: the key/value image, the counts, and lists as wide as the most
    tiles a block lists (the rules restated in bench.py give those counts)."""
    import importlib.util
    import os
    import workloads as wlmod
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    spec = importlib.util.spec_from_file_location("bench_module", os.path.join(root, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    wl = wlmod.custom(2, 40, (21, 45, 80), 128, (44, 42, 42))
    base = va.vidattn_fwd_workspace_size(va.BF16, 2, 40, N5, 128, 1)
    W = va.WindowDesc.make((21, 45, 80), (1, 4, 4), "rows")
    wsb = va.vidattn_fwd_window_workspace_size(va.BF16, 2, 40, N5, 128, 1, W)
    nqb, cap = -(-N5 // 256), max(bench.window_plan_counts(wl, (1, 4, 4), "rows"))
    assert wsb == base + (nqb * 4 + 255) // 256 * 256 + nqb * cap * 4
    WP = va.WindowDesc.make((21, 45, 80), (1, 4, 4), "patches")
    wsp = va.vidattn_fwd_window_workspace_size(va.BF16, 2, 40, N5, 128, 1, WP)
    pqb, pkt = 21 * 3 * 5, 21 * 6 * 10
    pcap = max(bench.window_plan_counts(wl, (1, 4, 4), "patches"))
    assert pcap == 3 * 4 * 4
    assert wsp == 2 * 40 * 256 * 128 * pkt + (pqb * 4 + 255) // 256 * 256 + pqb * pcap * 4
    assert va.vidattn_fwd_window_workspace_size(va.F32, 2, 40, N5, 128, 1, W) == 0
    win = lambda **kw: va.vidattn_fwd_window(**{**dict(
        q=QF, k=QF + T // 4, v=QF + T // 2, o=OF, dt=va.BF16, B=2, heads=40, N=N5, d=128, softmax_scale=0.1,
        rope=GOOD, window=W, workspace=WSF, workspace_bytes=wsb), **kw})
    assert win(dt=va.F32) == 2
    assert win(window=None) == 1 and "window" in va.vidattn_last_error()
    assert win(window=va.WindowDesc.make((21, 45, 81), (1, 1, 1))) == 1 and "N" in va.vidattn_last_error()
    assert win(window=va.WindowDesc.make((21, 45, 80), (-1, 1, 1))) == 1 and "radii" in va.vidattn_last_error()
    assert win(rope=Rope3dDesc.make((21, 80, 45), (44, 42, 42), 1e4)) == 1 and "grids differ" in va.vidattn_last_error()
    assert win(workspace_bytes=wsb - 1) == 3
    assert win(workspace_bytes=base) == 3
    assert win(softmax_scale=0.0) == 1
    assert win(window=va.WindowDesc.make((21, 45, 80), (1, 4, 4), 7)) == 1 and "layout" in va.vidattn_last_error()
    # the patch layout needs its own (larger) image: the row layout's size is short
    assert win(window=WP, workspace_bytes=wsp - 1) == 3
    # a grid of 2^22 or more key patches cannot take the patch layout
    big = va.WindowDesc.make((1 << 24, 1, 1), (0, 0, 1), "patches")
    assert win(window=big, N=1 << 24, rope=None) == 2 and "2^22" in va.vidattn_last_error()


def test_single_hip_runtime_whatever_the_import_order():
    """Importing the binding before torch must not map a second HIP runtime
    (torch bundles its own libamdhip64 under the system soname)."""
    import subprocess
    import sys
    code = ("import video_diffusion_transformer_rope3d_amd as va, torch; "
            "r = va._loaded_hip_runtimes(); print(len(r)); assert len(r) == 1, r")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr[-2000:]


def test_library_imports_no_allocation_copy_or_sync():
    """The library allocates, copies and synchronizes nothing: of the HIP
    runtime it imports only kernel and variable registration, launch, error
    strings, and the current device and device address of its fixed scratch
    array (the no-allocation entry point)."""
    import shutil
    import subprocess
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    out = subprocess.run([nm, "-D", "--undefined-only", va.lib_path()], capture_output=True, text=True,
                         check=True).stdout
    hip = sorted({line.split()[-1].split("@")[0] for line in out.splitlines() if "hip" in line.lower()})
    allowed = {"__hipPopCallConfiguration", "__hipPushCallConfiguration", "__hipRegisterFatBinary",
               "__hipRegisterFunction", "__hipUnregisterFatBinary", "hipGetErrorString", "hipGetLastError",
               "hipLaunchKernel", "__hipRegisterVar", "hipGetDevice", "hipGetSymbolAddress"}
    assert set(hip) <= allowed, sorted(set(hip) - allowed)


def test_build_entry_checks_the_binding_abi():
    """The build entry point compares the library's ABI with the binding's
    constant, not with a number of its own that could fall behind."""
    import importlib.util
    import os
    path = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "__graft_entry__.py")
    spec = importlib.util.spec_from_file_location("_graft_entry_probe", path)
    entry = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(entry)
    import inspect
    src = inspect.getsource(entry.build)
    assert "va.ABI_VERSION" in src and "== 3" not in src


def test_workspace_writers_reject_q_in_the_workspace():
    """The calls that write the workspace before the attention kernel reads q
    (the fused call, the window call, the block-mask list building) reject a
    q that overlaps what they write; the attend phase, which only reads the
    workspace, accepts it up to the launch (not made here)."""
    wsb = va.vidattn_fwd_workspace_size(va.BF16, 2, 40, N5, 128, 1)
    KF, VF = QF + T // 4, QF + T // 2
    s = va.vidattn_fwd(WSF + 4096, KF, VF, OF, va.BF16, 2, 40, N5, 128, 0.1, GOOD, WSF, wsb)
    assert s == 1 and "q overlaps the workspace" in va.vidattn_last_error()
    s = va.vidattn_fwd(WSF - 4096, KF, VF, OF, va.BF16, 2, 40, N5, 128, 0.1, GOOD, WSF, wsb)
    assert s == 1 and "q overlaps the workspace" in va.vidattn_last_error()
    W = va.WindowDesc.make((21, 45, 80), (1, 4, 4))
    wwsb = va.vidattn_fwd_window_workspace_size(va.BF16, 2, 40, N5, 128, 1, W)
    s = va.vidattn_fwd_window(WSF + wwsb - 4096, KF, VF, OF, va.BF16, 2, 40, N5, 128, 0.1, GOOD, W, WSF, wwsb)
    assert s == 1 and "q overlaps the workspace" in va.vidattn_last_error()
    need = va.vidattn_fwd_block_mask_workspace_size(va.BF16, 2, 40, N5, 128, True)
    MK = 6 << 40
    s = va.vidattn_fwd_attend_block_mask(WSF + wsb, MK, WSF, OF, va.BF16, 2, 40, N5, 128, 0.1, GOOD, need, None)
    assert s == 1 and "q overlaps the list part" in va.vidattn_last_error()


def test_noalloc_rejects_before_any_device_work():
    """The no-allocation entry point refuses a call whose workspace exceeds
    its fixed scratch (naming the limit), and passes malformed arguments on
    to vidattn_fwd's checks, all before any HIP call (these fail validation;
    the pointers are fake)."""
    assert va.NOALLOC_SCRATCH_BYTES == 64 << 20
    KF, VF = QF + T // 4, QF + T // 2
    s = va.vidattn_fwd_noalloc(QF, KF, VF, OF, va.BF16, 2, 40, N5, 128, 0.1, GOOD)
    assert s == 3 and str(64 << 20) in va.vidattn_last_error()
    s = va.vidattn_fwd_noalloc(QF, KF, VF, OF, va.BF16, 2, 40, N5, 96, 0.1, GOOD)
    assert s == 2 and "head dim" in va.vidattn_last_error()
    s = va.vidattn_fwd_noalloc(None, KF, VF, OF, va.BF16, 2, 40, N5, 128, 0.1, GOOD)
    assert s == 3  # the size check comes first for this shape


def test_header_compiles_as_c_and_matches_the_binding_layouts(tmp_path):
    """include/vidattn.h is a C header: it compiles as pedantic C99, and the
    size and field offsets of each descriptor struct equal those of the
    binding's ctypes structures (and the layout constants agree)."""
    import ctypes
    import os
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    inc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
    src = tmp_path / "layout.c"
    src.write_text(
        '#include <stddef.h>\n#include <stdio.h>\n#include "vidattn.h"\n'
        "int main(void) {\n"
        '  printf("%zu %zu %zu %zu %zu\\n", sizeof(vidattn_rope3d_desc), offsetof(vidattn_rope3d_desc, H),'
        " offsetof(vidattn_rope3d_desc, d_t), offsetof(vidattn_rope3d_desc, d_w), offsetof(vidattn_rope3d_desc, theta));\n"
        '  printf("%zu %zu %zu %zu %zu\\n", sizeof(vidattn_window_desc), offsetof(vidattn_window_desc, W),'
        " offsetof(vidattn_window_desc, r_f), offsetof(vidattn_window_desc, r_w), offsetof(vidattn_window_desc, layout));\n"
        '  printf("%d %d %d %d\\n", VIDATTN_WINDOW_AUTO, VIDATTN_WINDOW_ROWS, VIDATTN_WINDOW_PATCHES, VIDATTN_ABI_VERSION);\n'
        "  return 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", inc, str(src), "-o", str(exe)],
                   check=True, capture_output=True, text=True)
    rope, win, consts = (list(map(int, line.split())) for line in
                         subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.splitlines())
    R, W = va.Rope3dDesc, va.WindowDesc
    assert rope == [ctypes.sizeof(R), R.H.offset, R.d_t.offset, R.d_w.offset, R.theta.offset]
    assert win == [ctypes.sizeof(W), W.W.offset, W.r_f.offset, W.r_w.offset, W.layout.offset]
    assert consts == [va.WINDOW_AUTO, va.WINDOW_ROWS, va.WINDOW_PATCHES, va.ABI_VERSION]
