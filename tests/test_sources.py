"""Checks on the device sources that need no GPU."""
import glob
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "video_diffusion_transformer_rope3d_amd", "csrc")


def test_no_bit_cast_of_a_vector_element():
    """hipcc (ROCm 7.2) compiles __builtin_bit_cast(T, v[i]) on an element of
    an ext_vector_type value as a cast of element 0. Element values are
    copied into a scalar first; this keeps the pattern out of the sources."""
    bad = []
    for path in glob.glob(os.path.join(CSRC, "*")):
        for n, line in enumerate(open(path), 1):
            if re.search(r"__builtin_bit_cast\([^,]+,\s*[\w.]+\s*(\[[^\]]*\]\s*){1,}\)", line):
                bad.append(f"{os.path.basename(path)}:{n}: {line.strip()}")
    assert not bad, "\n".join(bad)


def test_m0_is_set_only_by_the_lds_copy():
    """The direct-to-LDS copy is inline assembly that writes m0, a register
    the compiler reserves. That is sound only while the compiled kernels
    keep nothing in m0 of their own: no compiler-written m0 set-up and no
    instruction that reads m0 implicitly outside those copy blocks."""
    import shutil
    import subprocess
    import sys
    import tempfile

    import pytest
    if not (os.path.exists("/opt/rocm/bin/hipcc") or shutil.which("hipcc")):
        pytest.skip("hipcc not available")
    sys.path.insert(0, os.path.join(ROOT, "video_diffusion_transformer_rope3d_amd"))
    import build
    with tempfile.TemporaryDirectory() as tmp:
        out = os.path.join(tmp, "vidattn.s")
        try:
            build.assembly(out)
        except subprocess.CalledProcessError as e:
            raise AssertionError(e.stderr.decode(errors="replace")[-2000:])
        lines = [ln.strip() for ln in open(out)]
    implicit = re.compile(r"\b(s_movrel\w*|v_movrel\w*|s_sendmsg\w*|ds_gws\w*|ds_append|ds_consume|ds_ordered\w*|"
                          r"\w+_load_lds\w*)\b")
    in_asm, copies, bad = False, 0, []
    for n, ln in enumerate(lines):
        if ln.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if ln.startswith(";;#ASMEND"):
            in_asm = False
            continue
        if ln.startswith((";", ".", "//")) or not ln:
            continue
        if in_asm and re.match(r"s_mov_b32 m0, s\d+$", ln):
            if lines[n + 1] != "s_nop 0" or not lines[n + 2].startswith("global_load_lds_dwordx4 "):
                bad.append(f"{n}: {ln} (not followed by the copy)")
            copies += 1
            continue
        if in_asm and (ln == "s_nop 0" or ln.startswith("global_load_lds_dwordx4 ")):
            continue
        if re.search(r"\bm0\b", ln) or implicit.search(ln):
            bad.append(f"{n}: {ln}")
    assert copies > 0, "no direct-to-LDS copy found in the assembly"
    assert not bad, "\n".join(bad[:20])
