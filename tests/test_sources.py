"""Checks on the device sources that need no GPU."""
import glob
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "video_diffusion_transformer_rope3d_amd", "csrc")


@pytest.fixture(scope="module")
def assembly_lines():
    """The library's gfx950 assembly, compiled once for the checks below."""
    import shutil
    import subprocess
    import sys
    import tempfile

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
        return [ln.strip() for ln in open(out)]


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


def test_m0_is_set_only_by_the_lds_copy(assembly_lines):
    """The direct-to-LDS copy is inline assembly that writes m0, a register
    the compiler reserves. That is sound only while the compiled kernels
    keep nothing in m0 of their own: no compiler-written m0 set-up and no
    instruction that reads m0 implicitly outside those copy blocks."""
    lines = assembly_lines
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


def _mfma_hand_offs(body, window=40):
    """(distance, kind, earlier, later) for every pair of matrix-core
    instructions with different opcodes where the later one takes as
    accumulator input a register the earlier one writes (RAW), or writes a
    register the earlier one takes as accumulator input (WAR), along the
    fall-through path of a kernel body. Distance counts instructions, an
    s_nop N as N + 1 wait states."""
    def regs(tok):
        m = re.match(r"v\[(\d+):(\d+)\]$", tok)
        if m:
            return frozenset(range(int(m.group(1)), int(m.group(2)) + 1))
        m = re.match(r"v(\d+)$", tok)
        return frozenset({int(m.group(1))}) if m else frozenset()

    seq, out = [], []
    for ln in body:
        t = ln.split(";")[0].strip()
        if not t or t.startswith(".") or t.endswith(":"):
            continue  # directives and labels; control falls through labels
        op = t.split()[0]
        if op == "s_nop":
            seq.extend([None] * (int(t.split()[1]) + 1))
            continue
        if op.startswith("v_mfma"):
            p = t.replace(",", " ").split()
            d, c = regs(p[1]), regs(p[4])
            for j in range(max(0, len(seq) - window), len(seq)):
                e = seq[j]
                if e is None or e[0] == op:
                    continue
                if e[1] & c:
                    out.append((len(seq) - j, "RAW", e[2], t))
                if e[3] & d:
                    out.append((len(seq) - j, "WAR", e[2], t))
            seq.append((op, d, t, c))
        else:
            seq.append(None)
        if op in ("s_branch", "s_setpc_b64", "s_endpgm"):
            seq = [None] * window  # nothing falls through an unconditional branch
    return out


def test_matrix_core_accumulator_hand_offs_are_spaced(assembly_lines):
    """Found on gfx950 with this compiler: a 16x16x32 f16 product that took,
    as accumulator input, the result of a 16x16x16 bf16 product one
    instruction earlier (and a 16x16x16 product that overwrote an
    accumulator input a 16x16x32 product had just read) gave wrong scores;
    the compiler inserted no wait states there. The attention kernels fence
    such hand-offs: every pair of different matrix-core opcodes that shares
    an accumulator register is at least 8 wait states apart on every
    fall-through path (builds that passed every GPU test had 9 and more; the
    failing one had 1)."""
    text = "\n".join(assembly_lines)
    kernels = re.findall(r"^(_Z\w*attn_fwd_bf16_pp_kernel\w*):[^\n]*\n(.*?)^s_endpgm", text, re.S | re.M)
    assert len(kernels) >= 8, [k[0] for k in kernels]
    bad = []
    for name, body in kernels:
        close = [p for p in _mfma_hand_offs(body.split("\n")) if p[0] < 8]
        bad += [f"{name[:60]}: {p}" for p in close[:3]]
    assert not bad, "\n".join(bad)


def test_hand_off_check_sees_the_pattern():
    """The check above flags the failing pattern and passes the fenced one."""
    failing = ["v_mfma_f32_16x16x16_bf16 v[62:65], v[150:151], v[72:73], v[50:53]",
               "v_mfma_f32_16x16x32_f16 v[66:69], v[26:29], v[10:13], v[62:65]",
               "v_mfma_f32_16x16x16_bf16 v[62:65], v[150:151], v[70:71], v[50:53]"]
    kinds = sorted(p[1] for p in _mfma_hand_offs(failing))
    assert kinds == ["RAW", "WAR"] and all(p[0] == 1 for p in _mfma_hand_offs(failing))
    fenced = failing[:1] + ["s_nop 7"] + failing[1:2]
    assert [p[0] for p in _mfma_hand_offs(fenced)] == [9]
    branch = failing[:1] + ["s_branch .LBB0_1", ".LBB0_2:"] + failing[1:2]
    assert _mfma_hand_offs(branch) == []
