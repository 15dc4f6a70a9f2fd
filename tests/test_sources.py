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
