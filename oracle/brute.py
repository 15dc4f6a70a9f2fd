"""Pure-Python brute-force twin of the oracle, for tiny inputs.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Written independently of ``reference.py`` (no NumPy, no shared helper): the
rotation is a complex multiply (x[2j] + i x[2j+1]) * exp(i*phi) with
``cmath``, token positions come from explicit nested loops over the grid, and
every sum is ``math.fsum``. Inputs are nested lists of floats.
"""
from __future__ import annotations

import cmath
import math


def positions(F, H, W):
    out = []
    for f in range(F):
        for y in range(H):
            for x in range(W):
                out.append((f, y, x))
    return out


def rotate_token(vec, pos, split, theta):
    """Rotate one token vector (list of d floats) at pos = (f, y, x)."""
    out = []
    start = 0
    for axis, width in enumerate(split):
        for j in range(width // 2):
            w = theta ** (-(2.0 * j) / width)
            z = complex(vec[start + 2 * j], vec[start + 2 * j + 1])
            z = z * cmath.exp(1j * pos[axis] * w)
            out.append(z.real)
            out.append(z.imag)
        start += width
    return out


def rope(xs, grid, split, theta):
    return [rotate_token(x, p, split, theta) for x, p in zip(xs, positions(*grid))]


def attend(qs, ks, vs, scale):
    """softmax(q k^T * scale) v, one query at a time, with fsum."""
    d_v = len(vs[0])
    out = []
    for q in qs:
        logits = [scale * math.fsum(a * b for a, b in zip(q, k)) for k in ks]
        mx = max(logits)
        w = [math.exp(s - mx) for s in logits]
        z = math.fsum(w)
        out.append([math.fsum(w[j] * vs[j][c] for j in range(len(vs))) / z for c in range(d_v)])
    return out


def rope_attend(qs, ks, vs, grid, split, theta, scale):
    return attend(rope(qs, grid, split, theta), rope(ks, grid, split, theta), vs, scale)
