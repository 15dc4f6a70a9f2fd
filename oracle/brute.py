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


def rope_attend_subset(q, q_index, k, v, grid, split, theta, scale):
    """Query-subset attention: query row r sits at token q_index[r] of the
    grid and attends to every key; explicit loops and math.fsum."""
    F, H, W = grid
    pos = positions(F, H, W)
    qr = [rotate_token(q[r], pos[q_index[r]], split, theta) for r in range(len(q))]
    kr = [rotate_token(k[j], pos[j], split, theta) for j in range(len(k))]
    return attend(qr, kr, v, scale)


def block_sparse_attend(q, k, v, grid, split, theta, scale, kv_blocks, kv_count, q_block, k_block):
    """Block-sparse attention: token i attends to token j only when j's key
    block (j // k_block) is listed for i's query block (i // q_block) among
    the first kv_count entries; a token with no listed key gets zeros. Keys
    and queries are rotated first when grid is given."""
    if grid is not None:
        q = rope(q, grid, split, theta)
        k = rope(k, grid, split, theta)
    d_v = len(v[0])
    out = []
    for i in range(len(q)):
        listed = set(kv_blocks[i // q_block][:kv_count[i // q_block]])
        keys = [j for j in range(len(k)) if j // k_block in listed]
        if not keys:
            out.append([0.0] * d_v)
            continue
        s = [scale * math.fsum(a * b for a, b in zip(q[i], k[j])) for j in keys]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        tot = math.fsum(e)
        out.append([math.fsum(e[n] * v[j][c] for n, j in enumerate(keys)) / tot for c in range(d_v)])
    return out


def window_attend(q, k, v, grid, split, theta, scale, radius):
    """Local-window attention with explicit loops: token i attends to the
    tokens whose grid coordinates differ from its own by at most the radius
    on every axis."""
    F, H, W = grid
    pos = positions(F, H, W)
    qr = rope(q, grid, split, theta)
    kr = rope(k, grid, split, theta)
    d_v = len(v[0])
    out = []
    for i in range(len(qr)):
        keys = [j for j in range(len(kr)) if all(abs(pos[i][a] - pos[j][a]) <= radius[a] for a in range(3))]
        s = [scale * math.fsum(a * b for a, b in zip(qr[i], kr[j])) for j in keys]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        tot = math.fsum(e)
        out.append([math.fsum(e[n] * v[j][c] for n, j in enumerate(keys)) / tot for c in range(d_v)])
    return out
