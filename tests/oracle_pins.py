"""Pins of the CPU oracle against facts that do not come from the oracle
itself: hand-derived closed forms (tests/golden/*.json), invariants of
rotations and of softmax attention, and the independent brute-force twin.

Each pin takes an ``impl`` namespace exposing ``grid_positions``,
``rope3d_at``, ``attention_probs`` and ``attention`` with the signatures of
``oracle.reference``, so the same pins can be run on deliberately broken
copies of the oracle (tests/test_oracle_mutants.py) to show that they catch
plausible mistakes. A pin raises AssertionError on failure.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

from oracle import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

ROPE_TOL = 1e-12


def _rng(seed):
    return np.random.default_rng(seed)


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


# ----------------------------------------------------------------- rotation

def pin_rope_golden(impl):
    cases = json.load(open(os.path.join(GOLDEN, "rope3d_hand.json")))["cases"]
    fn = {
        "cos": math.cos, "sin": math.sin, "-sin": lambda a: -math.sin(a),
        "cos-sin": lambda a: math.cos(a) - math.sin(a),
        "sin+cos": lambda a: math.sin(a) + math.cos(a),
        "zero": lambda a: 0.0, "const": lambda a: a,
    }
    for c in cases:
        x = np.array([c["x"]], dtype=np.float64)
        pos = np.array([c["pos"]], dtype=np.int64)
        got = impl.rope3d_at(x, pos, c["split"], c["theta"])[0]
        want = [fn[k](a) for k, a in c["expected"]]
        _close(got, want, ROPE_TOL, f"golden rope '{c['name']}'")


def pin_rope_origin_identity(impl):
    x = _rng(1).standard_normal((3, 24))
    pos = np.zeros((3, 3), dtype=np.int64)
    _close(impl.rope3d_at(x, pos, (8, 8, 8), 10000.0), x, 0.0, "rotation at (0,0,0)")


def pin_rope_1d_reduction(impl):
    """F = H = 1: frame and row chunks are untouched, the column chunk is a
    1D rotary embedding z_j * exp(i * x * theta**(-2j/d_w))."""
    W, split, theta = 7, (4, 6, 8), 50.0
    x = _rng(2).standard_normal((W, 18))
    got = impl.rope3d_at(x, impl.grid_positions((1, 1, W)), split, theta)
    _close(got[:, :10], x[:, :10], 0.0, "1D reduction: frame/row chunks")
    z = x[:, 10::2] + 1j * x[:, 11::2]
    ang = np.arange(W)[:, None] * theta ** (-np.arange(4)[None, :] * 2.0 / 8)
    zr = z * np.exp(1j * ang)
    _close(got[:, 10::2], zr.real, ROPE_TOL, "1D reduction: even")
    _close(got[:, 11::2], zr.imag, ROPE_TOL, "1D reduction: odd")


def pin_rope_norm(impl):
    x = _rng(3).standard_normal((40, 20))
    pos = _rng(4).integers(-50, 80, size=(40, 3))
    y = impl.rope3d_at(x, pos, (6, 8, 6), 10000.0)
    nx = x[:, 0::2] ** 2 + x[:, 1::2] ** 2
    ny = y[:, 0::2] ** 2 + y[:, 1::2] ** 2
    _close(ny, nx, 1e-12, "per-pair norm")


def pin_rope_relative(impl):
    """<R(p) q, R(p') k> = <q, R(p' - p) k>, also for shifted and negative
    positions."""
    g = _rng(5)
    split, theta = (6, 4, 6), 300.0
    q = g.standard_normal((30, 16))
    k = g.standard_normal((30, 16))
    p = g.integers(-30, 30, size=(30, 3))
    pp = g.integers(-30, 30, size=(30, 3))
    lhs = np.sum(impl.rope3d_at(q, p, split, theta) * impl.rope3d_at(k, pp, split, theta), axis=1)
    rhs = np.sum(q * impl.rope3d_at(k, pp - p, split, theta), axis=1)
    _close(lhs, rhs, 1e-11, "relative-offset invariance")
    shift = np.array([[7, -3, 11]])
    lhs2 = np.sum(impl.rope3d_at(q, p + shift, split, theta)
                  * impl.rope3d_at(k, pp + shift, split, theta), axis=1)
    _close(lhs2, lhs, 1e-11, "common shift invariance")


def pin_rope_group(impl):
    g = _rng(6)
    split, theta = (4, 4, 8), 10000.0
    x = g.standard_normal((25, 16))
    p = g.integers(-20, 20, size=(25, 3))
    pp = g.integers(-20, 20, size=(25, 3))
    _close(impl.rope3d_at(impl.rope3d_at(x, p, split, theta), -p, split, theta), x, 1e-12,
           "R(-p) R(p) = I")
    _close(impl.rope3d_at(impl.rope3d_at(x, p, split, theta), pp, split, theta),
           impl.rope3d_at(x, p + pp, split, theta), 1e-12, "R(p') R(p) = R(p + p')")


def pin_rope_brute(impl):
    grid, split, theta = (2, 3, 4), (4, 4, 4), 10000.0
    x = _rng(7).standard_normal((24, 12))
    got = impl.rope3d_at(x, impl.grid_positions(grid), split, theta)
    want = brute.rope(x.tolist(), grid, split, theta)
    _close(got, want, 1e-12, "rope vs brute force (2x3x4, d=12)")
    grid2, split2 = (3, 2, 2), (2, 6, 4)
    x2 = _rng(8).standard_normal((12, 12))
    got2 = impl.rope3d_at(x2, impl.grid_positions(grid2), split2, 77.0)
    _close(got2, brute.rope(x2.tolist(), grid2, split2, 77.0), 1e-12,
           "rope vs brute force (3x2x2, split 2/6/4)")


def pin_flatten_order(impl):
    for grid in [(2, 3, 4), (3, 1, 5), (1, 4, 2)]:
        got = impl.grid_positions(grid)
        want = np.array(brute.positions(*grid))
        assert got.shape == want.shape and np.array_equal(got, want), f"flatten order {grid}"


# ---------------------------------------------------------------- attention

def pin_attn_golden(impl):
    cases = json.load(open(os.path.join(GOLDEN, "attention_hand.json")))["cases"]
    for c in cases:
        q, k, v = (np.array(c[n], dtype=np.float64) for n in ("q", "k", "v"))
        out = []
        for row in c["logits"]:
            w = [math.exp(s) for s in row]
            z = sum(w)
            out.append([sum(w[j] * v[j][col] for j in range(len(w))) / z for col in range(v.shape[1])])
        _close(impl.attention(q, k, v, c["scale"]), out, 1e-14, f"golden attention '{c['name']}'")


def pin_attn_rows_sum_to_one(impl):
    g = _rng(10)
    p = impl.attention_probs(g.standard_normal((9, 8)), g.standard_normal((13, 8)), 0.7)
    assert p.shape == (9, 13), "P shape"
    assert np.all(p >= 0), "P negative"
    _close(p.sum(axis=1), np.ones(9), 1e-14, "rows of P sum to 1")


def pin_attn_zero_query(impl):
    g = _rng(11)
    k, v = g.standard_normal((17, 8)), g.standard_normal((17, 5))
    _close(impl.attention(np.zeros((4, 8)), k, v, 0.3), np.repeat(v.mean(0, keepdims=True), 4, 0),
           1e-14, "Q = 0 -> mean of V")


def pin_attn_identical_keys(impl):
    g = _rng(12)
    k = np.repeat(g.standard_normal((1, 8)), 11, axis=0)
    v = g.standard_normal((11, 6))
    _close(impl.attention(g.standard_normal((5, 8)), k, v, 1.1),
           np.repeat(v.mean(0, keepdims=True), 5, 0), 1e-14, "identical keys -> mean of V")


def pin_attn_ones(impl):
    g = _rng(13)
    _close(impl.attention(g.standard_normal((6, 8)), g.standard_normal((19, 8)), np.ones((19, 4)), 0.9),
           np.ones((6, 4)), 1e-14, "V = 1 -> O = 1")


def pin_attn_single_key(impl):
    g = _rng(14)
    v = g.standard_normal((1, 7))
    _close(impl.attention(g.standard_normal((3, 8)), g.standard_normal((1, 8)), v, 2.0),
           np.repeat(v, 3, 0), 1e-15, "N = 1 -> O = V")


def pin_attn_permutation(impl):
    g = _rng(15)
    q, k, v = g.standard_normal((7, 8)), g.standard_normal((23, 8)), g.standard_normal((23, 5))
    perm = g.permutation(23)
    _close(impl.attention(q, k[perm], v[perm], 0.4), impl.attention(q, k, v, 0.4), 1e-13,
           "joint permutation of K and V")


def pin_attn_linear_in_v(impl):
    g = _rng(16)
    q, k = g.standard_normal((7, 8)), g.standard_normal((12, 8))
    v1, v2 = g.standard_normal((12, 5)), g.standard_normal((12, 5))
    lhs = impl.attention(q, k, 2.0 * v1 - 3.0 * v2, 0.5)
    rhs = 2.0 * impl.attention(q, k, v1, 0.5) - 3.0 * impl.attention(q, k, v2, 0.5)
    _close(lhs, rhs, 1e-12, "linearity in V")


def pin_attn_dominant_key(impl):
    """One key aligned with the query and scaled far above the rest: the
    output is that key's value row (also exercises very large logits)."""
    g = _rng(17)
    q = np.zeros((1, 8)); q[0, 0] = 1.0
    k = g.standard_normal((20, 8)) * 0.01
    k[13] = 0; k[13, 0] = 1e4
    v = g.standard_normal((20, 5))
    _close(impl.attention(q, k, v, 1.0), v[13:14], 1e-12, "dominant key -> its V row")


def pin_attn_scale(impl):
    g = _rng(18)
    q, k, v = g.standard_normal((5, 8)), g.standard_normal((9, 8)), g.standard_normal((9, 3))
    _close(impl.attention(q * 3.0, k, v, 0.25), impl.attention(q, k, v, 0.75), 1e-13,
           "scale acts on the logits")


def pin_attn_rows_subset(impl):
    g = _rng(19)
    q, k, v = g.standard_normal((12, 8)), g.standard_normal((30, 8)), g.standard_normal((30, 4))
    rows = np.array([0, 5, 11])
    _close(impl.attention(q, k, v, 0.6, rows=rows), impl.attention(q, k, v, 0.6)[rows], 1e-15,
           "row subset")


def pin_attn_brute(impl):
    g = _rng(20)
    q, k, v = g.standard_normal((6, 12)), g.standard_normal((24, 12)), g.standard_normal((24, 12))
    _close(impl.attention(q, k, v, 0.3), brute.attend(q.tolist(), k.tolist(), v.tolist(), 0.3), 1e-12,
           "attention vs brute force")


def pin_rope_attention_brute(impl):
    grid, split, theta, scale = (2, 3, 4), (4, 4, 4), 10000.0, 1 / math.sqrt(12)
    g = _rng(21)
    q, k, v = (g.standard_normal((24, 12)) for _ in range(3))
    pos = impl.grid_positions(grid)
    got = impl.attention(impl.rope3d_at(q, pos, split, theta), impl.rope3d_at(k, pos, split, theta), v, scale)
    want = brute.rope_attend(q.tolist(), k.tolist(), v.tolist(), grid, split, theta, scale)
    _close(got, want, 1e-12, "rope + attention vs brute force")


ROPE_PINS = [pin_rope_golden, pin_rope_origin_identity, pin_rope_1d_reduction, pin_rope_norm,
             pin_rope_relative, pin_rope_group, pin_rope_brute, pin_flatten_order]
ATTN_PINS = [pin_attn_golden, pin_attn_rows_sum_to_one, pin_attn_zero_query, pin_attn_identical_keys,
             pin_attn_ones, pin_attn_single_key, pin_attn_permutation, pin_attn_linear_in_v,
             pin_attn_dominant_key, pin_attn_scale, pin_attn_rows_subset, pin_attn_brute]
ALL_PINS = ROPE_PINS + ATTN_PINS + [pin_rope_attention_brute]
