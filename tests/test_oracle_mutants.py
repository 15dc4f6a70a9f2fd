"""Plant plausible mistakes in copies of the oracle (on the CPU) and check
that the pins catch every one of them: a pin set that a dropped term, a wrong
sign or index, a swapped axis or a transposed operand slips through would not
pin the oracle."""
import types

import numpy as np
import pytest

from oracle import reference
from tests import oracle_pins


def rope_variant(x, pos, split, theta, *, sign=1.0, width="axis", expo=2.0, pairing="interleaved",
                 pos_offset=0, swap_cs=False, axis_perm=(0, 1, 2), j_offset=0):
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    pos = np.asarray(pos, dtype=np.float64)[:, list(axis_perm)] + pos_offset
    out = x.copy()
    start = 0
    for a, w in enumerate(split):
        w = int(w)
        j = np.arange(w // 2, dtype=np.float64) + j_offset
        denom = w if width == "axis" else d
        om = float(theta) ** (-expo * j / denom)
        phi = pos[:, a:a + 1] * om[None, :]
        c, s = np.cos(phi), np.sin(phi)
        if swap_cs:
            c, s = s, c
        if pairing == "interleaved":
            i0 = start + 2 * np.arange(w // 2)
            i1 = i0 + 1
        else:  # rotate-half inside the chunk
            i0 = start + np.arange(w // 2)
            i1 = i0 + w // 2
        x0, x1 = x[..., i0], x[..., i1]
        out[..., i0] = x0 * c - sign * x1 * s
        out[..., i1] = sign * x0 * s + x1 * c
        start += w
    return out


def positions_variant(grid, order="fhw"):
    F, H, W = grid
    if order == "fhw":
        return reference.grid_positions(grid)
    f, y, x = np.meshgrid(np.arange(F), np.arange(H), np.arange(W), indexing="ij")
    if order == "whf":  # column-fastest reversed: x slowest
        f, y, x = (a.transpose(2, 1, 0) for a in (f, y, x))
    return np.stack([f.ravel(), y.ravel(), x.ravel()], axis=1)


def probs_variant(q, k, scale, *, use_scale=True, axis=1, sub_max=True, base="e", transpose=False):
    s = (np.asarray(q, np.float64) @ np.asarray(k, np.float64).T)
    if use_scale:
        s = s * scale
    if sub_max:
        s = s - s.max(axis=axis, keepdims=True)
    e = np.exp2(s) if base == "2" else np.exp(s)
    p = e / e.sum(axis=axis, keepdims=True)
    return p


def attention_variant(q, k, v, scale, rows=None, *, normalize=True, v_from_k=False, transpose=False, **kw):
    q = np.asarray(q, np.float64)
    if rows is not None:
        q = q[np.asarray(rows)]
    p = probs_variant(q, k, scale, **kw)
    if not normalize:
        s = q @ np.asarray(k, np.float64).T * scale
        p = np.exp(s - s.max(axis=1, keepdims=True))
    vv = np.asarray(k if v_from_k else v, np.float64)
    if transpose and p.shape[0] == p.shape[1]:
        p = p.T
    return p @ vv


def make_impl(rope_kw=None, pos_kw=None, attn_kw=None):
    rope_kw, pos_kw, attn_kw = rope_kw or {}, pos_kw or {}, attn_kw or {}
    pk = {k: v for k, v in attn_kw.items() if k in ("use_scale", "axis", "sub_max", "base")}
    return types.SimpleNamespace(
        rope3d_at=lambda x, pos, split, theta: rope_variant(x, pos, split, theta, **rope_kw),
        grid_positions=lambda grid: positions_variant(grid, **pos_kw),
        attention_probs=lambda q, k, scale: probs_variant(q, k, scale, **pk),
        attention=lambda q, k, v, scale, rows=None: attention_variant(q, k, v, scale, rows, **attn_kw),
    )


MUTANTS = {
    "rope: sign of sin flipped": dict(rope_kw=dict(sign=-1.0)),
    "rope: frequency over full head width": dict(rope_kw=dict(width="full")),
    "rope: exponent j/d instead of 2j/d": dict(rope_kw=dict(expo=1.0)),
    "rope: rotate-half pairs": dict(rope_kw=dict(pairing="half")),
    "rope: 1-based positions": dict(rope_kw=dict(pos_offset=1)),
    "rope: cos and sin swapped": dict(rope_kw=dict(swap_cs=True)),
    "rope: frame and column axes swapped": dict(rope_kw=dict(axis_perm=(2, 1, 0))),
    "rope: pair index off by one": dict(rope_kw=dict(j_offset=1)),
    "grid: column-major flatten": dict(pos_kw=dict(order="whf")),
    "attn: scale dropped": dict(attn_kw=dict(use_scale=False)),
    "attn: softmax over queries": dict(attn_kw=dict(axis=0)),
    "attn: no max subtraction": dict(attn_kw=dict(sub_max=False)),
    "attn: base-2 exponential": dict(attn_kw=dict(base="2")),
    "attn: no normalisation": dict(attn_kw=dict(normalize=False)),
    "attn: P transposed": dict(attn_kw=dict(transpose=True)),
    "attn: V taken from K": dict(attn_kw=dict(v_from_k=True)),
}


def _failures(impl):
    failed = []
    with np.errstate(all="ignore"):
        for pin in oracle_pins.ALL_PINS:
            try:
                pin(impl)
            except (AssertionError, ValueError, IndexError, FloatingPointError):
                failed.append(pin.__name__)
    return failed


def test_unmutated_variant_passes_every_pin():
    assert _failures(make_impl()) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    failed = _failures(make_impl(**MUTANTS[name]))
    assert failed, f"no pin catches mutant '{name}'"
