"""The CPU oracle against its pins (closed forms, invariants, brute force)."""
import types

import numpy as np
import pytest

import oracle
from oracle import brute, reference
from tests import oracle_pins

IMPL = types.SimpleNamespace(grid_positions=reference.grid_positions, rope3d_at=reference.rope3d_at,
                             attention_probs=reference.attention_probs, attention=reference.attention)


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(IMPL)


def test_rope_attention_rows_match_full():
    """rope_attention on a row subset equals the same rows of the full
    evaluation (the subset path rotates only the chosen query rows)."""
    g = np.random.default_rng(30)
    grid, split = (3, 4, 5), (8, 4, 4)
    q, k, v = (g.standard_normal((60, 16)) for _ in range(3))
    full = oracle.rope_attention(q, k, v, grid, split, 1e4, 0.25)
    rows = np.array([0, 7, 33, 59])
    sub = oracle.rope_attention(q, k, v, grid, split, 1e4, 0.25, rows=rows)
    assert np.max(np.abs(full[rows] - sub)) <= 1e-15


def test_rope_attention_vs_brute_odd_grid():
    g = np.random.default_rng(31)
    grid, split, theta, scale = (1, 3, 5), (2, 2, 4), 500.0, 0.4
    q, k, v = (g.standard_normal((15, 8)) for _ in range(3))
    got = oracle.rope_attention(q, k, v, grid, split, theta, scale)
    want = brute.rope_attend(q.tolist(), k.tolist(), v.tolist(), grid, split, theta, scale)
    assert np.max(np.abs(got - np.array(want))) <= 1e-12


def test_decode_bf16_exact():
    bits = np.array([0x3F80, 0xBF80, 0x0000, 0x8000, 0x4049, 0x7F7F, 0x0001], dtype=np.uint16)
    want = [1.0, -1.0, 0.0, -0.0, 3.140625, 3.3895313892515355e38, 9.183549615799121e-41]
    got = oracle.decode_bf16(bits)
    assert got.dtype == np.float64
    assert list(got) == want


def test_v_not_rotated():
    """Only q and k are rotated: with q = 0 the output is the mean of the raw
    (unrotated) V rows."""
    g = np.random.default_rng(32)
    grid = (2, 2, 3)
    k, v = g.standard_normal((12, 8)), g.standard_normal((12, 8))
    out = oracle.rope_attention(np.zeros((12, 8)), k, v, grid, (2, 2, 4), 1e4, 0.5)
    assert np.max(np.abs(out - v.mean(0))) <= 1e-14
