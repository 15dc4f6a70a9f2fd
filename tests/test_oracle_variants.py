"""Pins of the oracle's query-subset and block-sparse attention (CPU), and
planted mistakes that the pins must catch.

The pins compare against computations that do not share the functions under
test: the dense rotary attention of the oracle on rearranged or sliced
inputs, closed forms (all-zero output for an empty key list), and the
pure-Python brute-force twin."""
import math
import types

import numpy as np
import pytest

from oracle import brute, reference

GRID, SPLIT, THETA = (2, 3, 4), (4, 4, 4), 10000.0
N, D = 24, 12
SCALE = 1 / math.sqrt(D)
QB, KB = 8, 6  # query / key block sizes of the tiny cases (unequal, to catch a swap)

IMPL = types.SimpleNamespace(subset=reference.rope_attention_subset, sparse=reference.block_sparse_attention)


def _data(seed, nq=N):
    g = np.random.default_rng(seed)
    return g.standard_normal((nq, D)), g.standard_normal((N, D)), g.standard_normal((N, D))


def _close(a, b, tol, what):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


# ---------------------------------------------------------------- query subset

def pin_subset_identity(impl):
    q, k, v = _data(1)
    _close(impl.subset(q, np.arange(N), k, v, GRID, SPLIT, THETA, SCALE),
           reference.rope_attention(q, k, v, GRID, SPLIT, THETA, SCALE), 1e-14, "identity subset == dense")


def pin_subset_permutation(impl):
    q, k, v = _data(2)
    perm = np.random.default_rng(3).permutation(N)[:10]
    _close(impl.subset(q[perm], perm, k, v, GRID, SPLIT, THETA, SCALE),
           reference.rope_attention(q, k, v, GRID, SPLIT, THETA, SCALE)[perm], 1e-14, "gathered rows == dense rows")


def pin_subset_duplicates(impl):
    q, k, v = _data(4, nq=1)
    q2 = np.repeat(q, 3, axis=0)
    out = impl.subset(q2, np.array([5, 5, 17]), k, v, GRID, SPLIT, THETA, SCALE)
    _close(out[0], out[1], 0.0, "same token twice")
    assert np.max(np.abs(out[0] - out[2])) > 1e-6, "a different position must change the result"


def pin_subset_brute(impl):
    q, k, v = _data(5, nq=7)
    idx = [3, 0, 23, 11, 11, 7, 19]
    _close(impl.subset(q, np.array(idx), k, v, GRID, SPLIT, THETA, SCALE),
           brute.rope_attend_subset(q.tolist(), idx, k.tolist(), v.tolist(), GRID, SPLIT, THETA, SCALE), 1e-12,
           "subset vs brute force")


# ---------------------------------------------------------------- block sparse

def _lists(seed, nqb, nkb, maxb):
    g = np.random.default_rng(seed)
    blocks = np.full((nqb, maxb), -1, dtype=np.int64)
    count = np.zeros(nqb, dtype=np.int64)
    for i in range(nqb):
        c = int(g.integers(0, maxb + 1))
        blocks[i, :c] = np.sort(g.choice(nkb, size=c, replace=False))
        count[i] = c
    return blocks, count


def pin_sparse_all_blocks_is_dense(impl):
    q, k, v = _data(6)
    nqb, nkb = -(-N // QB), -(-N // KB)
    blocks = np.tile(np.arange(nkb), (nqb, 1))
    _close(impl.sparse(q, k, v, GRID, SPLIT, THETA, SCALE, blocks, np.full(nqb, nkb), QB, KB),
           reference.rope_attention(q, k, v, GRID, SPLIT, THETA, SCALE), 1e-14, "all blocks == dense")


def pin_sparse_single_block_is_slice(impl):
    """With one key block listed, a query attends exactly to the rotated keys
    of that block: plain attention on the sliced rotated keys and values."""
    q, k, v = _data(7)
    nqb = -(-N // QB)
    blocks = np.array([[2], [0], [3]])[:nqb]
    got = impl.sparse(q, k, v, GRID, SPLIT, THETA, SCALE, blocks, np.ones(nqb, dtype=np.int64), QB, KB)
    pos = reference.grid_positions(GRID)
    qr, kr = reference.rope3d_at(q, pos, SPLIT, THETA), reference.rope3d_at(k, pos, SPLIT, THETA)
    for i in range(N):
        j0 = int(blocks[i // QB, 0]) * KB
        want = reference.attention(qr[i:i + 1], kr[j0:j0 + KB], v[j0:j0 + KB], SCALE)
        _close(got[i:i + 1], want, 1e-14, f"row {i} against its single key block")


def pin_sparse_empty_is_zero(impl):
    q, k, v = _data(8)
    nqb = -(-N // QB)
    blocks = np.array([[1, 2], [0, 0], [3, 0]])
    count = np.array([2, 0, 1])
    out = impl.sparse(q, k, v, GRID, SPLIT, THETA, SCALE, blocks, count, QB, KB)
    _close(out[QB:2 * QB], np.zeros((QB, D)), 0.0, "query block without keys")
    assert np.all(np.abs(out[:QB]).sum(axis=1) > 0)


def pin_sparse_brute(impl):
    q, k, v = _data(9)
    nqb, nkb = -(-N // QB), -(-N // KB)
    blocks, count = _lists(10, nqb, nkb, 3)
    count[0] = max(count[0], 1)
    _close(impl.sparse(q, k, v, GRID, SPLIT, THETA, SCALE, blocks, count, QB, KB),
           brute.block_sparse_attend(q.tolist(), k.tolist(), v.tolist(), GRID, SPLIT, THETA, SCALE,
                                     blocks.tolist(), count.tolist(), QB, KB), 1e-12, "block-sparse vs brute force")


PINS = [pin_subset_identity, pin_subset_permutation, pin_subset_duplicates, pin_subset_brute,
        pin_sparse_all_blocks_is_dense, pin_sparse_single_block_is_slice, pin_sparse_empty_is_zero,
        pin_sparse_brute]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(IMPL)


# ---------------------------------------------------------------- planted mistakes

def _subset_row_positions(q, q_index, k, v, grid, split, theta, scale, rows=None):
    """mistake: rotates query row r at token r instead of q_index[r]"""
    return reference.rope_attention_subset(q, np.arange(len(q)), k, v, grid, split, theta, scale)


def _sparse_with(mask_fn=None, count_shift=0, swap_blocks=False, masked_logit=None):
    def impl(q, k, v, grid, split, theta, scale, kv_blocks, kv_count, q_block=256, k_block=64, rows=None):
        n = np.asarray(q).shape[0]
        qb, kb = (k_block, q_block) if swap_blocks else (q_block, k_block)
        count = np.clip(np.asarray(kv_count) + count_shift, 0, np.asarray(kv_blocks).shape[1])
        vis = (mask_fn or reference.block_sparse_mask)(n, kv_blocks, count, qb, kb)
        pos = reference.grid_positions(grid)
        qr, kr = reference.rope3d_at(q, pos, split, theta), reference.rope3d_at(k, pos, split, theta)
        s = scale * (qr @ kr.T)
        if masked_logit is None:
            s = np.where(vis, s, -np.inf)
        else:
            s = np.where(vis, s, masked_logit)
        out = np.zeros((n, np.asarray(v).shape[1]))
        for i in range(n):
            if not np.isfinite(s[i]).any():
                continue
            e = np.exp(s[i] - np.max(s[i][np.isfinite(s[i])]))
            out[i] = (e / e.sum()) @ v
        return out
    return impl


def _transposed_mask(n, kv_blocks, kv_count, q_block, k_block):
    return reference.block_sparse_mask(n, kv_blocks, kv_count, q_block, k_block).T


MUTANTS = {
    "subset ignores q_index": types.SimpleNamespace(subset=_subset_row_positions, sparse=reference.block_sparse_attention),
    "sparse mask transposed": types.SimpleNamespace(subset=reference.rope_attention_subset,
                                                    sparse=_sparse_with(mask_fn=_transposed_mask)),
    "sparse count off by one": types.SimpleNamespace(subset=reference.rope_attention_subset,
                                                     sparse=_sparse_with(count_shift=-1)),
    "sparse block sizes swapped": types.SimpleNamespace(subset=reference.rope_attention_subset,
                                                        sparse=_sparse_with(swap_blocks=True)),
    "sparse masked logits kept at 0": types.SimpleNamespace(subset=reference.rope_attention_subset,
                                                            sparse=_sparse_with(masked_logit=0.0)),
}


def test_reference_sparse_matches_its_mutant_harness():
    """The harness that plants the mistakes reproduces the oracle when no
    mistake is planted, so each mutant differs by its planted change only."""
    q, k, v = _data(11)
    nqb, nkb = -(-N // QB), -(-N // KB)
    blocks, count = _lists(12, nqb, nkb, 3)
    count[:] = np.maximum(count, 1)
    _close(_sparse_with()(q, k, v, GRID, SPLIT, THETA, SCALE, blocks, count, QB, KB),
           reference.block_sparse_attention(q, k, v, GRID, SPLIT, THETA, SCALE, blocks, count, QB, KB), 1e-14,
           "harness without mistakes")


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch(name):
    caught = []
    for pin in PINS:
        try:
            pin(MUTANTS[name])
        except (AssertionError, IndexError, ValueError):  # a pin that fails or cannot run on the mutant catches it
            caught.append(pin.__name__)
    assert caught, f"no pin catches: {name}"


# ---------------------------------------------------------------- local window

WIMPL = types.SimpleNamespace(window=reference.window_attention)


def pin_window_large_radius_is_dense(impl):
    q, k, v = _data(20)
    _close(impl.window(q, k, v, GRID, SPLIT, THETA, SCALE, (GRID[0], GRID[1], GRID[2])),
           reference.rope_attention(q, k, v, GRID, SPLIT, THETA, SCALE), 1e-14, "unbounded window == dense")


def pin_window_zero_radius_is_identity_on_v(impl):
    q, k, v = _data(21)
    _close(impl.window(q, k, v, GRID, SPLIT, THETA, SCALE, (0, 0, 0)), v, 1e-15, "each token sees only itself")


def pin_window_1d_band(impl):
    """On a 1 x 1 x N grid the window is a band |i - j| <= r in token order:
    plain attention of each row on the rotated keys of its band."""
    g1, r = (1, 1, N), 3
    q, k, v = _data(22)
    got = impl.window(q, k, v, g1, SPLIT, THETA, SCALE, (0, 0, r))
    pos = reference.grid_positions(g1)
    qr, kr = reference.rope3d_at(q, pos, SPLIT, THETA), reference.rope3d_at(k, pos, SPLIT, THETA)
    for i in range(N):
        lo, hi = max(0, i - r), min(N, i + r + 1)
        _close(got[i:i + 1], reference.attention(qr[i:i + 1], kr[lo:hi], v[lo:hi], SCALE), 1e-14, f"band row {i}")


def pin_window_brute(impl):
    q, k, v = _data(23)
    radius = (0, 1, 2)  # unequal per axis, to catch a swapped axis
    _close(impl.window(q, k, v, GRID, SPLIT, THETA, SCALE, radius),
           brute.window_attend(q.tolist(), k.tolist(), v.tolist(), GRID, SPLIT, THETA, SCALE, radius), 1e-12,
           "window vs brute force")


def test_window_visibility_is_symmetric_and_contains_self():
    vis = reference.window_visible((3, 4, 5), (1, 0, 2))
    assert np.array_equal(vis, vis.T) and np.all(np.diag(vis))


WPINS = [pin_window_large_radius_is_dense, pin_window_zero_radius_is_identity_on_v, pin_window_1d_band,
         pin_window_brute]


@pytest.mark.parametrize("pin", WPINS, ids=lambda p: p.__name__)
def test_window_pin(pin):
    pin(WIMPL)


def _window_with(vis_fn):
    def impl(q, k, v, grid, split, theta, scale, radius, rows=None, rope=True):
        pos = reference.grid_positions(grid)
        qr, kr = reference.rope3d_at(q, pos, split, theta), reference.rope3d_at(k, pos, split, theta)
        vis = vis_fn(pos, np.asarray(radius))
        out = np.zeros((len(qr), np.asarray(v).shape[1]))
        for i in range(len(qr)):
            if not vis[i].any():
                raise ValueError("no visible key")
            s = scale * (kr[vis[i]] @ qr[i])
            e = np.exp(s - s.max())
            out[i] = (e / e.sum()) @ np.asarray(v)[vis[i]]
        return out
    return impl


WMUTANTS = {
    "strict inequality": _window_with(lambda p, r: np.all(np.abs(p[:, None] - p[None]) < r, axis=2)),
    "radius axes reversed": _window_with(lambda p, r: np.all(np.abs(p[:, None] - p[None]) <= r[::-1], axis=2)),
    "window anchored at the query, not centred": _window_with(
        lambda p, r: np.all((p[None] - p[:, None] >= 0) & (p[None] - p[:, None] <= r), axis=2)),
    "radius on the flat token index": _window_with(
        lambda p, r: np.abs(np.arange(len(p))[:, None] - np.arange(len(p))[None]) <= r.sum()),
}


@pytest.mark.parametrize("name", sorted(WMUTANTS))
def test_window_pins_catch(name):
    caught = []
    for pin in WPINS:
        try:
            pin(types.SimpleNamespace(window=WMUTANTS[name]))
        except (AssertionError, IndexError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches: {name}"


def test_window_harness_without_mistake_is_the_oracle():
    q, k, v = _data(24)
    exact = _window_with(lambda p, r: np.all(np.abs(p[:, None] - p[None]) <= r, axis=2))
    _close(exact(q, k, v, GRID, SPLIT, THETA, SCALE, (1, 1, 2)),
           reference.window_attention(q, k, v, GRID, SPLIT, THETA, SCALE, (1, 1, 2)), 1e-14, "harness")


# ---------------------------------------------------------------- block-sparse attention from a bit mask

def _mask_from_lists(blocks, count, nkb):
    m = np.zeros((len(count), nkb), dtype=bool)
    for i, c in enumerate(count):
        m[i, blocks[i, :c]] = True
    return m


def mask_pins(fn):
    """Pins of block_mask_attention (fn has its signature)."""
    q, k, v = _data(21)
    nqb, nkb = -(-N // QB), -(-N // KB)
    # against the pure-Python brute force, with the mask's set bits as lists
    blocks, count = _lists(22, nqb, nkb, 3)
    count[0] = max(count[0], 1)
    mask = _mask_from_lists(blocks, count, nkb)
    _close(fn(q, k, v, GRID, SPLIT, THETA, SCALE, mask, QB, KB),
           brute.block_sparse_attend(q.tolist(), k.tolist(), v.tolist(), GRID, SPLIT, THETA, SCALE,
                                     blocks.tolist(), count.tolist(), QB, KB), 1e-12, "bit mask vs brute force")
    # every bit set: the dense attention
    _close(fn(q, k, v, GRID, SPLIT, THETA, SCALE, np.ones((nqb, nkb), dtype=bool), QB, KB),
           reference.rope_attention(q, k, v, GRID, SPLIT, THETA, SCALE), 1e-12, "full mask vs dense")
    # a query block whose row is empty outputs 0; an asymmetric pattern
    m = np.zeros((nqb, nkb), dtype=bool)
    m[0, 1] = True
    m[2, 0] = m[2, 3] = True
    out = fn(q, k, v, GRID, SPLIT, THETA, SCALE, m, QB, KB)
    _close(out[QB:2 * QB], np.zeros((QB, D)), 0.0, "empty mask row")
    _close(out, brute.block_sparse_attend(q.tolist(), k.tolist(), v.tolist(), GRID, SPLIT, THETA, SCALE,
                                          [[1, 0], [0, 0], [0, 3]], [1, 0, 2], QB, KB), 1e-12, "asymmetric mask")


def test_block_mask_pins():
    mask_pins(reference.block_mask_attention)


def _mask_mutant(transpose=False, swap_blocks=False, invert=False):
    def fn(q, k, v, grid, split, theta, scale, mask, q_block=256, k_block=64, rows=None):
        m = np.asarray(mask, dtype=bool)
        if invert:
            m = ~m
        if transpose:
            full = np.zeros((max(m.shape), max(m.shape)), dtype=bool)
            full[:m.shape[0], :m.shape[1]] = m
            m = full.T[:m.shape[0], :m.shape[1]]
        qb, kb = (k_block, q_block) if swap_blocks else (q_block, k_block)
        nq = -(-np.asarray(q).shape[0] // qb)
        nk = -(-np.asarray(q).shape[0] // kb)
        mm = np.zeros((nq, nk), dtype=bool)
        mm[:min(nq, m.shape[0]), :min(nk, m.shape[1])] = m[:nq, :nk]
        return reference.block_mask_attention(q, k, v, grid, split, theta, scale, mm, qb, kb, rows)
    return fn


@pytest.mark.parametrize("mutant", [dict(transpose=True), dict(swap_blocks=True), dict(invert=True)],
                         ids=lambda m: next(iter(m)))
def test_block_mask_pins_catch(mutant):
    with pytest.raises((AssertionError, IndexError, ValueError)):
        mask_pins(_mask_mutant(**mutant))
