"""Plain float64 definition of 3D-RoPE + full softmax attention.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): no product code may
import this module.

What is computed, and where it comes from (vidax paper summary,
paperlayer.ai/abs/2609.18077v1):

* Tokens are 3D patches of a video latent ("1 Introduction", "Motivation and
  gap"). The pages do not give a flatten order; this oracle reads the grid
  frame-major: token n = (f*H + y)*W + x.
* 3D rotary position embedding ("2 System Architecture & Design", heading
  "3D RoPE, 3D VAEs, and flash attention") is named but not written out. The
  plainest reading, used here: the head dimension splits into three
  contiguous chunks of widths d_t | d_h | d_w for the frame, row and column
  axes; inside a chunk of width d_a, the pair (2j, 2j+1) is rotated by the
  angle pos_a * theta**(-2j/d_a), with pos_a the 0-based integer grid index
  on that axis.
* Attention is full, non-causal softmax(Q K^T * scale) V over all tokens
  (the ScalingAttention abstract on thelatestinai.com/papers/2606.17566
  names "3D full attention"); flash attention ("3D RoPE, 3D VAEs, and flash
  attention") reaches the same result without the N x N matrix, so the
  oracle is that plain result computed in float64 from the exact input
  values.

All arithmetic is float64; inputs given as bf16 bit patterns are widened
exactly.
"""
from __future__ import annotations

import numpy as np


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def grid_positions(grid) -> np.ndarray:
    """(N, 3) integer positions (f, y, x) of every token of an F x H x W grid,
    in frame-major order n = (f*H + y)*W + x."""
    F, H, W = (int(g) for g in grid)
    f, y, x = np.meshgrid(np.arange(F), np.arange(H), np.arange(W), indexing="ij")
    return np.stack([f.ravel(), y.ravel(), x.ravel()], axis=1).astype(np.int64)


def axis_of_pairs(split) -> np.ndarray:
    """Axis (0 = frame, 1 = row, 2 = column) of each rotated pair, for a head
    dimension split into contiguous chunks d_t | d_h | d_w."""
    d_t, d_h, d_w = (int(s) for s in split)
    return np.concatenate([np.full(d_t // 2, 0), np.full(d_h // 2, 1),
                           np.full(d_w // 2, 2)]).astype(np.int64)


def pair_frequencies(split, theta) -> np.ndarray:
    """Angular frequency of each rotated pair: theta**(-2j/d_a) for pair j of
    an axis chunk of width d_a (each axis uses its own width)."""
    out = []
    for d_a in split:
        d_a = int(d_a)
        j = np.arange(d_a // 2, dtype=np.float64)
        out.append(np.power(float(theta), -2.0 * j / d_a))
    return np.concatenate(out)


def rope3d_at(x: np.ndarray, pos: np.ndarray, split, theta) -> np.ndarray:
    """Rotate x (..., N, d) whose N tokens sit at integer (or any real)
    positions pos (N, 3). Pairs are adjacent elements (2p, 2p+1) of the head
    dimension; pair p belongs to axis axis_of_pairs(split)[p]."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    if sum(int(s) for s in split) != d or any(int(s) % 2 for s in split):
        raise ValueError("split must be even widths summing to d")
    pos = np.asarray(pos, dtype=np.float64)
    axis = axis_of_pairs(split)                         # (d/2,)
    omega = pair_frequencies(split, theta)              # (d/2,)
    phi = pos[:, axis] * omega[None, :]                 # (N, d/2)
    c, s = np.cos(phi), np.sin(phi)
    x0 = x[..., 0::2]
    x1 = x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def rope3d(x: np.ndarray, grid, split, theta) -> np.ndarray:
    """3D rotary embedding of x (..., N, d) with N = F*H*W tokens."""
    return rope3d_at(x, grid_positions(grid), split, theta)


def attention_probs(q: np.ndarray, k: np.ndarray, scale: float) -> np.ndarray:
    """Explicit softmax matrix P (Nq, Nk) of q (Nq, d) against k (Nk, d),
    row-wise softmax of scale * q k^T (max subtracted for stability)."""
    s = float(scale) * (np.asarray(q, np.float64) @ np.asarray(k, np.float64).T)
    s = s - s.max(axis=1, keepdims=True)
    e = np.exp(s)
    return e / e.sum(axis=1, keepdims=True)


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
              rows=None, chunk: int = 512) -> np.ndarray:
    """Full non-causal attention softmax(q k^T * scale) v for the query rows
    ``rows`` (default: all), each against all keys. q, k, v are (N, d)
    already rotated where rotation applies. Rows are processed in chunks so
    the (rows x N) logits never get large."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    if rows is not None:
        q = q[np.asarray(rows)]
    out = np.empty((q.shape[0], v.shape[1]), dtype=np.float64)
    for r0 in range(0, q.shape[0], chunk):
        p = attention_probs(q[r0:r0 + chunk], k, scale)
        out[r0:r0 + chunk] = p @ v
    return out


def rope_attention(q, k, v, grid, split, theta, scale, rows=None) -> np.ndarray:
    """One (batch, head) slice of the hot path: rotate q and k by 3D RoPE
    (v is not rotated), then full attention. Only the requested query rows
    are rotated and evaluated; every key is."""
    pos = grid_positions(grid)
    kr = rope3d_at(k, pos, split, theta)
    if rows is None:
        qr = rope3d_at(q, pos, split, theta)
    else:
        rows = np.asarray(rows)
        qr = rope3d_at(np.asarray(q)[rows], pos[rows], split, theta)
    return attention(qr, kr, v, scale)


# ---------------------------------------------------------------- query subset (key/value-cache synchronisation)

def rope_attention_subset(q, q_index, k, v, grid, split, theta, scale, rows=None) -> np.ndarray:
    """Query-subset attention of one (batch, head) slice: query row r is the
    token q_index[r] of the grid (its rotary position), and every row attends
    to all N keys. This is the key/value-cache synchronisation of
    Heterogeneous Step Allocation (its abstract on the paper listing
    thelatestinai.com/papers/2606.17566): active tokens attend to the full
    sequence. q is (Nq, d); k, v are (N, d)."""
    pos = grid_positions(grid)
    q_index = np.asarray(q_index, dtype=np.int64)
    q = np.asarray(q, np.float64)
    if rows is not None:
        rows = np.asarray(rows)
        q, q_index = q[rows], q_index[rows]
    qr = rope3d_at(q, pos[q_index], split, theta)
    kr = rope3d_at(k, pos, split, theta)
    return attention(qr, kr, v, scale)


# ---------------------------------------------------------------- block-sparse attention

def block_sparse_mask(N: int, kv_blocks, kv_count, q_block: int, k_block: int) -> np.ndarray:
    """Boolean (N, N) visibility of one (batch, head) slice: query token i
    sees key token j when j's key block (j // k_block) is among the first
    kv_count[i // q_block] entries of kv_blocks[i // q_block]."""
    kv_blocks = np.asarray(kv_blocks, dtype=np.int64)
    kv_count = np.asarray(kv_count, dtype=np.int64)
    allowed = np.zeros((kv_count.shape[0], -(-N // k_block)), dtype=bool)
    for i, c in enumerate(kv_count):
        allowed[i, kv_blocks[i, :c]] = True
    qi = np.arange(N) // q_block
    kj = np.arange(N) // k_block
    return allowed[qi][:, kj]


def block_sparse_attention(q, k, v, grid, split, theta, scale, kv_blocks, kv_count, q_block=256, k_block=64,
                           rows=None) -> np.ndarray:
    """Block-sparse attention of one (batch, head) slice, the block-sparse
    video-DiT attention of ScalingAttention (its abstract on
    thelatestinai.com/papers/2606.17566) and of Sparse Forcing's Persistent
    Block-Sparse Attention (its abstract on thelatestinai.com/papers/2609.18077): the
    logits of keys outside the listed blocks are -inf before the softmax. A
    query whose block lists no key block has no attended key; its output is
    defined as 0 (a reading: the pages leave that case open). q, k, v are
    (N, d) before rotation; kv_blocks (nqb, max_blocks) and kv_count (nqb,)
    are the lists of this slice."""
    N = np.asarray(q).shape[0]
    rows = np.arange(N) if rows is None else np.asarray(rows)
    q = np.asarray(q, np.float64)[rows]
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    if grid is not None:
        pos = grid_positions(grid)
        q = rope3d_at(q, pos[rows], split, theta)
        k = rope3d_at(k, pos, split, theta)
    # listed[i, c]: key block c is listed for query block i
    kv_blocks = np.asarray(kv_blocks, dtype=np.int64)
    kv_count = np.asarray(kv_count, dtype=np.int64)
    listed = np.zeros((kv_count.shape[0], -(-N // k_block)), dtype=bool)
    for i, c in enumerate(kv_count):
        listed[i, kv_blocks[i, :c]] = True
    key_block = np.arange(N) // k_block
    out = np.zeros((rows.shape[0], v.shape[1]), dtype=np.float64)
    for n, i in enumerate(rows):
        seen = listed[i // q_block][key_block]
        if not seen.any():
            continue
        s = float(scale) * (k[seen] @ q[n])
        e = np.exp(s - s.max())
        out[n] = (e / e.sum()) @ v[seen]
    return out


def block_mask_attention(q, k, v, grid, split, theta, scale, mask, q_block=256, k_block=64, rows=None) -> np.ndarray:
    """Block-sparse attention driven by a bit mask (the per-head block mask of
    ScalingAttention's bit-wise block-sparse kernel, its abstract on
    thelatestinai.com/papers/2606.17566): query token i sees key token j when
    mask[i // q_block, j // k_block] is true; logits of the other keys are
    -inf before the softmax, and a query that sees no key outputs 0 (the same
    reading as block_sparse_attention). mask is a boolean (nqb, nkb) array of
    one (batch, head) slice; q, k, v are (N, d) before rotation."""
    N = np.asarray(q).shape[0]
    rows = np.arange(N) if rows is None else np.asarray(rows)
    mask = np.asarray(mask, dtype=bool)
    q = np.asarray(q, np.float64)[rows]
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    if grid is not None:
        pos = grid_positions(grid)
        q = rope3d_at(q, pos[rows], split, theta)
        k = rope3d_at(k, pos, split, theta)
    key_block = np.arange(N) // k_block
    out = np.zeros((rows.shape[0], v.shape[1]), dtype=np.float64)
    for n, i in enumerate(rows):
        seen = mask[i // q_block, key_block]
        if not seen.any():
            continue
        s = float(scale) * (k[seen] @ q[n])
        e = np.exp(s - s.max())
        out[n] = (e / e.sum()) @ v[seen]
    return out


# ---------------------------------------------------------------- local-window attention

def window_visible(grid, radius, rows=None) -> np.ndarray:
    """Boolean (len(rows), N) visibility of a sliding 3D window: query token
    at (f, y, x) sees key token (f', y', x') when |f - f'| <= r_f,
    |y - y'| <= r_h and |x - x'| <= r_w (clipped at the grid border)."""
    pos = grid_positions(grid)
    rows = np.arange(pos.shape[0]) if rows is None else np.asarray(rows)
    r = np.asarray(radius, dtype=np.int64)
    diff = np.abs(pos[rows][:, None, :] - pos[None, :, :])  # (rows, N, 3)
    return np.all(diff <= r[None, None, :], axis=2)


def window_attention(q, k, v, grid, split, theta, scale, radius, rows=None, rope=True) -> np.ndarray:
    """Local-window attention of one (batch, head) slice: each query attends
    only to the keys inside a box of radii (r_f, r_h, r_w) around its own
    grid position (the windowed-attention primitive of the vidax summary,
    "3D RoPE, 3D VAEs, and flash attention", and the sliding local windows of
    Sparse Forcing's abstract on thelatestinai.com/papers/2609.18077; the
    pages give no window shape, a centred box clipped at the border is the
    plainest reading). Every query sees at least itself."""
    N = np.asarray(q).shape[0]
    rows = np.arange(N) if rows is None else np.asarray(rows)
    q = np.asarray(q, np.float64)[rows]
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    if rope:
        pos = grid_positions(grid)
        q = rope3d_at(q, pos[rows], split, theta)
        k = rope3d_at(k, pos, split, theta)
    out = np.empty((rows.shape[0], v.shape[1]), dtype=np.float64)
    for c0 in range(0, rows.shape[0], 256):
        vis = window_visible(grid, radius, rows[c0:c0 + 256])
        for n in range(vis.shape[0]):
            seen = vis[n]
            s = float(scale) * (k[seen] @ q[c0 + n])
            e = np.exp(s - s.max())
            out[c0 + n] = (e / e.sum()) @ v[seen]
    return out
