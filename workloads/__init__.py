"""Seeded synthetic workloads for 3D-RoPE video attention.

This module only *produces input data*: the five workload shapes and the
seeded draws of Q, K, V (and the sampled query rows that checks look at).
It holds none of the method's arithmetic (no rotation, no softmax), so both
the CPU oracle and the HIP path may take their inputs from here without
sharing any computation.

Workloads. The vidax paper summary ("Experimental setup", "B Full benchmark
table") runs video DiTs at batch 1 with classifier-free guidance, i.e. an
internal batch of two, over "tens of thousands" of 3D-patch tokens
("Motivation and gap"); it prints no token grid, head count or head width,
so the grids, head counts and head widths below are synthetic stand-ins of
that scale:

  id  B  heads  grid (F,H,W)  N      d    split (t/h/w)  dtype  distribution
  1   1  4      4x8x8         256    64   16/24/24       f32    N(0,1)
  2   2  12     21x30x52      32760  128  44/42/42       bf16   N(0,1)*0.5
  3   2  10     21x45x80      75600  128  44/42/42       bf16   N(0,1)*0.5
  4   2  40     21x30x52      32760  128  44/42/42       bf16   N(0,1); 1% K rows x8
  5   2  40     21x45x80      75600  128  44/42/42       bf16   N(0,1)*0.5

Seeding: base seed 1000 + id; every (tensor, b, head) slice has its own
PCG64 stream keyed by SeedSequence([seed, tensor_id, b, head]), so any slice
can be regenerated alone. Draws are float32 standard normals, scaled by an
exact power of two, then rounded to bf16 with round-to-nearest-even (bf16
workloads) or kept as float32 (f32 workload).
"""
from __future__ import annotations

import hashlib
import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

# stream ids inside a workload's seed
T_Q, T_K, T_V, T_PEAKY, T_ROWS, T_SUBSET, T_BLOCKS = 0, 1, 2, 3, 4, 5, 6
TENSOR_IDS = {"q": T_Q, "k": T_K, "v": T_V}

SAMPLE_ROWS = 256  # query rows per (b, head) checked on large workloads


@dataclass(frozen=True)
class Workload:
    id: int
    name: str
    B: int
    heads: int
    grid: tuple  # (F, H, W)
    d: int
    split: tuple  # (d_t, d_h, d_w)
    theta: float
    dtype: str  # "bf16" | "f32"
    std: tuple  # multiplier of the standard normal for (q, k, v)
    peaky_frac: float = 0.0  # fraction of K rows per (b, head) multiplied by peaky_mult
    peaky_mult: float = 1.0
    full_rows: bool = False  # checks cover every query row

    @property
    def N(self) -> int:
        F, H, W = self.grid
        return F * H * W

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def seed(self) -> int:
        return 1000 + self.id

    @property
    def flops(self) -> float:
        """Algorithmic FLOPs of one attention call: 2*N*N*d for Q.K^T plus
        2*N*N*d for P.V, per (b, head)."""
        return 4.0 * self.B * self.heads * self.N * self.N * self.d

    @property
    def peaky_rows(self) -> int:
        return int(round(self.peaky_frac * self.N))

    def describe(self) -> dict:
        return {
            "workload": self.name,
            "B": self.B,
            "heads": self.heads,
            "grid": list(self.grid),
            "N": self.N,
            "d": self.d,
            "split": list(self.split),
            "theta": self.theta,
            "scale": self.scale,
            "dtype": self.dtype,
        }


WORKLOADS = {
    1: Workload(1, "rope3d-attn-4x8x8-h4-d64-f32", 1, 4, (4, 8, 8), 64, (16, 24, 24), 1e4,
                "f32", (1.0, 1.0, 1.0), full_rows=True),
    2: Workload(2, "rope3d-attn-21x30x52-b2-h12-d128-bf16", 2, 12, (21, 30, 52), 128,
                (44, 42, 42), 1e4, "bf16", (0.5, 0.5, 0.5)),
    3: Workload(3, "rope3d-attn-21x45x80-b2-h10-d128-bf16", 2, 10, (21, 45, 80), 128,
                (44, 42, 42), 1e4, "bf16", (0.5, 0.5, 0.5)),
    4: Workload(4, "rope3d-attn-21x30x52-b2-h40-d128-bf16-peakyK", 2, 40, (21, 30, 52), 128,
                (44, 42, 42), 1e4, "bf16", (1.0, 1.0, 1.0), peaky_frac=0.01, peaky_mult=8.0),
    5: Workload(5, "rope3d-attn-21x45x80-b2-h40-d128-bf16", 2, 40, (21, 45, 80), 128,
                (44, 42, 42), 1e4, "bf16", (0.5, 0.5, 0.5)),
}


def custom(B, heads, grid, d, split, dtype="bf16", theta=1e4, std=(0.5, 0.5, 0.5),
           seed_id=100, peaky_frac=0.0, peaky_mult=1.0, name=None) -> Workload:
    """A workload of arbitrary shape (tests use these for ragged tails and
    edge cases). ``seed_id`` plays the role of the id in the seed."""
    nm = name or f"custom-{grid[0]}x{grid[1]}x{grid[2]}-b{B}-h{heads}-d{d}-{dtype}-s{seed_id}"
    return Workload(seed_id, nm, B, heads, tuple(grid), d, tuple(split), theta, dtype,
                    tuple(std), peaky_frac=peaky_frac, peaky_mult=peaky_mult, full_rows=True)


def _rng(wl: Workload, tensor_id: int, b: int, h: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([wl.seed, tensor_id, b, h])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); returns the
    16-bit patterns. Inputs are finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def peaky_row_index(wl: Workload, b: int, h: int) -> np.ndarray:
    """Distinct K rows of one (b, head) that are multiplied by ``peaky_mult``."""
    n = wl.peaky_rows
    if n == 0:
        return np.zeros(0, dtype=np.int64)
    g = _rng(wl, T_PEAKY, b, h)
    return np.sort(g.choice(wl.N, size=n, replace=False)).astype(np.int64)


def slice_f32(wl: Workload, tensor: str, b: int, h: int) -> np.ndarray:
    """(N, d) float32 draw of one slice before any rounding to bf16."""
    tid = TENSOR_IDS[tensor]
    g = _rng(wl, tid, b, h)
    x = g.standard_normal((wl.N, wl.d), dtype=np.float32)
    s = wl.std[tid]
    if s != 1.0:
        x *= np.float32(s)
    if tensor == "k" and wl.peaky_rows:
        x[peaky_row_index(wl, b, h)] *= np.float32(wl.peaky_mult)
    return x


def slice_values(wl: Workload, tensor: str, b: int, h: int) -> np.ndarray:
    """The input values of one slice as they are stored: uint16 bf16 bit
    patterns for bf16 workloads, float32 for f32 workloads."""
    x = slice_f32(wl, tensor, b, h)
    if wl.dtype == "bf16":
        return f32_to_bf16_bits(x)
    return x


def full(wl: Workload, tensor: str, threads: int | None = None) -> np.ndarray:
    """All B*heads slices of one tensor as a (B, heads, N, d) array (uint16
    bf16 bits or float32), generated slice by slice on a thread pool."""
    dt = np.uint16 if wl.dtype == "bf16" else np.float32
    out = np.empty((wl.B, wl.heads, wl.N, wl.d), dtype=dt)

    def one(i):
        b, h = divmod(i, wl.heads)
        out[b, h] = slice_values(wl, tensor, b, h)

    n = wl.B * wl.heads
    threads = threads or min(16, len(os.sched_getaffinity(0)))
    if n == 1 or threads == 1:
        for i in range(n):
            one(i)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(one, range(n)))
    return out


def sample_rows(wl: Workload, b: int, h: int) -> np.ndarray:
    """Query rows checked for one (b, head): every row for small workloads,
    else rows 0 and N-1 plus 254 distinct rows drawn uniformly from the rest."""
    N = wl.N
    if wl.full_rows or N <= SAMPLE_ROWS:
        return np.arange(N, dtype=np.int64)
    g = _rng(wl, T_ROWS, b, h)
    mid = g.choice(np.arange(1, N - 1), size=SAMPLE_ROWS - 2, replace=False)
    return np.sort(np.concatenate([[0, N - 1], mid])).astype(np.int64)


def slice_sha256(arr: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(arr).tobytes()).hexdigest()


# ---------------------------------------------------------------- inputs of the attention variants

def subset_index(wl: Workload, n_active: int) -> np.ndarray:
    """Token indices of the active queries of a query-subset attention: a
    seeded draw of ``n_active`` distinct tokens of the grid, ascending (the
    tokens that still take a denoising step; the rest are skipped)."""
    g = _rng(wl, T_SUBSET, 0, 0)
    return np.sort(g.choice(wl.N, size=n_active, replace=False)).astype(np.int32)


def block_lists(wl: Workload, q_block: int, k_block: int, window: int, n_global: int,
                max_blocks: int | None = None) -> tuple[np.ndarray, np.ndarray]:
    """Seeded block-sparse key lists, one per (b, head, query block): the key
    blocks whose tokens fall in a band of ``window`` key blocks around the
    query block's tokens (a local neighbourhood in token order) plus
    ``n_global`` key blocks drawn uniformly (a persistent salient set), as
    ascending lists padded with -1. Returns (kv_blocks [B, heads, nqb,
    max_blocks] int32, kv_count [B, heads, nqb] int32)."""
    N = wl.N
    nqb, nkb = -(-N // q_block), -(-N // k_block)
    lists = []
    for b in range(wl.B):
        for h in range(wl.heads):
            g = _rng(wl, T_BLOCKS, b, h)
            glob = g.choice(nkb, size=min(n_global, nkb), replace=False)
            for i in range(nqb):
                c0 = (i * q_block) // k_block
                c1 = min(nkb - 1, (min(N, (i + 1) * q_block) - 1) // k_block)
                lo, hi = max(0, c0 - window), min(nkb - 1, c1 + window)
                lists.append(np.union1d(np.arange(lo, hi + 1), glob))
    width = max_blocks or max(len(x) for x in lists)
    blocks = np.full((wl.B * wl.heads * nqb, width), -1, dtype=np.int32)
    count = np.zeros(wl.B * wl.heads * nqb, dtype=np.int32)
    for r, x in enumerate(lists):
        x = x[:width]
        blocks[r, :len(x)] = x
        count[r] = len(x)
    return blocks.reshape(wl.B, wl.heads, nqb, width), count.reshape(wl.B, wl.heads, nqb)


def block_mask_words(mask) -> np.ndarray:
    """Pack a boolean key-block mask [..., n_query_blocks, n_key_blocks] into
    uint32 words [..., n_query_blocks, ceil(n_key_blocks / 32)]: bit j % 32
    of word j // 32 is key block j (the layout the bit-mask attention reads)."""
    m = np.asarray(mask, dtype=bool)
    nkb = m.shape[-1]
    words = -(-nkb // 32)
    padded = np.zeros(m.shape[:-1] + (words * 32,), dtype=bool)
    padded[..., :nkb] = m
    bits = padded.reshape(m.shape[:-1] + (words, 32)).astype(np.uint64) << np.arange(32, dtype=np.uint64)
    return bits.sum(axis=-1).astype(np.uint32)



# ---------------------------------------------------------------- planted keys (softmax edge cases)

PLANT_SEED = 4242


def planted_keys(N: int, d: int, heads: int, plants, seed: int = PLANT_SEED):
    """Inputs whose softmax takes a chosen course: q, k, v ~ N(0,1)*0.5 and
    every query row shifted by +1 in each component, so that a key row set to
    c * (1, ..., 1) scores about c * d above the others (times the softmax
    scale). ``plants`` lists, per head, (key index, c) pairs; c must be exact
    in bf16. Keys planted with the same c are identical rows, so their logits
    tie exactly. Returns bf16 bit patterns (1, heads, N, d) for q, k, v."""
    out = {}
    for name, tid in (("q", T_Q), ("k", T_K), ("v", T_V)):
        arr = np.empty((1, heads, N, d), dtype=np.uint16)
        for h in range(heads):
            g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tid, N, h])))
            x = g.standard_normal((N, d), dtype=np.float32) * np.float32(0.5)
            if name == "q":
                x += np.float32(1.0)
            if name == "k":
                for j, c in plants[h]:
                    assert float(np.float32(c)) == float(bf16_bits_to_f32(f32_to_bf16_bits(np.float32([c])))[0])
                    x[j] = np.float32(c)
            arr[0, h] = f32_to_bf16_bits(x)
        out[name] = arr
    return out["q"], out["k"], out["v"]
