"""CPU oracle for 3D-RoPE full spatiotemporal attention.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports, links or
executes anything under ``oracle/``; only the tests, the smoke check and the
benchmark's CPU-baseline leg do. The oracle shares no code with the HIP path.

``reference``  plain float64 NumPy definition (rotation, logits, softmax, P.V;
               also the query-subset, block-sparse and local-window
               variants)
``brute``      an independent pure-Python twin (complex-number rotation,
               explicit loops, ``math.fsum``) for tiny inputs

Every function is pinned by the CPU tests in ``tests/test_oracle_*.py``
against closed forms, invariants and the brute-force twin. Parity unpinned:
the rotary convention itself (pair layout, per-axis frequencies, flatten
order), which the pages do not fix; the oracle follows the plainest reading.
"""
from .reference import (  # noqa: F401
    axis_of_pairs,
    attention,
    attention_probs,
    decode_bf16,
    grid_positions,
    pair_frequencies,
    rope3d,
    block_mask_attention,
    block_sparse_attention,
    block_sparse_mask,
    rope3d_at,
    rope_attention,
    rope_attention_subset,
    window_attention,
    window_visible,
)
