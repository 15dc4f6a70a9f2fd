"""Helpers shared by the GPU parity tests: upload seeded workloads, run the
HIP path through the C ABI binding, evaluate the oracle on the same inputs
(sampled rows, one (b, head) slice at a time, on a thread pool) and reduce
the differences to the two figures the tolerances are stated in:

  max-abs   max |o_gpu - o_ref| over the checked elements
  mean-rel  sum |o_gpu - o_ref| / sum |o_ref|   (an L1 ratio: a per-element
            mean of relative errors is dominated by outputs near zero)

Tolerances (fp64 oracle vs GPU): fp32 max-abs <= 1e-5; bf16 max-abs <= 2e-2
and mean-rel <= 5e-3.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle
import workloads as wlmod

TOL = {"f32": dict(max_abs=1e-5, mean_rel=1e-6), "bf16": dict(max_abs=2e-2, mean_rel=5e-3)}


def threads() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def to_torch(arr, device="cuda"):
    import torch
    if arr.dtype == np.uint16:
        return torch.from_numpy(arr.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(arr).to(device)


def from_torch(t) -> np.ndarray:
    """Device tensor -> float64 numpy (exact widening)."""
    import torch
    if t.dtype == torch.bfloat16:
        return oracle.decode_bf16(t.view(torch.int16).cpu().numpy().view(np.uint16))
    return t.double().cpu().numpy()


def host_inputs(wl):
    return {n: wlmod.full(wl, n) for n in ("q", "k", "v")}


def decode(wl, arr) -> np.ndarray:
    return oracle.decode_bf16(arr) if wl.dtype == "bf16" else arr.astype(np.float64)


def run_gpu(wl, host, rope=True, out=None, workspace=None):
    import video_diffusion_transformer_rope3d_amd as va
    q, k, v = (to_torch(host[n]) for n in ("q", "k", "v"))
    kw = dict(grid=wl.grid, split=wl.split, theta=wl.theta) if rope else {}
    o = va.attention(q, k, v, scale=wl.scale, out=out, workspace=workspace, **kw)
    return o


def oracle_rows(wl, host, b, h, rows, rope=True):
    q, k, v = (decode(wl, host[n][b, h]) for n in ("q", "k", "v"))
    if rope:
        return oracle.rope_attention(q, k, v, wl.grid, wl.split, wl.theta, wl.scale, rows=rows)
    return oracle.attention(q, k, v, wl.scale, rows=rows)


def compare(wl, host, o_gpu_t, rope=True, slices=None):
    """Compare sampled rows of every (b, head) slice (or of ``slices``).
    Returns dict(max_abs, mean_rel, checked, finite)."""
    from threadpoolctl import threadpool_limits
    import torch
    finite = bool(torch.isfinite(o_gpu_t.float()).all().item())
    pairs = slices or [(b, h) for b in range(wl.B) for h in range(wl.heads)]
    rows = {bh: wlmod.sample_rows(wl, *bh) for bh in pairs}
    gpu = {}
    for (b, h) in pairs:
        idx = torch.from_numpy(rows[(b, h)]).to(o_gpu_t.device)
        gpu[(b, h)] = from_torch(o_gpu_t[b, h].index_select(0, idx))

    def one(bh):
        ref = oracle_rows(wl, host, bh[0], bh[1], rows[bh], rope)
        e = np.abs(gpu[bh] - ref)
        return float(e.max()), float(e.sum()), float(np.abs(ref).sum()), e.size

    with threadpool_limits(1):
        with ThreadPoolExecutor(threads()) as ex:
            res = list(ex.map(one, pairs))
    mx = max(r[0] for r in res)
    se = sum(r[1] for r in res)
    sr = sum(r[2] for r in res)
    return dict(max_abs=mx, mean_rel=se / sr if sr > 0 else 0.0, checked=sum(r[3] for r in res), finite=finite)


def within(wl, stats) -> bool:
    t = TOL[wl.dtype]
    return stats["finite"] and stats["max_abs"] <= t["max_abs"] and stats["mean_rel"] <= t["mean_rel"]
