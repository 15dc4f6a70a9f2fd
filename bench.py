#!/usr/bin/env python3
"""Benchmark of 3D-RoPE full attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload ID]

A step is one fused ``vidattn_fwd`` call with the rotary descriptor (key
pre-pass + attention kernel with the query rotation fused) over the whole
workload, inputs resident in HBM. Default workload: 2 x 40 heads x 75600
tokens (21x45x80 grid), head dim 128, bf16. FLOPs per call = 4*B*H*N^2*d.

Prints ONE JSON line with the throughput, the roofline of the attention
kernel (its own launches timed with HIP events on the stream it runs on),
a sampled parity check against the oracle, and the oracle's own throughput
on a bounded sample on the host cores (``cpu_baseline``).
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention TFLOP/s on 1 MI355X and % of bf16 MFMA peak; ms per DiT attention call"
PEAK_TFLOPS = 2500.0  # MI355X dense bf16/fp16 MFMA
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
KERNEL = "attn_fwd_bf16_pp_kernel"


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "video_diffusion_transformer_rope3d_amd", "csrc")
    for p in sorted(glob.glob(os.path.join(csrc, "*"))):
        with open(p, "rb") as f:
            h.update(os.path.basename(p).encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def committed_summary(pattern: str, workload_name: str, kernel: str, keys) -> dict | None:
    """Figures from a committed rocprofv3 summary under profiles/ (file name
    matching ``pattern``) taken on the current kernel source, this workload
    and this kernel: the file, the kernel's duration in that profiled run
    (``kernel_ms``) and the requested keys; None if there is none."""
    src = kernel_source_hash()
    for p in sorted(glob.glob(os.path.join(ROOT, "profiles", pattern))):
        text = open(p).read()

        def field(k):
            m = re.search(r"(?:^|\n)-?\s*" + re.escape(k) + r":\s*(\S+)", text)
            return m.group(1) if m else None

        if field("kernel_source_sha256") != src or field("workload") != workload_name:
            continue
        if field("kernel") not in (None, kernel):
            continue
        out = {"file": os.path.relpath(p, ROOT)}
        for k in ("kernel_ms", *keys):
            v = field(k)
            if v is not None:
                out[k] = float(v)
        return out
    return None


def profile_block(workload_name: str, kernel: str, kernel_ms: float, this_run: str = "kernel") -> tuple:
    """(traffic bytes per launch or None, the 'profile' block of the roofline):
    counters of separate rocprofv3 runs on the same kernel source, labelled
    with their file and the kernel time in those runs, which may have been on
    another board (boards of this GPU differ by several per cent). kernel_ms
    is this run's time of the kernel (this_run="kernel") or of the whole call
    it sits in (this_run="call")."""
    tr = committed_summary("*traffic*.md", workload_name, kernel, ("traffic_bytes_per_launch",))
    ct = committed_summary("*counters*.md", workload_name, kernel, ("mfma_busy_frac", "clock_ghz"))
    block = {}
    traffic = None
    if tr and "traffic_bytes_per_launch" in tr:
        traffic = tr["traffic_bytes_per_launch"]
        block["traffic_file"] = tr["file"]
        if "kernel_ms" in tr:
            block["traffic_run_kernel_ms"] = tr["kernel_ms"]
    if ct:
        block["counters_file"] = ct["file"]
        for k in ("kernel_ms", "mfma_busy_frac", "clock_ghz"):
            if k in ct:
                block[{"kernel_ms": "counters_run_kernel_ms"}.get(k, k)] = ct[k]
    if block:
        block[f"this_run_{this_run}_ms"] = round(kernel_ms, 3)
        block["note"] = ("counters from separate rocprofv3 runs of the same kernel source (files above); "
                         "achieved and frac are this run's")
    return traffic, (block or None)


def cpu_baseline(wl, host, budget_s: float):
    """The oracle as it stands, on sampled query rows of whole (b, head)
    slices (every key), for about ``budget_s`` seconds of wall time: the
    slices are spread over a pool of one worker per host core (up to 16),
    each running the oracle with a single BLAS thread."""
    import numpy as np
    import oracle
    import workloads as wlmod
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits

    cores = len(os.sched_getaffinity(0))
    workers = max(1, min(16, cores))
    dec = oracle.decode_bf16 if wl.dtype == "bf16" else (lambda a: a.astype(np.float64))
    pairs = [(b, h) for b in range(wl.B) for h in range(wl.heads)]

    def one(bh):
        b, h = bh
        rows = wlmod.sample_rows(wl, b, h)
        q, k, v = (dec(host[n][b, h]) for n in ("q", "k", "v"))
        oracle.rope_attention(q, k, v, wl.grid, wl.split, wl.theta, wl.scale, rows=rows)
        return rows.size

    rows_total, slices = 0, 0
    t0 = time.perf_counter()
    with threadpool_limits(1), ThreadPoolExecutor(workers) as ex:
        for w0 in range(0, len(pairs), workers):
            rows_total += sum(ex.map(one, pairs[w0:w0 + workers]))
            slices += len(pairs[w0:w0 + workers])
            if time.perf_counter() - t0 >= budget_s:
                break
    wall = time.perf_counter() - t0
    flops = 4.0 * rows_total * wl.N * wl.d
    return {
        "value": flops / wall / 1e12,
        "unit": "TFLOP/s",
        "cores": workers,
        "kind": "oracle",
        "sample": f"{slices} (b, head) slices x {rows_total // max(slices, 1)} sampled query rows against all "
                  f"{wl.N} keys (fp64 NumPy, keys rotated in full per slice), {workers} slices at a time on "
                  f"{workers} worker threads with 1 BLAS thread each; {wall:.1f} s wall; {cores} host cores "
                  f"available",
        "workers": workers,
        "blas_threads_per_worker": 1,
        "seconds": wall,
        "ms_per_call_extrapolated": wall / rows_total * wl.N * wl.B * wl.heads * 1e3,
    }


def gemm_context(dev, attention_tflops: float, n: int = 8192, seconds: float = 1.5):
    """Rate of a plain bf16 matrix product (torch.mm, the vendor BLAS) on the
    same GPU, run after the timed region: the sustained matrix-core rate of
    this particular board under its power limit, against which the attention
    kernel's rate can be read (boards of one model differ by several %)."""
    import torch

    a = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    b = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    c = torch.empty(n, n, device=dev, dtype=torch.bfloat16)
    for _ in range(3):
        torch.mm(a, b, out=c)
    torch.cuda.synchronize()
    flop = 2.0 * n ** 3
    reps = max(3, int(seconds * 1.2e15 / flop))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        torch.mm(a, b, out=c)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    tflops = flop / (ms * 1e-3) / 1e12
    del a, b, c
    return {"op": f"torch.mm bf16 {n}x{n}x{n}", "reps": reps, "ms": round(ms, 4), "tflops": round(tflops, 1),
            "attention_kernel_over_gemm": round(attention_tflops / tflops, 4)}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="host time budget of the oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parity", action="store_true")
    ap.add_argument("--variant", choices=("dense", "subset", "sparse", "window", "rope3d", "prepass"),
                    default="dense",
                    help="subset: a quarter of the query tokens attend to all keys; sparse: block-sparse lists "
                         "(a band of 96 key blocks each side of the query block plus 96 global key blocks); "
                         "window: local window of radius (1, 7, 7) around each query; rope3d: the standalone "
                         "rotation of Q (bf16 to bf16); prepass: the key/value pre-pass alone (both HBM-bound)")
    ap.add_argument("--window-layout", choices=("auto", "rows", "patches"), default="auto",
                    help="tiling of the window variant (auto: the one that visits fewer key tiles)")
    ap.add_argument("--no-gemm-context", action="store_true",
                    help="skip the same-box torch.mm bf16 reference rate reported after the timed region")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="before the timed region, run one plain device-to-device copy of this many MiB "
                         "(a kernel of known traffic for scaling memory counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this attention path has no multi-GPU mode "
              "(each GPU would hold its own (batch, head) share); run with --gpus 1", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import video_diffusion_transformer_rope3d_amd as va
    import workloads as wlmod

    wl = wlmod.WORKLOADS[args.workload]
    assert wl.dtype == "bf16", "the benchmark workload is a bf16 one"
    t0 = time.time()
    host = {n: wlmod.full(wl, n) for n in ("q", "k", "v")}
    print(f"# inputs generated in {time.time() - t0:.1f} s", file=sys.stderr, flush=True)

    dev = torch.device("cuda:0")
    q, k, v = (torch.from_numpy(host[n].view(np.int16)).to(dev).view(torch.bfloat16) for n in ("q", "k", "v"))
    o = torch.empty_like(q)
    ws = va.workspace_for(q, True)
    rope = dict(grid=wl.grid, split=wl.split, theta=wl.theta)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()

    if args.calibration_copy_mib > 0:
        n = args.calibration_copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if args.variant != "dense":
        return variant_bench(args, va, wl, host, q, k, v, ws, rope, stream)

    def fused():
        va.attention(q, k, v, scale=wl.scale, out=o, workspace=ws, stream=stream, **rope)

    for _ in range(args.warmup):
        fused()
    torch.cuda.synchronize()

    # ---- timed region: K fused calls
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        ev[i][0].record(stream)
        fused()
        ev[i][1].record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    per_call = [a.elapsed_time(b) for a, b in ev]
    ms_per_step = total_ms / args.steps
    tflops = wl.flops / (ms_per_step * 1e-3) / 1e12

    # ---- the two kernels apart: pre-pass and attention launches, same stream
    def timed(fn, n):
        es = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for a, b in es:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in es]

    prep_ms = timed(lambda: va.prepare(k, v, workspace=ws, stream=stream, **rope), args.steps)
    attn_ms = timed(lambda: va.attend(q, k, v, ws, scale=wl.scale, out=o, stream=stream, **rope), args.steps)
    attn_mean = statistics.mean(attn_ms)
    achieved = wl.flops / (attn_mean * 1e-3) / 1e12

    result = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {**wl.describe(), "qk_mfma": "f16", "pv_mfma": "bf16", "flops_per_call": wl.flops},
        "pct_of_bf16_peak": round(100.0 * tflops / PEAK_TFLOPS, 2),
        "ms_per_call": {"mean": round(statistics.mean(per_call), 3), "median": round(statistics.median(per_call), 3),
                        "min": round(min(per_call), 3)},
        "breakdown_ms": {"kv_prepass": round(statistics.mean(prep_ms), 3), "attention_kernel": round(attn_mean, 3)},
        "roofline": {"kernel": KERNEL, "bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS, 4), "traffic": None},
    }
    # counter-derived figures (committed rocprofv3 summaries of this kernel source, else absent)
    traffic, prof = profile_block(wl.name, KERNEL, attn_mean)
    result["roofline"]["traffic"] = traffic
    if traffic is not None:
        result["roofline"]["hbm_gb_s"] = round(traffic / (attn_mean * 1e-3) / 1e9, 1)
    if prof:
        result["roofline"]["profile"] = prof

    if not args.no_gemm_context:
        result["gemm_context"] = gemm_context(dev, achieved)

    if not args.no_parity:
        sys.path.insert(0, os.path.join(ROOT, "tests"))
        from tests import parity
        st = parity.compare(wl, host, o, slices=[(0, 0), (wl.B - 1, wl.heads - 1)])
        result["parity_sample"] = {k2: (round(v2, 7) if isinstance(v2, float) else v2) for k2, v2 in st.items()}
        result["parity_sample"]["slices"] = "(0,0) and (B-1,heads-1), 256 rows each"

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, host, args.cpu_seconds)

    print(json.dumps(result), flush=True)
    return 0


def variant_bench(args, va, wl, host, q, k, v, ws, rope, stream) -> int:
    """One line for the query-subset or block-sparse attention on the same
    workload: a call is the key/value pre-pass plus the variant's attention;
    FLOPs count only the query-key pairs the variant visits."""
    import numpy as np
    import torch

    import oracle
    import workloads as wlmod

    QB, KB = va.SPARSE_Q_BLOCK, va.SPARSE_K_BLOCK
    if args.variant in ("rope3d", "prepass"):
        return hbm_bench(args, va, wl, q, k, v, ws, rope, stream)
    if args.variant == "window":
        return window_bench(args, va, wl, host, q, k, v, rope, stream)
    if args.variant == "subset":
        idx = wlmod.subset_index(wl, wl.N // 4)
        q_sub = torch.from_numpy(np.ascontiguousarray(host["q"][:, :, idx]).view(np.int16)).cuda().view(torch.bfloat16)
        idx_t = torch.from_numpy(idx).cuda()
        o = torch.empty_like(q_sub)
        flops = 4.0 * wl.B * wl.heads * len(idx) * wl.N * wl.d
        attend = lambda: va.attend_subset(q_sub, idx_t, ws, wl.N, scale=wl.scale, out=o, stream=stream, **rope)
        name = f"{wl.name}-subset{len(idx)}"
        detail = {"active_queries": int(len(idx)), "selection": "seeded distinct tokens, a quarter of N"}
    else:
        blocks, count = wlmod.block_lists(wl, QB, KB, window=96, n_global=96)
        rows_in = np.minimum(QB, wl.N - QB * np.arange(count.shape[-1]))
        ksize = np.minimum(KB, wl.N - KB * np.arange(-(-wl.N // KB)))
        keys = np.where(blocks >= 0, ksize[np.maximum(blocks, 0)], 0).sum(axis=-1)
        flops = 4.0 * wl.d * float((rows_in[None, None, :] * keys).sum())
        bt, ct = torch.from_numpy(blocks).cuda(), torch.from_numpy(count).cuda()
        o = torch.empty_like(q)
        attend = lambda: va.attend_block_sparse(q, ws, bt, ct, scale=wl.scale, out=o, stream=stream, **rope)
        name = f"{wl.name}-blocksparse-w96g96"
        detail = {"max_blocks": int(blocks.shape[-1]), "density": round(flops / wl.flops, 4),
                  "lists": "band of 96 key blocks each side of the query block + 96 seeded global key blocks"}
    prep = lambda: va.prepare(k, v, workspace=ws, stream=stream, **rope)

    for _ in range(args.warmup):
        prep()
        attend()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        prep()
        attend()
    end.record(stream)
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(end) / args.steps
    es = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for a, b in es:
        a.record(stream)
        attend()
        b.record(stream)
    torch.cuda.synchronize()
    attn_mean = statistics.mean(a.elapsed_time(b) for a, b in es)
    achieved = flops / (attn_mean * 1e-3) / 1e12
    mask_path = None
    if args.variant == "sparse":
        # the same blocks as a bit mask: list building on the device + the same attention
        nkb = -(-wl.N // KB)
        mask = np.zeros(count.shape + (nkb,), dtype=bool)
        for ix in np.ndindex(count.shape):
            mask[ix][blocks[ix][:count[ix]]] = True
        words = torch.from_numpy(wlmod.block_mask_words(mask).view(np.int32)).cuda()
        wsm = va.block_mask_workspace_for(q, True)
        va.prepare(k, v, workspace=wsm, stream=stream, **rope)
        om = torch.empty_like(q)
        call_m = lambda: va.attend_block_mask(q, wsm, words, scale=wl.scale, out=om, stream=stream, **rope)
        call_m()
        torch.cuda.synchronize()
        es_m = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        for a, b in es_m:
            a.record(stream)
            call_m()
            b.record(stream)
        torch.cuda.synchronize()
        ms_m = statistics.mean(a.elapsed_time(b) for a, b in es_m)
        mask_path = {"attend_block_mask_ms": round(ms_m, 3), "tflops": round(flops / (ms_m * 1e-3) / 1e12, 2),
                     "bitwise_equal_to_lists": bool(torch.equal(om.view(torch.int16), o.view(torch.int16)))}
        del wsm
    result = {
        "metric": METRIC, "value": round(flops / (ms_per_step * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {**wl.describe(), "workload": name, "variant": args.variant, **detail, "flops_per_call": flops},
        "breakdown_ms": {"attention_kernel": round(attn_mean, 3)},
        "roofline": {"kernel": KERNEL, "bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS, 4), "traffic": None},
    }
    traffic, prof = profile_block(name, KERNEL, attn_mean)
    result["roofline"]["traffic"] = traffic
    if prof:
        result["roofline"]["profile"] = prof
    if mask_path is not None:
        result["bit_mask_path"] = mask_path
    if not args.no_parity:
        from threadpoolctl import threadpool_limits
        dec = oracle.decode_bf16
        worst = dict(max_abs=0.0, mean_rel=0.0)
        for (b, h) in [(0, 0), (wl.B - 1, wl.heads - 1)]:
            with threadpool_limits(16):
                if args.variant == "subset":
                    rows = np.sort(np.random.default_rng(b * 100 + h).choice(len(idx), size=256, replace=False))
                    ref = oracle.rope_attention_subset(dec(host["q"][b, h][idx]), idx, dec(host["k"][b, h]),
                                                       dec(host["v"][b, h]), wl.grid, wl.split, wl.theta, wl.scale,
                                                       rows=rows)
                else:
                    rows = wlmod.sample_rows(wl, b, h)
                    ref = oracle.block_sparse_attention(dec(host["q"][b, h]), dec(host["k"][b, h]),
                                                        dec(host["v"][b, h]), wl.grid, wl.split, wl.theta, wl.scale,
                                                        blocks[b, h], count[b, h], QB, KB, rows=rows)
            got = oracle.decode_bf16(o[b, h, torch.from_numpy(rows).cuda()].view(torch.int16).cpu().numpy()
                                     .view(np.uint16))
            e = np.abs(got - ref)
            worst["max_abs"] = max(worst["max_abs"], float(e.max()))
            worst["mean_rel"] = max(worst["mean_rel"], float(e.sum() / np.abs(ref).sum()))
        result["parity_sample"] = {**{k2: round(v2, 7) for k2, v2 in worst.items()},
                                   "slices": "(0,0) and (B-1,heads-1), 256 rows each"}
    print(json.dumps(result), flush=True)
    return 0


def hbm_bench(args, va, wl, q, k, v, ws, rope, stream) -> int:
    """One of the two HBM-bound kernels alone, at the workload's shape: the
    standalone rotation of Q (reads and writes B*heads*N*d bf16 values) or
    the key/value pre-pass (reads K and V, writes the fp16 rotated keys and
    the transposed V into the workspace). GB/s of algorithmic bytes against
    the 8 TB/s HBM peak."""
    import torch

    n_el = wl.B * wl.heads * wl.N * wl.d
    if args.variant == "rope3d":
        out = torch.empty_like(q)
        call = lambda: va.rope3d(q, wl.grid, wl.split, wl.theta, out=out, stream=stream)  # noqa: E731
        nbytes = 2.0 * n_el * 2
        kernel = "rope3d_kernel"
        what = "standalone rotation of Q, bf16 in, bf16 out"
    else:
        call = lambda: va.prepare(k, v, workspace=ws, stream=stream, **rope)  # noqa: E731
        nbytes = 2.0 * n_el * 2 + ws.numel()
        kernel = "prep_kv_kernel"
        what = "key/value pre-pass: K and V read, rotated fp16 keys and transposed V written"
    for _ in range(max(args.warmup, 1)):
        call()
    torch.cuda.synchronize()
    es = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for a, b in es:
        a.record(stream)
        call()
        b.record(stream)
    torch.cuda.synchronize()
    ms = statistics.mean(a.elapsed_time(b) for a, b in es)
    gbs = nbytes / (ms * 1e-3) / 1e9
    result = {
        "metric": f"{kernel} GB/s on 1 MI355X and % of HBM peak", "value": round(gbs, 1), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {**wl.describe(), "workload": f"{wl.name}-{args.variant}", "variant": args.variant,
                   "bytes_per_call": nbytes, "what": what},
        "roofline": {"kernel": kernel, "bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None},
    }
    traffic, prof = profile_block(result["config"]["workload"], kernel, ms)
    result["roofline"]["traffic"] = traffic
    if prof:
        result["roofline"]["profile"] = prof
    print(json.dumps(result), flush=True)
    return 0


def window_plan_lists(wl, radius):
    """The 64-key tiles the window attention's plan lists for each 256-query
    block, ascending (the planning rule restated: every row within r_h of a
    row that the block's queries of a frame within r_f occupy)."""
    F, H, W = wl.grid
    hw, N = H * W, wl.N
    rf, rh, _ = radius
    lists = []
    for i in range(-(-N // 256)):
        q0, q1 = 256 * i, min(N, 256 * i + 256) - 1
        fa, fb = q0 // hw, q1 // hw
        ya, yb = (q0 - fa * hw) // W, (q1 - fb * hw) // W
        tiles = set()

        def emit(f, lo, hi):
            lo, hi = max(lo, 0), min(hi, H - 1)
            if lo <= hi:
                tiles.update(range(((f * H + lo) * W) // 64, ((f * H + hi) * W + W - 1) // 64 + 1))

        for f in range(max(0, fa - rf), min(F - 1, fb + rf) + 1):
            ga, gb = max(fa, f - rf), min(fb, f + rf)
            if max(ga, fa + 1) <= min(gb, fb - 1):
                emit(f, 0, H - 1)
            elif fa == fb:
                emit(f, ya - rh, yb + rh)
            elif ga == fa and gb == fb:
                if yb + rh >= ya - rh - 1:
                    emit(f, 0, H - 1)
                else:
                    emit(f, 0, yb + rh)
                    emit(f, ya - rh, H - 1)
            elif ga == fa:
                emit(f, ya - rh, H - 1)
            else:
                emit(f, 0, yb + rh)
        lists.append(sorted(tiles))
    return lists


def window_patch_lists(wl, radius):
    """The patch layout's plan restated: for each 16 x 16 query patch
    (f, py, px) of one frame, frame-major, every 8 x 8 key patch
    (tf, ty, tx), tile index (tf*ceil(H/8) + ty)*ceil(W/8) + tx, of frames
    within r_f whose rows and columns meet the patch's rows and columns
    widened by r_h and r_w (clipped to the grid), ascending."""
    F, H, W = wl.grid
    rf, rh, rw = (min(r, n) for r, n in zip(radius, wl.grid))
    tyn, txn = -(-H // 8), -(-W // 8)

    def span(p, n, r):
        return max(0, 16 * p - r) // 8, min(n - 1, min(16 * p + 15, n - 1) + r) // 8

    lists = []
    for f in range(F):
        for py in range(-(-H // 16)):
            for px in range(-(-W // 16)):
                (y0, y1), (x0, x1) = span(py, H, rh), span(px, W, rw)
                lists.append([(tf * tyn + ty) * txn + tx for tf in range(max(0, f - rf), min(F - 1, f + rf) + 1)
                              for ty in range(y0, y1 + 1) for tx in range(x0, x1 + 1)])
    return lists


def window_layout(wl, radius):
    """The layout the library picks for this window: patches when they list
    fewer key tiles in all (ties: rows)."""
    F, H, W = wl.grid
    if F * -(-H // 8) * -(-W // 8) >= 1 << 22 or F * -(-H // 16) * -(-W // 16) >= 1 << 22:
        return "rows"
    rows = sum(len(t) for t in window_plan_lists(wl, radius))
    patches = sum(len(t) for t in window_patch_lists(wl, radius))
    return "patches" if patches < rows else "rows"


def window_plan_counts(wl, radius, layout="rows"):
    lists = window_patch_lists(wl, radius) if layout == "patches" else window_plan_lists(wl, radius)
    return [len(t) for t in lists]


def window_block_rows(wl, layout):
    """Grid tokens (real query rows) of each query block of the layout."""
    F, H, W = wl.grid
    if layout == "rows":
        return [min(wl.N, 256 * i + 256) - 256 * i for i in range(-(-wl.N // 256))]
    return [(min(H, 16 * py + 16) - 16 * py) * (min(W, 16 * px + 16) - 16 * px)
            for _ in range(F) for py in range(-(-H // 16)) for px in range(-(-W // 16))]


def window_tiles(wl, radius, layout="rows"):
    """Query-key pairs the window attention visits (the tiles its plan lists
    per query block, times the block's real query rows) and the pairs inside
    the windows."""
    F, H, W = wl.grid
    rf, rh, rw = radius
    visited = sum(c * 64 * r for c, r in zip(window_plan_counts(wl, radius, layout), window_block_rows(wl, layout)))
    ext = lambda n, r: sum(min(n - 1, c + r) - max(0, c - r) + 1 for c in range(n))
    inside = ext(F, rf) * ext(H, rh) * ext(W, rw)
    return visited, inside


def window_bench(args, va, wl, host, q, k, v, rope, stream) -> int:
    """Local-window attention of radius (1, 7, 7): a call is pre-pass + plan
    + attention. The value counts the method's own work, the query-key pairs
    inside the windows; the pairs of the visited 64-key tiles (what the
    matrix cores compute) are reported beside it, for the whole call and for
    the attention kernel alone (timed on its own from the same workspace)."""
    import numpy as np
    import torch

    import oracle
    import workloads as wlmod

    radius = (1, 7, 7)
    layout = args.window_layout if args.window_layout != "auto" else window_layout(wl, radius)
    visited, inside = window_tiles(wl, radius, layout)
    flops = 4.0 * wl.B * wl.heads * visited * wl.d
    flops_in = 4.0 * wl.B * wl.heads * inside * wl.d
    desc = va.WindowDesc.make(wl.grid, radius, args.window_layout)
    n = va.vidattn_fwd_window_workspace_size(va.BF16, wl.B, wl.heads, wl.N, wl.d, True, desc)
    wws = torch.empty(n, dtype=torch.uint8, device=q.device)
    o = torch.empty_like(q)
    call = lambda: va.window_attention(q, k, v, radius, grid=wl.grid, split=wl.split, theta=wl.theta,
                                       scale=wl.scale, layout=args.window_layout, workspace=wws, out=o,
                                       stream=stream)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    # the FLOP count above restates the planning rule: check it against the
    # tile counts the planning kernel wrote (the workspace tail starts with them)
    want = window_plan_counts(wl, radius, layout)
    nqb = len(want)
    nkt = (wl.N + 63) // 64 if layout == "rows" else wl.grid[0] * -(-wl.grid[1] // 8) * -(-wl.grid[2] // 8)
    base = 256 * wl.d * wl.B * wl.heads * nkt  # the key/value image comes first
    # then the counts, and lists as wide as the most tiles a block lists
    if n != base + (4 * nqb + 255) // 256 * 256 + 4 * nqb * max(want):
        raise RuntimeError(f"window workspace size does not match the {layout} layout")
    if args.warmup > 0:
        got = wws[base:base + 4 * nqb].view(torch.int32).cpu().tolist()
        if got != want:
            raise RuntimeError("window plan tile counts differ from the FLOP-count rule")
    es = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for a, b in es:
        a.record(stream)
        call()
        b.record(stream)
    torch.cuda.synchronize()
    ms = statistics.mean(a.elapsed_time(b) for a, b in es)
    tflops = lambda f, t: f / (t * 1e-3) / 1e12  # noqa: E731
    result = {
        "metric": METRIC, "value": round(tflops(flops_in, ms), 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {**wl.describe(), "workload": f"{wl.name}-window-r{radius[0]}{radius[1]}{radius[2]}",
                   "variant": "window", "radius": list(radius), "layout": layout, "flops_per_call": flops_in,
                   "flops_per_call_visited_tiles": flops,
                   "visited_fraction": round(visited / wl.N ** 2, 4),
                   "pairs_inside_windows_fraction": round(inside / wl.N ** 2, 5)},
        "roofline": {"kernel": KERNEL, "bound": "mfma", "achieved": round(tflops(flops_in, ms), 2),
                     "peak": PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(tflops(flops_in, ms) / PEAK_TFLOPS, 4),
                     "traffic": None,
                     "note": "whole call (pre-pass + plan + attention) against the FLOPs of the pairs inside the "
                             "windows; visited_* count every pair of the visited 64-key tiles",
                     "visited_achieved": round(tflops(flops, ms), 2),
                     "visited_frac": round(tflops(flops, ms) / PEAK_TFLOPS, 4)},
    }
    # the attention kernel's own traffic and counters (committed summaries of
    # this kernel source), beside this run's whole-call time
    traffic, prof = profile_block(result["config"]["workload"], KERNEL, ms, this_run="call")
    result["roofline"]["traffic"] = traffic
    if prof:
        result["roofline"]["profile"] = prof
    if not args.no_parity:
        from threadpoolctl import threadpool_limits
        worst = dict(max_abs=0.0, mean_rel=0.0)
        for (b, h) in [(0, 0), (wl.B - 1, wl.heads - 1)]:
            rows = wlmod.sample_rows(wl, b, h)
            with threadpool_limits(16):
                ref = oracle.window_attention(*(oracle.decode_bf16(host[t][b, h]) for t in ("q", "k", "v")),
                                              wl.grid, wl.split, wl.theta, wl.scale, radius, rows=rows)
            got = oracle.decode_bf16(o[b, h, torch.from_numpy(rows).cuda()].view(torch.int16).cpu().numpy()
                                     .view(np.uint16))
            e = np.abs(got - ref)
            worst["max_abs"] = max(worst["max_abs"], float(e.max()))
            worst["mean_rel"] = max(worst["mean_rel"], float(e.sum() / np.abs(ref).sum()))
        result["parity_sample"] = {**{k2: round(v2, 7) for k2, v2 in worst.items()},
                                   "slices": "(0,0) and (B-1,heads-1), 256 rows each"}
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
