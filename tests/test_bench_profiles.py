"""bench.py's use of committed rocprofv3 summaries (CPU): a summary counts
only for the kernel source, workload and kernel it was taken on, and its
figures reach the bench line labelled with their file and the kernel time of
the profiled run."""
import importlib.util
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
_spec = importlib.util.spec_from_file_location("bench_module", os.path.join(ROOT, "bench.py"))
bench = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(bench)


def _write(d, name, text):
    os.makedirs(os.path.join(d, "profiles"), exist_ok=True)
    with open(os.path.join(d, "profiles", name), "w") as f:
        f.write(text)


def test_profile_block_matches_source_workload_and_kernel(tmp_path, monkeypatch):
    d = str(tmp_path)
    monkeypatch.setattr(bench, "ROOT", d)
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "abc123")
    _write(d, "k-w-traffic.md", "# t\n- workload: W\n- kernel: attn_fwd_bf16_pp_kernel\n- kernel_ms: 180.5\n"
                                "- traffic_bytes_per_launch: 3.4e10\nkernel_source_sha256: abc123\n")
    _write(d, "k-w-counters.md", "# c\n- workload: W\n- kernel_ms: 181.0\n- mfma_busy_frac: 0.7\n"
                                 "- clock_ghz: 1.9\nkernel_source_sha256: abc123\n")
    _write(d, "old-w-counters.md", "- workload: W\n- mfma_busy_frac: 0.1\nkernel_source_sha256: 000000\n")
    _write(d, "other-traffic.md", "- workload: W\n- kernel: prep_kv_kernel\n- traffic_bytes_per_launch: 1\n"
                                  "kernel_source_sha256: abc123\n")
    traffic, block = bench.profile_block("W", "attn_fwd_bf16_pp_kernel", 179.0)
    assert traffic == 3.4e10
    assert block["traffic_file"] == os.path.join("profiles", "k-w-traffic.md")
    assert block["traffic_run_kernel_ms"] == 180.5
    assert block["counters_file"] == os.path.join("profiles", "k-w-counters.md")
    assert block["mfma_busy_frac"] == 0.7 and block["clock_ghz"] == 1.9
    assert block["counters_run_kernel_ms"] == 181.0 and block["this_run_kernel_ms"] == 179.0
    assert bench.profile_block("W", "prep_kv_kernel", 1.0)[0] == 1.0
    assert bench.profile_block("other", "attn_fwd_bf16_pp_kernel", 1.0) == (None, None)
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "def456")
    assert bench.profile_block("W", "attn_fwd_bf16_pp_kernel", 1.0) == (None, None)
