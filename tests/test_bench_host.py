"""Host-side pieces of bench.py on the CPU: the trace form of the hidden hand-off (copy intervals
covered by product intervals), the attention core's causal flop count, the refusal of more than one
GPU, and the recorded-traffic lookup (only a summary taken on the current GEMM source counts)."""
import hashlib
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def rec(kind, s, e):
    return {"kind": kind, "start_ms": s, "end_ms": e}


def test_hidden_copy_share_from_intervals():
    recs = [rec("product", 1.0, 3.0), rec("product", 2.5, 3.5), rec("product", 5.0, 6.0),
            rec("copy", 0.0, 2.0), rec("copy", 3.0, 5.5), rec("copy", 7.0, 8.0)]
    share, tot = bench.hidden_from_trace(recs)
    # products cover [1, 3.5] and [5, 6]: 1 of the first copy, 0.5 + 0.5 of the second, 0 of the third
    assert tot == pytest.approx(5.5)
    assert share == pytest.approx(2.0 / 5.5)
    assert bench.hidden_from_trace([rec("product", 0.0, 1.0)]) == (None, 0.0)
    # a copy inside one product is hidden whole; overlapping products count once
    share, _ = bench.hidden_from_trace([rec("product", 0.0, 10.0), rec("product", 1.0, 9.0), rec("copy", 2.0, 4.0)])
    assert share == pytest.approx(1.0)


def test_union_merges_touching_intervals():
    assert bench.union([(3, 4), (0, 1), (1, 2), (5, 6), (5.5, 7)]) == [[0, 2], [3, 4], [5, 7]]


def test_core_flops_counts_the_causal_pairs():
    class W:
        q_heads_shard = 8
        tokens = 4 * 16

    fwd, bwd = bench.core_flops(W, 16)
    # per head and sequence: 16 * 17 / 2 = 136 causal pairs, 2 * 128 flops each per product
    per = 136 * 2 * 128 * 8 * 4
    assert fwd == 2 * per and bwd == 4 * per
    # brute force over the pairs of one sequence
    assert sum(1 for t in range(16) for s in range(16) if s <= t) == 136


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "measures one GPU" in r.stderr and r.stdout == ""


def test_recorded_traffic_needs_the_current_gemm_source(tmp_path, monkeypatch):
    sha = hashlib.sha256(open(os.path.join(ROOT, "comm_overlap_amd", "csrc", "gemm.hip"), "rb").read()).hexdigest()
    (tmp_path / "profiles").mkdir()
    (tmp_path / "comm_overlap_amd" / "csrc").mkdir(parents=True)
    (tmp_path / "comm_overlap_amd" / "csrc" / "gemm.hip").write_bytes(
        open(os.path.join(ROOT, "comm_overlap_amd", "csrc", "gemm.hip"), "rb").read())
    kernel = "gemm_kernel<Tile<256, 256, 2, 2, 1>, 1, 0> grid 256 x 256"
    summary = tmp_path / "profiles" / "gemm_kernel_w_traffic.txt"
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.recorded_traffic("w", kernel) is None  # no summary
    summary.write_text(f"kernel: {kernel}\ngemm.hip sha256: {sha}\noutput:\n  traffic_bytes_per_launch: 1\n"
                       f"later line:\ntraffic_bytes_per_launch: 253095995\n")
    assert bench.recorded_traffic("w", kernel) == 253095995.0  # the last such line
    assert bench.recorded_traffic("w", kernel.replace("1, 0>", "0, 0>")) is None  # another kernel
    summary.write_text(f"kernel: {kernel}\ngemm.hip sha256: {'0' * 64}\ntraffic_bytes_per_launch: 5\n")
    assert bench.recorded_traffic("w", kernel) is None  # taken on another source
