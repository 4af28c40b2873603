"""bench.py on the CPU: the one-GPU contract, the algorithmic byte and flop
model behind its roofline fractions, and the lookup of committed traffic
counters (reported only while the kernel sources they were taken on are
unchanged)."""
import hashlib
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from block_diffusion_speculative_amd import configs as C  # noqa: E402
from block_diffusion_speculative_amd import inputs as I  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_step_model_qwen3_8b_batch1():
    """The batch-1 workload's bytes and flops: weights once (fc, five
    layers), the lm_head twice (draft head and verify head), the KV cache
    read after injecting 9 rows, the appended rows, features and target
    hidden states."""
    w = C.get("qwen3-8b-b1")
    d = w.dims
    m = bench.step_model(d, 1, np.array([2048]), np.array([9]))
    H, I_, V, hd = 4096, 12288, 151936, 128
    layer = (32 + 2 * 8) * hd * H + H * 32 * hd + 3 * I_ * H
    weights = (H * 5 * H + 5 * layer + 2 * V * H) * 2
    kv = (2048 + 9) * 5 * 2 * 8 * hd * 2 + 9 * 5 * 2 * 8 * hd * 2
    io = 9 * 5 * H * 2 + 17 * H * 2
    assert m["weight_bytes"] == weights
    assert m["bytes"] == weights + kv + io == 4629291008
    flops = 2 * (9 * H * 5 * H + 9 * H * 5 * 2 * 8 * hd) + 2 * 16 * 5 * layer + 2 * 16 * V * H \
        + 2 * 17 * V * H + 4 * 32 * 16 * (2048 + 9 + 16) * hd * 5
    assert m["flops"] == flops


def test_step_model_is_linear_in_ragged_contexts():
    w = C.get("qwen3-8b-b32")
    d = w.dims
    ctx = I.context_lengths(w, 0)
    rows = I.new_row_counts(w, 0, 0)
    m = bench.step_model(d, w.batch, ctx, rows)
    m1 = bench.step_model(d, w.batch, ctx + 1, rows)
    per_pos = w.batch * d.n_layers * 2 * d.n_kv_heads * d.head_dim * 2
    assert m1["bytes"] - m["bytes"] == per_pos


def _write_summary(path, value, sources, digest):
    with open(path, "w") as fh:
        fh.write("# summary\n\n```\n")
        fh.write(f"traffic_bytes_per_launch: {value}\n")
        if sources is not None:
            fh.write(f"sources: {' '.join(sources)}\n")
        fh.write(f"sources_sha256: {digest}\n```\n")


def test_traffic_lookup_follows_the_sources(tmp_path, monkeypatch):
    csrc = os.path.join(ROOT, "block_diffusion_speculative_amd", "csrc")
    srcs = ["gemm_tiled.hip", "common.hpp"]
    h = hashlib.sha256()
    for f in srcs:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic_{}.md"))
    _write_summary(tmp_path / "traffic_good.md", 123456789, srcs, h.hexdigest())
    _write_summary(tmp_path / "traffic_stale.md", 123456789, srcs, "0" * 64)
    assert bench.measured_traffic("good") == 123456789
    assert bench.measured_traffic("stale") is None
    assert bench.measured_traffic("absent") is None
    # a summary that names no sources was taken on the skinny GEMM's files
    h2 = hashlib.sha256()
    for f in bench.TRAFFIC_SOURCES:
        with open(os.path.join(csrc, f), "rb") as fh:
            h2.update(fh.read())
    _write_summary(tmp_path / "traffic_default.md", 42, None, h2.hexdigest())
    assert bench.measured_traffic("default") == 42


def test_block_size_outside_the_sweep_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "qwen3-8b-b1",
                        "--block-size", "4"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "not swept" in r.stderr and r.stdout == ""


def test_head_label_follows_the_routing_rule():
    """The heads run skinny up to 32 rows while two row tiles of activations
    fit the registers (hidden 4096: one sequence's 17 verify rows, two
    anchored blocks) and tiled above (34 rows, two sequences' verify rows);
    at hidden 5120 they switch above 17 rows (40 verify rows of the batch-8,
    B = 4 workload are tiled, and so are 32)."""
    assert bench.HEAD_TILED_MIN_ROWS == 32 and bench.STEP_TILED_MIN_ROWS == 17
    assert bench.head_kernel_label(17).startswith("gemm_kernel<")
    assert bench.head_kernel_label(32).startswith("gemm_kernel<")
    assert bench.head_kernel_label(34).startswith("gemm_tiled_kernel<")
    assert bench.head_kernel_label(17, 5120).startswith("gemm_kernel<")
    assert bench.head_kernel_label(32, 5120).startswith("gemm_tiled_kernel<")
    assert bench.head_kernel_label(40, 5120).startswith("gemm_tiled_kernel<")
    api = open(os.path.join(ROOT, "block_diffusion_speculative_amd", "csrc", "api.hip")).read()
    assert "constexpr int HEAD_TILED_MIN_ROWS = 32;" in api
    assert "constexpr int STEP_TILED_MIN_ROWS = 17;" in api
    hpp = open(os.path.join(ROOT, "block_diffusion_speculative_amd", "csrc", "kernels.hpp")).read()
    assert "(MT * planes <= 2 && per <= 16)" in hpp


def test_extras_default_list_covers_the_measured_workloads():
    names = {(n, b) for n, b in bench.EXTRAS}
    assert ("qwen3-8b-b32", 16) in names and ("qwen3-8b-long", 16) in names
    assert {("larger-b8", b) for b in (4, 8, 16)} <= names
    for n, b in names:
        assert b in C.get(n).block_sizes
