"""bench.py's host logic on the CPU: the algorithmic work it prices the
kernels with, its percentiles, the digest check that keeps stale counter
summaries out of the JSON line, and the single-GPU contract."""
import os
import subprocess
import sys

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_work_of_the_default_workload():
    """K3: D N (N - 1) unique-pair flops plus 2 G alpha N D logit flops per
    slice; bytes N D e + G alpha D e + 12 N. K5: 4 D e per moved row. At 256
    slices of N = 1152 this is 45.9 GFLOP and 81.1 MB, and 266.5 MB for the
    260,278 rows the default input moves."""
    w = synth.WORKLOADS["llama8b_b1"]
    kernels, roofline = bench.kernel_table(w, [1152], 260278, [0.080, 0.013, 0.045])
    N, D, G, A = 1152, 128, 4, 8
    assert kernels["gram"]["flops"] == 256 * (D * N * (N - 1) + 2 * G * A * N * D)
    assert abs(kernels["gram"]["flops"] / 1e9 - 45.9) < 0.05
    assert abs(kernels["gram"]["bytes"] / 1e6 - 81.1) < 0.05
    assert kernels["compact"]["bytes"] == 4 * 128 * 2 * 260278
    assert abs(kernels["gram"]["achieved"] - kernels["gram"]["flops"] / 80e-6 / 1e12) < 1e-6
    assert roofline["kernel"] == "gram" and roofline["unit"] == "TFLOP/s" and roofline["peak"] == 2500.0
    assert abs(roofline["frac"] - kernels["gram"]["achieved"] / 2500.0) < 1e-12


def test_ragged_batch_prices_evicting_sequences_only():
    w = synth.WORKLOADS["llama8b_b32_ragged"]
    lens = [1100, 1152]
    kernels, _ = bench.kernel_table(w, lens, 0, [1.0, 1.0, 1.0])
    per = w.num_layers * w.num_kv_heads
    assert kernels["gram"]["flops"] == per * sum(128 * n * (n - 1) + 2 * 4 * 8 * n * 128 for n in lens)


def test_percentile_is_the_nearest_rank():
    xs = [5.0, 1.0, 4.0, 2.0, 3.0]
    assert bench.percentile(xs, 0) == 1.0
    assert bench.percentile(xs, 50) == 3.0
    assert bench.percentile(xs, 100) == 5.0
    assert bench.percentile([7.0], 90) == 7.0


def test_counter_summaries_need_the_current_kernel_digest(tmp_path, monkeypatch):
    digest = bench.kernel_source_digest("gram")
    assert len(digest) == 16 and digest == bench.kernel_source_digest("gram")
    assert digest != bench.kernel_source_digest("compact")
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    path = tmp_path / "gram_wl_hbm_traffic.md"
    path.write_text(f"# x\n\n- source_digest: `{digest}`\n- traffic_bytes_per_launch: 1234\n")
    assert bench.measured_traffic("gram", "wl") == 1234
    path.write_text("# x\n\n- source_digest: `0000000000000000`\n- traffic_bytes_per_launch: 1234\n")
    assert bench.measured_traffic("gram", "wl") is None
    assert bench.measured_traffic("gram", "missing") is None
    (tmp_path / "gram_wl_mfma_counters.md").write_text(f"- source_digest: `{digest}`\n- mfma_busy_fraction: 0.25\n")
    assert bench.measured_mfma_busy("wl") == 0.25


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr or "single" in r.stderr
    assert r.stdout.strip() == ""


def test_fused_step_is_the_dominant_kernel():
    """With the fused step the roofline describes that one launch: the scoring
    flops over its whole duration, and the time its flops at the MFMA peak
    plus its bytes (scoring, selection and compaction) at the HBM peak would
    take."""
    w = synth.WORKLOADS["qwen14b_b8"]
    kernels, roofline = bench.kernel_table(w, [4224] * 8, 1000, [7.7, 0.09, 2.28], fused_ms=9.0)
    f = kernels["fused_step"]
    assert roofline["kernel"] == "fused_step" and roofline["bound"] == "mfma" and roofline["unit"] == "TFLOP/s"
    assert abs(f["achieved"] - kernels["gram"]["flops"] / 9.0e-3 / 1e12) < 1e-6
    assert f["bytes"] == kernels["gram"]["bytes"] + kernels["select"]["bytes"] + kernels["compact"]["bytes"]
    ideal_us = (kernels["gram"]["flops"] / 2.5e15 + f["bytes"] / 8e12) * 1e6
    assert abs(f["serial_ideal_us"] - ideal_us) < 1e-6
    assert abs(roofline["frac_serial_ideal"] - ideal_us / 9000.0) < 1e-12
    assert abs(roofline["frac"] - f["achieved"] / 2500.0) < 1e-12
    # without it, the staged scoring kernel stays the dominant one
    _, staged = bench.kernel_table(w, [4224] * 8, 1000, [7.7, 0.09, 2.28])
    assert staged["kernel"] == "gram"
