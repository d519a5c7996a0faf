"""Smoke tests of bench.py on the CPU: the one-GPU guard, the byte and flop accounting behind its roofline figures
(against the storage and adapter counts the pages print), the lookup of committed profile figures, and the
CPU-oracle baseline leg on a small layer. The GPU side of the bench is covered by tests/test_gpu_bench.py."""
import hashlib
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    for n in (2, 8):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)], capture_output=True,
                           text=True, timeout=300)
        assert r.returncode == 2
        assert "one GPU" in r.stderr and r.stdout == ""


def test_projection_bytes_match_the_pages():
    # "QeRL: When Quantized Weights Help Reinforcement Learning, and Where the Evidence Stops" §3.1: P NVFP4 weights
    # take 4P/8 bytes of codes plus one byte per 16 weights, 9P/16; for P = 4096 x 4096 that is 9,437,184 bytes
    # (plus the one f32 tensor scale the accounting here adds)
    assert bench.proj_bytes(4096, 4096, 0, 0) == 9_437_184 + 4
    # same page §2.1: rank 32 on a 4096 x 4096 matrix adds 32 (4096 + 4096) = 262,144 adapter parameters (bf16)
    assert bench.proj_bytes(4096, 4096, 0, 32) - bench.proj_bytes(4096, 4096, 0, 0) == 2 * 262_144
    # M bf16 activations in (K wide) and out (N wide)
    assert bench.proj_bytes(1024, 4096, 16, 0) - bench.proj_bytes(1024, 4096, 0, 0) == 2 * 16 * (1024 + 4096)


def test_headline_accounting():
    from nvfp4_weight_only_amd.layer import QWEN25_7B as S
    # the gate|up launch at 16 tokens: two 18,944 x 3,584 NVFP4 weights, two rank-32 LoRA-B, x in and the product out
    assert bench.gateup_main_bytes(S, 16) == 79_527_944
    # the layer step: the seven projections (q 3584, k and v 512, o 3584 wide; gate, up 18,944; down 3,584 wide
    # over 18,944), two norms' gamma and noise
    assert bench.layer_bytes(S, 16) == sum(bench.proj_bytes(n, k, 16, 32) for n, k in [
        (3584, 3584), (512, 3584), (512, 3584), (3584, 3584), (18944, 3584), (18944, 3584), (3584, 18944)]) + 12 * 3584
    assert 139.7e6 < bench.layer_bytes(S, 16) < 139.9e6
    # prefill: 2 M N K per weight plus the LoRA, 2.248 TFLOP for the 7B gate|up at 8,192 tokens
    assert abs(bench.prefill_flops(S, 8192) / 1e12 - 2.248) < 1e-3


def test_profile_figures_are_used_only_for_the_current_kernel_source(tmp_path):
    sha = hashlib.sha256(open(bench.KERNEL_SOURCE, "rb").read()).hexdigest()
    p = tmp_path / "summary.md"
    p.write_text(f"avg_duration_us[k_x] = 20.42 (linear.hip sha256 {sha})\n"
                 f"avg_duration_us[k_y] = 11.00 (linear.hip sha256 {'0' * 64})\n")
    assert bench.profile_value(str(p), "avg_duration_us", "k_x") == pytest.approx(20.42)
    assert bench.profile_value(str(p), "avg_duration_us", "k_y") is None  # taken on another kernel source
    assert bench.profile_value(str(p), "avg_duration_us", "k_z") is None
    assert bench.profile_value(str(tmp_path / "missing.md"), "avg_duration_us", "k_x") is None


def test_cpu_baseline_leg_on_a_small_layer():
    from nvfp4_weight_only_amd.layer import LayerShape
    shape = LayerShape(hidden=256, q_dim=256, kv_dim=128, inter=512, head_dim=64, rank=16)
    for threads in (1, 2):
        r = bench.cpu_baseline(shape, 4, 0.01, row_stride=2, threads=threads)
        assert r["kind"] == "oracle" and r["cores"] == threads and r["value"] > 0
        assert r["unit"] == "tokens/s (28-layer equivalent)"
        assert r["value"] == pytest.approx(4 / (28 * r["layer_step_s"]))
