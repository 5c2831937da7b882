"""Host-side checks of bench.py: the multi-GPU refusal and the per-kernel
algorithmic work it divides by (no GPU needed)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import moe_inputs as mi  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_gemm_flops_sum_to_the_layer():
    # forward 6 M H I (two products, the first 2I wide), backward 12 M H I
    d = mi.CONFIGS[2]
    f = bench.gemm_flops(d)
    MHI = d.M * d.H * d.I
    assert f["gemm1_swiglu"] + f["gemm2"] == 6 * MHI
    assert sum(f.values()) == 18 * MHI


def test_combine_bytes():
    # k expert rows read and one token row written per token, bf16, plus the
    # per-slot row index and gate (combine) or index only (unpermute)
    d = mi.CONFIGS[2]
    b = bench.hbm_bytes(d)
    rows = (d.T * d.k + d.T) * d.H * 2
    assert b["combine"] == rows + d.T * d.k * 8
    assert b["unpermute_reduce"] == rows + d.T * d.k * 4
