"""Host-side parts of bench.py: the one-GPU refusal and the algorithmic work the
roofline figures are computed from (no GPU is touched)."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused_with_a_message(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert r.stdout == ""
    assert "one GPU" in r.stderr and f"--gpus {n}" in r.stderr


def test_algorithmic_work_of_the_q_proj_layer():
    a = bench.algorithmic(4096, 4096, 262144, 4)
    # symmetric Hessian: N n (n + 1) multiply-adds counted once each way = 4.40e12 flops
    assert a["hessian_flop"] == 262144 * 4096 * 4097
    assert abs(a["hessian_flop"] - 4.40e12) / 4.40e12 < 2e-3
    # X streamed once as bf16: 2.15 GB
    assert a["x_bytes"] == 2 * 262144 * 4096
    # factor and inverse 2 n^3 / 3; quantize loop rows * cols^2, of it the trailing update
    assert a["factor_flop"] == pytest.approx(2 * 4096 ** 3 / 3)
    assert a["quantize_flop"] == 4096.0 ** 3
    assert a["trailing_flop"] == 4096.0 * 4096 * (4096 - 128)
    assert a["total_flop"] == pytest.approx(a["hessian_flop"] + a["factor_flop"] + a["quantize_flop"])


def test_algorithmic_work_of_a_single_block_layer():
    # 128 columns: one block, so no trailing update at all
    a = bench.algorithmic(256, 128, 512, 4)
    assert a["trailing_flop"] == 0.0
    assert a["hessian_flop"] == 512 * 128 * 129


def test_traffic_figure_only_for_the_measured_workload():
    # the stored counter figure belongs to one workload and token count; any other reports none
    t = bench.SYRK_TRAFFIC
    assert bench.syrk_traffic("mlp_7b", t["tokens"]) is None
    assert bench.syrk_traffic(t["workload"], t["tokens"] // 2) is None


def test_cpu_baseline_reports_host_and_stages():
    """The oracle leg on the small 256x256 workload, in full: every stage timed on its own, the host's
    cores, CPU model and BLAS recorded."""
    import argparse

    from post_weight_quantization_03_amd import synth
    wl = synth.workload("linear256")
    lin, acts = wl.linears[0], wl.hessians["x"]
    args = argparse.Namespace(cpu_full=True, cpu_tokens=16384, cpu_rows=512)
    r = bench.cpu_baseline(lin.weight(), acts, 256, 256, acts.tokens, 4, args, x_bf16=False, w_bf16=False)
    assert r["kind"] == "oracle" and r["measured_in_full"] and r["value"] > 0
    assert set(r["stage_seconds"]) == {"hessian", "factor", "quantize_loop"}
    assert all(v > 0 for v in r["stage_seconds"].values())
    assert r["seconds_full_layer"] == pytest.approx(sum(r["stage_seconds"].values()))
    h = r["host"]
    assert h["cpu_count"] == os.cpu_count() and h["cpu_model"] and r["cores"] >= 1
