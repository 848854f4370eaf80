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


def test_traffic_figure_belongs_to_the_committed_kernel_sources():
    # the counters were taken on the Hessian sources as committed; a change to them must come
    # with new counters (or the line reports no traffic figure)
    t = bench.SYRK_TRAFFIC
    assert bench.syrk_sources_sha256() == t["sources_sha256"]
    assert bench.syrk_traffic(t["workload"], t["tokens"]) == t["fetch_bytes"] + t["write_bytes"]


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


def test_trace_decoding_on_a_synthetic_buffer():
    """bench.trace_summary on records laid out as gptq_trace_set describes, with known phases."""
    import numpy as np
    R = bench.TRACE_REC
    recs = []

    def add(kind, wg, tag, stamps):
        r = np.zeros(R, dtype=np.int64)
        r[:4] = (kind, wg, tag, len(stamps))
        r[4:4 + len(stamps)] = stamps
        recs.append(r)

    # two loop workgroups of block 1: phases of 5, 1, 0.1, 0.5, 7, 1.5 us (stamps in 10 ns ticks)
    for wg in range(2):
        base = 1000 * wg
        add(bench.TRACE_LOOP, wg, 1, np.cumsum([base, 500, 100, 10, 50, 700, 150]))
    # diagonal factors of blocks 0 and 1: load 2 us, panels 1.5 us, updates 0.5 us, write 1 us
    for k in range(2):
        st = [100000 * k, 100000 * k + 200]
        for p in range(8):
            st.append(st[-1] + 150)
            if p < 7:
                st.append(st[-1] + 50)
        st.append(st[-1] + 100)
        add(bench.TRACE_POTRF, 0, k, st)
    p0_end = 200 + 8 * 150 + 7 * 50 + 100  # end of the diagonal factor of block 0
    # solve of block 0: 2 us after the factor, spanning 6 us; update of block 1: 3 us later, 2 us long
    add(bench.TRACE_TRSM, 0, 0, [p0_end + 200, p0_end + 300, p0_end + 800])
    add(bench.TRACE_DIAG, 0, 1, [p0_end + 1100, p0_end + 1300])
    words = np.zeros(R * (len(recs) + 1), dtype=np.int64)
    words[0] = 100
    words[R:] = np.concatenate(recs)
    out = bench.trace_summary(words, len(recs))
    lw = out["loop_workgroup_us"]
    assert lw["operands_and_near_update"] == 5.0 and lw["steps_128"] == 7.0 and abs(lw["total"] - 15.1) < 1e-9
    df = out["diagonal_factor_us"]
    assert df["load"] == 2.0 and df["panels"] == 12.0 and df["updates"] == 3.5 and df["write"] == 1.0
    assert out["block_solve_workgroup_us"] == {"fill_and_rows": 1.0, "steps_128": 5.0}
    ch = out["chain_step_us"]
    assert ch["steps"] == 1 and ch["solve_span"] == 6.0 and ch["diagonal_update_span"] == 2.0
    # gaps: factor end -> solve 2 us, solve end -> update 3 us, update end -> next factor
    assert abs(ch["gaps_between_launches"] - (2.0 + 3.0 + (100000 - (p0_end + 1300)) / 100.0)) < 1e-9


def test_batch_trace_decoding_on_a_synthetic_buffer():
    """bench.trace_batch_summary on batch-product records (kind 6) with known phases and start times;
    records of other kinds and short records are ignored."""
    import numpy as np
    R = bench.TRACE_REC
    recs = []

    def add(kind, wg, tag, stamps):
        r = np.zeros(R, dtype=np.int64)
        r[:4] = (kind, wg, tag, len(stamps))
        r[4:4 + len(stamps)] = stamps
        recs.append(r)

    # four workgroups: two start at 1 us (ticks of 10 ns), two at 21 us; phases 1, 3, 1, 2, 4, 1 us
    for wg, t0 in enumerate((100, 100, 2100, 2100)):
        add(bench.TRACE_MMA, wg, wg, np.cumsum([t0, 100, 300, 100, 200, 400, 100]))
    add(bench.TRACE_LOOP, 0, 1, np.cumsum([0, 1, 2, 3, 4, 5, 6]))       # another kind
    add(bench.TRACE_MMA, 9, 9, [5, 6, 7])                                # too few stamps
    words = np.zeros(R * (len(recs) + 1), dtype=np.int64)
    words[0] = 100
    words[R:] = np.concatenate(recs)
    out = bench.trace_batch_summary(words, len(recs))
    assert out["workgroups"] == 4
    assert out["kernel_span_us"] == 32.0                  # last end 21 + 12 us, from the first start at 1 us
    assert out["phase_median_us"] == {"x_loads_issued": 1.0, "scale_and_code_loads_issued": 3.0, "lds_zeroed": 1.0,
                                      "staged": 2.0, "chunks_applied": 4.0, "rows_combined_and_written": 1.0}
    assert out["start_us_percentiles"][0] == 0.0 and out["start_us_percentiles"][-1] == 20.0
    assert out["lifetime_us_percentiles"] == [12.0] * 5
    assert out["alive"][0] == 2 and out["alive"][-1] == 0 and max(out["alive"]) == 2
    assert bench.trace_batch_summary(words[:R], 0) == {"workgroups": 0}
