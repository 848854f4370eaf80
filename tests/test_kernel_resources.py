"""The counted waits of the direct-to-LDS pipelines, checked on the compiled gfx950 assembly.

The software pipelines of the Hessian's SYRK (k_hessian.hip), the fp32 GEMM tile (gemm_tile.h,
used by k_gemm.hip and the factor) and the split-bf16 GEMM tile (sgemm_tile.h, used by the quantize
loop) queue `global_load_lds_dwordx4` loads a few stages ahead and retire one stage at each
barrier with `s_waitcnt vmcnt(N)`, N being the number of loads the wave queued for the newest
stage.  Loads complete in issue order, so the wait retires every older stage exactly when every
stage queues N loads; any other vector-memory operation in the loop (a spill's scratch load or
store) only makes it stricter, but costs the pipeline time.  Checked here on the assembly hipcc
produces for gfx950 (host-only: hipcc cross-compiles without a GPU):

  * in every such loop whose body is one basic block (the steady state), the only vector-memory
    instructions are the direct-to-LDS loads, and the loads issued between consecutive counted
    barriers number exactly the count of the later barrier;
  * other vector-memory operations in the prologue and tail loops (spill traffic) are counted:
    they can only make a counted wait stricter;
  * the pipelined kernels outside the Hessian (the fp32 GEMM tiles, the factor's step, the
    quantize launch with its split tiles) use no scratch memory at all.
"""

from __future__ import annotations

import os
import re
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "post_weight_quantization_03_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FILES = ["k_hessian.hip", "k_gemm.hip", "k_factor.hip", "k_quant.hip"]

VMEM = re.compile(r"^\s*(global_|buffer_|scratch_|flat_)\w+")
DMA = re.compile(r"^\s*global_load_lds_dword")
COUNTED = re.compile(r"^\s*s_waitcnt vmcnt\((\d+)\)")
LABEL = re.compile(r"^(\.LBB\d+_\d+):")
BRANCH = re.compile(r"^\s*s_(?:cbranch_\w+|branch)\s+(\.LBB\d+_\d+)")


def _asm(src, tmp_path):
    out = tmp_path / (src + ".s")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++20", "-fPIC", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "--cuda-device-only", "-S",
           os.path.join(CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:]
    return out.read_text().splitlines()


def _kernels(lines):
    """kernel symbol -> its instruction lines (from its label to s_endpgm)."""
    out, name, body = {}, None, []
    for ln in lines:
        m = re.match(r"^(_Z\w+):", ln)
        if m:
            name, body = m.group(1), []
            continue
        if name is not None:
            body.append(ln)
            if re.match(r"^\s*s_endpgm", ln):
                out[name] = body
                name = None
    return out


def _counted_barriers(body, a, b):
    """(line index, N) of every `s_waitcnt vmcnt(N)` with N > 0 followed by s_barrier in body[a:b]."""
    res = []
    for i in range(a, b - 1):
        m = COUNTED.match(body[i])
        if m and int(m.group(1)) > 0 and re.match(r"^\s*s_barrier", body[i + 1]):
            res.append((i, int(m.group(1))))
    return res


def _loops(body):
    """(header index, back-edge index) of every loop: a label branched to from below."""
    labels = {}
    loops = []
    for i, ln in enumerate(body):
        m = LABEL.match(ln)
        if m:
            labels[m.group(1)] = i
        m = BRANCH.match(ln)
        if m and m.group(1) in labels and labels[m.group(1)] < i:
            loops.append((labels[m.group(1)], i))
    return loops


def check_file(lines):
    """Returns (pipelined loops found, steady single-block loops checked, extra vector-memory ops
    found in the other pipelined loops).

    Steady-state loops (one basic block) must hold only the direct loads, the count of each stage
    equal to the wait that retires the stage before it.  The other loops that hold counted barriers
    (prologue and tail stages) may hold other vector-memory operations, such as the spill traffic of
    a tail: an extra operation only makes a counted wait stricter (it cannot leave an older load of
    the pipeline outstanding, since loads complete in issue order), so they are counted, not refused.
    """
    checked = single = extra = 0
    for name, body in _kernels(lines).items():
        for a, b in _loops(body):
            bars = _counted_barriers(body, a, b + 1)
            if not bars:
                continue
            checked += 1
            inner_labels = [i for i in range(a + 1, b + 1) if LABEL.match(body[i])]
            inner_branches = [i for i in range(a, b) if BRANCH.match(body[i])]
            others = [body[i].strip() for i in range(a, b + 1) if VMEM.match(body[i]) and not DMA.match(body[i])]
            if inner_labels or inner_branches:
                extra += len(others)
                continue
            assert not others, f"{name}: vector-memory op inside a steady counted pipeline: {others[0]}"
            single += 1
            # cyclic: the loads queued between consecutive counted barriers of the steady body
            for k, (i, n) in enumerate(bars):
                j = bars[k - 1][0]
                span = list(range(j + 1, i)) if k > 0 else list(range(j + 1, b + 1)) + list(range(a, i))
                loads = sum(1 for t in span if DMA.match(body[t]))
                assert loads == n, f"{name}: {loads} direct loads before a vmcnt({n}) barrier"
    return checked, single, extra


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    tmp = tmp_path_factory.mktemp("asm")
    with ThreadPoolExecutor(max_workers=len(FILES)) as ex:
        return dict(zip(FILES, ex.map(lambda f: _asm(f, tmp), FILES)))


def scratch_sizes(lines):
    """kernel symbol -> (private segment bytes per lane, whether it issues direct-to-LDS loads)."""
    dma = {name: any(DMA.match(ln) for ln in body) for name, body in _kernels(lines).items()}
    out, cur = {}, None
    for ln in lines:
        m = re.match(r"^\s*\.amdhsa_kernel (\S+)", ln)
        if m:
            cur = m.group(1)
            continue
        m = re.match(r"^\s*\.amdhsa_private_segment_fixed_size (\d+)", ln)
        if m and cur is not None:
            out[cur] = (int(m.group(1)), dma.get(cur, False))
            cur = None
    return out


def test_pipelined_tiles_use_no_scratch(asm):
    """A tile that keeps its operands' addresses in scratch memory (for instance a copy of its job
    indexed at run time) issues scratch loads inside its pipeline; outside the Hessian's kernels,
    whose epilogues spill, no pipelined kernel may use scratch at all."""
    seen = 0
    for f in ("k_gemm.hip", "k_factor.hip", "k_quant.hip"):
        for name, (nbytes, dma) in scratch_sizes(asm[f]).items():
            if dma:
                seen += 1
                assert nbytes == 0, f"{f}: {name} uses {nbytes} bytes of scratch per lane"
    assert seen >= 6, seen  # four GEMM tiles, the factor step, the quantize launches


def test_counted_pipelines_hold_only_their_own_loads(asm):
    totals = {f: check_file(lines) for f, lines in asm.items()}
    print(totals)
    # every file with such a pipeline has its steady-state loops checked
    for f in ("k_hessian.hip", "k_gemm.hip", "k_quant.hip"):
        assert totals[f][0] > 0, (f, totals[f])
    assert totals["k_hessian.hip"][1] >= 4, totals  # bf16 Hessian and cross term, two tile kinds each


def test_checker_catches_a_planted_spill_and_a_miscount():
    """The checker itself, on a hand-written loop: a spill inside the pipeline and a stage with one
    load fewer than its wait assumes must both fail."""
    good = """_Zk:
.LBB0_1:                               ; =>This Inner Loop Header: Depth=1
\ts_waitcnt vmcnt(2) lgkmcnt(0)
\ts_barrier
\tglobal_load_lds_dwordx4 v1, s[2:3]
\tglobal_load_lds_dwordx4 v2, s[2:3]
\tv_mfma_f32_32x32x16_bf16 a[0:15], v[4:7], v[8:11], a[0:15]
\ts_waitcnt vmcnt(2) lgkmcnt(0)
\ts_barrier
\tglobal_load_lds_dwordx4 v1, s[4:5]
\tglobal_load_lds_dwordx4 v2, s[4:5]
\ts_cbranch_scc0 .LBB0_1
\ts_endpgm""".splitlines()
    assert check_file(good) == (1, 1, 0)
    spill = good[:6] + ["\tscratch_store_dword off, v3, off offset:4"] + good[6:]
    with pytest.raises(AssertionError):
        check_file(spill)
    short = [ln for k, ln in enumerate(good) if k != 9]
    with pytest.raises(AssertionError):
        check_file(short)
