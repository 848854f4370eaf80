"""The Hessian kernels' work decomposition (syrk_plan.h), checked on the host.

The header holds the plan of token splits and pieces, the work item -> (tile, token range,
partial slot) map, each tile's partial slots and the orders in which items take tiles, as plain
constexpr C++ that the kernels compile for the device.  Here g++ compiles the same header beside a
driver (tests/syrk_plan_driver.cpp) that checks:

  * the supertile order, the off-diagonal-first order and the row-major order are bijections onto
    the upper tiles, and the cross term's square supertile order onto all tiles, for 1 ... 139 block
    rows (up to 35584 columns of 256);
  * for 2184 plans (widths 1 ... 11008, 1 ... 262144 tokens, bf16 and fp32, Hessian and cross
    term, 80, 256 and 304 compute units): every partial slot is written by exactly one work item,
    every tile's items cover its tokens exactly once, and tile_slots names exactly the slots of a
    tile's items (the order in which the reduction sums them).
"""

from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "post_weight_quantization_03_amd", "csrc")


def test_work_decomposition(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not found")
    exe = tmp_path / "syrk_plan"
    subprocess.run([gxx, "-std=c++20", "-O2", "-Wall", "-Werror", "-I", CSRC,
                    os.path.join(ROOT, "tests", "syrk_plan_driver.cpp"), "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    print(r.stdout)
    assert r.returncode == 0, r.stdout[-3000:]
    assert "failures 0" in r.stdout
