"""Builds the native libraries in-tree.

libgptq.so       -- the HIP kernels and the C ABI (hipcc, gfx950)
libgptq_trace.so -- the same, built with GPTQ_TRACE: phase timestamps of the column
                    loop and the factor's chain (gptq_trace_set; bench.py --trace)
libsynth.so      -- the seeded input generator (gcc, OpenMP)
"""

from __future__ import annotations

import glob
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++20", "-fPIC", "-shared",
    # packed fp32 VALU forms stay off on this target
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")
    return out


def build_gptq(trace: bool = False) -> str:
    """Compiles each kernel file to an object (in parallel), then links the shared library."""
    from concurrent.futures import ThreadPoolExecutor

    srcs = sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))
    obj_dir = os.path.join(ROOT, "_build", "gptq_trace" if trace else "gptq")
    os.makedirs(obj_dir, exist_ok=True)
    cflags = [f for f in HIP_FLAGS if f != "-shared"] + (["-DGPTQ_TRACE"] if trace else [])

    def compile_one(src):
        obj = os.path.join(obj_dir, os.path.basename(src) + ".o")
        _run([HIPCC, *cflags, "-I", os.path.join(ROOT, "include"), "-c", src, "-o", obj])
        return obj

    jobs = max(1, min(len(srcs), os.cpu_count() or 1, 16))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_one, srcs))
    out = os.path.join(PKG, "libgptq_trace.so" if trace else "libgptq.so")
    tmp = out + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-fPIC", "-shared", *objs, "-o", tmp])
    os.replace(tmp, out)
    return out


def build_synth() -> str:
    src = os.path.join(PKG, "synth", "synth.c")
    out = os.path.join(PKG, "synth", "libsynth.so")
    tmp = out + ".tmp"
    _run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", src, "-o", tmp, "-lm"])
    os.replace(tmp, out)
    return out


def build_all():
    return [build_synth(), build_gptq(), build_gptq(trace=True)]


if __name__ == "__main__":
    for p in build_all():
        print(p)
