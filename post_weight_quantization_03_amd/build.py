"""Builds the native libraries in-tree.

libgptq.so  -- the HIP kernels and the C ABI (hipcc, gfx950)
libsynth.so -- the seeded input generator (gcc, OpenMP)
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


def build_gptq() -> str:
    srcs = sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))
    out = os.path.join(PKG, "libgptq.so")
    tmp = out + ".tmp"
    _run([HIPCC, *HIP_FLAGS, "-I", os.path.join(ROOT, "include"), *srcs, "-o", tmp, "-L/opt/rocm/lib",
          "-lhipblaslt"])
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
    return [build_synth(), build_gptq()]


if __name__ == "__main__":
    for p in build_all():
        print(p)
