"""The trace build (libgptq_trace.so, GPTQ_TRACE) on the GPU: a layer quantized through it records
every kind of phase stamp and gives the plain library's outputs bit for bit (the stamps change no
arithmetic).  The trace library runs in a child process, since the binding loads one library per
process."""

import json
import os
import subprocess
import sys

import numpy as np
import pytest

from gpuhelp import gpu_quantize, say
from post_weight_quantization_03_amd import synth

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import hashlib, json, os, sys
import numpy as np
sys.path.insert(0, sys.argv[1])
import torch
import post_weight_quantization_03_amd as g
g.LIB_PATH = os.path.join(os.path.dirname(g.__file__), "libgptq_trace.so")
KEYS = ("codes", "scales", "zeros", "w_hat", "row_loss", "H_after")
W = np.load(sys.argv[2])
H = np.load(sys.argv[3])
dev = torch.device("cuda:0")
Wd = torch.from_numpy(W.view(np.int16)).to(dev).view(torch.bfloat16)
Hd = torch.from_numpy(H).to(dev)
cap = 1 << 16
buf = torch.zeros(32 * (cap + 1), dtype=torch.int64, device=dev)
buf[0] = cap
g.gptq_trace_set(buf)
o = g.quantize(Wd, Hd, g.Params(bits=4, groupsize=128))
torch.cuda.synchronize()
g.gptq_trace_set(None)
w = buf.cpu().numpy()
n = int(min(w[1], cap))
rec = w[32:32 * (n + 1)].reshape(n, 32)
kinds = sorted(set(int(k) for k in rec[:, 0]))
ok_order = bool(np.all(rec[:, 4] <= rec[np.arange(n), 3 + rec[:, 3]]))
o["H_after"] = Hd
dig = {k: hashlib.sha256(o[k].cpu().numpy().tobytes()).hexdigest() for k in KEYS}
print(json.dumps({"records": int(w[1]), "kinds": kinds, "stamps_ordered": ok_order, "digest": dig}))
"""


def test_trace_build_records_and_matches_plain(tmp_path):
    import hashlib
    rows, cols = 40, 1100  # 9 blocks, the last ragged: every kernel of the chain and loop
    a = synth.Activations(seed=3, tensor=synth.T_X, n=cols, tokens=4 * cols, dist=synth.STUDENT_T4,
                          outliers=11, outlier_factor=20.0, bf16=True)
    X = synth.bf16_to_f32(a.full()).astype(np.float64)
    H = (2.0 * (X.T @ X)).astype(np.float32)
    W = synth.rows(3, synth.T_W, synth.NORMAL, 0.02, cols, 0, rows, bf16=True)
    np.save(tmp_path / "W.npy", W)
    np.save(tmp_path / "H.npy", H)
    say("trace build: quantize 40x1100 through libgptq_trace.so in a child process")
    r = subprocess.run([sys.executable, "-c", CHILD, ROOT, str(tmp_path / "W.npy"),
                        str(tmp_path / "H.npy")], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    child = json.loads(r.stdout.strip().splitlines()[-1])
    say(f"   {child['records']} records, kinds {child['kinds']}")
    assert child["kinds"] == [1, 2, 3, 4, 5]
    assert child["stamps_ordered"]
    out = gpu_quantize(W, H, 4, 128, w_bf16=True)
    for k in ("codes", "scales", "zeros", "w_hat", "row_loss", "H_after"):
        assert hashlib.sha256(np.ascontiguousarray(out[k]).tobytes()).hexdigest() == child["digest"][k], k
