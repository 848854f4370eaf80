"""Shared helpers of the GPU parity tests: device marshalling, the parity gates and their checks.

Gates (stated here once, used by every parity test):
  H_RTOL      relative Frobenius error of H against the fp64 oracle
  TAU         a code flip is a rounding tie when the oracle's pre-rounding value w/s lies
              within TAU code units of a rounding boundary
  IDENT_MIN   minimum fraction of identical codes (replay protocol)
  SCALE_RTOL  relative error of scales
  LERR_RTOL   |e_gpu / e_oracle - 1| for the relative layer output error
"""

from __future__ import annotations

import sys

import numpy as np

H_RTOL = 1e-4
TAU = 1e-3
IDENT_MIN = 0.999
SCALE_RTOL = 1e-5
LERR_RTOL = 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def torch_dev():
    import torch
    return torch, torch.device("cuda:0")


def to_dev(a):
    torch, dev = torch_dev()
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def bf16_dev(bits):
    torch, dev = torch_dev()
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


def gpu_hessian(X, bf16: bool, chunks=1, ldx_pad=0):
    """H from X on the GPU, optionally in several calls and with a padded row stride."""
    import post_weight_quantization_03_amd as g
    torch, dev = torch_dev()
    n = X.shape[1]
    H = torch.zeros((n, n), dtype=torch.float32, device=dev)
    if ldx_pad:
        Xp = np.zeros((X.shape[0], n + ldx_pad), dtype=X.dtype)
        Xp[:, :n] = X
        Xd_full = bf16_dev(Xp) if bf16 else to_dev(Xp)
        Xd = Xd_full[:, :n]
    else:
        Xd = bf16_dev(X) if bf16 else to_dev(X)
    bounds = np.linspace(0, X.shape[0], chunks + 1).astype(int)
    for a, b in zip(bounds[:-1], bounds[1:]):
        g.gptq_accumulate_hessian(H, Xd[a:b])
    torch.cuda.synchronize()
    return H.cpu().numpy()


def gpu_quantize(W, H32, bits, groupsize, w_bf16=False, damp=0.01, flags=0):
    """Runs gptq_quantize_layer on copies of W and H; returns numpy outputs and the factor."""
    import post_weight_quantization_03_amd as g
    torch, dev = torch_dev()
    Wd = bf16_dev(W) if w_bf16 else to_dev(W.astype(np.float32))
    Hd = to_dev(H32.astype(np.float32))
    out = g.quantize(Wd, Hd, g.Params(bits=bits, groupsize=groupsize, damp=damp, flags=flags))
    torch.cuda.synchronize()
    res = {k: v.cpu().numpy() for k, v in out.items() if v is not None}
    res["U"] = np.triu(Hd.cpu().numpy())
    res["H_after"] = Hd.cpu().numpy()
    return res


def check_quantize(W64, H32, bits, groupsize, out, rows_sel=None, blocked=True, lerr=True):
    """Replay the oracle against the GPU outputs and assert every gate.  Returns the stats."""
    from oracle import gptq_quantize, layer_error, replay_compare
    H64 = H32.astype(np.float32).astype(np.float64)
    ref = gptq_quantize(W64, H64, bits, groupsize, 0.01, blocksize=128 if blocked else None, decision=np.float32)
    sel = slice(None) if rows_sel is None else rows_sel
    st = replay_compare(ref["W_staged"], ref["U"], bits, groupsize, out["codes"][sel].astype(np.int64),
                        out["scales"][sel], out["zeros"][sel], TAU, rows_sel=rows_sel)
    st.pop("what")
    say("   replay:", {k: (round(v, 8) if isinstance(v, float) else v) for k, v in st.items()})
    assert st["hard_flips"] == 0, st
    assert st["zero_hard"] == 0, st
    assert st["identical_frac"] >= IDENT_MIN, st
    assert st["max_scale_rel"] <= SCALE_RTOL, st
    maxq = 2 ** bits - 1
    assert out["codes"].max() <= maxq and out["zeros"].max() <= maxq
    if lerr:
        e_or = layer_error(ref["W_staged"], ref["what"], H64)
        e_gpu = layer_error(ref["W_staged"], out["w_hat"].astype(np.float64), H64)
        if e_or == 0.0:
            # every group exact (a one-value group quantizes without error): so must the GPU's be
            say(f"   layer error gpu {e_gpu:.6e} oracle 0")
            assert e_gpu == 0.0
        else:
            say(f"   layer error gpu {e_gpu:.6e} oracle {e_or:.6e} ratio-1 {e_gpu / e_or - 1:.2e}")
            assert abs(e_gpu / e_or - 1.0) <= LERR_RTOL
        st["lerr_gpu"], st["lerr_oracle"] = e_gpu, e_or
    # the w_hat output decodes the codes with the group grid, bit for bit
    g = W64.shape[1] if groupsize == -1 else groupsize
    s = np.repeat(out["scales"], g, axis=1)[:, :W64.shape[1]].astype(np.float32)
    z = np.repeat(out["zeros"].astype(np.float32), g, axis=1)[:, :W64.shape[1]]
    np.testing.assert_array_equal(out["w_hat"], (s * (out["codes"].astype(np.float32) - z)).astype(np.float32))
    st["ref"] = ref
    return st
