"""gptq_accumulate_hessian_static -- the Hessian entry point that allocates nothing -- through the
C ABI, against gptq_accumulate_hessian on the same inputs.

Two calls in a row, the second with a smaller input (the fixed array keeps the first call's
partials; the second must not read them), then a call past the array's limit, which must be
refused without touching H.  The two entry points run the same work split and kernels, so H
must agree bit for bit; the first case is also checked against the oracle's fp64 Hessian.
"""

from __future__ import annotations

import numpy as np
import pytest

from gpuhelp import H_RTOL, bf16_dev, say, to_dev, torch_dev
from oracle import hessian_ref
from post_weight_quantization_03_amd import synth

pytestmark = pytest.mark.gpu


def _acts(n, tokens, seed, bf16):
    a = synth.Activations(seed=seed, tensor=synth.T_X, n=n, tokens=tokens, dist=synth.STUDENT_T4,
                          outliers=max(1, n // 100), outlier_factor=20.0, bf16=bf16)
    return a.full()


def _both(X, bf16):
    import post_weight_quantization_03_amd as g
    torch, dev = torch_dev()
    n = X.shape[1]
    Xd = bf16_dev(X) if bf16 else to_dev(X)
    H_ws = torch.zeros((n, n), dtype=torch.float32, device=dev)
    g.gptq_accumulate_hessian(H_ws, Xd)
    H_st = torch.full((n, n), 0.0, dtype=torch.float32, device=dev)
    g.gptq_accumulate_hessian_static(H_st, Xd)
    torch.cuda.synchronize()
    return H_ws.cpu().numpy(), H_st.cpu().numpy()


def test_static_hessian_two_calls_then_limit():
    import post_weight_quantization_03_amd as g
    torch, dev = torch_dev()
    cases = [(1024, 65536, True, 31), (300, 5000, True, 32), (256, 4096, False, 33)]
    for i, (n, tokens, bf16, seed) in enumerate(cases):
        need = g.gptq_hessian_workspace_bytes(n, tokens, g.GPTQ_BF16 if bf16 else g.GPTQ_F32)
        say(f"static-scratch Hessian call {i + 1}: n={n} tokens={tokens} bf16={bf16} partials={need >> 20} MiB")
        assert 0 < need <= g.GPTQ_HESSIAN_STATIC_BYTES
        X = _acts(n, tokens, seed, bf16)
        H_ws, H_st = _both(X, bf16)
        assert np.array_equal(H_st, H_ws), f"max |diff| {np.abs(H_st - H_ws).max()}"
        if i == 0:
            H0 = hessian_ref([synth.bf16_to_f32(X) if bf16 else X], n)
            rel = np.linalg.norm(H_st.astype(np.float64) - H0) / np.linalg.norm(H0)
            say(f"   rel Frobenius vs oracle {rel:.3e}")
            assert rel <= H_RTOL
    # past the limit: refused before any work, H untouched
    n, tokens = 2048, 8192
    say(f"static-scratch Hessian past the limit: n={n} tokens={tokens}")
    H = torch.full((n, n), 5.0, dtype=torch.float32, device=dev)
    Xd = torch.zeros((tokens, n), dtype=torch.bfloat16, device=dev)
    with pytest.raises(g.GptqError) as ei:
        g.gptq_accumulate_hessian_static(H, Xd)
    assert ei.value.status == g.GPTQ_EWORKSPACE
    torch.cuda.synchronize()
    assert bool(torch.all(H == 5.0))
