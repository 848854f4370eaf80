"""GPU parity of the fixed randomised Hadamard rotation against the oracle.

Tolerances, from the kernels' arithmetic (u = 2^-24, kb = log2 b):
  rows     out_j = sum over j's block of +-x_k d_k, through kb butterfly
           additions, times fl(1/sqrt b): |err_j| <= (kb + 2) u sum_blk |x_k| / sqrt b.
  Hessian  two such passes: |err_ij| <= (2 kb + 4) u (|Q|^T |H| |Q|)_ij, where
           (|Q|^T |H| |Q|)_ij = sum_{k in blk(i), l in blk(j)} |H_kl| / b.
"""

import numpy as np
import pytest

from gpuhelp import bf16_dev, check_quantize, gpu_quantize, say, to_dev, torch_dev
from oracle import rotate_hessian_ref, rotate_rows_ref, rotation_ref
from post_weight_quantization_03_amd import synth

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24


def _lib():
    import post_weight_quantization_03_amd as g
    g.lib()
    return g


def _signs(n, seed):
    return np.where(np.random.default_rng(seed).random(n) < 0.5, -1.0, 1.0).astype(np.float32)


def _block_abs_sums(A, b):
    """sum over each element's b-block of |A| (rows of A), broadcast back to the elements."""
    m, n = A.shape
    s = np.abs(A).reshape(m, n // b, b).sum(axis=2)
    return np.repeat(s, b, axis=1)


def _rows_bound(A64, b):
    kb = int(np.log2(b))
    return (kb + 2) * U32 * _block_abs_sums(A64, b) / np.sqrt(b)


def _gpu_rows(A, d, b, bf16=False, pad=0, inplace=False):
    g = _lib()
    torch, dev = torch_dev()
    rows, n = A.shape
    if bf16 and pad:
        full = torch.zeros((rows, n + pad), dtype=torch.bfloat16, device=dev)
        full[:, :n] = bf16_dev(A)
        src = full[:, :n]
    elif bf16:
        src = bf16_dev(A)
    elif pad:
        full = torch.zeros((rows, n + pad), dtype=torch.float32, device=dev)
        full[:, :n] = to_dev(A)
        src = full[:, :n]
    else:
        src = to_dev(A)
    out = src if inplace else None
    if pad and not inplace:
        out = torch.full((rows, n + 2 * pad), float("nan"), dtype=torch.float32, device=dev)[:, :n]
    res = g.gptq_hadamard_rows(src, to_dev(d), b, out=out)
    torch.cuda.synchronize()
    return res.cpu().numpy()


@pytest.mark.parametrize("rows,n,b,bf16,pad,inplace", [
    (5, 256, 256, False, 0, False),
    (3, 4096, 4096, True, 0, False),      # one full chunk from bf16
    (7, 11008, 128, True, 0, False),      # 2 full chunks + a 2816-element chunk of 128-blocks
    (4, 8192, 4096, False, 0, False),     # two chunks, two blocks
    (2, 96, 32, False, 3, False),         # padded row strides
    (9, 40, 8, False, 0, True),           # in place
    (6, 300, 4, False, 0, False),
    (3, 12288, 2048, False, 0, True),
    (1, 5120, 1024, False, 0, False),     # one input vector x^T -> (Q^T x)^T
    (2, 1002, 2, False, 0, False),        # width not a multiple of 4: element-wise path
    (3, 4096, 4096, True, 2, False),      # bf16 rows not 8-byte aligned: element-wise path
])
def test_hadamard_rows_parity(rows, n, b, bf16, pad, inplace):
    say(f"hadamard rows rows={rows} n={n} block={b} bf16={bf16} pad={pad} inplace={inplace}")
    A = synth.Activations(seed=n + b, tensor=synth.T_X, n=n, tokens=rows, dist=synth.STUDENT_T4,
                          outliers=max(1, n // 100), outlier_factor=20.0, bf16=bf16).full()
    if bf16:
        A64 = synth.bf16_to_f32(A).astype(np.float64)
        out = _gpu_rows(A, _signs(n, 1), b, bf16=True, pad=pad)
    else:
        A64 = A.astype(np.float64)
        out = _gpu_rows(A, _signs(n, 1), b, pad=pad, inplace=inplace)
    ref = rotate_rows_ref(A64, _signs(n, 1).astype(np.float64), b)
    err = np.abs(out - ref)
    bound = _rows_bound(A64, b)
    say(f"   max err/bound {np.max(err / bound):.3f}")
    assert np.all(np.isfinite(out)) and np.all(err <= bound)


def test_hadamard_rows_block1_is_the_sign_flip():
    say("hadamard rows block=1")
    A = np.random.default_rng(1).standard_normal((3, 1000)).astype(np.float32)
    d = _signs(1000, 2)
    np.testing.assert_array_equal(_gpu_rows(A, d, 1), A * d)


def test_hadamard_rows_q_proj_full_size():
    """The q_proj weights (4096 x 4096 bf16) as the rotated pipeline rotates them: every output."""
    say("hadamard rows q_proj 4096x4096 bf16 block=4096")
    wl = synth.workload("q_proj_4096", tokens=64)
    W_bits = wl.linears[0].weight()
    W64 = synth.bf16_to_f32(W_bits).astype(np.float64)
    d = _signs(4096, 3)
    out = _gpu_rows(W_bits, d, 4096, bf16=True)
    ref = rotate_rows_ref(W64, d.astype(np.float64), 4096)
    err = np.abs(out - ref)
    bound = _rows_bound(W64, 4096)
    say(f"   max err/bound {np.max(err / bound):.3f}")
    assert np.all(err <= bound)


def _hess_bound(H64, b):
    kb = int(np.log2(b))
    n = H64.shape[0]
    nb = n // b
    blk = np.abs(H64).reshape(nb, b, nb, b).sum(axis=(1, 3)) / b
    return (2 * kb + 4) * U32 * np.kron(blk, np.ones((b, b)))


def _gpu_hessian_rot(H32, d, b):
    g = _lib()
    torch, dev = torch_dev()
    Hd = to_dev(H32)
    g.gptq_hadamard_hessian(Hd, to_dev(d), b)
    torch.cuda.synchronize()
    return Hd.cpu().numpy()


@pytest.mark.parametrize("n,b,tokens", [(256, 256, 600), (300, 4, 700), (200, 8, 100), (4096, 4096, 8192),
                                          (302, 2, 500)])  # width not a multiple of 4: element-wise tile pairs
def test_hadamard_hessian_parity(n, b, tokens):
    say(f"hadamard hessian n={n} block={b}")
    X = synth.Activations(seed=5, tensor=synth.T_X, n=n, tokens=tokens, dist=synth.STUDENT_T4,
                          outliers=max(1, n // 100), outlier_factor=20.0, bf16=False).full()
    X64 = X.astype(np.float64)
    H32 = (2.0 * X64.T @ X64).astype(np.float32)
    H32 = np.triu(H32) + np.triu(H32, 1).T  # exactly symmetric input
    d = _signs(n, 4)
    out = _gpu_hessian_rot(H32, d, b)
    H64 = H32.astype(np.float64)
    ref = rotate_hessian_ref(H64, d.astype(np.float64), b)
    err = np.abs(out - ref)
    bound = _hess_bound(H64, b)
    say(f"   max err/bound {np.max(err / bound):.3f}")
    assert np.array_equal(out, out.T), "rotated H not exactly symmetric"
    assert np.all(err <= bound)


def test_hadamard_hessian_sampled_blocks_11008():
    """The MLP width (11008 = 86 x 128): sampled 128-block pairs of Q^T H Q, each Q_I^T H_IJ Q_J."""
    n, b = 11008, 128
    say(f"hadamard hessian n={n} block={b}, sampled block pairs")
    X = synth.Activations(seed=6, tensor=synth.T_X, n=n, tokens=256, dist=synth.STUDENT_T4,
                          outliers=n // 100, outlier_factor=20.0, bf16=False).full()
    X64 = X.astype(np.float64)
    H32 = (2.0 * X64.T @ X64).astype(np.float32)
    H32 = np.triu(H32) + np.triu(H32, 1).T
    d = _signs(n, 8)
    out = _gpu_hessian_rot(H32, d, b)
    assert np.array_equal(out, out.T)
    H64 = H32.astype(np.float64)
    q = rotation_ref(b, np.ones(b), b)  # blockdiag(H_b)/sqrt(b) restricted to one block
    for I, J in [(0, 0), (0, 85), (85, 0), (17, 42), (85, 85), (40, 41)]:
        sI, sJ = slice(I * b, (I + 1) * b), slice(J * b, (J + 1) * b)
        QI = d[sI].astype(np.float64)[:, None] * q
        QJ = d[sJ].astype(np.float64)[:, None] * q
        ref = QI.T @ H64[sI, sJ] @ QJ
        bound = (2 * 7 + 4) * U32 * np.abs(H64[sI, sJ]).sum() / b
        assert np.all(np.abs(out[sI, sJ] - ref) <= bound), (I, J)


def test_rotated_layer_quantizes_to_oracle_parity():
    """W and H rotated on the GPU, then quantized there, against the oracle's quantization of
    its own fp64 rotation of the same W and H (256 x 256, 4-bit g128)."""
    say("rotated 256x256 layer: GPU rotate + quantize vs oracle rotate + quantize")
    g = _lib()
    torch, dev = torch_dev()
    wl = synth.workload("linear256")
    X = wl.hessians["x"].full().astype(np.float64)
    H32 = (2.0 * X.T @ X).astype(np.float32)
    H32 = np.triu(H32) + np.triu(H32, 1).T
    W = wl.linears[0].weight()  # fp32
    d = _signs(256, 9)
    Wr = g.gptq_hadamard_rows(to_dev(W), to_dev(d), 256)
    Hr = to_dev(H32)
    g.gptq_hadamard_hessian(Hr, to_dev(d), 256)
    torch.cuda.synchronize()
    out = gpu_quantize(Wr.cpu().numpy(), Hr.cpu().numpy(), 4, 128, w_bf16=False)
    W64r = rotate_rows_ref(W.astype(np.float64), d.astype(np.float64), 256)
    H32r = rotate_hessian_ref(H32.astype(np.float64), d.astype(np.float64), 256).astype(np.float32)
    check_quantize(W64r, H32r, 4, 128, out, blocked=False)
