"""GPTQ layer quantizer for AMD Instinct MI355X (gfx950).

A thin Python binding over the C ABI of ``libgptq.so`` (declared in
``include/gptq.h``).  The functions carry the C names; they only marshal
arguments -- device pointers and the current HIP stream of PyTorch-ROCm
tensors -- and raise ``GptqError`` on a non-zero status.  Every step of the
quantizer runs in the library's HIP kernels; there is no other code path.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgptq.so")

GPTQ_OK, GPTQ_EINVAL, GPTQ_ENOTPD, GPTQ_EWORKSPACE, GPTQ_EUNSUPPORTED, GPTQ_EHIP = range(6)
GPTQ_BF16, GPTQ_F32 = 0, 1
GPTQ_H_IS_FACTOR = 1
GPTQ_FACTOR_F64 = 2


class GptqError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {gptq_status_string(status)} (status {status})")


class gptq_params(ctypes.Structure):
    _fields_ = [("bits", ctypes.c_int32), ("groupsize", ctypes.c_int32), ("blocksize", ctypes.c_int32),
                ("damp", ctypes.c_float), ("flags", ctypes.c_int32)]


@dataclass
class Params:
    """GPTQ(wbits, groupsize) knobs; see gptq_params in include/gptq.h."""

    bits: int = 4
    groupsize: int = 128
    blocksize: int = 128
    damp: float = 0.01
    flags: int = 0

    def c(self) -> gptq_params:
        return gptq_params(self.bits, self.groupsize, self.blocksize, self.damp, self.flags)


_lib = None


def lib():
    """The loaded libgptq.so.  Raises if it has not been built: there is no fallback."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with post_weight_quantization_03_amd.build")
    # PyTorch-ROCm ships its own HIP runtime under the same soname.  Loading torch first
    # makes the library bind to that already-loaded runtime, so tensors, streams and the
    # library's launches share one runtime instead of two in one process.
    import torch  # noqa: F401
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    L.gptq_hessian_workspace_bytes.argtypes = [i64, i64, ctypes.c_int]
    L.gptq_hessian_workspace_bytes.restype = sz
    L.gptq_accumulate_hessian.argtypes = [vp, i64, vp, ctypes.c_int, i64, i64, vp, sz, vp]
    L.gptq_accumulate_hessian.restype = ctypes.c_int
    L.gptq_accumulate_hessian_static.argtypes = [vp, i64, vp, ctypes.c_int, i64, i64, vp]
    L.gptq_accumulate_hessian_static.restype = ctypes.c_int
    L.gptq_quantize_workspace_bytes.argtypes = [i64, i64, ctypes.POINTER(gptq_params)]
    L.gptq_quantize_workspace_bytes.restype = sz
    L.gptq_quantize_layer.argtypes = [vp, ctypes.c_int, i64, i64, vp, ctypes.POINTER(gptq_params), vp, vp, vp,
                                      vp, vp, vp, sz, vp, vp]
    L.gptq_quantize_layer.restype = ctypes.c_int
    L.gptq_pack.argtypes = [vp, i64, i64, i32, vp, vp]
    L.gptq_pack.restype = ctypes.c_int
    L.gptq_dequant_gemv.argtypes = [vp, vp, vp, i64, i64, i32, i32, vp, ctypes.c_int, vp, vp]
    L.gptq_dequant_gemv.restype = ctypes.c_int
    L.gptq_dequant_gemm_workspace_bytes.argtypes = [i64, i64, i32, i32, i64]
    L.gptq_dequant_gemm_workspace_bytes.restype = ctypes.c_size_t
    L.gptq_dequant_gemm.argtypes = [vp, vp, vp, i64, i64, i32, i32, vp, ctypes.c_int, i64, i64, vp, i64, vp,
                                    ctypes.c_size_t, vp]
    L.gptq_dequant_gemm.restype = ctypes.c_int
    L.gptq_hadamard_rows.argtypes = [vp, ctypes.c_int, i64, vp, i64, i64, i64, vp, i32, vp]
    L.gptq_hadamard_rows.restype = ctypes.c_int
    L.gptq_hadamard_hessian.argtypes = [vp, i64, vp, i32, vp]
    L.gptq_hadamard_hessian.restype = ctypes.c_int
    L.gptq_cross_workspace_bytes.argtypes = [i64, i64, ctypes.c_int]
    L.gptq_cross_workspace_bytes.restype = sz
    L.gptq_accumulate_cross.argtypes = [vp, i64, vp, vp, ctypes.c_int, i64, i64, vp, sz, vp]
    L.gptq_accumulate_cross.restype = ctypes.c_int
    L.gptq_qep_workspace_bytes.argtypes = [i64, i64]
    L.gptq_qep_workspace_bytes.restype = sz
    L.gptq_qep_correct.argtypes = [vp, ctypes.c_int, i64, i64, vp, vp, ctypes.c_float, ctypes.c_float, vp, vp, sz,
                                   vp, vp]
    L.gptq_qep_correct.restype = ctypes.c_int
    L.gptq_status_string.argtypes = [ctypes.c_int]
    L.gptq_status_string.restype = ctypes.c_char_p
    L.gptq_version.argtypes = []
    L.gptq_version.restype = ctypes.c_int
    L.gptq_trace_set.argtypes = [vp]
    L.gptq_trace_set.restype = ctypes.c_int
    _lib = L
    return L


# --------------------------------------------------------------------------- marshalling helpers

def _torch():
    import torch
    return torch


def _stream(stream=None):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return GPTQ_BF16
    if t.dtype == torch.float32:
        return GPTQ_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _check_dev(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous device tensors")


def _workspace(nbytes, like, stream=None):
    """A temporary workspace, freed when the caller drops it.  PyTorch's caching allocator ties a
    block to the stream current at allocation; when the library's work runs on another stream,
    the block is recorded on that stream too, so it is not handed out again before that work is
    done."""
    torch = _torch()
    ws = torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=like.device)
    if stream is not None:
        ws.record_stream(stream)
    return ws


# --------------------------------------------------------------------------- entry points

def gptq_status_string(status: int) -> str:
    return lib().gptq_status_string(int(status)).decode()


def gptq_version() -> int:
    return int(lib().gptq_version())


def gptq_trace_set(buf) -> None:
    """Points the trace build's phase timestamps at buf (an int64 device tensor laid out as
    gptq_trace_set in gptq.h describes), or stops them (None).  Raises GptqError with
    GPTQ_EUNSUPPORTED on the library built without tracing."""
    st = lib().gptq_trace_set(None if buf is None else _ptr(buf))
    if st:
        raise GptqError(st, "gptq_trace_set")


def gptq_hessian_workspace_bytes(n: int, tokens: int, x_dtype: int) -> int:
    return int(lib().gptq_hessian_workspace_bytes(n, tokens, x_dtype))


def gptq_accumulate_hessian(H, X, workspace=None, stream=None):
    """H [n, n] fp32 += 2 X^T X for X [tokens, n] (bf16 or fp32, unit column stride)."""
    _check_dev(H)
    if not X.is_cuda or X.stride(1) != 1:
        raise ValueError("X must be a device tensor with unit column stride")
    n = H.shape[0]
    if H.dtype != _torch().float32 or H.shape != (n, n) or X.shape[1] != n:
        raise ValueError("shape or dtype mismatch")
    dt = _dtype_code(X)
    need = gptq_hessian_workspace_bytes(n, X.shape[0], dt)
    if workspace is None:
        workspace = _workspace(need, H, stream)
    st = lib().gptq_accumulate_hessian(_ptr(H), n, _ptr(X), dt, X.shape[0], X.stride(0), _ptr(workspace),
                                       workspace.numel(), _stream(stream))
    if st:
        raise GptqError(st, "gptq_accumulate_hessian")
    return H


GPTQ_HESSIAN_STATIC_BYTES = 64 << 20


def gptq_accumulate_hessian_static(H, X, stream=None):
    """gptq_accumulate_hessian with the partial tiles in the library's fixed device array: no
    workspace and no allocation, for calls whose workspace need fits GPTQ_HESSIAN_STATIC_BYTES."""
    _check_dev(H)
    if not X.is_cuda or X.stride(1) != 1:
        raise ValueError("X must be a device tensor with unit column stride")
    n = H.shape[0]
    if H.dtype != _torch().float32 or H.shape != (n, n) or X.shape[1] != n:
        raise ValueError("shape or dtype mismatch")
    st = lib().gptq_accumulate_hessian_static(_ptr(H), n, _ptr(X), _dtype_code(X), X.shape[0], X.stride(0),
                                              _stream(stream))
    if st:
        raise GptqError(st, "gptq_accumulate_hessian_static")
    return H


def gptq_quantize_workspace_bytes(rows: int, cols: int, params: Params) -> int:
    p = params.c()
    return int(lib().gptq_quantize_workspace_bytes(rows, cols, ctypes.byref(p)))


def gptq_quantize_layer(W, H, params: Params, codes, scales, zeros, w_hat=None, row_loss=None, workspace=None,
                        d_status=None, stream=None):
    """Quantize W [rows, cols] against H [cols, cols]; H is overwritten by the factor.

    With ``d_status`` (a device int32 tensor) the call is asynchronous and the final
    status lands there; without it the call synchronizes and raises on failure.
    """
    _check_dev(W, H, codes, scales, zeros, w_hat, row_loss, d_status)
    rows, cols = W.shape
    p = params.c()
    need = int(lib().gptq_quantize_workspace_bytes(rows, cols, ctypes.byref(p)))
    if workspace is None:
        workspace = _workspace(need, W, stream)
    st = lib().gptq_quantize_layer(_ptr(W), _dtype_code(W), rows, cols, _ptr(H), ctypes.byref(p), _ptr(codes),
                                   _ptr(scales), _ptr(zeros), _ptr(w_hat), _ptr(row_loss), _ptr(workspace),
                                   workspace.numel(), _ptr(d_status), _stream(stream))
    if st:
        raise GptqError(st, "gptq_quantize_layer")
    return codes


def gptq_pack(codes, bits: int, packed, stream=None):
    """codes [rows, cols] uint8 -> packed [rows, cols*bits/32] (int32 tensor holding uint32 words)."""
    _check_dev(codes, packed)
    rows, cols = codes.shape
    st = lib().gptq_pack(_ptr(codes), rows, cols, bits, _ptr(packed), _stream(stream))
    if st:
        raise GptqError(st, "gptq_pack")
    return packed


def gptq_dequant_gemv(packed, scales, zeros, bits: int, groupsize: int, x, y, stream=None):
    """y [rows] fp32 = W^ x with W^ decoded from packed [rows, cols*bits/32] codes, scales and zeros [rows, G];
    x [cols] bf16 or fp32."""
    _check_dev(packed, scales, zeros, x, y)
    torch = _torch()
    rows, cols = packed.shape[0], x.shape[0]
    if (y.dtype != torch.float32 or scales.dtype != torch.float32
            or zeros.dtype != torch.uint8 or y.shape != (rows,) or x.dim() != 1
            or packed.dim() != 2 or packed.shape[1] * 32 != cols * bits or packed.element_size() != 4
            or scales.shape != zeros.shape or scales.shape[0] != rows):
        raise ValueError("shape or dtype mismatch")
    st = lib().gptq_dequant_gemv(_ptr(packed), _ptr(scales), _ptr(zeros), rows, cols, bits, groupsize, _ptr(x),
                                 _dtype_code(x), _ptr(y), _stream(stream))
    if st:
        raise GptqError(st, "gptq_dequant_gemv")
    return y


def gptq_dequant_gemm_workspace_bytes(rows: int, cols: int, bits: int, groupsize: int, batch: int) -> int:
    return int(lib().gptq_dequant_gemm_workspace_bytes(rows, cols, bits, groupsize, batch))


def gptq_dequant_gemm(packed, scales, zeros, bits: int, groupsize: int, X, Y, workspace=None, stream=None):
    """Y [batch, rows] fp32 = (W^ X^T)^T for X [batch, cols] bf16 or fp32 (unit column stride).
    workspace: a device tensor of at least gptq_dequant_gemm_workspace_bytes bytes; allocated here
    (through torch, tied to the stream the kernels run on) when None."""
    _check_dev(packed, scales, zeros, Y)
    torch = _torch()
    rows = packed.shape[0]
    if X.dim() != 2 or not X.is_cuda or X.stride(1) != 1:
        raise ValueError("X must be a 2-D device tensor with unit column stride")
    batch, cols = X.shape
    if (Y.dtype != torch.float32 or Y.shape != (batch, rows) or scales.dtype != torch.float32
            or zeros.dtype != torch.uint8 or packed.dim() != 2 or packed.shape[1] * 32 != cols * bits
            or packed.element_size() != 4 or scales.shape != zeros.shape or scales.shape[0] != rows):
        raise ValueError("shape or dtype mismatch")
    ldx = X.stride(0) if batch > 1 else cols
    need = gptq_dequant_gemm_workspace_bytes(rows, cols, bits, groupsize, batch)
    if workspace is None and need:
        workspace = _workspace(need, Y, stream)
    wsz = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().gptq_dequant_gemm(_ptr(packed), _ptr(scales), _ptr(zeros), rows, cols, bits, groupsize, _ptr(X),
                                 _dtype_code(X), ldx, batch, _ptr(Y), Y.stride(0) if batch > 1 else rows,
                                 None if workspace is None else _ptr(workspace), wsz, _stream(stream))
    if st:
        raise GptqError(st, "gptq_dequant_gemm")
    return Y


def gptq_hadamard_rows(inp, signs, block: int, out=None, stream=None):
    """out [rows, n] fp32 = inp Q (inp bf16 or fp32 with unit column stride); out may be inp (fp32)."""
    torch = _torch()
    if inp.dim() != 2 or not inp.is_cuda or inp.stride(1) != 1:
        raise ValueError("inp must be a 2-D device tensor with unit column stride")
    rows, n = inp.shape
    if out is None:
        out = torch.empty((rows, n), dtype=torch.float32, device=inp.device)
    if (out.dtype != torch.float32 or out.shape != (rows, n) or out.stride(1) != 1 or not out.is_cuda
            or signs.dtype != torch.float32 or signs.shape != (n,)):
        raise ValueError("shape or dtype mismatch")
    _check_dev(signs)
    # a one-row tensor may carry any stride on its first axis (NumPy gives 0 for x[None, :])
    ld_in = inp.stride(0) if rows > 1 else n
    ld_out = out.stride(0) if rows > 1 else n
    st = lib().gptq_hadamard_rows(_ptr(inp), _dtype_code(inp), ld_in, _ptr(out), ld_out, rows, n,
                                  _ptr(signs), block, _stream(stream))
    if st:
        raise GptqError(st, "gptq_hadamard_rows")
    return out


def gptq_hadamard_hessian(H, signs, block: int, stream=None):
    """H [n, n] fp32 := Q^T H Q in place."""
    _check_dev(H, signs)
    n = H.shape[0]
    torch = _torch()
    if H.dtype != torch.float32 or H.shape != (n, n) or signs.dtype != torch.float32 or signs.shape != (n,):
        raise ValueError("shape or dtype mismatch")
    st = lib().gptq_hadamard_hessian(_ptr(H), n, _ptr(signs), block, _stream(stream))
    if st:
        raise GptqError(st, "gptq_hadamard_hessian")
    return H


def gptq_cross_workspace_bytes(n: int, tokens: int, x_dtype: int) -> int:
    return int(lib().gptq_cross_workspace_bytes(n, tokens, x_dtype))


def gptq_accumulate_cross(C, X, Xq, workspace=None, stream=None):
    """C [n, n] fp32 += 2 X^T Xq for X, Xq [tokens, n] (same dtype, unit column stride, same row stride)."""
    _check_dev(C)
    n = C.shape[0]
    torch = _torch()
    if (C.dtype != torch.float32 or C.shape != (n, n) or X.shape != Xq.shape or X.shape[1] != n
            or X.dtype != Xq.dtype or X.stride() != Xq.stride() or X.stride(1) != 1 or not X.is_cuda
            or not Xq.is_cuda):
        raise ValueError("shape, dtype or stride mismatch")
    if workspace is None:
        workspace = _workspace(gptq_cross_workspace_bytes(n, X.shape[0], _dtype_code(X)), C, stream)
    st = lib().gptq_accumulate_cross(_ptr(C), n, _ptr(X), _ptr(Xq), _dtype_code(X), X.shape[0], X.stride(0),
                                     _ptr(workspace), workspace.numel(), _stream(stream))
    if st:
        raise GptqError(st, "gptq_accumulate_cross")
    return C


def gptq_qep_workspace_bytes(rows: int, cols: int) -> int:
    return int(lib().gptq_qep_workspace_bytes(rows, cols))


def gptq_qep_correct(W, C, H, alpha: float, damp: float = 0.01, W_out=None, workspace=None, d_status=None,
                     stream=None):
    """W_out = W + alpha W (C - H) H_d^-1; afterwards C holds C - H and H the factor (for GPTQ_H_IS_FACTOR)."""
    _check_dev(W, C, H, W_out, d_status)
    torch = _torch()
    rows, cols = W.shape
    if C.shape != (cols, cols) or H.shape != (cols, cols) or C.dtype != torch.float32 or H.dtype != torch.float32:
        raise ValueError("shape or dtype mismatch")
    if W_out is None:
        W_out = torch.empty((rows, cols), dtype=torch.float32, device=W.device)
    if workspace is None:
        workspace = _workspace(gptq_qep_workspace_bytes(rows, cols), W, stream)
    st = lib().gptq_qep_correct(_ptr(W), _dtype_code(W), rows, cols, _ptr(C), _ptr(H), damp, alpha, _ptr(W_out),
                                _ptr(workspace), workspace.numel(), _ptr(d_status), _stream(stream))
    if st:
        raise GptqError(st, "gptq_qep_correct")
    return W_out


def quantize(W, H, params: Params, stream=None, want_what=True):
    """Allocates the outputs on W's device and runs gptq_quantize_layer synchronously."""
    torch = _torch()
    rows, cols = W.shape
    g = cols if params.groupsize == -1 else params.groupsize
    G = -(-cols // g)
    dev = W.device
    out = {
        "codes": torch.empty((rows, cols), dtype=torch.uint8, device=dev),
        "scales": torch.empty((rows, G), dtype=torch.float32, device=dev),
        "zeros": torch.empty((rows, G), dtype=torch.uint8, device=dev),
        "w_hat": torch.empty((rows, cols), dtype=torch.float32, device=dev) if want_what else None,
        "row_loss": torch.empty((rows,), dtype=torch.float32, device=dev),
    }
    gptq_quantize_layer(W, H, params, out["codes"], out["scales"], out["zeros"], out["w_hat"], out["row_loss"],
                        stream=stream)
    return out
