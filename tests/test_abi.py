"""The C ABI on the host (no GPU): every declared symbol is exported, and argument
errors are reported before any device work.  Pointers passed here are never
dereferenced: every call below returns from its host-side checks."""

import ctypes
import os
import re

import pytest

import post_weight_quantization_03_amd as g

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "gptq.h")
FAKE = ctypes.c_void_p(0x1000)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gptq_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    lib = g.lib()
    names = declared_functions()
    assert set(names) == {"gptq_hessian_workspace_bytes", "gptq_accumulate_hessian", "gptq_accumulate_hessian_static",
                          "gptq_quantize_workspace_bytes", "gptq_quantize_layer", "gptq_pack",
                          "gptq_dequant_gemv", "gptq_dequant_gemm_workspace_bytes", "gptq_dequant_gemm",
                          "gptq_hadamard_rows", "gptq_hadamard_hessian",
                          "gptq_cross_workspace_bytes", "gptq_accumulate_cross", "gptq_qep_workspace_bytes",
                          "gptq_qep_correct", "gptq_status_string", "gptq_version", "gptq_trace_set"}
    for n in names:
        assert hasattr(lib, n), n
    # the trace build exports the same symbols
    trace = ctypes.CDLL(os.path.join(os.path.dirname(g.LIB_PATH), "libgptq_trace.so"))
    for n in names:
        assert hasattr(trace, n), n


def test_trace_entry_is_refused_by_the_plain_build():
    """The library built without GPTQ_TRACE records nothing and says so (no device call)."""
    assert g.lib().gptq_trace_set(None) == g.GPTQ_EUNSUPPORTED
    with pytest.raises(g.GptqError):
        g.gptq_trace_set(None)


def test_version_and_status_strings():
    assert g.gptq_version() == 100
    for s in range(6):
        assert g.gptq_status_string(s)
    assert g.gptq_status_string(99) == "unknown status"


def _q(rows, cols, p, W=FAKE, H=FAKE, codes=FAKE, ws=FAKE, ws_bytes=1 << 40):
    return g.lib().gptq_quantize_layer(W, 0, rows, cols, H, ctypes.byref(p), codes, FAKE, FAKE, None, None, ws,
                                       ws_bytes, None, None)


def test_quantize_argument_errors():
    P = g.gptq_params
    assert _q(8, 256, P(5, 128, 128, 0.01, 0)) == g.GPTQ_EINVAL            # bits
    assert _q(8, 256, P(4, 0, 128, 0.01, 0)) == g.GPTQ_EINVAL              # groupsize 0
    assert _q(8, 256, P(4, -2, 128, 0.01, 0)) == g.GPTQ_EINVAL             # groupsize < -1
    assert _q(8, 256, P(4, 96, 128, 0.01, 0)) == g.GPTQ_EUNSUPPORTED       # groupsize 96
    assert _q(8, 256, P(4, 128, 64, 0.01, 0)) == g.GPTQ_EUNSUPPORTED       # blocksize
    assert _q(8, 256, P(4, 128, 128, -1.0, 0)) == g.GPTQ_EINVAL            # damp
    assert _q(8, 256, P(4, 128, 128, float("nan"), 0)) == g.GPTQ_EINVAL
    assert _q(8, 256, P(4, 128, 128, 0.01, 8)) == g.GPTQ_EINVAL            # unknown flag
    assert _q(8, 256, P(4, 128, 128, 0.01, 4)) == g.GPTQ_EINVAL
    assert _q(8, 2, P(4, 128, 128, 0.01, 1)) == g.GPTQ_EINVAL              # shared factor needs cols >= 3
    assert _q(-1, 256, P(4, 128, 128, 0.01, 0)) == g.GPTQ_EINVAL
    assert _q(8, 256, P(4, 128, 128, 0.01, 0), W=None) == g.GPTQ_EINVAL
    assert _q(8, 256, P(4, 128, 128, 0.01, 0), codes=None) == g.GPTQ_EINVAL
    assert _q(8, 256, P(4, 128, 128, 0.01, 0), ws_bytes=16) == g.GPTQ_EWORKSPACE
    assert _q(0, 256, P(4, 128, 128, 0.01, 0), W=None) == g.GPTQ_OK        # empty: no work
    assert _q(8, 0, P(4, 128, 128, 0.01, 0), W=None) == g.GPTQ_OK


def test_quantize_workspace_sizes():
    p = g.Params(bits=4, groupsize=128)
    a = g.gptq_quantize_workspace_bytes(4096, 4096, p)
    b = g.gptq_quantize_workspace_bytes(4096, 4096, g.Params(bits=4, groupsize=128, flags=g.GPTQ_H_IS_FACTOR))
    # working W + error block + the two n x n factor buffers and the doubling scratch
    assert a >= 4096 * 4096 * 4 + 4096 * 128 * 4 + 2 * 4096 * 4096 * 4
    assert b < a and b >= 4096 * 4096 * 4
    assert g.gptq_quantize_workspace_bytes(4096, 4096, g.Params(bits=5)) == 0
    assert g.gptq_quantize_workspace_bytes(0, 4096, p) == 0
    # the fp64 factor option: the work matrix and the diagonal-block buffers in fp64
    c = g.gptq_quantize_workspace_bytes(4096, 4096, g.Params(bits=4, groupsize=128, flags=g.GPTQ_FACTOR_F64))
    assert c - a == 4096 * 4096 * 4 + 32 * 128 * 128 * 4
    d = g.gptq_quantize_workspace_bytes(4096, 4096, g.Params(bits=4, groupsize=128,
                                                             flags=g.GPTQ_FACTOR_F64 | g.GPTQ_H_IS_FACTOR))
    assert d == b


def test_hessian_argument_errors_and_workspace():
    L = g.lib()
    assert L.gptq_accumulate_hessian(FAKE, 64, FAKE, 7, 10, 64, None, 0, None) == g.GPTQ_EINVAL  # dtype
    assert L.gptq_accumulate_hessian(FAKE, 64, FAKE, 0, 10, 32, None, 0, None) == g.GPTQ_EINVAL  # ldx < n
    assert L.gptq_accumulate_hessian(None, 64, FAKE, 0, 10, 64, None, 0, None) == g.GPTQ_EINVAL
    assert L.gptq_accumulate_hessian(FAKE, 64, FAKE, 0, 0, 64, None, 0, None) == g.GPTQ_OK       # no tokens
    need = g.gptq_hessian_workspace_bytes(4096, 262144, g.GPTQ_BF16)
    assert need > 0
    assert L.gptq_accumulate_hessian(FAKE, 4096, FAKE, 0, 262144, 4096, FAKE, need - 1, None) == g.GPTQ_EWORKSPACE
    assert g.gptq_hessian_workspace_bytes(11008, 131072, g.GPTQ_BF16) == 0  # enough tiles: no split


def test_hessian_static_argument_errors_and_limit():
    """The entry point without allocation checks its arguments and its fixed array's limit on the
    host, before any device work."""
    L = g.lib()
    f = L.gptq_accumulate_hessian_static
    assert f(FAKE, 64, FAKE, 7, 10, 64, None) == g.GPTQ_EINVAL       # dtype
    assert f(FAKE, 64, FAKE, 0, 10, 32, None) == g.GPTQ_EINVAL       # ldx < n
    assert f(None, 64, FAKE, 0, 10, 64, None) == g.GPTQ_EINVAL
    assert f(FAKE, -1, FAKE, 0, 10, 64, None) == g.GPTQ_EINVAL
    assert f(FAKE, 64, FAKE, 0, 0, 64, None) == g.GPTQ_OK            # no tokens: no work
    # partials beyond the fixed array: rejected
    assert g.gptq_hessian_workspace_bytes(4096, 4096, g.GPTQ_BF16) > g.GPTQ_HESSIAN_STATIC_BYTES
    assert f(FAKE, 4096, FAKE, 0, 4096, 4096, None) == g.GPTQ_EWORKSPACE
    assert g.gptq_hessian_workspace_bytes(2048, 8192, g.GPTQ_BF16) > g.GPTQ_HESSIAN_STATIC_BYTES
    assert f(FAKE, 2048, FAKE, 0, 8192, 2048, None) == g.GPTQ_EWORKSPACE
    # the limit stated in the header is the one the binding uses
    text = open(HEADER).read()
    assert re.search(r"#define GPTQ_HESSIAN_STATIC_BYTES \(\(size_t\)64 << 20\)", text)
    assert g.GPTQ_HESSIAN_STATIC_BYTES == 64 << 20


@pytest.mark.parametrize("bits,cols", [(3, 40), (4, 12), (5, 64), (2, 8)])
def test_pack_argument_errors(bits, cols):
    assert g.lib().gptq_pack(FAKE, 4, cols, bits, FAKE, None) == g.GPTQ_EINVAL


def _gemv(rows, cols, bits, groupsize, packed=FAKE, x=FAKE, y=FAKE, x_dtype=1):
    return g.lib().gptq_dequant_gemv(packed, FAKE, FAKE, rows, cols, bits, groupsize, x, x_dtype, y, None)


def test_dequant_gemv_argument_errors():
    assert _gemv(8, 256, 5, 128) == g.GPTQ_EINVAL              # bits
    assert _gemv(8, 256, 4, 0) == g.GPTQ_EINVAL                # groupsize 0
    assert _gemv(8, 256, 4, -3) == g.GPTQ_EINVAL               # groupsize < -1
    assert _gemv(8, 40, 3, -1) == g.GPTQ_EINVAL                # cols * bits not whole words
    assert _gemv(8, 12, 4, -1) == g.GPTQ_EINVAL
    assert _gemv(-1, 256, 4, 128) == g.GPTQ_EINVAL
    assert _gemv(8, 256, 4, 48) == g.GPTQ_EUNSUPPORTED         # groups must be whole 32-code runs
    assert _gemv(8, 256, 4, 128, packed=None) == g.GPTQ_EINVAL
    assert _gemv(8, 256, 4, 128, y=None) == g.GPTQ_EINVAL
    assert _gemv(8, 256, 4, 128, x=ctypes.c_void_p(0x1002)) == g.GPTQ_EINVAL  # misaligned
    assert _gemv(8, 256, 4, 128, x_dtype=5) == g.GPTQ_EINVAL  # x dtype
    assert _gemv(0, 256, 4, 128, packed=None) == g.GPTQ_OK     # no rows: no work


def test_dequant_gemm_argument_errors():
    L = g.lib()
    q = L.gptq_dequant_gemm
    assert q(FAKE, FAKE, FAKE, 8, 256, 4, 128, FAKE, 1, 128, 4, FAKE, 8, None, 0, None) == g.GPTQ_EINVAL   # ldx < cols
    assert q(FAKE, FAKE, FAKE, 8, 256, 4, 128, FAKE, 1, 256, 4, FAKE, 4, None, 0, None) == g.GPTQ_EINVAL   # ldy < rows
    assert q(FAKE, FAKE, FAKE, 8, 256, 4, 128, FAKE, 0, 257, 4, FAKE, 8, None, 0, None) == g.GPTQ_EINVAL   # odd bf16 ldx
    assert q(FAKE, FAKE, FAKE, 8, 256, 5, 128, FAKE, 1, 256, 4, FAKE, 8, None, 0, None) == g.GPTQ_EINVAL   # bits
    assert q(FAKE, FAKE, FAKE, 8, 256, 4, 48, FAKE, 1, 256, 4, FAKE, 8, None, 0, None) == g.GPTQ_EUNSUPPORTED
    assert q(FAKE, FAKE, FAKE, 8, 256, 4, 128, FAKE, 1, 256, -1, FAKE, 8, None, 0, None) == g.GPTQ_EINVAL  # batch
    assert q(None, None, None, 8, 256, 4, 128, None, 1, 256, 0, None, 8, None, 0, None) == g.GPTQ_OK      # no vectors
    # the matrix-core path splits the columns of a wide layer over workgroups: a short
    # workspace is refused before any launch
    need = L.gptq_dequant_gemm_workspace_bytes(64, 8192, 4, 128, 8)
    assert need >= 2 * 8 * 64 * 4 and need % 256 == 0
    assert q(FAKE, FAKE, FAKE, 64, 8192, 4, 128, FAKE, 1, 8192, 8, FAKE, 64, FAKE, need - 1, None) == \
        g.GPTQ_EWORKSPACE
    assert q(FAKE, FAKE, FAKE, 64, 8192, 4, 128, FAKE, 1, 8192, 8, FAKE, 64, None, need, None) == g.GPTQ_EWORKSPACE
    assert q(FAKE, FAKE, FAKE, 64, 8192, 4, 128, FAKE, 1, 8192, 8, FAKE, 64, ctypes.c_void_p(0x1002), need,
             None) == g.GPTQ_EINVAL                                                                # misaligned
    # no workspace where the path is not taken: one vector, groups of 64, or one slice
    assert L.gptq_dequant_gemm_workspace_bytes(64, 8192, 4, 128, 1) == 0
    assert L.gptq_dequant_gemm_workspace_bytes(64, 8192, 4, 64, 8) == 0
    assert L.gptq_dequant_gemm_workspace_bytes(64, 256, 4, 128, 8) == 0
    assert L.gptq_dequant_gemm_workspace_bytes(64, 8192, 4, -1, 8) == need
    # up to 16 vectors share a launch: the workspace stops growing there
    assert L.gptq_dequant_gemm_workspace_bytes(64, 8192, 4, 128, 40) == L.gptq_dequant_gemm_workspace_bytes(
        64, 8192, 4, 128, 16)


def test_hadamard_argument_errors():
    L = g.lib()
    B, F = g.GPTQ_BF16, g.GPTQ_F32
    assert L.gptq_hadamard_rows(FAKE, F, 256, FAKE, 256, 4, 256, FAKE, 3, None) == g.GPTQ_EINVAL     # block
    assert L.gptq_hadamard_rows(FAKE, F, 256, FAKE, 256, 4, 256, FAKE, 8192, None) == g.GPTQ_EINVAL  # > 4096
    assert L.gptq_hadamard_rows(FAKE, F, 96, FAKE, 96, 4, 96, FAKE, 64, None) == g.GPTQ_EINVAL       # 64 !| 96
    assert L.gptq_hadamard_rows(FAKE, 7, 256, FAKE, 256, 4, 256, FAKE, 64, None) == g.GPTQ_EINVAL    # dtype
    assert L.gptq_hadamard_rows(FAKE, F, 128, FAKE, 256, 4, 256, FAKE, 64, None) == g.GPTQ_EINVAL    # ld_in < n
    assert L.gptq_hadamard_rows(FAKE, B, 256, FAKE, 256, 4, 256, FAKE, 64, None) == g.GPTQ_EINVAL    # bf16 in place
    assert L.gptq_hadamard_rows(FAKE, F, 256, FAKE, 512, 4, 256, FAKE, 64, None) == g.GPTQ_EINVAL    # strides differ
    assert L.gptq_hadamard_rows(FAKE, F, 256, None, 256, 4, 256, FAKE, 64, None) == g.GPTQ_EINVAL
    assert L.gptq_hadamard_rows(None, F, 256, None, 256, 0, 256, None, 64, None) == g.GPTQ_OK        # no rows
    assert L.gptq_hadamard_hessian(FAKE, 100, FAKE, 8, None) == g.GPTQ_EINVAL                        # 8 !| 100
    assert L.gptq_hadamard_hessian(None, 128, FAKE, 8, None) == g.GPTQ_EINVAL
    assert L.gptq_hadamard_hessian(None, 0, None, 1, None) == g.GPTQ_OK


def test_qep_argument_errors():
    L = g.lib()
    F = g.GPTQ_F32
    T = 100000
    ws = L.gptq_cross_workspace_bytes(256, T, F)
    assert ws > 0
    assert L.gptq_cross_workspace_bytes(256, 10, F) == 0                   # too few tokens to split
    assert L.gptq_cross_workspace_bytes(256, T, 7) == 0                    # bad dtype
    # split partials over the whole square grid: at least the Hessian's upper-tile count
    assert ws >= g.gptq_hessian_workspace_bytes(256, T, F)
    assert L.gptq_accumulate_cross(FAKE, 256, FAKE, FAKE, 7, T, 256, FAKE, ws, None) == g.GPTQ_EINVAL    # dtype
    assert L.gptq_accumulate_cross(FAKE, 256, FAKE, FAKE, F, T, 128, FAKE, ws, None) == g.GPTQ_EINVAL    # ldx < n
    assert L.gptq_accumulate_cross(FAKE, 256, FAKE, None, F, T, 256, FAKE, ws, None) == g.GPTQ_EINVAL
    assert L.gptq_accumulate_cross(FAKE, 256, FAKE, FAKE, F, T, 256, FAKE, ws - 1, None) == g.GPTQ_EWORKSPACE
    assert L.gptq_accumulate_cross(FAKE, 256, FAKE, FAKE, F, 0, 256, None, 0, None) == g.GPTQ_OK         # no tokens
    need = L.gptq_qep_workspace_bytes(64, 256)
    assert need >= 2 * 64 * 256 * 4 + 256 * 256 * 4
    q = L.gptq_qep_correct
    assert q(FAKE, F, 64, 256, FAKE, FAKE, 0.01, 1.5, FAKE, FAKE, need, None, None) == g.GPTQ_EINVAL      # alpha > 1
    assert q(FAKE, F, 64, 256, FAKE, FAKE, -0.1, 0.5, FAKE, FAKE, need, None, None) == g.GPTQ_EINVAL      # damp < 0
    assert q(FAKE, 9, 64, 256, FAKE, FAKE, 0.01, 0.5, FAKE, FAKE, need, None, None) == g.GPTQ_EINVAL      # dtype
    assert q(FAKE, F, 64, 256, FAKE, None, 0.01, 0.5, FAKE, FAKE, need, None, None) == g.GPTQ_EINVAL
    assert q(FAKE, F, 64, 256, FAKE, FAKE, 0.01, 0.5, FAKE, FAKE, need - 1, None, None) == g.GPTQ_EWORKSPACE
    assert q(None, F, 0, 256, None, None, 0.01, 0.5, None, None, 0, None, None) == g.GPTQ_OK              # no rows


def test_product_path_has_no_oracle_import():
    """The package and its binding never reach for the oracle."""
    pkg = os.path.dirname(g.__file__)
    for root, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".c", ".cpp")):
                text = open(os.path.join(root, f)).read()
                assert "oracle" not in text.replace("the oracle", ""), f
