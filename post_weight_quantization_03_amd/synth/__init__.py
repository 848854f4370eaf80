"""Seeded synthetic weights and calibration activations.

This module only draws inputs; it holds none of the quantizer's arithmetic.
Both the HIP path and the oracle are fed from it.  The generator is
SplitMix64 in counter mode (see ``synth.c``), so a row range or a column
subset regenerates bit-identically on its own.

Workload presets follow the layer shapes and input laws of the pages'
workloads: Llama-2-7B layers (OneComp page: one-line API example) and a
Qwen3-32B down projection (OneComp page: verified model table), calibrated on
synthetic heavy-tailed activations in place of C4/WikiText (OneComp hub page,
code architecture: calibration loaders).  Weights and datasets of those models
are not used.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None

# Tensor ids that key independent streams.
T_W = 1
T_X = 2
T_X_MID = 3
T_OUTLIER = 101
T_OUTLIER_MID = 102
T_BITS = 201

NORMAL = 0
STUDENT_T4 = 1


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"{_LIB_PATH} is missing; build it first (python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(_LIB_PATH)
    u64, i64, i32, dbl, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int, ctypes.c_double, ctypes.c_void_p
    lib.synth_key.argtypes = [u64, u64]
    lib.synth_key.restype = u64
    lib.synth_hash.argtypes = [u64, i64, vp]
    lib.synth_hash.restype = None
    lib.synth_rows.argtypes = [u64, i32, dbl, vp, i64, i64, i64, vp, vp]
    lib.synth_rows.restype = None
    lib.synth_columns.argtypes = [u64, i32, dbl, vp, i64, i64, vp, i64, vp, vp]
    lib.synth_columns.restype = None
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def key(seed: int, tensor: int) -> int:
    return int(_load().synth_key(seed & (2**64 - 1), tensor))


def hashes(seed: int, tensor: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.uint64)
    _load().synth_hash(key(seed, tensor), n, _ptr(out))
    return out


def outlier_scale(seed: int, tensor: int, n: int, count: int, factor: float) -> np.ndarray:
    """Per-channel multipliers: the `count` channels with the smallest hash get `factor`."""
    s = np.ones(n, dtype=np.float64)
    if count > 0:
        idx = np.argsort(hashes(seed, tensor, n), kind="stable")[:count]
        s[idx] = factor
    return s


def rows(seed, tensor, dist, sigma, cols, r0, nrows, colscale=None, bf16=False):
    """Rows [r0, r0+nrows) of a [*, cols] tensor, as float32 or as bf16 bit patterns (uint16)."""
    lib = _load()
    cs = None if colscale is None else np.ascontiguousarray(colscale, dtype=np.float64)
    if bf16:
        out = np.empty((nrows, cols), dtype=np.uint16)
        lib.synth_rows(key(seed, tensor), dist, sigma, _ptr(cs), r0, nrows, cols, None, _ptr(out))
    else:
        out = np.empty((nrows, cols), dtype=np.float32)
        lib.synth_rows(key(seed, tensor), dist, sigma, _ptr(cs), r0, nrows, cols, _ptr(out), None)
    return out


def columns(seed, tensor, dist, sigma, cols, nrows, sel, colscale=None, bf16=False):
    """Columns `sel` of rows [0, nrows) of a [*, cols] tensor, shape [nrows, len(sel)]."""
    lib = _load()
    sel = np.ascontiguousarray(sel, dtype=np.int64)
    cs = None if colscale is None else np.ascontiguousarray(colscale, dtype=np.float64)
    if bf16:
        out = np.empty((nrows, len(sel)), dtype=np.uint16)
        lib.synth_columns(key(seed, tensor), dist, sigma, _ptr(cs), nrows, cols, _ptr(sel), len(sel), None, _ptr(out))
    else:
        out = np.empty((nrows, len(sel)), dtype=np.float32)
        lib.synth_columns(key(seed, tensor), dist, sigma, _ptr(cs), nrows, cols, _ptr(sel), len(sel), _ptr(out), None)
    return out


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


@dataclass
class Activations:
    """Calibration activations X [tokens, n] of one Hessian."""

    seed: int
    tensor: int
    n: int
    tokens: int
    dist: int
    outliers: int
    outlier_factor: float
    bf16: bool
    chunk: int = 8192
    _scale: np.ndarray | None = field(default=None, repr=False)

    def colscale(self):
        if self._scale is None:
            self._scale = outlier_scale(self.seed, self.tensor + 100, self.n, self.outliers, self.outlier_factor)
        return self._scale

    def block(self, t0, nt):
        return rows(self.seed, self.tensor, self.dist, 1.0, self.n, t0, nt, self.colscale(), self.bf16)

    def chunks(self):
        for t0 in range(0, self.tokens, self.chunk):
            yield self.block(t0, min(self.chunk, self.tokens - t0))

    def full(self):
        return self.block(0, self.tokens)

    def cols(self, sel, ntok=None):
        return columns(self.seed, self.tensor, self.dist, 1.0, self.n, self.tokens if ntok is None else ntok,
                       sel, self.colscale(), self.bf16)


@dataclass
class Linear:
    """One linear layer W [rows, cols] and the Hessian it is quantized against."""

    name: str
    rows: int
    cols: int
    sigma: float
    bits: int
    seed: int
    wtensor: int
    hessian: str
    bf16: bool = True

    def weight(self):
        return rows(self.seed, self.wtensor, NORMAL, self.sigma, self.cols, 0, self.rows, None, self.bf16)


@dataclass
class Workload:
    name: str
    description: str
    hessians: dict
    linears: list
    groupsize: int = 128
    blocksize: int = 128
    damp: float = 0.01


def _acts(seed, tensor, n, tokens, outliers, factor, dist=STUDENT_T4, bf16=True):
    return Activations(seed=seed, tensor=tensor, n=n, tokens=tokens, dist=dist, outliers=outliers,
                       outlier_factor=factor, bf16=bf16)


def stack_bits(seed: int, blocks: int = 32):
    """Per-layer bit widths {2,3,4}[hash mod 3] for a stack of blocks x 7 linears (q,k,v,o,gate,up,down)."""
    h = hashes(seed, T_BITS, 7 * blocks)
    return [(2, 3, 4)[int(x % np.uint64(3))] for x in h]


def workload(name: str, seed: int = 0, tokens: int | None = None, blocks: int = 32) -> Workload:
    """Named workloads.  `tokens` overrides the calibration token count (reduced-token variants)."""
    if name == "linear256":
        t = 512 if tokens is None else tokens
        return Workload(name, "single 256x256 linear, fp32 W ~N(0,0.02^2), fp32 X 512x256 ~N(0,1), 4 outlier channels x10, 4-bit g128",
                        {"x": _acts(seed, T_X, 256, t, 4, 10.0, dist=NORMAL, bf16=False)},
                        [Linear("linear", 256, 256, 0.02, 4, seed, T_W, "x", bf16=False)])
    if name == "q_proj_4096":
        t = 262144 if tokens is None else tokens
        return Workload(name, "Llama-2-7B q_proj 4096x4096 bf16 ~N(0,0.02^2), X 262144x4096 bf16 t4 with 41 outlier channels x20, 4-bit g128",
                        {"x": _acts(seed, T_X, 4096, t, 41, 20.0)},
                        [Linear("q_proj", 4096, 4096, 0.02, 4, seed, T_W, "x")])
    if name == "mlp_7b":
        t = 131072 if tokens is None else tokens
        return Workload(name, "Llama-2-7B MLP at 3-bit g128: gate/up 11008x4096 sharing a 4096^2 Hessian, down 4096x11008 with an 11008^2 Hessian, 131072 tokens",
                        {"x": _acts(seed, T_X, 4096, t, 41, 20.0), "mid": _acts(seed, T_X_MID, 11008, t, 110, 20.0)},
                        [Linear("gate_proj", 11008, 4096, 0.02, 3, seed, 10, "x"),
                         Linear("up_proj", 11008, 4096, 0.02, 3, seed, 11, "x"),
                         Linear("down_proj", 4096, 11008, 0.02, 3, seed, 12, "mid")])
    if name == "down_proj_32b":
        t = 131072 if tokens is None else tokens
        return Workload(name, "Qwen3-32B down_proj 5120x25600 bf16 ~N(0,0.015^2), X 131072x25600 bf16 t4 with 128 outlier channels x30, 4-bit g128",
                        {"x": _acts(seed, T_X, 25600, t, 128, 30.0)},
                        [Linear("down_proj", 5120, 25600, 0.015, 4, seed, T_W, "x")])
    if name == "stack_7b":
        t = 65536 if tokens is None else tokens
        bits = stack_bits(seed, blocks)
        hess, lins = {}, []
        for b in range(blocks):
            base = 1000 + 16 * b
            hess[f"b{b}.qkv"] = _acts(seed, base + 0, 4096, t, 41, 20.0)
            hess[f"b{b}.o"] = _acts(seed, base + 1, 4096, t, 41, 20.0)
            hess[f"b{b}.gateup"] = _acts(seed, base + 2, 4096, t, 41, 20.0)
            hess[f"b{b}.down"] = _acts(seed, base + 3, 11008, t, 110, 20.0)
            shapes = [("q_proj", 4096, 4096, "qkv"), ("k_proj", 4096, 4096, "qkv"), ("v_proj", 4096, 4096, "qkv"),
                      ("o_proj", 4096, 4096, "o"), ("gate_proj", 11008, 4096, "gateup"),
                      ("up_proj", 11008, 4096, "gateup"), ("down_proj", 4096, 11008, "down")]
            for i, (nm, r, c, h) in enumerate(shapes):
                lins.append(Linear(f"b{b}.{nm}", r, c, 0.02, bits[7 * b + i], seed, base + 4 + i, f"b{b}.{h}"))
        return Workload(name, f"Llama-2-7B-shaped stack, {blocks} blocks x 7 linears, bits from {{2,3,4}} by seed, g128, {t} tokens per Hessian",
                        hess, lins)
    raise KeyError(name)
