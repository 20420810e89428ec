"""Python side of the CPU oracle -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this module; the GPU library never does.  It loads
``oracle/libkq_oracle.so`` (plain C, fp64; built from ``kq_oracle.c`` with
gcc and no fast-math) and marshals numpy arrays.

Functions:
  dequant(qtype, rows, cols, gguf)      exact fp64 weights  w = d*sc*q - dmin*m  (Q4_K/Q5_K)
                                        or w = d*sc*(q-32) (Q6_K), [rows, cols]
  dequant_f32(...)                      the same rounded once to fp32 (RNE)
  gemv(qtype, rows, cols, gguf, x)      y = W x^T and a = sum |w x| in fp64, [batch, rows]
  silu(g), swiglu(g, u)                 the SwiGLU feed-forward's activation in fp64
  sigmoid(v)                            the attention output gate, fp64
  rmsnorm(x, eps)                       the weight-less RMSNorm, fp64
  head_rmsnorm(v, eps, head_rows)       the same per head of consecutive outputs (Q/K norm), fp64
  gemv_rmsnorm(...)                     W (rmsnorm(x)) from the fp64 dequantised W, fp64
  gather(qtype, rows, cols, gguf, ids)  rows ids of dequant_f32 (the embedding lookup)
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kq_oracle.c")
_LIB = os.path.join(_HERE, "libkq_oracle.so")
TYPE_ID = {"q4k": 1, "q5k": 2, "q6k": 3}
SB_BYTES = {"q4k": 144, "q5k": 176, "q6k": 210}
_default = None


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc (-O2, OpenMP, no FMA contraction, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        compile_c(_SRC, _LIB)
    return _LIB


def compile_c(src: str, out: str) -> None:
    tmp = out + f".tmp{os.getpid()}"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                           "-shared", "-fPIC", "-o", tmp, src, "-lm"])
    os.replace(tmp, out)


class Oracle:
    """One loaded copy of the C oracle (the tests also load deliberately broken copies)."""

    def __init__(self, path: str):
        L = ctypes.CDLL(path)
        L.kqo_f16_to_double.argtypes = [ctypes.c_uint16]
        L.kqo_f16_to_double.restype = ctypes.c_double
        L.kqo_bf16_to_double.argtypes = [ctypes.c_uint16]
        L.kqo_bf16_to_double.restype = ctypes.c_double
        L.kqo_dequant.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
        L.kqo_dequant.restype = ctypes.c_int
        L.kqo_gemv.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
                               ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        L.kqo_gemv.restype = ctypes.c_int
        self.L = L

    def f16_to_double(self, bits: int) -> float:
        return self.L.kqo_f16_to_double(int(bits) & 0xFFFF)

    def bf16_to_double(self, bits: int) -> float:
        return self.L.kqo_bf16_to_double(int(bits) & 0xFFFF)

    def dequant(self, qtype: str, rows: int, cols: int, gguf) -> np.ndarray:
        g = _bytes(gguf, qtype, rows, cols)
        w = np.empty((rows, cols), dtype=np.float64)
        rc = self.L.kqo_dequant(TYPE_ID[qtype], rows, cols, g.ctypes.data, w.ctypes.data)
        if rc:
            raise ValueError(f"oracle dequant failed (code {rc})")
        return w

    def dequant_f32(self, qtype: str, rows: int, cols: int, gguf) -> np.ndarray:
        return self.dequant(qtype, rows, cols, gguf).astype(np.float32)

    def gemv(self, qtype: str, rows: int, cols: int, gguf, x) -> tuple[np.ndarray, np.ndarray]:
        """x: float32 [batch, cols] or uint16 bf16 bit patterns [batch, cols] -> (y, a), each [batch, rows]."""
        g = _bytes(gguf, qtype, rows, cols)
        x = np.ascontiguousarray(x)
        if x.ndim != 2 or x.shape[1] != cols:
            raise ValueError("x must be [batch, cols]")
        if x.dtype == np.float32:
            xt = 0
        elif x.dtype == np.uint16:
            xt = 1
        else:
            raise TypeError("x must be float32 or uint16 (bf16 bits)")
        batch = x.shape[0]
        y = np.empty((batch, rows), dtype=np.float64)
        a = np.empty((batch, rows), dtype=np.float64)
        rc = self.L.kqo_gemv(TYPE_ID[qtype], rows, cols, g.ctypes.data, xt, x.ctypes.data, cols, batch,
                             y.ctypes.data, a.ctypes.data)
        if rc:
            raise ValueError(f"oracle gemv failed (code {rc})")
        return y, a


def _bytes(gguf, qtype, rows, cols) -> np.ndarray:
    g = np.ascontiguousarray(np.asarray(gguf, dtype=np.uint8)).reshape(-1)
    need = rows * (cols // 256) * SB_BYTES[qtype]
    if g.size != need:
        raise ValueError(f"expected {need} bytes, got {g.size}")
    return g


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle(build())
    return _default


def f16_to_double(bits):
    return default().f16_to_double(bits)


def bf16_to_double(bits):
    return default().bf16_to_double(bits)


def dequant(qtype, rows, cols, gguf):
    return default().dequant(qtype, rows, cols, gguf)


def dequant_f32(qtype, rows, cols, gguf):
    return default().dequant_f32(qtype, rows, cols, gguf)


def gemv(qtype, rows, cols, gguf, x):
    return default().gemv(qtype, rows, cols, gguf, x)


def silu(g):
    """silu(g) = g * sigmoid(g) = g / (1 + exp(-g)), in fp64: the gate activation of the SwiGLU
    feed-forward named on the "Muse-Glimmer-30B (text decoder) - Apple Core AI" card (section "The
    architecture, and what the port had to do about it"); the pages name it without a formula, and this
    is the standard one.  exp(-g) overflows to inf for g < -709, which gives -0 as the limit."""
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def sigmoid(v):
    """sigmoid(v) = 1 / (1 + exp(-v)) in fp64: the attention output gate of the same card and section
    (a sigmoid gate read from the hidden state that Q/K/V read)."""
    v = np.asarray(v, dtype=np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-v))


def rmsnorm(x, eps):
    """The weight-less RMSNorm of each row of x in fp64: x / sqrt(mean(x^2) + eps), no gain ("Muse-Glimmer-30B
    (text decoder) - Apple Core AI", section "The architecture, and what the port had to do about it": applied to
    the embedding output and to Q/K).  x: float rows [batch, K]."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def head_rmsnorm(v, eps, head_rows=128):
    """The weight-less RMSNorm of each head of `head_rows` consecutive outputs, per batch row, in fp64: the card's
    norm on Q/K, whose heads are 128 wide (head_dim).  v: [batch, rows] with rows a multiple of head_rows."""
    v = np.asarray(v, dtype=np.float64)
    b, r = v.shape
    if r % head_rows:
        raise ValueError("rows must be a multiple of head_rows")
    h = v.reshape(b, r // head_rows, head_rows)
    return (h / np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + eps)).reshape(b, r)


def gemv_rmsnorm(qtype, rows, cols, gguf, x, eps):
    """(y, a) = (W xn, |W| |xn|) per batch row, xn = rmsnorm(x, eps), W the fp64 dequantised matrix.
    x: float32 [batch, cols] or uint16 bf16 bit patterns."""
    x = np.ascontiguousarray(x)
    # a bf16 value is the upper half of the fp32 with the same bits
    xd = ((x.astype(np.uint32) << 16).view(np.float32) if x.dtype == np.uint16 else x).astype(np.float64)
    xn = rmsnorm(xd, eps)
    W = dequant(qtype, rows, cols, gguf)
    return xn @ W.T, np.abs(xn) @ np.abs(W).T


def swiglu(g, u):
    """The SwiGLU hidden activation silu(g) * u for gate output g and up output u, in fp64."""
    return silu(g) * np.asarray(u, dtype=np.float64)


def gather(qtype, rows, cols, gguf, ids):
    """The embedding lookup: rows `ids` of the fp32 dequantised matrix."""
    return dequant_f32(qtype, rows, cols, gguf)[np.asarray(ids)]
