"""Plain CPU oracle for the affine group-quantized matvec (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library never does, and
this package imports nothing from it: the two share no code.

The arithmetic lives in ``qmv_oracle.c`` (plain C, fp32 quantizer steps as the
mlx-cpu 0.30.1 ``quantized.h`` ``affine_quantize`` kernel states them, fp64
everything after dequantization).  This module compiles it with gcc when the
shared object is missing and wraps each routine for numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qmv_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# The oracle mutation test points this at a deliberately broken copy, built
# from an edited source, to check that the pins catch the mistake.
_ALT_LIB = os.environ.get("QMV_ORACLE_LIB")

_lib = None


def compile_source(src: str, out: str) -> None:
    """gcc, no fast-math, no FMA contraction: one IEEE operation per step."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared",
           "-ffp-contract=off", "-fno-fast-math", "-fno-finite-math-only",
           "-o", tmp, src, "-lm"]
    subprocess.check_call(cmd)
    os.replace(tmp, out)


def build(force: bool = False) -> str:
    """Compile the oracle (the library the package loads)."""
    if _ALT_LIB:
        return _ALT_LIB
    if force or not os.path.exists(_LIB):
        compile_source(_SRC, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        I = ctypes.c_int
        sig = {
            "oracle_bf16_from_f32": (ctypes.c_uint16, [ctypes.c_float]),
            "oracle_f64_from_bf16": (ctypes.c_double, [ctypes.c_uint16]),
            "oracle_quantize": (I, [P, I64, I64, I, I, P, P, P, P, P]),
            "oracle_pack": (I, [P, I64, I64, I, P]),
            "oracle_unpack": (I, [P, I64, I64, I, P]),
            "oracle_dequantize": (I, [P, P, P, I64, I64, I, I, P]),
            "oracle_qmv_f64": (I, [P, P, P, P, I64, I64, I64, I, I, P]),
            "oracle_qmv_rows_f64": (I, [P, P, P, P, I64, I64, I64, I, I, P,
                                        I64, P]),
            "oracle_qvm_f64": (I, [P, P, P, P, I64, I64, I64, I, I, P]),
            "oracle_silu_gate_resid_f64": (I, [P, P, P, P, P, P, I64, I64, I,
                                               I, P]),
            "oracle_gather_qmv_f64": (I, [P, I64, P, P, P, I64, P, P, I64,
                                          I64, I64, I64, I, I, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def _check(rc, name):
    if rc != 0:
        raise ValueError(f"{name} failed with code {rc}")


# ---------------------------------------------------------------- scalars
def bf16_from_f32(v: float) -> int:
    return int(_load().oracle_bf16_from_f32(float(v)))


def f64_from_bf16(h: int) -> float:
    return float(_load().oracle_f64_from_bf16(int(h)))


def bf16_bits_to_f64(a) -> np.ndarray:
    """Vector bf16-bits -> float64 (exact widening; no arithmetic)."""
    a = np.asarray(a, dtype=np.uint16)
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ---------------------------------------------------------------- quantize
def quantize(w: np.ndarray, group_size: int, bits: int):
    """-> codes uint8 [N,K], s32, b32 float32 [N,K/g], s16, b16 uint16."""
    w = _c(w, np.float32)
    N, K = w.shape
    G = K // group_size
    codes = np.empty((N, K), np.uint8)
    s32 = np.empty((N, G), np.float32)
    b32 = np.empty((N, G), np.float32)
    s16 = np.empty((N, G), np.uint16)
    b16 = np.empty((N, G), np.uint16)
    _check(_load().oracle_quantize(_ptr(w), N, K, group_size, bits,
                                   _ptr(codes), _ptr(s32), _ptr(b32),
                                   _ptr(s16), _ptr(b16)), "oracle_quantize")
    return codes, s32, b32, s16, b16


def pack(codes: np.ndarray, bits: int) -> np.ndarray:
    codes = _c(codes, np.uint8)
    N, K = codes.shape
    out = np.empty((N, K * bits // 32), np.uint32)
    _check(_load().oracle_pack(_ptr(codes), N, K, bits, _ptr(out)),
           "oracle_pack")
    return out


def unpack(w: np.ndarray, K: int, bits: int) -> np.ndarray:
    w = _c(w, np.uint32)
    N = w.shape[0]
    out = np.empty((N, K), np.uint8)
    _check(_load().oracle_unpack(_ptr(w), N, K, bits, _ptr(out)),
           "oracle_unpack")
    return out


def quantize_pack(w: np.ndarray, group_size: int, bits: int):
    """The full offline step: -> (w_q uint32, scales bf16 bits, biases bf16)."""
    codes, _, _, s16, b16 = quantize(w, group_size, bits)
    return pack(codes, bits), s16, b16


def dequantize(w_q, scales, biases, K: int, group_size: int, bits: int):
    w_q = _c(w_q, np.uint32)
    scales = _c(scales, np.uint16)
    biases = _c(biases, np.uint16)
    N = w_q.shape[0]
    out = np.empty((N, K), np.float64)
    _check(_load().oracle_dequantize(_ptr(w_q), _ptr(scales), _ptr(biases),
                                     N, K, group_size, bits, _ptr(out)),
           "oracle_dequantize")
    return out


# ---------------------------------------------------------------- products
def qmv(x_bits, w_q, scales, biases, group_size: int, bits: int):
    """y [M,N] fp64 = x @ W_hat^T; x given as bf16 bits [M,K]."""
    x_bits = np.atleast_2d(_c(x_bits, np.uint16))
    w_q = _c(w_q, np.uint32)
    M, K = x_bits.shape
    N = w_q.shape[0]
    y = np.empty((M, N), np.float64)
    _check(_load().oracle_qmv_f64(_ptr(x_bits), _ptr(w_q),
                                  _ptr(_c(scales, np.uint16)),
                                  _ptr(_c(biases, np.uint16)), M, N, K,
                                  group_size, bits, _ptr(y)), "oracle_qmv_f64")
    return y


def qmv_rows(x_bits, w_q, scales, biases, group_size: int, bits: int, rows):
    """y [M, len(rows)] fp64: only the listed output rows of x @ W_hat^T."""
    x_bits = np.atleast_2d(_c(x_bits, np.uint16))
    w_q = _c(w_q, np.uint32)
    rows = _c(rows, np.int64)
    M, K = x_bits.shape
    N = w_q.shape[0]
    y = np.empty((M, rows.size), np.float64)
    _check(_load().oracle_qmv_rows_f64(_ptr(x_bits), _ptr(w_q),
                                       _ptr(_c(scales, np.uint16)),
                                       _ptr(_c(biases, np.uint16)), M, N, K,
                                       group_size, bits, _ptr(rows),
                                       rows.size, _ptr(y)),
           "oracle_qmv_rows_f64")
    return y


def qvm(x_bits, w_q, scales, biases, N: int, group_size: int, bits: int):
    """y [M,N] fp64 = x @ W_hat with W [K,N] quantized along N."""
    x_bits = np.atleast_2d(_c(x_bits, np.uint16))
    w_q = _c(w_q, np.uint32)
    M, K = x_bits.shape
    y = np.empty((M, N), np.float64)
    _check(_load().oracle_qvm_f64(_ptr(x_bits), _ptr(w_q),
                                  _ptr(_c(scales, np.uint16)),
                                  _ptr(_c(biases, np.uint16)), M, N, K,
                                  group_size, bits, _ptr(y)), "oracle_qvm_f64")
    return y


def silu_gate_resid(gate_bits, up_bits, x_resid_bits, w_q, scales, biases,
                    group_size: int, bits: int):
    """y [N] fp64 = x_resid + W_hat @ (silu(gate) * up); x_resid may be None."""
    gate_bits = _c(gate_bits, np.uint16).ravel()
    up_bits = _c(up_bits, np.uint16).ravel()
    xr = None if x_resid_bits is None else _c(x_resid_bits, np.uint16).ravel()
    w_q = _c(w_q, np.uint32)
    N = w_q.shape[0]
    K = gate_bits.size
    y = np.empty((N,), np.float64)
    _check(_load().oracle_silu_gate_resid_f64(
        _ptr(gate_bits), _ptr(up_bits), _ptr(xr), _ptr(w_q),
        _ptr(_c(scales, np.uint16)), _ptr(_c(biases, np.uint16)), N, K,
        group_size, bits, _ptr(y)), "oracle_silu_gate_resid_f64")
    return y


def gather_qmv(x_bits, w_q, scales, biases, lhs, rhs, group_size: int,
               bits: int):
    """x [Bx,M,K] bf16 bits; w_q [E,N,K*bits/32]; -> y [P,M,N] fp64."""
    x_bits = _c(x_bits, np.uint16)
    if x_bits.ndim == 2:
        x_bits = x_bits[:, None, :]
    w_q = _c(w_q, np.uint32)
    lhs = _c(lhs, np.uint32).ravel()
    rhs = _c(rhs, np.uint32).ravel()
    Bx, M, K = x_bits.shape
    E, N = w_q.shape[0], w_q.shape[1]
    P = lhs.size
    y = np.empty((P, M, N), np.float64)
    _check(_load().oracle_gather_qmv_f64(
        _ptr(x_bits), Bx, _ptr(w_q), _ptr(_c(scales, np.uint16)),
        _ptr(_c(biases, np.uint16)), E, _ptr(lhs), _ptr(rhs), P, M, N, K,
        group_size, bits, _ptr(y)), "oracle_gather_qmv_f64")
    return y
