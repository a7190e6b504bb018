"""MI355X (gfx950) affine group-quantized matvec: Python binding of libqmv.so.

Argument marshalling only.  Every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/qmv.h``; torch supplies device
memory and the current stream.  If ``libqmv.so`` has not been built, importing
the functions raises ``ImportError``: there is no CPU fallback.

Names and defaults follow mlx's ``quantize`` / ``quantized_matmul`` /
``gather_qmm`` (transpose=True, group_size=64, bits=4) and the metrale
``QuantWeights`` fused methods.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "QmvError", "lib", "qmv_pack", "qmv", "qmv_gate_up", "qmv_silu_gate_resid",
    "gather_qmv", "qmv_dequantize", "qmv_unpack_codes", "qmv_workspace_bytes",
    "QMV_OK", "QMV_EINVAL",
    "QMV_EUNSUPPORTED", "QMV_EHIP", "QMV_OUT_BF16", "QMV_OUT_F32",
]

QMV_OK, QMV_EINVAL, QMV_EUNSUPPORTED, QMV_EHIP = 0, -1, -2, -3
QMV_OUT_BF16, QMV_OUT_F32 = 0, 1

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libqmv.so")

_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I = ctypes.c_int
SIGNATURES = {
    "qmv_pack": [_P, _I64, _I64, _I, _I, _P, _P, _P, _P],
    "qmv": [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I, _I, _I, _I, _P],
    "qmv_workspace_bytes": [_I64, _I64, _I64, _I, _I, _I, _P],
    "qmv_noalloc": [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I, _I, _I, _I, _P],
    "qmv_with_workspace": [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I, _I, _I, _I,
                           _P, ctypes.c_size_t, _P],
    "qmv_gate_up": [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I, _I, _P],
    "qmv_silu_gate_resid": [_P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I, _I, _I,
                            _P],
    "gather_qmv": [_P, _I64, _P, _P, _P, _I64, _P, _P, _I64, _P, _I64, _I64,
                   _I64, _I, _I, _I, _I, _I, _P],
    "qmv_dequantize": [_P, _P, _P, _P, _I64, _I64, _I, _I, _I, _P],
    "qmv_unpack_codes": [_P, _I64, _I64, _I, _P, _P],
}


class QmvError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


def lib() -> ctypes.CDLL:
    """The loaded C library (raises ImportError if it was never built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                "(or python bit_affine_quantized_amd/_build.py); there is no "
                "fallback implementation")
        L = ctypes.CDLL(LIB_PATH)
        for name, args in SIGNATURES.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = _I
        L.qmv_last_error.argtypes = []
        L.qmv_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _call(name: str, *args) -> None:
    L = lib()
    rc = getattr(L, name)(*args)
    if rc != QMV_OK:
        raise QmvError(rc, L.qmv_last_error().decode())


# ----------------------------------------------------------------- helpers
def _torch():
    import torch
    return torch


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, dtype, name):
    torch = _torch()
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _bits16(t, name):
    """bf16 tensors travel as their uint16 bit patterns (a view, no copy)."""
    torch = _torch()
    _need(t, torch.bfloat16, name)
    return t


def _out_code(out_dtype):
    torch = _torch()
    if out_dtype in (None, torch.bfloat16):
        return QMV_OUT_BF16, torch.bfloat16
    if out_dtype == torch.float32:
        return QMV_OUT_F32, torch.float32
    raise ValueError("out_dtype must be torch.bfloat16 or torch.float32")


# ----------------------------------------------------------------- API
def qmv_pack(w, group_size: int = 64, bits: int = 4, stream=None, out=None):
    """Quantize fp32 W [N, K] on the device -> (w_q uint32-as-int32 [N,
    K*bits/32], scales bf16 [N, K/g], biases bf16 [N, K/g]).  ``out`` may
    give the three output tensors."""
    torch = _torch()
    _need(w, torch.float32, "w")
    if w.dim() != 2:
        raise ValueError("w must be 2-D [N, K]")
    N, K = w.shape
    words = (K * bits) // 32 if bits > 0 else 0
    groups = K // group_size if group_size > 0 else 0
    if out is None:
        w_q = torch.empty((N, max(words, 1)), dtype=torch.int32, device=w.device)
        s = torch.empty((N, max(groups, 1)), dtype=torch.bfloat16, device=w.device)
        b = torch.empty_like(s)
    else:
        w_q, s, b = out
        _wq(w_q)
        _bits16(s, "scales")
        _bits16(b, "biases")
        if w_q.numel() < N * words or s.numel() < N * groups or b.numel() < N * groups:
            raise ValueError("qmv_pack: output tensors too small")
    _call("qmv_pack", _ptr(w), N, K, group_size, bits, _ptr(w_q), _ptr(s),
          _ptr(b), _stream(stream))
    return w_q, s, b


def _wq(t, name="w_q"):
    torch = _torch()
    if t.dtype not in (torch.int32, torch.uint32):
        raise ValueError(f"{name} must hold uint32 words (int32/uint32 dtype)")
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")
    return t


def qmv_workspace_bytes(M: int, N: int, K: int, group_size: int = 64,
                        bits: int = 4, transpose: bool = True) -> int:
    """Bytes of split-K workspace a qmv call of these sizes needs (0: none)."""
    out = ctypes.c_size_t(0)
    _call("qmv_workspace_bytes", M, N, K, group_size, bits,
          1 if transpose else 0, ctypes.byref(out))
    return int(out.value)


def qmv(x, w_q, scales, biases, transpose: bool = True, group_size: int = 64,
        bits: int = 4, out_dtype=None, y=None, stream=None, workspace=None):
    """y = x @ W_hat^T for x bf16 [..., M, K] (batch dims flattened into M).

    ``workspace``: an optional device tensor of at least
    ``qmv_workspace_bytes(...)`` bytes for the split-K paths; without it the
    library takes a stream-ordered allocation for the call."""
    torch = _torch()
    _bits16(x, "x")
    _wq(w_q)
    _bits16(scales, "scales")
    _bits16(biases, "biases")
    K = x.shape[-1]
    M = x.numel() // K if K else 0
    N = w_q.shape[0] if transpose else w_q.shape[-1] * 32 // bits
    code, dt = _out_code(out_dtype)
    if y is None:
        y = torch.empty((*x.shape[:-1], N), dtype=dt, device=x.device)
    args = (_ptr(x), _ptr(w_q), _ptr(scales), _ptr(biases), _ptr(y), M, N, K,
            group_size, bits, 1 if transpose else 0, code)
    if workspace is None:
        _call("qmv", *args, _stream(stream))
    else:
        if not workspace.is_cuda or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous device tensor")
        _call("qmv_with_workspace", *args, _ptr(workspace),
              workspace.numel() * workspace.element_size(), _stream(stream))
    return y


def qmv_gate_up(x, gate_w, up_w, group_size: int = 64, bits: int = 4,
                gate_y=None, up_y=None, stream=None):
    """(gate_y, up_y) = (W_gate x, W_up x) in one launch; *_w = (w_q, s, b)."""
    torch = _torch()
    _bits16(x, "x")
    wg, sg, bg = gate_w
    wu, su, bu = up_w
    _wq(wg, "gate w_q")
    _wq(wu, "up w_q")
    for t, n in ((sg, "gate scales"), (bg, "gate biases"), (su, "up scales"),
                 (bu, "up biases")):
        _bits16(t, n)
    if wg.shape != wu.shape or sg.shape != su.shape:
        raise ValueError("gate and up weights must have the same shape")
    N, K = wg.shape[0], x.shape[-1]
    if gate_y is None:
        gate_y = torch.empty((N,), dtype=torch.bfloat16, device=x.device)
    if up_y is None:
        up_y = torch.empty((N,), dtype=torch.bfloat16, device=x.device)
    _call("qmv_gate_up", _ptr(x), _ptr(wg), _ptr(sg), _ptr(bg), _ptr(wu),
          _ptr(su), _ptr(bu), _ptr(gate_y), _ptr(up_y), N, K, group_size,
          bits, _stream(stream))
    return gate_y, up_y


def qmv_silu_gate_resid(gate, up, x_resid, w_q, scales, biases,
                        group_size: int = 64, bits: int = 4, out_dtype=None,
                        y=None, stream=None):
    """y = x_resid + W_hat @ (silu(gate) * up); x_resid may be None."""
    torch = _torch()
    _bits16(gate, "gate")
    _bits16(up, "up")
    if x_resid is not None:
        _bits16(x_resid, "x_resid")
    _wq(w_q)
    _bits16(scales, "scales")
    _bits16(biases, "biases")
    if gate.numel() != up.numel():
        raise ValueError("gate and up must have the same length")
    N, K = w_q.shape[0], gate.numel()
    code, dt = _out_code(out_dtype)
    if y is None:
        y = torch.empty((N,), dtype=dt, device=gate.device)
    _call("qmv_silu_gate_resid", _ptr(gate), _ptr(up), _ptr(x_resid),
          _ptr(w_q), _ptr(scales), _ptr(biases), _ptr(y), N, K, group_size,
          bits, code, _stream(stream))
    return y


def gather_qmv(x, w_q, scales, biases, lhs_indices=None, rhs_indices=None,
               transpose: bool = True, group_size: int = 64, bits: int = 4,
               sorted_indices: bool = False, out_dtype=None, y=None,
               stream=None):
    """y[p] = x[lhs[p]] @ W_hat[rhs[p]]^T.  x: [Bx, M, K]; w_q: [E, N, K*b/32].
    Index arrays are flattened (they must already be broadcast together)."""
    torch = _torch()
    _bits16(x, "x")
    _wq(w_q)
    _bits16(scales, "scales")
    _bits16(biases, "biases")
    code, dt = _out_code(out_dtype)
    K = x.shape[-1]
    M = x.shape[-2] if x.dim() >= 2 else 1
    Bx = x.numel() // (M * K)
    if w_q.dim() == 2:
        E, N = 1, w_q.shape[0]
    else:
        E, N = w_q.shape[0], w_q.shape[1]
    if (lhs_indices is None) != (rhs_indices is None):
        raise ValueError("give both lhs_indices and rhs_indices, or neither")
    if lhs_indices is None:
        P = 1
        shape = (M, N)
    else:
        for t, n in ((lhs_indices, "lhs_indices"), (rhs_indices, "rhs_indices")):
            if t.dtype not in (torch.int32, torch.uint32) or not t.is_cuda \
                    or not t.is_contiguous():
                raise ValueError(f"{n} must be a contiguous device int32/uint32 tensor")
        if lhs_indices.shape != rhs_indices.shape:
            raise ValueError("lhs_indices and rhs_indices must have one shape")
        P = lhs_indices.numel()
        shape = (*lhs_indices.shape, M, N)
    if y is None:
        y = torch.empty(shape, dtype=dt, device=x.device)
    _call("gather_qmv", _ptr(x), Bx, _ptr(w_q), _ptr(scales), _ptr(biases), E,
          _ptr(lhs_indices), _ptr(rhs_indices), P, _ptr(y), M, N, K,
          group_size, bits, 1 if transpose else 0, 1 if sorted_indices else 0,
          code, _stream(stream))
    return y


def qmv_dequantize(w_q, scales, biases, group_size: int = 64, bits: int = 4,
                   out_dtype=None, out=None, stream=None):
    """W_hat [N, K] = scales * q + biases (bf16 or fp32), rounded once."""
    torch = _torch()
    _wq(w_q)
    _bits16(scales, "scales")
    _bits16(biases, "biases")
    N = w_q.shape[0]
    K = w_q.shape[-1] * 32 // bits
    code, dt = _out_code(out_dtype)
    if out is None:
        out = torch.empty((N, K), dtype=dt, device=w_q.device)
    _call("qmv_dequantize", _ptr(w_q), _ptr(scales), _ptr(biases), _ptr(out),
          N, K, group_size, bits, code, _stream(stream))
    return out


def qmv_unpack_codes(w_q, K: int, bits: int, stream=None):
    """Debug: the kernels' own unpacking -> codes uint8 [N, K]."""
    torch = _torch()
    _wq(w_q)
    N = w_q.shape[0]
    codes = torch.empty((N, K), dtype=torch.uint8, device=w_q.device)
    _call("qmv_unpack_codes", _ptr(w_q), N, K, bits, _ptr(codes),
          _stream(stream))
    return codes
