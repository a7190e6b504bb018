"""Conversions and tolerance rules shared by the GPU parity tests.

Tolerances (the oracle is fp64):
  T1, bf16 outputs: |y - y_ref| <= 1e-2 * RMS(y_ref) + ulp_bf16(y_ref)/2 for
      every element.  The 1e-2 * RMS budget covers the kernel's arithmetic;
      the half ulp is the single rounding to bf16 that even a perfectly
      computed output takes (|y| in [4, 8) has a half ulp of 2^-6 > 1e-2*RMS
      at these shapes, so the bare budget would reject exact answers).
  T2, fp32 outputs: max |y - y_ref| <= 1e-5 * RMS(y_ref).
  With RMS(y_ref) = 0 (every reference output is exactly zero) both rules
  reduce to exact equality, which is checked directly.
"""
import numpy as np


def to_dev_bf16(bits_u16, dev):
    import torch
    a = np.ascontiguousarray(bits_u16, dtype=np.uint16)
    return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)


def to_dev_u32(words, dev):
    import torch
    a = np.ascontiguousarray(words, dtype=np.uint32)
    return torch.from_numpy(a.view(np.int32)).to(dev)


def bf16_to_np_bits(t):
    import torch
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def u32_to_np(t):
    return t.detach().cpu().contiguous().numpy().view(np.uint32)


def bf16_bits_to_f64(bits):
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def half_ulp_bf16(ref):
    a = np.abs(np.asarray(ref, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return np.exp2(e - 8)


def rms(ref):
    return float(np.sqrt(np.mean(np.square(np.asarray(ref, np.float64)))))


def check_t1(y_bits, ref, what=""):
    got = bf16_bits_to_f64(y_bits)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    err = np.abs(got - ref)
    if rms(ref) == 0.0:
        assert np.all(got == 0.0), f"{what}: reference is all zero, got max |y| {err.max():.3e}"
        return 0.0, 0.0
    tol = 1e-2 * rms(ref) + half_ulp_bf16(ref)
    bad = np.argwhere(err > tol)
    assert bad.size == 0, (f"{what}: {bad.shape[0]} elements out of T1, first "
                           f"{bad[:4].tolist()}, max err {err.max():.3e}, "
                           f"rms {rms(ref):.3e}")
    return float(err.max()), float(np.max(err / (1e-2 * rms(ref))))


def check_t2(y_f32, ref, what=""):
    got = np.asarray(y_f32, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    err = np.abs(got - ref)
    if rms(ref) == 0.0:
        assert np.all(got == 0.0), f"{what}: reference is all zero, got max |y| {err.max():.3e}"
        return 0.0, 0.0
    tol = 1e-5 * rms(ref)
    assert err.max() <= tol, (f"{what}: max err {err.max():.3e} > T2 "
                              f"{tol:.3e} at {np.unravel_index(err.argmax(), err.shape)}")
    return float(err.max()), float(err.max() / tol)


def bf16_bits_rne_from_f64(v):
    """Round float64 values once to bf16 bits (nearest, ties to even), from
    the binary64 fields.  Normal bf16 range and zero only (a value outside
    raises): what exact dequantized weights need."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    u = v.view(np.uint64)
    sign = (u >> np.uint64(63)).astype(np.uint32)
    exp = ((u >> np.uint64(52)) & np.uint64(0x7FF)).astype(np.int64)
    m53 = (u & np.uint64((1 << 52) - 1)) | np.uint64(1 << 52)
    zero = (u & np.uint64((1 << 63) - 1)) == 0
    e = exp - 1023
    if np.any(~zero & ((e < -126) | (e > 127))):
        raise ValueError("value outside the normal bf16 range")
    keep = (m53 >> np.uint64(45)).astype(np.int64)           # 8 bits with the leading one
    rem = m53 & np.uint64((1 << 45) - 1)
    half = np.uint64(1 << 44)
    up = (rem > half) | ((rem == half) & ((keep & 1) == 1))
    keep = keep + up.astype(np.int64)
    carry = keep == 256
    keep = np.where(carry, 128, keep)
    e = e + carry.astype(np.int64)
    out = (sign << 15) | (((e + 127) & 0xFF).astype(np.uint32) << 7) | (keep & 0x7F).astype(np.uint32)
    out = np.where(zero, sign << 15, out)
    return out.astype(np.uint16)
