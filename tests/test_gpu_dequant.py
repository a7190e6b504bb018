"""GPU parity of qmv_dequantize: every output is the exact s*q + z rounded
once, so it must equal the oracle's exact (fp64) dequantized weight rounded
the same way, bit for bit (fp32: numpy's IEEE rounding; bf16:
tests.parity.bf16_bits_rne_from_f64)."""
import numpy as np
import pytest

import oracle
import synth
from tests.parity import (bf16_bits_rne_from_f64, bf16_to_np_bits, to_dev_bf16,
                          to_dev_u32)

pytestmark = pytest.mark.gpu

BITS = (2, 3, 4, 5, 6, 8)
GROUPS = (32, 64, 128)


def _dev_dequant(w_q, s16, b16, g, bits, dev, f32):
    import torch

    import bit_affine_quantized_amd as q
    out = q.qmv_dequantize(to_dev_u32(w_q, dev), to_dev_bf16(s16, dev),
                           to_dev_bf16(b16, dev), g, bits,
                           out_dtype=torch.float32 if f32 else None)
    if f32:
        return out.cpu().numpy()
    return bf16_to_np_bits(out)


def _check(w_q, s16, b16, K, g, bits, dev, what):
    exact = oracle.dequantize(w_q, s16, b16, K, g, bits)
    got16 = _dev_dequant(w_q, s16, b16, g, bits, dev, False)
    np.testing.assert_array_equal(got16, bf16_bits_rne_from_f64(exact), err_msg=what + " bf16")
    got32 = _dev_dequant(w_q, s16, b16, g, bits, dev, True)
    np.testing.assert_array_equal(got32.view(np.uint32), exact.astype(np.float32).view(np.uint32),
                                  err_msg=what + " f32")


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("g", GROUPS)
def test_dequantize_bit_exact(dev, bits, g):
    N, K = 37, 640 if g != 128 else 768          # ragged N, several chunks
    w = synth.weight((N, K), synth.SEED_W)
    w_q, s16, b16 = oracle.quantize_pack(w, g, bits)
    _check(w_q, s16, b16, K, g, bits, dev, f"b{bits} g{g}")


def test_dequantize_full_headline_shape(dev):
    w = synth.weight((14336, 4096), synth.SEED_W)
    w_q, s16, b16 = oracle.quantize_pack(w, 64, 4)
    _check(w_q, s16, b16, 4096, 64, 4, dev, "14336x4096 b4 g64")


@pytest.mark.parametrize("bits", (3, 4, 5, 6, 8))
def test_dequantize_midpoint_decided_by_the_rounding_error(dev, bits):
    """s*q lands exactly halfway between two bf16 values and a tiny z pushes
    the exact sum off the midpoint; the fp32 sum alone would round to even.
    s = 0.6015625 (bf16), q = 5: s*q = 3.0078125, halfway between 3.0 and
    3.015625.  z = +-2^-30 (bf16) is below half an fp32 ulp at 3."""
    g, K = 32, 128
    codes = np.full((4, K), 5, dtype=np.uint8)
    w_q = oracle.pack(codes, bits)
    s_val = [0.6015625, 0.6015625, -0.6015625, 0.6015625]
    z_val = [2.0 ** -30, -(2.0 ** -30), -(2.0 ** -30), 0.0]
    s16 = np.array([[oracle.bf16_from_f32(v)] * (K // g) for v in s_val], dtype=np.uint16)
    b16 = np.array([[oracle.bf16_from_f32(v)] * (K // g) for v in z_val], dtype=np.uint16)
    _check(w_q, s16, b16, K, g, bits, dev, f"midpoint b{bits}")
    got = _dev_dequant(w_q, s16, b16, g, bits, dev, False)
    # rows: above the midpoint -> 3.015625; below -> 3.0; negative mirror;
    # exactly on it -> ties to even (3.0)
    np.testing.assert_array_equal(got[:, 0], np.array([0x4041, 0x4040, 0xC041, 0x4040], dtype=np.uint16))
