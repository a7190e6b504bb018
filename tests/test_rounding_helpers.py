"""Pins of the test-side rounding helper that turns the oracle's exact fp64
dequantized weights into bf16 bits: crafted values with known bf16 images."""
import numpy as np

from tests.parity import bf16_bits_rne_from_f64


def test_exact_bf16_values_are_unchanged():
    bits = np.array([0x3F80, 0xBF80, 0x4040, 0x0080, 0x7F7F, 0x3C01, 0xC2F7], dtype=np.uint32)
    vals = (bits << 16).view(np.float32).astype(np.float64)
    np.testing.assert_array_equal(bf16_bits_rne_from_f64(vals), bits.astype(np.uint16))


def test_ties_go_to_even_and_off_ties_go_to_nearest():
    # 1 + 2^-8 is halfway between 1 (even mantissa) and 1 + 2^-7: ties to 1.
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 (odd) and 1 + 2^-6: ties up.
    # Anything beyond a midpoint, however little, goes to the far side.
    v = np.array([1 + 2.0**-8, 1 + 3 * 2.0**-8, 1 + 2.0**-8 + 2.0**-40,
                  1 + 2.0**-8 - 2.0**-40, -(1 + 2.0**-8 + 2.0**-40),
                  3.0078125 + 2.0**-30, 3.0078125 - 2.0**-30, 3.0078125])
    want = [0x3F80, 0x3F82, 0x3F81, 0x3F80, 0xBF81, 0x4041, 0x4040, 0x4040]
    np.testing.assert_array_equal(bf16_bits_rne_from_f64(v), np.array(want, dtype=np.uint16))


def test_carry_into_the_exponent_and_zero():
    v = np.array([2.0 - 2.0**-9, 2.0 - 2.0**-20, 0.0, -0.0])
    want = [0x4000, 0x4000, 0x0000, 0x8000]
    np.testing.assert_array_equal(bf16_bits_rne_from_f64(v), np.array(want, dtype=np.uint16))


def test_agrees_with_f32_rounding_where_no_double_rounding_can_occur():
    # values exactly representable in fp32: one rounding either way
    rng = np.random.default_rng(7)
    f = (rng.standard_normal(20000) * 3).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    ref = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    np.testing.assert_array_equal(bf16_bits_rne_from_f64(f.astype(np.float64)), ref)
