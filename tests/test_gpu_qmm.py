"""GPU parity of the matrix-core paths that qmv (transpose = 1) takes for 5 or
more rows of x, against the oracle's exact fp64 product: T1 for bf16 outputs,
T2 for the fp32 debugging mode.  Covers every bit width and group size,
partial 64-row W blocks and 8-chunk K blocks, x rows beyond one 64-row slab,
the split-K and single-slice launches, the one-pass form (4-bit, K = 2048 or
4096, up to 16 rows) and run-to-run determinism."""
import numpy as np
import pytest

import oracle
import synth
from tests.parity import (bf16_to_np_bits, check_t1, check_t2, to_dev_bf16,
                          to_dev_u32)

pytestmark = pytest.mark.gpu

BITS = (2, 3, 4, 5, 6, 8)
GROUPS = (32, 64, 128)


def _pack(N, K, g, bits, seed):
    return oracle.quantize_pack(synth.weight((N, K), seed), g, bits)


def _dev(w, dev):
    w_q, s, b = w
    return to_dev_u32(w_q, dev), to_dev_bf16(s, dev), to_dev_bf16(b, dev)


def _run(x_bits, dw, g, bits, dev, out_f32=False):
    import torch

    import bit_affine_quantized_amd as q
    y = q.qmv(to_dev_bf16(x_bits, dev), *dw, group_size=g, bits=bits,
              out_dtype=torch.float32 if out_f32 else None)
    return y.cpu().numpy() if out_f32 else bf16_to_np_bits(y)


def _check(N, K, g, bits, M, dev, seed):
    w = _pack(N, K, g, bits, seed)
    x = synth.activation_bf16((M, K), seed=seed + 1)
    ref = oracle.qmv(x, *w, g, bits)
    dw = _dev(w, dev)
    check_t1(_run(x, dw, g, bits, dev), ref, "bf16")
    check_t2(_run(x, dw, g, bits, dev, out_f32=True), ref, "f32")


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("g", GROUPS)
@pytest.mark.parametrize("M", (5, 6, 8, 12, 17, 64, 70))
def test_qmm_ragged_shapes(dev, bits, g, M):
    """N = 200 (three full 64-row W blocks and a partial one), K = 1152 (36
    chunks: four full 8-chunk K blocks and a half one); M = 70 spills into a
    second 64-row slab of x."""
    _check(200, 1152, g, bits, M, dev, seed=bits * 31 + g + M)


@pytest.mark.parametrize("bits", (4, 8, 3))
def test_qmm_single_slice_launch(dev, bits):
    """N = 32768: 512 W blocks, so K is not split (results go straight to y)."""
    _check(32768, 256, 64, bits, 12, dev, seed=11)


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("K,g", [(288, 32), (320, 64), (384, 128)])
def test_qmm_rows_off_16_byte_boundaries(dev, bits, K, g):
    """K / 32 = 9, 10 or 12 chunks: for odd bit widths (and 2 or 6 bits at 9
    chunks) a packed row is not a multiple of 16 bytes, so the rows start off
    16-byte boundaries; the rest start on them with a partial 8-chunk block."""
    _check(72, K, g, bits, 20, dev, seed=bits * 7 + K)


@pytest.mark.parametrize("bits,M", [(4, 64), (4, 128), (8, 16), (2, 32), (6, 48)])
def test_qmm_prefill_shapes(dev, bits, M):
    _check(4096, 4096, 64, bits, M, dev, seed=synth.SEED_W)


def test_qmm_repeated_calls_are_bit_identical(dev):
    N, K, g, bits, M = 2048, 4096, 64, 4, 32
    dw = _dev(_pack(N, K, g, bits, seed=3), dev)
    x = synth.activation_bf16((M, K), seed=4)
    a = _run(x, dw, g, bits, dev, out_f32=True)
    for _ in range(3):
        np.testing.assert_array_equal(_run(x, dw, g, bits, dev, out_f32=True).view(np.uint32),
                                      a.view(np.uint32))


def test_qmm_zero_x_gives_exact_zero(dev):
    N, K, g, bits, M = 512, 1024, 64, 4, 16
    dw = _dev(_pack(N, K, g, bits, seed=5), dev)
    x = np.zeros((M, K), dtype=np.uint16)
    np.testing.assert_array_equal(_run(x, dw, g, bits, dev), np.zeros((M, N), np.uint16))


@pytest.mark.parametrize("K", (2048, 4096))
@pytest.mark.parametrize("g", GROUPS)
@pytest.mark.parametrize("M", (5, 8, 13, 16))
def test_qmf_one_pass_shapes(dev, K, g, M):
    """4-bit codes, K = 2048 or 4096, 5-16 rows of x: the one-pass product (K
    split across the waves of a workgroup, no slices).  N = 1000 is not a
    multiple of its 16-row tile."""
    _check(1000, K, g, 4, M, dev, seed=M * 7 + g + K)


def test_qmf_one_row_tile_and_repeat(dev):
    """N = 17: a second tile holding one W row (the others re-read row 16 and
    are never stored); repeated calls are bit-identical."""
    N, K, g, bits, M = 17, 4096, 64, 4, 16
    w = _pack(N, K, g, bits, seed=9)
    dw = _dev(w, dev)
    x = synth.activation_bf16((M, K), seed=10)
    ref = oracle.qmv(x, *w, g, bits)
    a = _run(x, dw, g, bits, dev, out_f32=True)
    check_t2(a, ref, "f32")
    check_t1(_run(x, dw, g, bits, dev), ref, "bf16")
    for _ in range(3):
        np.testing.assert_array_equal(_run(x, dw, g, bits, dev, out_f32=True).view(np.uint32),
                                      a.view(np.uint32))
