"""GPU parity of the transpose = 0 product (qvm): y = x @ W_hat with W packed
[K, N] along N, through the C ABI, against the oracle's exact fp64 qvm.
T1 for bf16 outputs and T2 for the fp32 debugging mode; the split-K sum is
fixed-order, so repeated calls and graph replays give the same bits."""
import numpy as np
import pytest

import oracle
import synth
from tests.parity import (bf16_to_np_bits, check_t1, check_t2, to_dev_bf16,
                          to_dev_u32)

pytestmark = pytest.mark.gpu

BITS = (2, 3, 4, 5, 6, 8)
GROUPS = (32, 64, 128)


def _pack_kn(K, N, g, bits, seed):
    """Seeded W [K, N] quantized along N (the qvm layout)."""
    return oracle.quantize_pack(synth.weight((K, N), seed), g, bits)


def _run(x_bits, w, g, bits, dev, out_f32=False, y=None):
    import torch

    import bit_affine_quantized_amd as q
    out = q.qmv(to_dev_bf16(x_bits, dev), *w, transpose=False, group_size=g,
                bits=bits, out_dtype=torch.float32 if out_f32 else None, y=y)
    return out.cpu().numpy() if out_f32 else bf16_to_np_bits(out)


def _dev(w, dev):
    w_q, s, b = w
    return to_dev_u32(w_q, dev), to_dev_bf16(s, dev), to_dev_bf16(b, dev)


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("g", GROUPS)
@pytest.mark.parametrize("M", (1, 3, 5))
def test_qvm_ragged_shapes(dev, bits, g, M):
    """K = 300 rows (several split-K slices, the last one partial) and
    N = 1152 columns (3 column blocks of 512, the last one partial); M = 5
    runs as a 4-vector slab and a 1-vector slab."""
    K, N = 300, 1152
    w = _pack_kn(K, N, g, bits, seed=bits + 7 * g)
    x = synth.activation_bf16((M, K), seed=M)
    ref = oracle.qvm(x, *w, N, g, bits)
    dw = _dev(w, dev)
    check_t1(_run(x, dw, g, bits, dev), ref, "bf16")
    check_t2(_run(x, dw, g, bits, dev, out_f32=True), ref, "f32")


@pytest.mark.parametrize("K,N,g,bits,M", [(40, 256, 32, 4, 2), (1, 64, 64, 8, 1),
                                          (129, 32, 32, 3, 1), (4096, 96, 32, 6, 2)])
def test_qvm_small_edges(dev, K, N, g, bits, M):
    w = _pack_kn(K, N, g, bits, seed=K + N)
    x = synth.activation_bf16((M, K), seed=K)
    ref = oracle.qvm(x, *w, N, g, bits)
    dw = _dev(w, dev)
    check_t1(_run(x, dw, g, bits, dev), ref, "bf16")
    check_t2(_run(x, dw, g, bits, dev, out_f32=True), ref, "f32")


@pytest.mark.parametrize("K,N,bits,g,M", [(4096, 4096, 4, 64, 1), (4096, 4096, 4, 64, 4),
                                          (14336, 4096, 8, 64, 1)])
def test_qvm_decode_shapes(dev, K, N, bits, g, M):
    w = _pack_kn(K, N, g, bits, seed=synth.SEED_W)
    x = synth.activation_bf16((M, K), seed=synth.SEED_X)
    ref = oracle.qvm(x, *w, N, g, bits)
    dw = _dev(w, dev)
    check_t1(_run(x, dw, g, bits, dev), ref, "bf16")
    check_t2(_run(x, dw, g, bits, dev, out_f32=True), ref, "f32")


def test_qvm_repeated_calls_are_bit_identical(dev):
    K, N, g, bits = 4096, 2048, 64, 4
    dw = _dev(_pack_kn(K, N, g, bits, seed=3), dev)
    x = synth.activation_bf16((2, K), seed=4)
    a = _run(x, dw, g, bits, dev, out_f32=True)
    for _ in range(3):
        np.testing.assert_array_equal(_run(x, dw, g, bits, dev, out_f32=True).view(np.uint32),
                                      a.view(np.uint32))


def test_qvm_zero_x_gives_exact_zero(dev):
    K, N, g, bits = 512, 1024, 64, 4
    dw = _dev(_pack_kn(K, N, g, bits, seed=5), dev)
    x = np.zeros((1, K), dtype=np.uint16)
    np.testing.assert_array_equal(_run(x, dw, g, bits, dev), np.zeros((1, N), np.uint16))
