"""GPU parity of the matrix-core gather that gather_qmv takes when the routed
x vectors average 5 or more per expert (prefill-sized MoE), against the
oracle's exact fp64 gather: T1 / T2, sorted = unsorted bit for bit, experts
with more than 64 vectors (several passes), an expert with no pair, x with
two rows per batch entry, and a routing list longer than one 1024-pair
window."""
import numpy as np
import pytest

import oracle
import synth
from tests.parity import (bf16_to_np_bits, check_t1, check_t2, to_dev_bf16,
                          to_dev_u32)

pytestmark = pytest.mark.gpu

BITS = (2, 3, 4, 5, 6, 8)
GROUPS = (32, 64, 128)


def _experts(E, N, K, bits, g, seed0=2000):
    packs = [oracle.quantize_pack(synth.weight((N, K), seed0 + e), g, bits) for e in range(E)]
    return tuple(np.stack([p[i] for p in packs]) for i in range(3))


def _run(dev, x, ew, lhs, rhs, g, bits, sorted_indices=False, out_f32=False):
    import torch

    import bit_affine_quantized_amd as q
    w_q, s, b = ew
    y = q.gather_qmv(to_dev_bf16(x, dev), to_dev_u32(w_q, dev), to_dev_bf16(s, dev),
                     to_dev_bf16(b, dev), to_dev_u32(lhs, dev), to_dev_u32(rhs, dev),
                     group_size=g, bits=bits, sorted_indices=sorted_indices,
                     out_dtype=torch.float32 if out_f32 else None)
    return y.cpu().numpy() if out_f32 else bf16_to_np_bits(y)


def _check(dev, E, N, K, bits, g, T, top, M=1, seed=0, rhs=None):
    ew = _experts(E, N, K, bits, g, seed0=2000 + seed)
    x = synth.activation_bf16((T, M, K), seed=seed + 7)
    if rhs is None:
        lhs, rhs = synth.moe_indices(T, top, E, seed=seed + 9)
        lhs, rhs = lhs.ravel(), rhs.ravel()
    else:
        lhs = np.repeat(np.arange(T, dtype=np.uint32), top)
    assert lhs.size * M >= 5 * E             # the matrix-core gather is taken
    ref = oracle.gather_qmv(x, *ew, lhs, rhs, g, bits)
    y = _run(dev, x, ew, lhs, rhs, g, bits)
    check_t1(y, ref, "bf16")
    check_t2(_run(dev, x, ew, lhs, rhs, g, bits, out_f32=True), ref, "f32")
    perm = np.argsort(rhs, kind="stable")
    ys = _run(dev, x, ew, lhs[perm], rhs[perm], g, bits, sorted_indices=True)
    np.testing.assert_array_equal(ys, y[perm])


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("g", GROUPS)
def test_gather_qmm_parity(dev, bits, g):
    """8 experts of [200, 1152] (a partial 64-row W block, 36 chunks); 48
    tokens x top-2 = 96 pairs, 12 per expert on average."""
    _check(dev, 8, 200, 1152, bits, g, T=48, top=2, seed=bits + g)


@pytest.mark.parametrize("bits", (3, 5, 8))
def test_gather_qmm_rows_off_16_byte_boundaries(dev, bits):
    """K = 288 (9 chunks): 3- and 5-bit rows are not a multiple of 16 bytes."""
    _check(dev, 4, 72, 288, bits, 32, T=32, top=2, seed=bits + 50)


@pytest.mark.parametrize("T", (20, 40, 96, 160))
def test_gather_qmm_slab_heights(dev, T):
    """8 experts, top-2: 5, 10, 24 and 40 x vectors per expert on average,
    so the slabs are 16, 16, 32 and 64 vectors tall; expert 0 takes a
    quarter of the pairs, so its list spans several slabs."""
    E = 8
    rng = np.random.default_rng(T)
    rhs = rng.integers(0, E, T * 2).astype(np.uint32)
    rhs[: T // 2] = 0
    _check(dev, E, 136, 512, 4, 64, T=T, top=2, seed=T, rhs=rhs)


def test_gather_qmm_many_vectors_and_an_empty_expert(dev):
    """Expert 3 gets no pair; experts 0 and 1 get more than 64 vectors."""
    T, top, E = 160, 2, 6
    rng = np.random.default_rng(5)
    rhs = np.empty(T * top, np.uint32)
    for t in range(T):
        first = 0 if t % 2 == 0 else 1
        rhs[2 * t] = first
        rhs[2 * t + 1] = rng.choice([2, 4, 5])
    _check(dev, E, 256, 512, 4, 64, T=T, top=top, seed=3, rhs=rhs)


def test_gather_qmm_two_rows_per_token(dev):
    _check(dev, 4, 128, 1024, 4, 64, T=16, top=2, M=2, seed=4)


def test_gather_qmm_prefill_moe_shape(dev):
    """16 experts [512, 1024] b4 g64; 256 tokens x top-4 = 1024 pairs."""
    _check(dev, 16, 512, 1024, 4, 64, T=256, top=4, seed=6)


def test_gather_qmm_long_list_windows(dev):
    """2500 pairs on 2 experts: expert 0 holds more than one 1024-pair
    window."""
    T = 2500
    rhs = (np.arange(T) % 5 == 4).astype(np.uint32)
    _check(dev, 2, 128, 256, 4, 64, T=T, top=1, seed=8, rhs=rhs)
