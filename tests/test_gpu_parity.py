"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bit-exact: packed words, scale and bias bits, unpacked codes, gate_up versus
two qmv calls, sorted versus unsorted gather.  Floating point: T1 for bf16
outputs and T2 for the fp32 debugging mode (rules in tests/parity.py).
"""
import numpy as np
import pytest

import oracle
import synth
from tests.parity import (bf16_to_np_bits, check_t1, check_t2, to_dev_bf16,
                          to_dev_u32, u32_to_np)

pytestmark = pytest.mark.gpu

BITS = (2, 3, 4, 5, 6, 8)
GROUPS = (32, 64, 128)

_cache = {}


def q():
    import bit_affine_quantized_amd as mod
    return mod


def packed(N, K, bits, g, seed=synth.SEED_W):
    """(w fp32, oracle w_q, s16, b16) for a seeded weight, cached."""
    key = (N, K, bits, g, seed)
    if key not in _cache:
        w = synth.weight((N, K), seed)
        _cache[key] = (w,) + oracle.quantize_pack(w, g, bits)
    return _cache[key]


def crafted_weight(N, K, seed):
    """Seeded weight with special groups: all zero, all negative, a lattice
    with exact half-step ties, a constant group, and tiny values."""
    w = synth.weight((N, K), seed)
    L = min(128, K)
    w[0, :L] = 0.0
    w[1 % N, :L] = -np.abs(w[1 % N, :L])
    lat = (np.arange(L) % 16 - 5).astype(np.float32) * np.float32(2 ** -6)
    lat[3::16] += np.float32(2 ** -7)      # ties at half a step
    w[2 % N, :L] = lat
    w[3 % N, :L] = np.float32(0.03)
    w[4 % N, :L] *= np.float32(1e-6)
    return w


def dev_pack(w, g, bits, dev):
    import torch
    return q().qmv_pack(torch.from_numpy(np.ascontiguousarray(w)).to(dev), g,
                        bits)


def assert_pack_equal(dw, ds, db, ow, os_, ob):
    np.testing.assert_array_equal(u32_to_np(dw), ow)
    np.testing.assert_array_equal(bf16_to_np_bits(ds), os_)
    np.testing.assert_array_equal(bf16_to_np_bits(db), ob)


# ---------------------------------------------------------------- pack
@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("g", GROUPS)
def test_pack_bit_exact_crafted(dev, bits, g):
    w = crafted_weight(40, 1536, seed=bits * 131 + g)
    dw, ds, db = dev_pack(w, g, bits, dev)
    assert_pack_equal(dw, ds, db, *oracle.quantize_pack(w, g, bits))


FULL_PACKS = [(14336, 4096, 4, 64), (4096, 4096, 4, 64), (256, 512, 4, 64)] + \
    [(14336, 4096, b, g) for b in (2, 3, 5, 6, 8) for g in GROUPS]


@pytest.mark.parametrize("N,K,bits,g", FULL_PACKS)
def test_pack_bit_exact_full_size(dev, N, K, bits, g):
    w, ow, os_, ob = packed(N, K, bits, g)
    dw, ds, db = dev_pack(w, g, bits, dev)
    assert_pack_equal(dw, ds, db, ow, os_, ob)


# ---------------------------------------------------------------- unpack
@pytest.mark.parametrize("bits", BITS)
def test_unpack_codes_bit_exact(dev, bits):
    rng = np.random.default_rng(bits)
    N, K = 37, 4224
    words = rng.integers(0, 2 ** 32, size=(N, K * bits // 32),
                         dtype=np.uint64).astype(np.uint32)
    codes = q().qmv_unpack_codes(to_dev_u32(words, dev), K, bits)
    np.testing.assert_array_equal(codes.cpu().numpy(),
                                  oracle.unpack(words, K, bits))


# ---------------------------------------------------------------- qmv
def run_qmv(x_bits, w_q, s, b, g, bits, dev, out_f32=False):
    import torch
    y = q().qmv(to_dev_bf16(x_bits, dev), w_q, s, b, group_size=g, bits=bits,
                out_dtype=torch.float32 if out_f32 else None)
    if out_f32:
        return y.cpu().numpy()
    return bf16_to_np_bits(y)


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("g", GROUPS)
@pytest.mark.parametrize("M", (1, 2, 3, 4, 5))
def test_qmv_ragged_shapes(dev, bits, g, M):
    """N = 300 (not a multiple of the 16-row workgroup tile) and K = 4224
    (132 chunks: two full 64-lane steps and a 4-lane tail)."""
    N, K = 300, 4224
    w = crafted_weight(N, K, seed=bits + 7 * g)
    ow, os_, ob = oracle.quantize_pack(w, g, bits)
    x = synth.activation_bf16((M, K), seed=M)
    ref = oracle.qmv(x, ow, os_, ob, g, bits)
    dw, ds, db = to_dev_u32(ow, dev), to_dev_bf16(os_, dev), to_dev_bf16(ob, dev)
    check_t1(run_qmv(x, dw, ds, db, g, bits, dev), ref, "bf16")
    check_t2(run_qmv(x, dw, ds, db, g, bits, dev, out_f32=True), ref, "f32")


@pytest.mark.parametrize("N,K,g", [(4100, 4224, 32), (4100, 4096, 128), (300, 8192, 64),
                                   (300, 8256, 32), (77, 4160, 64)])
def test_qmv_two_bit_shapes(dev, N, K, g):
    """2-bit codes (8-byte chunks) past the tile and step boundaries: more
    than 4096 rows (two rows per wave) with a ragged lane tail (K = 4224),
    K = 8192 and 8256 past the straight-line kernel's 4096, and an odd
    number of groups per row (K = 4160 with 65 groups of 64)."""
    bits = 2
    w = crafted_weight(N, K, seed=N + K + g)
    ow, os_, ob = oracle.quantize_pack(w, g, bits)
    x = synth.activation_bf16((1, K), seed=3)
    ref = oracle.qmv(x, ow, os_, ob, g, bits)
    dw, ds, db = to_dev_u32(ow, dev), to_dev_bf16(os_, dev), to_dev_bf16(ob, dev)
    check_t1(run_qmv(x, dw, ds, db, g, bits, dev), ref, "bf16")
    check_t2(run_qmv(x, dw, ds, db, g, bits, dev, out_f32=True), ref, "f32")


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("N,K,g", [(1, 32, 32), (3, 64, 64), (17, 128, 128),
                                   (64, 96, 32), (5, 2048, 64)])
def test_qmv_small_edges(dev, bits, N, K, g):
    w = crafted_weight(N, K, seed=N + K)
    ow, os_, ob = oracle.quantize_pack(w, g, bits)
    x = synth.activation_bf16((2, K), seed=K)
    ref = oracle.qmv(x, ow, os_, ob, g, bits)
    dw, ds, db = to_dev_u32(ow, dev), to_dev_bf16(os_, dev), to_dev_bf16(ob, dev)
    check_t1(run_qmv(x, dw, ds, db, g, bits, dev), ref)
    check_t2(run_qmv(x, dw, ds, db, g, bits, dev, out_f32=True), ref)


def test_qmv_zero_x_gives_exact_zero(dev):
    N, K, g, bits = 64, 1024, 64, 4
    w, ow, os_, ob = packed(N, K, bits, g, seed=3)
    x = np.zeros((1, K), np.uint16)
    y = run_qmv(x, to_dev_u32(ow, dev), to_dev_bf16(os_, dev),
                to_dev_bf16(ob, dev), g, bits, dev, out_f32=True)
    assert np.all(y == 0.0)


@pytest.mark.parametrize("bits,M", [(4, 4), (8, 4), (3, 1)])
def test_qmv_long_k_lds_limit(dev, bits, M):
    """K = 32768: x for four vectors no longer fits in one workgroup's LDS,
    so the call is split into slabs of fewer vectors."""
    N, K, g = 48, 32768, 128
    w, ow, os_, ob = packed(N, K, bits, g, seed=5)
    x = synth.activation_bf16((M, K), seed=9)
    ref = oracle.qmv(x, ow, os_, ob, g, bits)
    dw, ds, db = to_dev_u32(ow, dev), to_dev_bf16(os_, dev), to_dev_bf16(ob, dev)
    check_t1(run_qmv(x, dw, ds, db, g, bits, dev), ref)
    check_t2(run_qmv(x, dw, ds, db, g, bits, dev, out_f32=True), ref)


CONFIGS = [("tiny", 256, 512, 4, 64, 1), ("decode_m1", 4096, 4096, 4, 64, 1),
           ("decode_m4", 4096, 4096, 4, 64, 4),
           ("headline", 14336, 4096, 4, 64, 1)] + \
    [(f"sweep_b{b}_g{g}", 14336, 4096, b, g, 1) for b in (2, 3, 5, 6, 8)
     for g in GROUPS]


@pytest.mark.parametrize("name,N,K,bits,g,M", CONFIGS,
                         ids=[c[0] for c in CONFIGS])
def test_qmv_workloads_full(dev, name, N, K, bits, g, M):
    """Every output of every workload, device-packed weights, both modes."""
    w, ow, os_, ob = packed(N, K, bits, g)
    dw, ds, db = dev_pack(w, g, bits, dev)
    x = synth.activation_bf16((M, K))
    ref = oracle.qmv(x, ow, os_, ob, g, bits)
    check_t1(run_qmv(x, dw, ds, db, g, bits, dev), ref, name)
    check_t2(run_qmv(x, dw, ds, db, g, bits, dev, out_f32=True), ref, name)


@pytest.mark.parametrize("bits", (3, 4, 8))
@pytest.mark.parametrize("M", (2, 3, 4))
def test_qmv_headline_matrix_decode_batch(dev, bits, M):
    """The 14336x4096 g64 matrix at decode batch 2-4: more than 4096 rows and
    2-4 rows of x run two rows per wave against a 2- or 4-vector slab (the
    4-value lane butterfly at two vectors, the 8-value one at four); 8-bit
    codes take the fp32-staged form.  Every output, both modes."""
    N, K, g = 14336, 4096, 64
    w, ow, os_, ob = packed(N, K, bits, g)
    dw, ds, db = to_dev_u32(ow, dev), to_dev_bf16(os_, dev), to_dev_bf16(ob, dev)
    x = synth.activation_bf16((M, K), seed=300 + M)
    ref = oracle.qmv(x, ow, os_, ob, g, bits)
    check_t1(run_qmv(x, dw, ds, db, g, bits, dev), ref, f"b{bits} M={M} bf16")
    check_t2(run_qmv(x, dw, ds, db, g, bits, dev, out_f32=True), ref,
             f"b{bits} M={M} f32")


@pytest.mark.parametrize("bits", (2, 4, 5, 8))
@pytest.mark.parametrize("M", (2, 4))
def test_qmv_ragged_rows_past_4096(dev, bits, M):
    """N = 4100 (past 4096, not a multiple of the two-row wave tile) and
    K = 1536 (24 chunks: a partial first lane step), at 2 and 4 rows of x."""
    N, K, g = 4100, 1536, 64
    w = crafted_weight(N, K, seed=bits * 11 + M)
    ow, os_, ob = oracle.quantize_pack(w, g, bits)
    dw, ds, db = to_dev_u32(ow, dev), to_dev_bf16(os_, dev), to_dev_bf16(ob, dev)
    x = synth.activation_bf16((M, K), seed=400 + M)
    ref = oracle.qmv(x, ow, os_, ob, g, bits)
    check_t1(run_qmv(x, dw, ds, db, g, bits, dev), ref, "bf16")
    check_t2(run_qmv(x, dw, ds, db, g, bits, dev, out_f32=True), ref, "f32")


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("M", (1, 2, 3, 4))
@pytest.mark.parametrize("N,g", [(1000, 64), (4100, 128)])
def test_qmv_vectors_partial_second_step(dev, bits, M, N, g):
    """K = 3968 (124 chunks: a second 64-lane step with 4 lanes idle) at 1-4
    rows of x, at most 4096 rows (one row per wave) and past it (two rows per
    wave): the straight-line kernel with a partial step (its x staged in
    16-byte pieces for 4- and 8-bit codes at one row per wave and for 8-bit
    codes at two), and the several-vector slab with a partial step and with
    3 of a 4-vector slab's slots filled."""
    K = 3968
    w = crafted_weight(N, K, seed=bits * 13 + M + g)
    ow, os_, ob = oracle.quantize_pack(w, g, bits)
    dw, ds, db = to_dev_u32(ow, dev), to_dev_bf16(os_, dev), to_dev_bf16(ob, dev)
    x = synth.activation_bf16((M, K), seed=500 + M)
    ref = oracle.qmv(x, ow, os_, ob, g, bits)
    check_t1(run_qmv(x, dw, ds, db, g, bits, dev), ref, "bf16")
    check_t2(run_qmv(x, dw, ds, db, g, bits, dev, out_f32=True), ref, "f32")


# ---------------------------------------------------------------- fused FFN
def _ffn_weights(dev, N=14336, K=4096, bits=8, g=64, down=True):
    wg = packed(N, K, bits, g, seed=synth.SEED_W)
    wu = packed(N, K, bits, g, seed=synth.SEED_UP)
    mats = [wg, wu]
    if down:
        mats.append(packed(K, N, bits, g, seed=synth.SEED_DOWN))
    on_dev = [tuple(f(a, dev) for f, a in zip((to_dev_u32, to_dev_bf16,
                                                 to_dev_bf16), p[1:]))
              for p in mats]
    return mats, on_dev


@pytest.mark.parametrize("bits,g", [(8, 64), (4, 64), (3, 32), (2, 32), (2, 128)])
def test_gate_up_equals_two_qmv_and_oracle(dev, bits, g):
    N, K = (14336, 4096) if bits == 8 else (2000, 2048)
    (wg, wu), (dg, du) = _ffn_weights(dev, N, K, bits, g, down=False)
    x = synth.activation_bf16((1, K))
    xd = to_dev_bf16(x, dev)
    gate_y, up_y = q().qmv_gate_up(xd[0], dg, du, group_size=g, bits=bits)
    g_bits, u_bits = bf16_to_np_bits(gate_y), bf16_to_np_bits(up_y)
    g2 = run_qmv(x, *dg, g, bits, dev)[0]
    u2 = run_qmv(x, *du, g, bits, dev)[0]
    np.testing.assert_array_equal(g_bits, g2)
    np.testing.assert_array_equal(u_bits, u2)
    check_t1(g_bits, oracle.qmv(x, *wg[1:], g, bits)[0], "gate")
    check_t1(u_bits, oracle.qmv(x, *wu[1:], g, bits)[0], "up")


def test_ffn_tail_workload(dev):
    """gate/up in one launch, then silu(gate)*up -> down + residual."""
    import torch
    bits, g, N, K = 8, 64, 14336, 4096
    (wg, wu, wd), (dg, du, dd) = _ffn_weights(dev, N, K, bits, g)
    x = synth.activation_bf16((1, K))
    xr = synth.activation_bf16((K,), seed=synth.SEED_XRESID)
    gate_y, up_y = q().qmv_gate_up(to_dev_bf16(x, dev)[0], dg, du,
                                   group_size=g, bits=bits)
    xr_d = to_dev_bf16(xr, dev)
    y = q().qmv_silu_gate_resid(gate_y, up_y, xr_d, *dd, group_size=g,
                                bits=bits)
    yf = q().qmv_silu_gate_resid(gate_y, up_y, xr_d, *dd, group_size=g,
                                 bits=bits, out_dtype=torch.float32)
    gb, ub = bf16_to_np_bits(gate_y), bf16_to_np_bits(up_y)
    ref = oracle.silu_gate_resid(gb, ub, xr, *wd[1:], g, bits)
    check_t1(bf16_to_np_bits(y), ref, "tail bf16")
    check_t2(yf.cpu().numpy(), ref, "tail f32")
    # end to end with the oracle's own gate/up rounded once to bf16
    gr = oracle.qmv(x, *wg[1:], g, bits)[0]
    ur = oracle.qmv(x, *wu[1:], g, bits)[0]
    to_bits = lambda v: bf16_to_np_bits(torch.from_numpy(v).to(torch.bfloat16))
    ref_e2e = oracle.silu_gate_resid(to_bits(gr), to_bits(ur), xr, *wd[1:], g,
                                     bits)
    check_t1(bf16_to_np_bits(y), ref_e2e, "ffn end to end")


@pytest.mark.parametrize("bits", BITS)
def test_silu_gate_resid_small(dev, bits):
    import torch
    N, K, g = 260, 4224, 64
    w = crafted_weight(N, K, seed=bits)
    ow, os_, ob = oracle.quantize_pack(w, g, bits)
    dd = (to_dev_u32(ow, dev), to_dev_bf16(os_, dev), to_dev_bf16(ob, dev))
    gate = synth.activation_bf16((K,), seed=1)
    up = synth.activation_bf16((K,), seed=2)
    xr = synth.activation_bf16((N,), seed=3)
    gd, ud, xd = (to_dev_bf16(a, dev) for a in (gate, up, xr))
    for resid in (True, False):
        ref = oracle.silu_gate_resid(gate, up, xr if resid else None, ow, os_,
                                     ob, g, bits)
        y = q().qmv_silu_gate_resid(gd, ud, xd if resid else None, *dd,
                                    group_size=g, bits=bits)
        check_t1(bf16_to_np_bits(y), ref)
        yf = q().qmv_silu_gate_resid(gd, ud, xd if resid else None, *dd,
                                     group_size=g, bits=bits,
                                     out_dtype=torch.float32)
        check_t2(yf.cpu().numpy(), ref)


def test_silu_zero_up_or_gate_returns_resid_exactly(dev):
    N, K, g, bits = 128, 2048, 64, 8
    w, ow, os_, ob = packed(N, K, bits, g, seed=4)
    dd = (to_dev_u32(ow, dev), to_dev_bf16(os_, dev), to_dev_bf16(ob, dev))
    xr = synth.activation_bf16((N,), seed=3)
    a = to_dev_bf16(synth.activation_bf16((K,), seed=8), dev)
    z = to_dev_bf16(np.zeros(K, np.uint16), dev)
    xd = to_dev_bf16(xr, dev)
    for gate, up in ((a, z), (z, a)):
        y = q().qmv_silu_gate_resid(gate, up, xd, *dd, group_size=g, bits=bits)
        np.testing.assert_array_equal(bf16_to_np_bits(y), xr)


# ---------------------------------------------------------------- gather
def _experts(E, N, K, bits, g, seed0=1000):
    ws = [packed(N, K, bits, g, seed=seed0 + e) for e in range(E)]
    w_q = np.stack([p[1] for p in ws])
    s = np.stack([p[2] for p in ws])
    b = np.stack([p[3] for p in ws])
    return w_q, s, b


def _run_gather(dev, x, ew, lhs, rhs, g, bits, sorted_indices, out_f32=False):
    import torch
    w_q, s, b = ew
    y = q().gather_qmv(to_dev_bf16(x, dev), to_dev_u32(w_q, dev),
                       to_dev_bf16(s, dev), to_dev_bf16(b, dev),
                       to_dev_u32(lhs, dev), to_dev_u32(rhs, dev),
                       group_size=g, bits=bits, sorted_indices=sorted_indices,
                       out_dtype=torch.float32 if out_f32 else None)
    return y.cpu().numpy() if out_f32 else bf16_to_np_bits(y)


def test_gather_moe_workload(dev):
    """64 experts [2048, 2048] b4 g64; 16 tokens x top-8; unsorted and
    stable-sorted pairs give identical bits after the inverse permutation."""
    cfg = synth.MOE
    E, N, K, bits, g = cfg["E"], cfg["N"], cfg["K"], cfg["bits"], cfg["group"]
    T, top = cfg["tokens"], cfg["top_k"]
    ew = _experts(E, N, K, bits, g)
    x = synth.activation_bf16((T, 1, K))
    lhs, rhs = synth.moe_indices(T, top, E)
    lhs, rhs = lhs.ravel(), rhs.ravel()
    ref = oracle.gather_qmv(x, *ew, lhs, rhs, g, bits)
    y_u = _run_gather(dev, x, ew, lhs, rhs, g, bits, False)
    check_t1(y_u, ref, "unsorted")
    check_t2(_run_gather(dev, x, ew, lhs, rhs, g, bits, False, True), ref, "f32")
    perm = np.argsort(rhs, kind="stable")
    y_s = _run_gather(dev, x, ew, lhs[perm], rhs[perm], g, bits, True)
    np.testing.assert_array_equal(y_s, y_u[perm])


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("M", (1, 2, 3))
def test_gather_small(dev, bits, M):
    # fewer than 5 vectors per expert on average: the matvec gather
    E, N, K, g = 7, 70, 1152, 64
    ew = _experts(E, N, K, bits, g, seed0=50 + bits)
    rng = np.random.default_rng(M * 10 + bits)
    Bx, P = 4, 11
    x = synth.activation_bf16((Bx, M, K), seed=M)
    lhs = rng.integers(0, Bx, P).astype(np.uint32)
    rhs = rng.integers(0, E, P).astype(np.uint32)
    rhs[:6] = 2            # one expert with more vectors than one batch
    ref = oracle.gather_qmv(x, *ew, lhs, rhs, g, bits)
    y = _run_gather(dev, x, ew, lhs, rhs, g, bits, False)
    check_t1(y, ref)
    check_t2(_run_gather(dev, x, ew, lhs, rhs, g, bits, False, True), ref)
    perm = np.argsort(rhs, kind="stable")
    np.testing.assert_array_equal(
        _run_gather(dev, x, ew, lhs[perm], rhs[perm], g, bits, True), y[perm])


@pytest.mark.parametrize("E,N,K,g,bits", [(3, 1, 64, 64, 4), (5, 7, 96, 32, 3),
                                          (4, 9, 2112, 64, 8), (2, 33, 320, 64, 6)])
def test_gather_row_and_k_edges(dev, E, N, K, g, bits):
    """Row counts below and just past one 8-row wave step (N = 1, 7, 9, 33)
    and K ranges that leave most lanes of a row segment idle (2 or 3
    chunks) or end one chunk into a step (66 and 10 chunks)."""
    ew = _experts(E, N, K, bits, g, seed0=300 + N)
    rng = np.random.default_rng(N + K)
    Bx, P = 3, 9                                   # under 5 pairs per expert
    x = synth.activation_bf16((Bx, 1, K), seed=N)
    lhs = rng.integers(0, Bx, P).astype(np.uint32)
    rhs = rng.integers(0, E, P).astype(np.uint32)
    ref = oracle.gather_qmv(x, *ew, lhs, rhs, g, bits)
    check_t1(_run_gather(dev, x, ew, lhs, rhs, g, bits, False), ref)
    check_t2(_run_gather(dev, x, ew, lhs, rhs, g, bits, False, True), ref)


@pytest.mark.parametrize("sorted_indices", (False, True))
def test_gather_long_pair_lists(dev, sorted_indices):
    """1400 pairs over 300 experts (4.7 per expert on average: the matvec
    gather), 1100 of them on expert 0: its list exceeds the 1024-pair
    routing window, so its rows are served in several windows."""
    E, N, K, g, bits = 300, 48, 256, 64, 4
    ew = _experts(E, N, K, bits, g, seed0=77)
    rng = np.random.default_rng(5)
    Bx, P = 40, 1400
    x = synth.activation_bf16((Bx, 1, K), seed=6)
    lhs = rng.integers(0, Bx, P).astype(np.uint32)
    rhs = rng.integers(1, E, P).astype(np.uint32)
    rhs[rng.choice(P, 1100, replace=False)] = 0
    if sorted_indices:
        perm = np.argsort(rhs, kind="stable")
        lhs, rhs = lhs[perm], rhs[perm]
    ref = oracle.gather_qmv(x, *ew, lhs, rhs, g, bits)
    check_t1(_run_gather(dev, x, ew, lhs, rhs, g, bits, sorted_indices), ref)
    check_t2(_run_gather(dev, x, ew, lhs, rhs, g, bits, sorted_indices, True),
             ref)


def test_gather_without_indices_is_qmv(dev):
    N, K, g, bits = 300, 2048, 64, 4
    w, ow, os_, ob = packed(N, K, bits, g, seed=12)
    x = synth.activation_bf16((2, K), seed=4)
    dw, ds, db = to_dev_u32(ow, dev), to_dev_bf16(os_, dev), to_dev_bf16(ob, dev)
    y = q().gather_qmv(to_dev_bf16(x, dev)[None], dw, ds, db, group_size=g,
                       bits=bits)
    np.testing.assert_array_equal(bf16_to_np_bits(y),
                                  run_qmv(x, dw, ds, db, g, bits, dev))
