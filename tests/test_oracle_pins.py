"""Pins for the CPU oracle: each check compares it with something other than
itself (the page's byte tables, closed forms derived by hand from the
quantizer's definition, exact rational arithmetic, library routines)."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from tests.page_layout import decode_words

BITS = (2, 3, 4, 5, 6, 8)
GROUPS = (32, 64, 128)


def _bf16_exact(h):
    return Fraction(float(synth.bf16_bits_to_f32(np.uint16(h))))


# ----------------------------------------------------------------- layout (P-1)
@pytest.mark.parametrize("bits", BITS)
def test_pack_matches_page_byte_layout(bits):
    """Oracle bit-stream pack, read back with the page's byte formulas."""
    rng = np.random.default_rng(bits)
    N, K = 5, 256
    codes = rng.integers(0, 1 << bits, size=(N, K), dtype=np.uint8)
    w_q = oracle.pack(codes, bits)
    assert w_q.shape == (N, K * bits // 32)
    np.testing.assert_array_equal(decode_words(w_q, K, bits), codes)


@pytest.mark.parametrize("bits", (2, 4, 8))
def test_pack_word_shift_layout(bits):
    """For power-of-two widths: word = OR of code_i << (bits*i) (the page's
    quantizer writes output |= val << bits*(i % pack_factor))."""
    rng = np.random.default_rng(7)
    per = 32 // bits
    codes = rng.integers(0, 1 << bits, size=(3, 4 * per), dtype=np.uint8)
    w_q = oracle.pack(codes, bits)
    for n in range(3):
        for wi in range(4):
            expect = 0
            for i in range(per):
                expect |= int(codes[n, wi * per + i]) << (bits * i)
            assert int(w_q[n, wi]) == expect


def test_pack_golden_3bit_hand_example():
    """Codes 0..7 at 3 bits: the page's 8-codes-in-3-bytes pack, by hand.
    code j at stream bit 3j: bytes = 0b10001000, 0b11000110, 0b11111010."""
    codes = np.arange(8, dtype=np.uint8)[None, :]
    codes = np.tile(codes, (1, 4))  # K = 32 -> 3 words
    w_q = oracle.pack(codes, 3)
    b = w_q.view(np.uint8).ravel()
    assert list(b[:3]) == [0x88, 0xC6, 0xFA]


# -------------------------------------------------------------- bijection (P-2)
@pytest.mark.parametrize("bits", BITS)
def test_pack_unpack_bijection(bits):
    rng = np.random.default_rng(100 + bits)
    N, K = 7, 384
    codes = rng.integers(0, 1 << bits, size=(N, K), dtype=np.uint8)
    np.testing.assert_array_equal(oracle.unpack(oracle.pack(codes, bits), K,
                                                bits), codes)
    words = rng.integers(0, 2**32, size=(N, K * bits // 32), dtype=np.uint64)
    words = words.astype(np.uint32)
    np.testing.assert_array_equal(oracle.pack(oracle.unpack(words, K, bits),
                                              bits), words)


# ------------------------------------------------------ quantizer closed forms
@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("g", GROUPS)
@pytest.mark.parametrize("z_frac", (0.0, 0.3, 0.5, 0.8, 1.0))
def test_quantize_lattice_group_is_exact(bits, g, z_frac):
    """Values (j - z) * 2^-7 with j covering 0 and 2^b - 1.  From the
    quantizer's steps: scale = +-2^-7, the codes are j (if |w_min| > |w_max|)
    or (2^b - 1) - j, and s*q + b reproduces every value exactly."""
    nb = (1 << bits) - 1
    delta = 2.0 ** -7
    z = int(round(z_frac * nb))
    rng = np.random.default_rng(bits * 1000 + g)
    j = rng.integers(0, nb + 1, size=g)
    j[0], j[1] = 0, nb
    v = ((j - z) * delta).astype(np.float32)[None, :]
    codes, s32, b32, s16, b16 = oracle.quantize(v, g, bits)
    side = z > nb - z
    exp_codes = j if side else nb - j
    np.testing.assert_array_equal(codes[0], exp_codes.astype(np.uint8))
    assert s32[0, 0] == np.float32(delta if side else -delta)
    assert b32[0, 0] == np.float32(-z * delta if side else (nb - z) * delta)
    w_hat = oracle.dequantize(oracle.pack(codes, bits), s16, b16, g, g, bits)
    np.testing.assert_array_equal(w_hat[0], v[0].astype(np.float64))


def test_quantize_all_zero_group():
    """w == 0: range 0 -> scale = eps = 1e-7, |0| > |0| is false so the
    scale turns negative, round(0 / -1e-7) == 0 -> bias 0, codes 0."""
    import torch
    v = np.zeros((1, 64), np.float32)
    codes, s32, b32, s16, b16 = oracle.quantize(v, 64, 4)
    assert not codes.any()
    assert s32[0, 0] == np.float32(-1e-7)
    assert b32[0, 0] == 0.0
    want = torch.tensor([-1e-7], dtype=torch.float32).to(torch.bfloat16)
    assert int(s16[0, 0]) == int(want.view(torch.int16).item()) & 0xFFFF
    assert int(b16[0, 0]) == 0


@pytest.mark.parametrize("bits", BITS)
def test_quantize_all_negative_group_keeps_zero_in_range(bits):
    """w_max starts at 0, so an all-negative group still spans [w_min, 0]:
    values -j*2^-7 with j in [1, nb] give scale 2^-7, bias -nb*2^-7 and codes
    nb - j.  (A w_max starting at -inf would give a different scale.)"""
    nb = (1 << bits) - 1
    delta = 2.0 ** -7
    rng = np.random.default_rng(bits)
    j = rng.integers(1, nb + 1, size=32)
    j[0], j[1] = 1, nb
    v = (-j * delta).astype(np.float32)[None, :]
    codes, s32, b32, _, _ = oracle.quantize(v, 32, bits)
    assert s32[0, 0] == np.float32(delta)
    assert b32[0, 0] == np.float32(-nb * delta)
    np.testing.assert_array_equal(codes[0], (nb - j).astype(np.uint8))


def test_quantize_rounds_half_away_from_zero_codes():
    """4-bit group {0, 15d, 6.5d}: scale -d, bias 15d, and 6.5d maps to
    (6.5d - 15d)/(-d) = 8.5 -> 9 (half away from zero; half-even gives 8)."""
    d = 2.0 ** -4
    v = np.zeros((1, 32), np.float32)
    v[0, 1] = 15 * d
    v[0, 2] = 6.5 * d
    codes, s32, b32, _, _ = oracle.quantize(v, 32, 4)
    assert s32[0, 0] == np.float32(-d) and b32[0, 0] == np.float32(15 * d)
    assert codes[0, 0] == 15 and codes[0, 1] == 0 and codes[0, 2] == 9


def test_quantize_rounds_half_away_from_zero_q0():
    """2-bit group {2.5, -0.5, 0...}: range/3 = 1, not side -> scale -1,
    edge 2.5, q0 = round(-2.5) = -3 (half-even would give -2), so the scale
    becomes 2.5 / -3 and the bias 2.5.  -0.5 maps to 3.6 -> 4 -> clamp 3."""
    v = np.zeros((1, 32), np.float32)
    v[0, 0] = 2.5
    v[0, 1] = -0.5
    codes, s32, b32, _, _ = oracle.quantize(v, 32, 2)
    assert s32[0, 0] == np.float32(2.5) / np.float32(-3.0)
    assert b32[0, 0] == np.float32(2.5)
    assert codes[0, 0] == 0 and codes[0, 1] == 3


# ---------------------------------------------------- round-trip bound (P-4)
@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("g", GROUPS)
def test_roundtrip_bound(bits, g):
    """|w - w_hat| <= c*|s| + 2^-8 (q|s| + |b|): c = 1/2 below the top code,
    1 at the top code (the clamp and the edge/q0 rescale), plus the bf16
    narrowing of s and b."""
    w = synth.weight((64, 4 * g), seed=bits * 7 + g)
    codes, s32, b32, s16, b16 = oracle.quantize(w, g, bits)
    w_hat = oracle.dequantize(oracle.pack(codes, bits), s16, b16, w.shape[1],
                              g, bits)
    nb = (1 << bits) - 1
    s = np.repeat(np.abs(s32.astype(np.float64)), g, axis=1)
    b = np.repeat(np.abs(b32.astype(np.float64)), g, axis=1)
    c = np.where(codes == nb, 1.0, 0.5)
    bound = c * s + 2.0 ** -8 * (codes * s + b)
    err = np.abs(w.astype(np.float64) - w_hat)
    assert np.all(err <= bound * (1 + 1e-12)), float((err - bound).max())


def test_bits8_near_identity():
    """At 8 bits every reconstruction is within 2.5 quantization steps
    (range/255) of the input, i.e. within 1% of the group's range: one half
    step of rounding, one more at the clamped top code, and the bf16
    narrowing of scale (up to 255 * 2^-9 steps) and bias."""
    w = synth.weight((128, 512), seed=3)
    codes, s32, b32, s16, b16 = oracle.quantize(w, 64, 8)
    w_hat = oracle.dequantize(oracle.pack(codes, 8), s16, b16, 512, 64, 8)
    rng = w.reshape(128, 8, 64).max(-1) - np.minimum(
        w.reshape(128, 8, 64).min(-1), 0)
    err = np.abs(w - w_hat).reshape(128, 8, 64).max(-1)
    assert np.all(err <= rng / 255 * 2.5)
    assert np.all(err <= 0.01 * rng)


# ------------------------------------------------------- brute force (P-5)
def _exact_qmv(x_bits, w_q, s16, b16, K, g, bits):
    codes = decode_words(w_q, K, bits)
    N = codes.shape[0]
    M = x_bits.shape[0]
    y = [[Fraction(0)] * N for _ in range(M)]
    y_fold = [[Fraction(0)] * N for _ in range(M)]
    for m in range(M):
        xs = [_bf16_exact(h) for h in x_bits[m]]
        for n in range(N):
            acc = Fraction(0)
            fold = Fraction(0)
            for gi in range(K // g):
                s = _bf16_exact(s16[n, gi])
                b = _bf16_exact(b16[n, gi])
                qx = sum((int(codes[n, k]) * xs[k]
                          for k in range(gi * g, gi * g + g)), Fraction(0))
                sx = sum(xs[gi * g:gi * g + g], Fraction(0))
                fold += s * qx + b * sx
                for k in range(gi * g, gi * g + g):
                    acc += (s * int(codes[n, k]) + b) * xs[k]
            y[m][n] = acc
            y_fold[m][n] = fold
    return y, y_fold


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("g", GROUPS)
def test_qmv_brute_force_rational(bits, g):
    N, K, M = 4, 128, 2
    w = synth.weight((N, K), seed=bits + g)
    x = synth.activation_bf16((M, K), seed=bits * g)
    w_q, s16, b16 = oracle.quantize_pack(w, g, bits)
    y = oracle.qmv(x, w_q, s16, b16, g, bits)
    exact, fold = _exact_qmv(x, w_q, s16, b16, K, g, bits)
    for m in range(M):
        for n in range(N):
            assert exact[m][n] == fold[m][n]
            assert abs(Fraction(float(y[m, n])) - exact[m][n]) <= \
                Fraction(1, 10**12) * (1 + abs(exact[m][n]))


# ------------------------------------------------------- addressing (P-6)
@pytest.mark.parametrize("bits", BITS)
def test_qmv_one_hot_and_ones(bits):
    N, K, g = 3, 64, 32
    w = synth.weight((N, K), seed=11 * bits)
    w_q, s16, b16 = oracle.quantize_pack(w, g, bits)
    codes = decode_words(w_q, K, bits)
    s = synth.bf16_bits_to_f32(s16).astype(np.float64)
    b = synth.bf16_bits_to_f32(b16).astype(np.float64)
    one = synth.f32_to_bf16_bits(np.ones(1, np.float32))[0]
    x = np.zeros((K, K), np.uint16)
    x[np.arange(K), np.arange(K)] = one
    y = oracle.qmv(x, w_q, s16, b16, g, bits)  # row k of y: column k of W_hat
    for k in range(K):
        col = s[:, k // g] * codes[:, k] + b[:, k // g]
        np.testing.assert_array_equal(y[k], col)
    ones = np.full((1, K), one, np.uint16)
    y1 = oracle.qmv(ones, w_q, s16, b16, g, bits)[0]
    rows = [sum(s[n, k // g] * float(codes[n, k]) + b[n, k // g]
                for k in range(K)) for n in range(N)]
    np.testing.assert_allclose(y1, rows, rtol=1e-14, atol=0)


def test_qmv_rows_matches_full():
    w = synth.weight((40, 256), seed=5)
    x = synth.activation_bf16((3, 256), seed=6)
    w_q, s16, b16 = oracle.quantize_pack(w, 64, 4)
    full = oracle.qmv(x, w_q, s16, b16, 64, 4)
    rows = np.array([0, 7, 39, 12])
    np.testing.assert_array_equal(
        oracle.qmv_rows(x, w_q, s16, b16, 64, 4, rows), full[:, rows])


# ------------------------------------------------------ transpose=False (qvm)
@pytest.mark.parametrize("bits", (3, 4, 8))
def test_qvm_brute_force(bits):
    K, N, g, M = 6, 64, 32, 2
    w = synth.weight((K, N), seed=bits)     # W [K, N], quantized along N
    x = synth.activation_bf16((M, K), seed=bits + 1)
    w_q, s16, b16 = oracle.quantize_pack(w, g, bits)
    y = oracle.qvm(x, w_q, s16, b16, N, g, bits)
    codes = decode_words(w_q, N, bits)
    for m in range(M):
        for n in range(N):
            exact = sum(_bf16_exact(x[m, k]) * (
                _bf16_exact(s16[k, n // g]) * int(codes[k, n]) +
                _bf16_exact(b16[k, n // g])) for k in range(K))
            assert abs(Fraction(float(y[m, n])) - exact) <= \
                Fraction(1, 10**12) * (1 + abs(exact))


# -------------------------------------------------------- FFN tail and gather
def _w_hat_pages(w_q, s16, b16, K, g, bits):
    codes = decode_words(w_q, K, bits).astype(np.float64)
    s = np.repeat(synth.bf16_bits_to_f32(s16).astype(np.float64), g, axis=1)
    b = np.repeat(synth.bf16_bits_to_f32(b16).astype(np.float64), g, axis=1)
    return s * codes + b


@pytest.mark.parametrize("bits", (4, 8))
def test_silu_gate_resid_against_torch_silu(bits):
    import torch
    N, K, g = 16, 256, 64
    w_q, s16, b16 = oracle.quantize_pack(synth.weight((N, K), 2), g, bits)
    gate = synth.activation_bf16((K,), 0)
    up = synth.activation_bf16((K,), 1)
    xr = synth.activation_bf16((N,), 101)
    y = oracle.silu_gate_resid(gate, up, xr, w_q, s16, b16, g, bits)
    g64 = torch.from_numpy(synth.bf16_bits_to_f32(gate).astype(np.float64))
    u64 = torch.from_numpy(synth.bf16_bits_to_f32(up).astype(np.float64))
    h = (torch.nn.functional.silu(g64) * u64).numpy()
    W = _w_hat_pages(w_q, s16, b16, K, g, bits)
    ref = synth.bf16_bits_to_f32(xr).astype(np.float64) + W @ h
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)
    y0 = oracle.silu_gate_resid(gate, up, None, w_q, s16, b16, g, bits)
    np.testing.assert_allclose(y0, W @ h, rtol=1e-12, atol=1e-12)


def test_silu_gate_resid_zero_up_or_gate_is_resid():
    N, K, g = 8, 128, 32
    w_q, s16, b16 = oracle.quantize_pack(synth.weight((N, K), 2), g, 8)
    xr = synth.activation_bf16((N,), 101)
    z = np.zeros(K, np.uint16)
    a = synth.activation_bf16((K,), 3)
    xr64 = synth.bf16_bits_to_f32(xr).astype(np.float64)
    np.testing.assert_array_equal(
        oracle.silu_gate_resid(a, z, xr, w_q, s16, b16, g, 8), xr64)
    np.testing.assert_array_equal(
        oracle.silu_gate_resid(z, a, xr, w_q, s16, b16, g, 8), xr64)


def test_gather_is_per_pair_product():
    E, N, K, g, bits = 5, 8, 128, 64, 4
    w = np.stack([synth.weight((N, K), seed=e) for e in range(E)])
    packs = [oracle.quantize_pack(w[e], g, bits) for e in range(E)]
    w_q = np.stack([p[0] for p in packs])
    s16 = np.stack([p[1] for p in packs])
    b16 = np.stack([p[2] for p in packs])
    x = synth.activation_bf16((3, 1, K), seed=9)
    lhs = np.array([2, 0, 1, 1, 2], np.uint32)
    rhs = np.array([4, 4, 0, 3, 1], np.uint32)
    y = oracle.gather_qmv(x, w_q, s16, b16, lhs, rhs, g, bits)
    assert y.shape == (5, 1, N)
    for p in range(5):
        W = _w_hat_pages(w_q[rhs[p]], s16[rhs[p]], b16[rhs[p]], K, g, bits)
        xv = synth.bf16_bits_to_f32(x[lhs[p], 0]).astype(np.float64)
        np.testing.assert_allclose(y[p, 0], W @ xv, rtol=1e-12, atol=1e-12)
    with pytest.raises(ValueError):
        oracle.gather_qmv(x, w_q, s16, b16, lhs, np.array([0, 0, 0, 0, 5],
                                                          np.uint32), g, bits)


def test_bf16_narrowing_matches_torch():
    import torch
    rng = np.random.default_rng(0)
    v = (rng.standard_normal(2000) * 10.0 ** rng.integers(-30, 30, 2000))
    v = v.astype(np.float32)
    # exact ties (low half 0x8000) with even and odd kept halves, and
    # values one ulp either side of a tie
    hi = rng.integers(0x0080, 0x7F00, 200).astype(np.uint32) << 16
    lows = np.array([0x8000, 0x7FFF, 0x8001], np.uint32)
    ties = (hi[:, None] | lows[None, :]).ravel().view(np.float32)
    v = np.concatenate([v, ties, -ties])
    ours = np.array([oracle.bf16_from_f32(float(t)) for t in v], np.uint16)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy()
    np.testing.assert_array_equal(ours, ref.view(np.uint16))


@pytest.mark.parametrize("M", (2, 3))
def test_gather_rows_per_entry_brute_force(M):
    """Gather with M > 1 rows per batch entry: x is [Bx, M, K], y is
    [P, M, N], and y[p, m] is row m of x[lhs[p]] against expert rhs[p]
    (quantized.h, adjust_matrix_offsets for the gather kernels: x moves by
    the lhs batch stride M*K, the output slot by N*M).  Every y[p, m, n] is
    an explicit dot product over the page-decoded weight.  Row m of each
    batch entry is made distinctive (one-hot at a row-dependent column plus
    noise) so that a wrong x or y stride changes the answer by at least one
    whole weight."""
    E, N, K, g, bits, Bx = 4, 6, 128, 32, 4, 3
    w = np.stack([synth.weight((N, K), seed=40 + e) for e in range(E)])
    packs = [oracle.quantize_pack(w[e], g, bits) for e in range(E)]
    w_q = np.stack([p[0] for p in packs])
    s16 = np.stack([p[1] for p in packs])
    b16 = np.stack([p[2] for p in packs])
    x = synth.activation_bf16((Bx, M, K), seed=77)
    one = synth.f32_to_bf16_bits(np.array([64.0], np.float32))[0]
    for bi in range(Bx):
        for m in range(M):
            x[bi, m, (5 * bi + 17 * m) % K] = one
    lhs = np.array([2, 0, 1, 2, 0, 1, 1], np.uint32)
    rhs = np.array([3, 3, 0, 1, 2, 0, 3], np.uint32)
    y = oracle.gather_qmv(x, w_q, s16, b16, lhs, rhs, g, bits)
    assert y.shape == (lhs.size, M, N)
    for p in range(lhs.size):
        W = _w_hat_pages(w_q[rhs[p]], s16[rhs[p]], b16[rhs[p]], K, g, bits)
        for m in range(M):
            xv = synth.bf16_bits_to_f32(x[lhs[p], m]).astype(np.float64)
            for n in range(N):
                ref = sum(W[n, k] * xv[k] for k in range(K))
                assert abs(y[p, m, n] - ref) <= 1e-12 * (1.0 + abs(ref)), \
                    (p, m, n, y[p, m, n], ref)
