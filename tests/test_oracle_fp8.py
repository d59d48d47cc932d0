"""Pins for the FP8 side of the oracle: the E4M3 codec against the format's
closed forms and torch's float8_e4m3fn, the Hadamard matrix against its
closed form and a butterfly transform, the rotation's orthogonality, and the
block quantiser and FP8 simulation on inputs where quantisation is lossless."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import (attention, block_quantize, dequantize, e4m3_decode, e4m3_encode,
                    hadamard_rotate_quant, rotate, sylvester_hadamard)


# ---------------------------------------------------------------- E4M3 codec
# Closed-form values of the OCP E4M3FN encoding (1.4.3, bias 7).
KNOWN = {
    0x00: 0.0, 0x01: 2.0 ** -9, 0x02: 2.0 ** -8, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6,
    0x38: 1.0, 0x39: 1.125, 0x3C: 1.5, 0x3F: 1.875, 0x40: 2.0, 0x70: 128.0, 0x78: 256.0,
    0x7E: 448.0, 0x80: -0.0, 0xB8: -1.0, 0xFE: -448.0,
}


def test_decode_known_values():
    for code, val in KNOWN.items():
        got = float(e4m3_decode(np.uint8(code)))
        assert got == val and math.copysign(1, got) == math.copysign(1, val), hex(code)
    assert np.isnan(e4m3_decode(np.uint8(0x7F))) and np.isnan(e4m3_decode(np.uint8(0xFF)))


def test_decode_exhaustive_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert set(np.nonzero(nan)[0]) == {0x7F, 0xFF}
    np.testing.assert_array_equal(np.isnan(ours), nan)
    np.testing.assert_array_equal(ours[~nan], ref[~nan])


def test_decode_is_monotone_and_bounded():
    pos = e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)
    assert pos.max() == 448.0


def test_encode_round_trip_on_representable_values():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = e4m3_decode(codes)
    np.testing.assert_array_equal(e4m3_encode(vals), codes)


# ---------------------------------------------------------------- E5M2 codec
# Closed-form values of the OCP E5M2 encoding (1.5.2, bias 15).
KNOWN_E5M2 = {
    0x00: 0.0, 0x01: 2.0 ** -16, 0x02: 2.0 ** -15, 0x03: 3 * 2.0 ** -16, 0x04: 2.0 ** -14,
    0x3C: 1.0, 0x3D: 1.25, 0x3E: 1.5, 0x3F: 1.75, 0x40: 2.0, 0x78: 32768.0, 0x7B: 57344.0,
    0x7C: math.inf, 0x80: -0.0, 0xBC: -1.0, 0xFB: -57344.0, 0xFC: -math.inf,
}


def test_e5m2_decode_known_values():
    for code, val in KNOWN_E5M2.items():
        got = float(oracle.e5m2_decode(np.uint8(code)))
        assert got == val and math.copysign(1, got) == math.copysign(1, val), hex(code)
    for code in (0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF):
        assert np.isnan(oracle.e5m2_decode(np.uint8(code)))


def test_e5m2_decode_exhaustive_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e5m2_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e5m2).to(torch.float64).numpy()
    nan = np.isnan(ref)
    np.testing.assert_array_equal(np.isnan(ours), nan)
    np.testing.assert_array_equal(ours[~nan], ref[~nan])


def test_e5m2_encode_round_trip_ties_and_saturation():
    pos = oracle.e5m2_decode(np.arange(0x7C, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0) and pos.max() == 57344.0
    finite = np.array([c for c in range(256) if (c & 0x7F) < 0x7C], np.uint8)
    np.testing.assert_array_equal(oracle.e5m2_encode(oracle.e5m2_decode(finite)), finite)
    cases = {1.125: 0x3C, 1.375: 0x3E, 1.625: 0x3E, 1.875: 0x40, 2.0 ** -17: 0x00,
             3 * 2.0 ** -17: 0x02, 60000.0: 0x7B, 1e9: 0x7B, -1e9: 0xFB, -1.125: 0xBC}
    for x, code in cases.items():
        assert int(oracle.e5m2_encode(np.float64(x))) == code, x
    assert int(oracle.e5m2_encode(np.float64(np.nan))) == 0x7F


def test_e5m2_encode_matches_torch_after_clamp():
    x = np.random.default_rng(5).standard_normal(20000) * np.exp2(np.random.default_rng(6).uniform(-20, 17, 20000))
    xc = np.clip(x, -57344.0, 57344.0)
    ref = torch.from_numpy(xc).to(torch.float8_e5m2).view(torch.uint8).numpy()
    np.testing.assert_array_equal(oracle.e5m2_encode(xc), ref)


def test_e5m2_block_max_encodes_to_57344():
    x = np.random.default_rng(7).standard_normal((2, 300, 64)) * 3
    codes, scales, _ = block_quantize(x, 128, fmt="e5m2")
    for b in range(3):
        blk = codes[:, 128 * b:128 * (b + 1)]
        xb = x[:, 128 * b:128 * (b + 1)]
        amax = np.abs(xb).max(axis=(-2, -1))
        np.testing.assert_allclose(scales[:, b], amax / 57344.0, rtol=0, atol=0)
        for h in range(2):
            i = np.unravel_index(np.argmax(np.abs(xb[h])), xb[h].shape)
            assert blk[h][i] in (0x7B, 0xFB)
    back = dequantize(codes, scales, 128, fmt="e5m2")
    # 2 mantissa bits: relative error at most 2^-3 for normal values
    big = np.abs(x) > np.abs(x).max() * 2.0 ** -14
    assert np.all(np.abs(back - x)[big] <= np.abs(x)[big] * 2.0 ** -3 + 1e-12)


def test_encode_ties_to_even_and_saturation():
    cases = {1.0625: 0x38, 1.1875: 0x3A, 2.0 ** -10: 0x00, 3 * 2.0 ** -10: 0x02,
             1.9375: 0x40, 15 * 2.0 ** -10: 0x08, 460.0: 0x7E, 1e6: 0x7E, -1e6: 0xFE,
             -1.0625: 0xB8, 449.0: 0x7E, 432.0: 0x7E, 424.0: 0x7D}
    for x, code in cases.items():
        assert int(e4m3_encode(np.float64(x))) == code, x
    assert int(e4m3_encode(np.float64(np.nan))) == 0x7F


def test_encode_matches_torch_after_clamp():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * s for s in (1e-3, 0.05, 1, 30, 300)])
    x = np.clip(x, -448, 448)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(e4m3_encode(x), ref)


def test_encode_error_bound():
    # Round to nearest: |x - decode(encode(x))| <= half the local spacing.
    x = np.random.default_rng(1).uniform(-448, 448, 50000)
    err = np.abs(e4m3_decode(e4m3_encode(x)) - x)
    ax = np.abs(x)
    spacing = np.where(ax < 2 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(ax, 2 ** -6))) - 3))
    assert np.all(err <= spacing / 2 + 1e-12)


# ---------------------------------------------------------------- Hadamard
@pytest.mark.parametrize("d", [1, 2, 8, 64, 128, 256])
def test_hadamard_closed_form_and_orthogonality(d):
    h = sylvester_hadamard(d)
    i = np.arange(d)
    pop = np.vectorize(lambda t: bin(t).count("1"))(i[:, None] & i[None, :])
    np.testing.assert_array_equal(h, (-1.0) ** pop)
    np.testing.assert_array_equal(h @ h.T, d * np.eye(d))


def test_hadamard_rejects_non_power_of_two():
    with pytest.raises(ValueError):
        sylvester_hadamard(96)


def _fwht(x):
    """In-place butterfly fast Walsh-Hadamard transform over the last axis."""
    x = np.array(x, dtype=np.float64)
    d = x.shape[-1]
    hlen = 1
    while hlen < d:
        y = x.reshape(*x.shape[:-1], d // (2 * hlen), 2, hlen)
        a, b = y[..., 0, :].copy(), y[..., 1, :].copy()
        y[..., 0, :], y[..., 1, :] = a + b, a - b
        x = y.reshape(*x.shape)
        hlen *= 2
    return x


@pytest.mark.parametrize("d", [64, 128, 256])
def test_rotation_equals_butterfly_fwht(d):
    rng = np.random.default_rng(d)
    x = rng.standard_normal((5, 7, d))
    signs = rng.integers(0, 2, d) * 2 - 1
    np.testing.assert_allclose(rotate(x, signs), _fwht(x * signs) / math.sqrt(d), atol=1e-12)


def test_rotation_preserves_inner_products_and_norms():
    rng = np.random.default_rng(3)
    d = 128
    q, k = rng.standard_normal((40, d)), rng.standard_normal((30, d))
    q[:, 5] *= 20
    k[:, 5] *= 20
    signs = rng.integers(0, 2, d) * 2 - 1
    qr, kr = rotate(q, signs), rotate(k, signs)
    np.testing.assert_allclose(qr @ kr.T, q @ k.T, rtol=0, atol=1e-10)
    np.testing.assert_allclose(np.linalg.norm(qr, axis=1), np.linalg.norm(q, axis=1), rtol=1e-14)
    # different sign vectors for Q and K break the identity
    other = -signs
    other[0] = signs[0]
    assert np.abs(rotate(q, signs) @ rotate(k, other).T - q @ k.T).max() > 1.0


def test_rotation_spreads_an_outlier_channel():
    d = 128
    x = np.zeros((1, d))
    x[0, 17] = 20.0
    signs = np.ones(d)
    xr = rotate(x, signs)
    np.testing.assert_allclose(np.abs(xr), 20.0 / math.sqrt(d), rtol=1e-14)


# ---------------------------------------------------------------- block quantisation
def test_block_scale_and_max_element():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((2, 3, 300, 64))       # 300 rows: blocks of 128, 128, 44
    codes, scales, y = block_quantize(x, 128)
    assert scales.shape == (2, 3, 3)
    for b, (r0, r1) in enumerate([(0, 128), (128, 256), (256, 300)]):
        blk = x[:, :, r0:r1, :]
        amax = np.abs(blk).max(axis=(-2, -1))
        np.testing.assert_allclose(scales[..., b], amax / 448.0, rtol=1e-15)
        cb = codes[:, :, r0:r1, :].reshape(2, 3, -1)
        flat = blk.reshape(2, 3, -1)
        idx = np.abs(flat).argmax(-1)
        top = np.take_along_axis(cb, idx[..., None], -1)[..., 0]
        sgn = np.take_along_axis(flat, idx[..., None], -1)[..., 0] < 0
        np.testing.assert_array_equal(top, np.where(sgn, 0xFE, 0x7E))
        assert np.all(np.abs(e4m3_decode(cb)) <= 448)


def test_exact_rounding_ties_resolve_to_even():
    """Values lying exactly on an E4M3 rounding midpoint round to the even
    code.  amax = 63/16: x = 153/16384 gives x * 448 / amax = 17/16 exactly
    (between 1.0 = 0x38 and 1.125 = 0x39) and x = 225/8192 gives 25/8
    (between 3.0 = 0x44 and 3.25 = 0x45).  amax = 3.125: x = 0.002288818359375
    gives 0.328125 (between 0x2A and 0x2B); multiplying by a rounded 448/amax
    instead would land just above that midpoint and give 0x2B."""
    x = np.zeros((2, 1, 128, 8))
    x[0, 0, 0, 0] = 63 / 16
    x[0, 0, 1, 1] = 153 / 16384
    x[0, 0, 2, 2] = -153 / 16384
    x[0, 0, 3, 3] = 225 / 8192
    x[1, 0, 0, 0] = 3.125
    x[1, 0, 5, 5] = 0.002288818359375
    codes, scales, y = block_quantize(x, 128)
    assert y[0, 0, 1, 1] == 17 / 16 and y[0, 0, 3, 3] == 25 / 8 and y[1, 0, 5, 5] == 0.328125
    assert codes[0, 0, 1, 1] == 0x38 and codes[0, 0, 2, 2] == 0xB8 and codes[0, 0, 3, 3] == 0x44
    assert codes[1, 0, 5, 5] == 0x2A
    assert codes[0, 0, 0, 0] == 0x7E and codes[1, 0, 0, 0] == 0x7E


def test_zero_block_gets_zero_scale():
    # s = amax / 448 with amax = 0: the block dequantises to exact zeros
    x = np.zeros((1, 1, 256, 8))
    x[0, 0, 200, 3] = -2.5
    codes, scales, _ = block_quantize(x, 128)
    assert scales[0, 0, 0] == 0.0 and np.all(e4m3_decode(codes[0, 0, :128]) == 0)
    assert scales[0, 0, 1] == 2.5 / 448
    np.testing.assert_array_equal(dequantize(codes, scales, 128), x)


def _grid_exact(shape, seed, block_rows=128):
    """Inputs that block quantisation represents exactly: E4M3 grid values
    times a power-of-two block scale, with one +-448 per block."""
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 0x7F, shape).astype(np.uint8) | (rng.integers(0, 2, shape) << 7).astype(np.uint8)
    vals = e4m3_decode(codes)
    n = shape[-2]
    for r0 in range(0, n, block_rows):
        vals[..., r0, 0] = 448.0
        vals[..., r0:r0 + block_rows, :] *= 2.0 ** rng.integers(-12, -4)
    return vals


def test_quantisation_is_lossless_on_grid_inputs():
    x = _grid_exact((2, 2, 260, 32), 5)
    for t in (False, True):
        codes, scales, _ = hadamard_rotate_quant(x, None, 128, transpose_out=t)
        if t:
            assert codes.shape == (2, 2, 32, 260)
        np.testing.assert_array_equal(dequantize(codes, scales, 128, transposed=t), x)


def test_fp8_simulation_equals_exact_when_lossless():
    """Rotated Q~, K~ and V on the E4M3 grid: the simulated FP8 attention then
    equals the exact attention of the unrotated inputs (orthogonality)."""
    B, H, N, d = 1, 2, 256, 64
    rng = np.random.default_rng(6)
    signs = rng.integers(0, 2, d) * 2 - 1
    qt, kt, v = (_grid_exact((B, H, N, d), s) for s in (7, 8, 9))
    h = sylvester_hadamard(d) / math.sqrt(d)
    q = (qt @ h) * signs            # inverse of x~ = H D x  is  x = D H x~
    k = (kt @ h) * signs
    np.testing.assert_allclose(rotate(q, signs), qt, atol=1e-12)
    scale = 1 / math.sqrt(d)
    o_sim, lse_sim = oracle.attention_fp8_simulated(q, k, v, signs, scale)
    o_ex, lse_ex = attention(q, k, v, scale)
    np.testing.assert_allclose(o_sim, o_ex, rtol=0, atol=1e-9)
    np.testing.assert_allclose(lse_sim, lse_ex, rtol=0, atol=1e-9)


def test_fp8_simulation_error_is_small_but_nonzero():
    B, H, N, d = 1, 1, 256, 64
    rng = np.random.default_rng(10)
    q, k, v = (rng.standard_normal((B, H, N, d)) for _ in range(3))
    signs = rng.integers(0, 2, d) * 2 - 1
    o_ex, _ = attention(q, k, v, 0.125)
    o_sim, _ = oracle.attention_fp8_simulated(q, k, v, signs, 0.125)
    err = oracle.rel_rms(o_sim, o_ex)
    # E4M3 keeps 3 mantissa bits: per-value relative error ~2-3 %.
    assert 0.005 < err < 0.1
    o_p, lse_p = oracle.attention_fp8_simulated(q, k, v, signs, 0.125, quantize_p=True)
    assert 0 < oracle.rel_rms(o_p, o_sim) < 0.06
    # rounded P in the row sums: l moves by at most the E4M3 relative rounding
    # (2^-4 for values in the normal range, which the gain of 256 keeps the
    # row maximum and everything within 2^-14 of it in)
    _, lse_sim = oracle.attention_fp8_simulated(q, k, v, signs, 0.125)
    dl = np.abs(lse_p - lse_sim)
    assert 0 < dl.max() <= np.log1p(2.0 ** -4)


def test_fp8_simulation_quantized_p_keeps_constant_v():
    # with the rounded P in both the numerator and the row sums, the output is
    # a convex combination of V rows: a constant V comes out unchanged (V's
    # codes are all 448 and its scale |c| / 448, so V dequantises exactly)
    B, H, N, d = 1, 2, 200, 64
    rng = np.random.default_rng(11)
    q, k = (rng.standard_normal((B, H, N, d)) * 3 for _ in range(2))
    v = np.full((B, H, N, d), -1.75)
    signs = rng.integers(0, 2, d) * 2 - 1
    for causal in (False, True):
        o_p, _ = oracle.attention_fp8_simulated(q, k, v, signs, 0.125, causal=causal, quantize_p=True)
        np.testing.assert_allclose(o_p, v, rtol=1e-13, atol=0)


def test_quantized_probabilities_closed_forms():
    """The rounded weights of the FP8 second product on hand-computed rows
    (one block).  Scores 0 and ln 0.3 (log2: 0 and -1.737): M = 0,
    P' = E4M3(256) = 256 and E4M3(76.8) = 80 (spacing 8 in [64, 128)), so
    P~ = (1, 80/256).  A V block scale of 0.75 of the largest makes the
    second gain 192: E4M3(57.6) = 56 (spacing 4 in [32, 64)), P~ = 56/192.
    A zero scale counts as the largest one."""
    s = np.array([[0.0, np.log(0.3)]])
    pq, m = oracle.quantized_probabilities(s, np.array([2.0, 2.0]))
    assert m[0] == 0.0
    np.testing.assert_array_equal(pq, [[1.0, 80 / 256]])
    pq, _ = oracle.quantized_probabilities(s, np.array([2.0, 1.5]))
    np.testing.assert_array_equal(pq, [[1.0, 56 / 192]])
    pq, _ = oracle.quantized_probabilities(s, np.array([2.0, 0.0]))
    np.testing.assert_array_equal(pq, [[1.0, 80 / 256]])
    pq, _ = oracle.quantized_probabilities(s, np.array([0.0, 0.0]))
    np.testing.assert_array_equal(pq, [[1.0, 80 / 256]])
    # the reference is the row maximum rounded UP to a power of two: scores
    # log2 0.7 and -inf (masked) give M = 0, P' = E4M3(179.2) = 176 (spacing
    # 16 in [128, 256)); the masked key weighs exactly 0
    pq, m = oracle.quantized_probabilities(np.array([[np.log(0.7), -np.inf]]), np.array([1.0, 1.0]))
    assert m[0] == 0.0
    np.testing.assert_array_equal(pq, [[176 / 256, 0.0]])
    # weights far below the row maximum fall into E4M3's subnormals (spacing
    # 2^-9 of the gained value): 2^-12 * 256 = 2^-4 is still normal,
    # 2^-17.5 * 256 = 0.707 * 2^-9 rounds up to one subnormal step and
    # 2^-18.5 * 256 = 0.354 * 2^-9 to zero
    def w2(t2):
        return oracle.quantized_probabilities(np.array([[0.0, t2 * np.log(2.0)]]), np.array([1.0, 1.0]))[0][0, 1]
    assert w2(-12.0) == 2.0 ** -12
    assert w2(-17.5) == 2.0 ** -17
    assert w2(-18.5) == 0.0


def test_quantized_probabilities_running_reference():
    """Blocks of 2 keys: the weights of block 0 are rounded against the
    running maximum after block 0, not the row's final maximum.  Block 0
    holds t = -16.3 and -16 (log2), block 1 holds 0 and -inf.  M^0 = -16:
    2^-0.3 * 256 = 207.9 rounds to 208, weight 208/256 * 2^-16.  Against the
    final reference M = 0 it would be the subnormal 2^-16.3 * 256 = 0.0032,
    rounded to 2 * 2^-9, weight 2^-16.  In the normal range the two agree
    (the grid is the same up to a power of two)."""
    t = np.array([[-16.3, -16.0, 0.0, -np.inf]])
    pq, m = oracle.quantized_probabilities(t * np.log(2.0), np.ones(4), block=2)
    assert m[0] == 0.0
    np.testing.assert_array_equal(pq, [[208 / 256 * 2.0 ** -16, 2.0 ** -16, 1.0, 0.0]])
    pq1, _ = oracle.quantized_probabilities(t * np.log(2.0), np.ones(4), block=4)
    assert pq1[0, 0] == 2.0 ** -16
    t = np.array([[-2.5, -2.0, 0.0, -1.0]])
    pa, _ = oracle.quantized_probabilities(t * np.log(2.0), np.ones(4), block=2)
    pb, _ = oracle.quantized_probabilities(t * np.log(2.0), np.ones(4), block=4)
    np.testing.assert_array_equal(pa, pb)


def test_quantized_probabilities_power_of_two_shift():
    """Shifting a row's scores by k ln 2 (k an integer) moves M by k and
    leaves the rounded weights unchanged: the grid is tied to powers of two,
    not to the exact maximum.  A non-integer shift changes them."""
    rng = np.random.default_rng(3)
    s = rng.standard_normal((5, 300)) * 3
    w = rng.uniform(0.2, 1.0, 300)
    for block in (7, 128, 300):
        pq, m = oracle.quantized_probabilities(s, w, block)
        for kk in (-3, 1, 7):
            pk, mk = oracle.quantized_probabilities(s + kk * np.log(2.0), w, block)
            np.testing.assert_array_equal(mk, m + kk)
            np.testing.assert_allclose(pk, pq, rtol=1e-12, atol=0)
        p_half, _ = oracle.quantized_probabilities(s + 0.5 * np.log(2.0), w, block)
        assert np.abs(p_half / np.exp(0.5 * np.log(2.0)) - pq).max() > 1e-3


def test_rel_rms():
    assert oracle.rel_rms([3.0, 4.0], [3.0, 4.0]) == 0.0
    assert oracle.rel_rms([3.0, 4.0 + 5.0], [3.0, 4.0]) == pytest.approx(1.0)


@pytest.mark.parametrize("frac", [0.0, 0.005, 0.02, 0.05])
def test_rotation_lowers_simulated_error_with_outliers(frac):
    """Direction of the pages' claim that incoherent processing lowers the FP8
    error ("FlashAttention-3" page, section "FP8 路径与低精度误差", about 2.6x
    against a baseline): with outlier channels in Q and K the simulated
    error drops several-fold when Q and K are rotated first, for per-block
    (128 rows) and per-tensor (one scale per head) quantisation alike; with
    no outliers the rotation changes little.  The magnitude is not pinned, and
    a single outlier channel (0.5 % of d = 128) is reported only: whether it
    hurts the unrotated codes depends on the draw (on 4 heads x 1024 rows of
    seed 11 the rotation is the worse of the two)."""
    from exact_attention_forward_06_amd.inputs import make_inputs, to_f64
    B, H, N, d = 1, 4, 256, 128      # four heads: one outlier channel's effect varies with the draw
    inp = make_inputs(B, H, N, d, "fp8", seed=11, outlier_frac=frac)
    q, k, v = (to_f64(inp[n]) for n in ("q", "k", "v"))
    signs = inp["signs"].numpy()
    s = 1 / np.sqrt(d)
    exact, _ = attention(q, k, v, s)
    for block_rows in (128, N):
        rot = oracle.rel_rms(oracle.attention_fp8_simulated(q, k, v, signs, s, block_rows=block_rows)[0], exact)
        unrot = oracle.rel_rms(oracle.attention_fp8_simulated(q, k, v, None, s, block_rows=block_rows)[0], exact)
        assert np.isfinite(rot) and np.isfinite(unrot)
        if frac == 0.0:
            assert 0.8 <= unrot / rot <= 1.25, (block_rows, rot, unrot)
        elif frac >= 0.02:
            assert unrot / rot >= 2.0, (block_rows, rot, unrot)
