"""Pins of the RoPE oracle (oracle.rope) against what the RoPE definition and
the mathematics fix, not against a retyping of its formula:

  * the complex form: pair i as z = a + i b becomes z * exp(i n theta_i),
    with theta_i computed here in plain Python from base^(-2i/d);
  * the relative-position property that defines RoPE: the score of a query at
    position m and a key at position n depends on m - n only, and equals the
    score of the unrotated query with the key rotated to position n - m;
  * each pair keeps its length (a rotation), position 0 is the identity, and
    at d = 2 the angle is the position itself (theta_0 = 1);
  * the two pairings are the same map up to a channel permutation;
  * composed with the orthogonal H D of the FP8 pre-pass, scores are those of
    the position-encoded Q and K.
Each plausible slip (a sign of sin, an exponent, a swapped pair, an off-by-one
position) fails at least one of these.
"""
import cmath
import math

import numpy as np
import pytest

from oracle.fp8 import rotate
from oracle.rope import rope, rope_angles, rope_hadamard_rotate_quant

STYLES = ["interleaved", "half"]


def _complex_rope(x, base, pos_offset, style):
    """Pure-Python complex-form RoPE of a 2-D array (rows = positions)."""
    n, d = x.shape
    out = np.empty_like(x, dtype=np.float64)
    for r in range(n):
        pos = pos_offset + r
        for i in range(d // 2):
            theta = base ** (-(2.0 * i) / d)
            if style == "interleaved":
                j0, j1 = 2 * i, 2 * i + 1
            else:
                j0, j1 = i, i + d // 2
            z = complex(float(x[r, j0]), float(x[r, j1])) * cmath.exp(1j * pos * theta)
            out[r, j0], out[r, j1] = z.real, z.imag
    return out


@pytest.mark.parametrize("style", STYLES)
@pytest.mark.parametrize("d,base,off", [(8, 10000.0, 0), (16, 500.0, 7), (64, 10000.0, 8000)])
def test_rope_equals_complex_form(style, d, base, off):
    x = np.random.default_rng(d).standard_normal((5, d))
    np.testing.assert_allclose(rope(x, base, off, style), _complex_rope(x, base, off, style),
                               rtol=0, atol=1e-11)


@pytest.mark.parametrize("style", STYLES)
def test_relative_position_property(style):
    d = 32
    rng = np.random.default_rng(1)
    q, k = rng.standard_normal((1, d)), rng.standard_normal((1, d))
    for m, n, t in [(3, 11, 5), (100, 2, 1000), (0, 0, 9)]:
        s = (rope(q, pos_offset=m, style=style) @ rope(k, pos_offset=n, style=style).T).item()
        s_shift = (rope(q, pos_offset=m + t, style=style) @ rope(k, pos_offset=n + t, style=style).T).item()
        s_rel = (q @ rope(k, pos_offset=n - m, style=style).T).item()
        assert abs(s - s_shift) <= 1e-10 * (1 + abs(s))
        assert abs(s - s_rel) <= 1e-10 * (1 + abs(s))
    # and it does depend on the offset (the rotation is not trivial)
    s1 = (q @ rope(k, pos_offset=1, style=style).T).item()
    s0 = (q @ k.T).item()
    assert abs(s1 - s0) > 1e-3


@pytest.mark.parametrize("style", STYLES)
def test_rotation_invariants(style):
    d = 16
    x = np.random.default_rng(2).standard_normal((40, d))
    y = rope(x, pos_offset=3, style=style)
    i0 = np.arange(0, d, 2) if style == "interleaved" else np.arange(d // 2)
    i1 = i0 + 1 if style == "interleaved" else i0 + d // 2
    np.testing.assert_allclose(x[:, i0] ** 2 + x[:, i1] ** 2, y[:, i0] ** 2 + y[:, i1] ** 2, rtol=1e-12)
    # position 0 (row 0 with no offset) is the identity
    np.testing.assert_array_equal(rope(x, style=style)[0], x[0])


def test_d2_angle_is_the_position():
    ang = rope_angles(6, 2, base=12345.0, pos_offset=4)
    np.testing.assert_array_equal(ang[:, 0], np.arange(4, 10, dtype=np.float64))
    x = np.array([[1.0, 0.0]] * 3)
    y = rope(x, pos_offset=1)
    for r in range(3):
        assert abs(y[r, 0] - math.cos(1 + r)) < 1e-15 and abs(y[r, 1] - math.sin(1 + r)) < 1e-15


def test_styles_are_a_permutation_of_each_other():
    d = 16
    x = np.random.default_rng(3).standard_normal((7, d))
    perm = np.empty(d, np.int64)      # half-split channel of interleaved channel c
    perm[0::2] = np.arange(d // 2)
    perm[1::2] = np.arange(d // 2) + d // 2
    y_half = rope(x, pos_offset=5, style="half")
    y_int = rope(x[:, perm], pos_offset=5, style="interleaved")
    np.testing.assert_allclose(y_int, y_half[:, perm], rtol=0, atol=1e-13)


def test_fused_pass_scores_are_rope_scores():
    d, n = 64, 20
    rng = np.random.default_rng(4)
    q, k = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    signs = rng.integers(0, 2, d) * 2 - 1
    qr, kr = rope(q, pos_offset=10), rope(k, pos_offset=10)
    s_ref = qr @ kr.T
    s_rot = rotate(qr, signs) @ rotate(kr, signs).T
    np.testing.assert_allclose(s_rot, s_ref, rtol=0, atol=1e-10)
    # the fused oracle rounds exactly those rotated values
    _, _, y = rope_hadamard_rotate_quant(q, signs, block_rows=128, pos_offset=10)
    amax = np.abs(rotate(qr, signs)).max()
    np.testing.assert_allclose(y, rotate(qr, signs) * 448 / amax, rtol=1e-14, atol=1e-12)
