"""fp64 CPU oracle for rotary position embedding (RoPE) as the first step of
the fused FP8 producer pass: x -> RoPE(x) -> H D -> per-block FP8 codes.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import this module; the HIP path never does.

Source and readings.  The "FlashAttention-3" page, section "为什么 Hadamard
适合放到内核里", says only that the Hadamard transform, itself bandwidth-bound,
can be fused with a pre-processing stage such as RoPE that is already
bandwidth-bound.  It gives no formula for RoPE, so RoPE is taken from its
published definition (Su et al., "RoFormer: Enhanced Transformer with Rotary
Position Embedding", 2021): the head dimension is split into d/2 pairs; pair
i at position n is rotated by the angle n * theta_i with

    theta_i = base^(-2 i / d),   i = 0 .. d/2 - 1,   base = 10000 by default,
    (a, b) -> (a cos(n theta_i) - b sin(n theta_i),  a sin(n theta_i) + b cos(n theta_i)).

Two pairings are in common use and both are provided:
  * "interleaved": pair i is (x[2i], x[2i+1])  (the RoFormer paper's form);
  * "half":        pair i is (x[i], x[i + d/2])  (the split-halves form).
Position n of row r of a [..., N, d] tensor is pos_offset + r.  Readings
(not on the pages): RoPE is applied to Q and K before the rotation H D (it
belongs to the model, incoherent processing to the quantisation); V is not
position-encoded.  Since H D is orthogonal and shared by Q and K, the
scores of the rotated, position-encoded Q and K are those of RoPE(Q) and
RoPE(K).
"""
from __future__ import annotations

import numpy as np

STYLES = ("interleaved", "half")


def rope_angles(n_rows, d, base=10000.0, pos_offset=0):
    """Angles n * theta_i, fp64 [n_rows, d/2], for positions pos_offset .. pos_offset + n_rows - 1."""
    if d % 2:
        raise ValueError("d must be even")
    i = np.arange(d // 2, dtype=np.float64)
    theta = np.power(float(base), -2.0 * i / d)
    pos = np.arange(n_rows, dtype=np.float64) + float(pos_offset)
    return pos[:, None] * theta[None, :]


def _pair_index(d, style):
    """(first, second) channel indices of the d/2 pairs."""
    if style == "interleaved":
        return np.arange(0, d, 2), np.arange(1, d, 2)
    if style == "half":
        return np.arange(d // 2), np.arange(d // 2, d)
    raise ValueError(f"unknown RoPE style {style!r}")


def rope(x, base=10000.0, pos_offset=0, style="interleaved"):
    """RoPE of the rows of x[..., N, d] (fp64 result)."""
    x = np.asarray(x, dtype=np.float64)
    n, d = x.shape[-2:]
    ang = rope_angles(n, d, base, pos_offset)
    c, s = np.cos(ang), np.sin(ang)
    i0, i1 = _pair_index(d, style)
    a, b = x[..., i0], x[..., i1]
    out = np.empty_like(x)
    out[..., i0] = a * c - b * s
    out[..., i1] = a * s + b * c
    return out


def rope_hadamard_rotate_quant(x, signs=None, block_rows=128, fmt="e4m3", base=10000.0, pos_offset=0,
                               style="interleaved"):
    """The fused producer pass: RoPE, then (signs given) x~ = (H / sqrt(d)) D x,
    then per-block FP8 codes.  Returns (codes [..., N, d], scales, y) as
    oracle.fp8.hadamard_rotate_quant does."""
    from .fp8 import hadamard_rotate_quant
    return hadamard_rotate_quant(rope(x, base, pos_offset, style), signs, block_rows, fmt=fmt)
