"""fp64 CPU oracle for the FP8 variant: incoherent processing, per-block
E4M3 quantisation, and a step-by-step simulation of FP8 attention.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import this module; the HIP path never does.

Sources and readings:

  * Incoherent processing x~ = H D x, with D a random +-1 diagonal and H a
    Hadamard transform, applied to Q and K before quantisation: the
    "FlashAttention-3" page (lyirs.cc), section "FP8 路径与低精度误差",
    subsections "Incoherent processing 在做什么" and "为什么 Hadamard 适合放到内核里";
    also the "FlashAttention-2/3" page, section "FlashAttention-3：拥抱 Hopper",
    特性二 (a random orthogonal rotation).
    Readings: H is the Sylvester-order Hadamard matrix,
    H[i, j] = (-1)^popcount(i & j), normalised to be orthonormal (H / sqrt(d));
    one D vector is shared by Q and K (needed for (HDq).(HDk) = q.k); V is
    not rotated.
  * Per-block quantisation with one scale per block: the "FlashAttention-2/3"
    page, 特性三 (block-level online quantisation).  Readings: a block is
    128 consecutive rows of one (b, h) over all d columns; the stored
    dequantisation scale is s = amax / 448 (so an all-zero block has s = 0
    and all codes zero: it dequantises to zero exactly); code = E4M3
    round-to-nearest-even of x * 448 / amax, saturating at +-448.
  * E4M3 itself: the FP8 formats named on the "FlashAttention-2/3" page
    (特性二).  The codec below is the OCP "E4M3FN" encoding, written from
    its definition: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa
    bits, subnormals m * 2^-9, no infinities, S.1111.111 is NaN, largest
    finite value 448.
  * E5M2, the other format that page names: the OCP E5M2 encoding, from its
    definition: 1 sign bit, 5 exponent bits with bias 15, 2 mantissa bits,
    subnormals m * 2^-16, S.11111.00 is infinity, S.11111.{01,10,11} NaN,
    largest finite value 57344.  Same block rule with 57344 in place of 448
    (fmt="e5m2").  P, where the simulation rounds it, stays E4M3.
"""
from __future__ import annotations

import numpy as np

from .attention import attention as _attention_exact

E4M3_MAX = 448.0
E4M3_BIAS = 7


def e4m3_decode(codes):
    """Decode uint8 E4M3FN codes to fp64 (NaN for 0x7F / 0xFF)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    sub = m.astype(np.float64) * 2.0 ** (1 - E4M3_BIAS - 3)          # m/8 * 2^-6
    nrm = (1.0 + m / 8.0) * np.exp2((e - E4M3_BIAS).astype(np.float64))
    val = np.where(e == 0, sub, nrm)
    val = np.where((e == 0xF) & (m == 0x7), np.nan, val)
    return sign * val


# Non-negative finite values in code order (codes 0x00 .. 0x7E); the codes
# are monotone in value, so a code's parity is its mantissa's parity.
_POS_VALUES = e4m3_decode(np.arange(0x7F, dtype=np.uint8))


def e4m3_encode(x):
    """Round fp64 values to the nearest E4M3FN value, ties to the even code,
    saturating at +-448.  NaN maps to 0x7F.  Negative values (including
    those that round to zero, and -0.0) carry the sign bit."""
    x = np.asarray(x, dtype=np.float64)
    ax = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(_POS_VALUES, ax, side="left")      # first value >= ax
    hi = np.minimum(hi, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = ax - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - ax
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(ax == _POS_VALUES[hi], hi, code)        # exact hits
    code = code.astype(np.uint8)
    code = np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)
    return np.where(np.isnan(x), np.uint8(0x7F), code).astype(np.uint8)


E5M2_MAX = 57344.0
E5M2_BIAS = 15


def e5m2_decode(codes):
    """Decode uint8 OCP E5M2 codes to fp64 (+-inf for S.11111.00, NaN for
    the other three codes of exponent 31)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 2) & 0x1F
    m = c & 0x3
    sub = m.astype(np.float64) * 2.0 ** (1 - E5M2_BIAS - 2)          # m/4 * 2^-14
    nrm = (1.0 + m / 4.0) * np.exp2((e - E5M2_BIAS).astype(np.float64))
    val = np.where(e == 0, sub, nrm)
    val = np.where((e == 0x1F) & (m == 0), np.inf, val)
    val = np.where((e == 0x1F) & (m != 0), np.nan, val)
    return sign * val


_POS_VALUES_E5M2 = e5m2_decode(np.arange(0x7C, dtype=np.uint8))   # finite: 0x00 .. 0x7B


def e5m2_encode(x):
    """Round fp64 values to the nearest finite E5M2 value, ties to the even
    code, saturating at +-57344 (the block rule never exceeds it).  NaN maps
    to 0x7F."""
    x = np.asarray(x, dtype=np.float64)
    ax = np.minimum(np.abs(x), E5M2_MAX)
    hi = np.searchsorted(_POS_VALUES_E5M2, ax, side="left")
    hi = np.minimum(hi, len(_POS_VALUES_E5M2) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = ax - _POS_VALUES_E5M2[lo]
    d_hi = _POS_VALUES_E5M2[hi] - ax
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(ax == _POS_VALUES_E5M2[hi], hi, code)
    code = code.astype(np.uint8)
    code = np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)
    return np.where(np.isnan(x), np.uint8(0x7F), code).astype(np.uint8)


# format name -> (encode, decode, largest finite value)
FORMATS = {"e4m3": (e4m3_encode, e4m3_decode, E4M3_MAX), "e5m2": (e5m2_encode, e5m2_decode, E5M2_MAX)}


def sylvester_hadamard(d):
    """Dense unnormalised Sylvester Hadamard matrix, H_{2n} = [[H, H], [H, -H]]."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    h = np.ones((1, 1), np.float64)
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def rotate(x, signs):
    """Incoherent processing of the rows of x[..., d]: x~ = (H / sqrt(d)) D x.

    Row vectors: x~ = (x * D) @ H^T / sqrt(d) (H is symmetric)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    h = sylvester_hadamard(d)
    dx = x * np.asarray(signs, dtype=np.float64)
    return (dx @ h.T) / np.sqrt(d)


def block_quantize(x, block_rows=128, fmt="e4m3"):
    """Per-(..., row block) FP8 quantisation of x[..., N, d] (E4M3, or E5M2
    with 57344 in place of 448).

    Returns (codes uint8 [..., N, d], scales fp64 [..., ceil(N/block_rows)],
    y fp64 [..., N, d]) where y = x * 448 / amax is the value each code
    rounds (kept so that tests can locate rounding boundaries)."""
    encode, _, qmax = FORMATS[fmt]
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[-2]
    nb = -(-n // block_rows)
    lead = x.shape[:-2]
    codes = np.empty(x.shape, np.uint8)
    y = np.empty(x.shape, np.float64)
    scales = np.empty(lead + (nb,), np.float64)
    for b in range(nb):
        r0, r1 = b * block_rows, min(n, (b + 1) * block_rows)
        blk = x[..., r0:r1, :]
        amax = np.max(np.abs(blk), axis=(-2, -1))
        safe = np.where(amax > 0, amax, 1.0)
        # the quotient (x * 448) / amax: x * 448 is exact in fp64 for every
        # input of at most 50 significant bits and the division is correctly
        # rounded, so a value that lies exactly on a rounding midpoint stays
        # there and is decided by the ties-to-even rule
        yb = np.where((amax > 0)[..., None, None], (blk * qmax) / safe[..., None, None], 0.0)
        y[..., r0:r1, :] = yb
        codes[..., r0:r1, :] = encode(yb)
        scales[..., b] = amax / qmax
    return codes, scales, y


def hadamard_rotate_quant(x, signs=None, block_rows=128, transpose_out=False, fmt="e4m3"):
    """The FP8 pre-pass: optional incoherent processing (signs given), then
    per-block quantisation to `fmt`.  Returns (codes, scales, y) with codes in
    [..., N, d] or, if transpose_out, [..., d, N] order."""
    xr = rotate(x, signs) if signs is not None else np.asarray(x, dtype=np.float64)
    codes, scales, y = block_quantize(xr, block_rows, fmt)
    if transpose_out:
        codes = np.swapaxes(codes, -1, -2).copy()
        y = np.swapaxes(y, -1, -2).copy()
    return codes, scales, y


def dequantize(codes, scales, block_rows=128, transposed=False, fmt="e4m3"):
    """x^ = decode(code) * scale of its row block."""
    c = np.swapaxes(codes, -1, -2) if transposed else codes
    val = FORMATS[fmt][1](c)
    n = val.shape[-2]
    row_scale = np.repeat(scales, block_rows, axis=-1)[..., :n]
    return val * row_scale[..., :, None]


def attention_fp8_simulated(q, k, v, signs, scale, causal=False, block_rows=128,
                            quantize_p=False, fmt="e4m3", p_block=128):
    """Step-by-step simulation of FP8 attention.

    1. Rotate Q and K with the shared signs (skipped if signs is None).
    2. Block-quantise Q~, K~ and V and dequantise them.
    3. Evaluate the exact definition on the dequantised values.

    With quantize_p the probabilities of the second product are rounded to
    E4M3 as well (the pages put both products on the FP8 path but leave the
    rounding of P open).  Reading: the weights are rounded as the tiled
    online softmax of the "FlashAttention-2/3" page (section "技术原理")
    produces them, block by block of p_block keys, against the running row
    maximum after that block, rounded up to a power of two; each V block's
    dequantisation scale is folded into the weight before rounding
    (quantized_probabilities states the rounding); the rounded weights serve
    both the product with V and the row sums, so O is normalised by exactly
    the weights it used (a constant V comes out unchanged) and
    LSE = M ln 2 + ln l.
    Returns fp64 (O, LSE).
    """
    qc, qs, _ = hadamard_rotate_quant(q, signs, block_rows, fmt=fmt)
    kc, ks, _ = hadamard_rotate_quant(k, signs, block_rows, fmt=fmt)
    vc, vs, _ = hadamard_rotate_quant(v, None, block_rows, fmt=fmt)
    qh = dequantize(qc, qs, block_rows, fmt=fmt)
    kh = dequantize(kc, ks, block_rows, fmt=fmt)
    vh = dequantize(vc, vs, block_rows, fmt=fmt)
    if not quantize_p:
        return _attention_exact(qh, kh, vh, scale, causal)
    lead = qh.shape[:-2]
    n, d = qh.shape[-2:]
    qf, kf, vf = (a.reshape(-1, a.shape[-2], a.shape[-1]) for a in (qh, kh, vh))
    vsf = np.asarray(vs, np.float64).reshape(qf.shape[0], -1)
    o = np.empty((qf.shape[0], n, vf.shape[-1]))
    lse = np.empty((qf.shape[0], n))
    for h in range(qf.shape[0]):
        s = (qf[h] @ kf[h].T) * scale
        if causal:
            s = np.where(np.arange(n)[None, :] > np.arange(n)[:, None], -np.inf, s)
        w = np.repeat(vsf[h], block_rows)[:n]
        pq, m = quantized_probabilities(s, w, p_block)
        l = pq.sum(1)
        o[h] = (pq @ vf[h]) / l[:, None]
        lse[h] = m * np.log(2.0) + np.log(l)
    return o.reshape(*lead, n, -1), lse.reshape(*lead, n)


P_GAIN = 256.0   # largest E4M3 weight: 256 <= 448, so nothing saturates


def quantized_probabilities(s, w, block=128):
    """The E4M3-rounded weights of the FP8 second product.

    s: scores [Nq, Nk] in natural units (masked entries -inf); w: [Nk] the
    dequantisation scale of each key's V block; block: keys per block of the
    online pass.  With t = s log2(e) and b(j) the block of key j:
      * M_i^b = ceil(max of t_ik over the keys k of blocks 0..b): the running
        row maximum after block b (the online softmax's m), rounded up to a
        whole power of two;
      * gain g_j = 256 w_j / svmax (svmax the largest V block scale; a zero
        scale, an all-zero block whose values contribute nothing, counts as
        svmax; svmax = 1 if every scale is zero);
      * P'_ij = E4M3(2^(t_ij - M_i^b(j)) g_j): at most 256, no saturation;
        weights far below the running maximum fall into E4M3's subnormals;
      * weight_ij = P'_ij / g_j * 2^(M_i^b(j) - M_i), M_i = M_i^last.
    Returns (weights [Nq, Nk], M [Nq]): the weights relative to 2^M_i."""
    s = np.asarray(s, np.float64)
    w = np.asarray(w, np.float64)
    nq, nk = s.shape
    t = s * np.log2(np.e)
    nb = -(-nk // block)
    bmax = np.stack([np.max(t[:, b * block:(b + 1) * block], axis=1) for b in range(nb)], axis=1)
    ref_blk = np.ceil(np.maximum.accumulate(bmax, axis=1))          # [Nq, nb], -inf while all masked
    ref = np.repeat(ref_blk, block, axis=1)[:, :nk]
    m = ref_blk[:, -1]
    svmax = float(np.max(w)) if np.max(w) > 0 else 1.0
    w = np.where(w > 0, w, svmax)
    gain = P_GAIN * w / svmax
    seen = np.isfinite(t)
    arg = np.where(seen, t - np.where(seen, ref, 0.0), -np.inf)
    pq = e4m3_decode(e4m3_encode(np.exp2(arg) * gain[None, :])) / gain[None, :]
    pq = pq * np.exp2(np.where(seen, ref - m[:, None], 0.0))
    return pq, m


def rel_rms(a, b):
    """||a - b||_F / ||b||_F."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.sqrt(np.sum((a - b) ** 2)) / np.sqrt(np.sum(b ** 2)))
