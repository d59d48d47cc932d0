"""GPU parity of the FP8 path: hadamard_rotate_quant codes/scales against the
oracle codec, and attn_fwd_fp8 against the oracle's step-by-step FP8
simulation (rotate -> per-block E4M3 -> softmax on the dequantised values,
with the probabilities of the second product rounded to E4M3 as
oracle.quantized_probabilities states: the kernel's reading).

Code parity: a code must equal the oracle's, except where the exact value
x~ * 448 / amax lies within fp32 rounding of a rounding midpoint; there the
adjacent code is also accepted (the kernel forms x~ in fp32, the oracle in
fp64).  Scales: relative 2e-6.

Attention parity against that simulation (the rotated path and every
input without outlier channels): relative RMS of O <= 3e-3; LSE mean
|err| <= 3e-4 and 99th percentile <= 1e-2.  What separates the two is the
bf16 rounding of O (1.66e-3 relative RMS on Gaussian values by itself),
fp32 accumulation, and weights whose exponent lies within the arithmetic's
error of an E4M3 rounding midpoint: rare, but when it is a row's dominant
weight it moves that row's sum by up to an E4M3 step, hence a percentile
rather than a max for the LSE.  Rows with outlier-sized scores (|s log2 e|
in the hundreds) widen that error: the FP8 MFMA adds its 64 products with
less precision than fp32 when one product dominates (measured on gfx950: up
to ~1 code unit on sums of ~5e3, where an fp32 sum is within 1e-2), so the
exponents of such rows carry errors of ~1e-3..1e-2.  The unrotated codes of
the outlier workload, where every score is dominated by the outlier
channel's product, are checked at relative RMS <= 1e-2 and LSE mean
<= 1e-2 for that reason.

The error against EXACT attention is a property of the format, measured and
reported beside the gate the method was set (relative RMS <= 3e-2): on the
FP8 workload the quantisation alone puts the result well above it.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from exact_attention_forward_06_amd import (attn_fwd_fp8, attn_fwd_fp8_e2e, attn_fwd_fp8_qrot, hadamard_rotate_quant,
                                            rope_hadamard_rotate_quant)
from exact_attention_forward_06_amd.inputs import WORKLOADS, make_inputs, random_signs, to_f64, workload_inputs

from oracle_pool import fp8_head_errors, map_heads, reduce_fp8

O_TOL = 3e-3          # relative RMS of O against the simulation with rounded P
LSE_TOL = 1e-2        # 99th percentile of |LSE err| against the same
LSE_MEAN_TOL = 3e-4   # mean |LSE err| against the same
UNROT_TOL = 1e-2      # O relative RMS and LSE mean, unrotated codes of outlier inputs

pytestmark = pytest.mark.gpu

_DT = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}


def _codes_match(c_gpu, c_ref, y_ref, band, what, max_frac=1e-3, fmt="e4m3"):
    """c_gpu, c_ref: uint8 arrays; y_ref: the fp64 values the oracle rounded;
    band: absolute distance from a rounding midpoint within which the fp32
    kernel may land on either side."""
    decode = oracle.FORMATS[fmt][1]
    c_gpu = np.asarray(c_gpu)
    same = (c_gpu == c_ref) | ((c_gpu & 0x7F) == 0) & ((c_ref & 0x7F) == 0)
    bad = ~same
    if bad.any():
        vg = decode(c_gpu[bad])
        vo = decode(c_ref[bad])
        y = y_ref[bad]
        band = np.broadcast_to(band, y_ref.shape)[bad]
        mid = 0.5 * (vg + vo)
        adjacent = np.abs(np.abs(vg - y) - np.abs(vo - y)) <= 2 * band + 1e-12
        near_tie = np.abs(y - mid) <= band
        ok = adjacent & near_tie
        assert ok.all(), (f"{what}: {int((~ok).sum())} codes differ beyond the rounding band; "
                          f"e.g. gpu {c_gpu[bad][~ok][:5]} oracle {c_ref[bad][~ok][:5]} y {y[~ok][:5]}")
        assert bad.sum() <= max(2, max_frac * c_gpu.size), f"{what}: {int(bad.sum())} tie flips"
    return int(bad.sum())


def _band(y_ref, d, rotated, qmax=448.0):
    """fp32 error of the value the kernel rounds, in code units: the rotated
    path sums log2(d) butterfly stages in fp32 (absolute error ~ 2^-24 * qmax
    per stage, block-relative); the unrotated path only rounds the quotient."""
    if rotated:
        return qmax * 2.0 ** -24 * 4 * math.log2(d)
    return 2.0 ** -22 * np.abs(y_ref)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("dtype", ["bf16", "fp32", "fp16"])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("rot,trans", [(True, False), (False, True), (False, False), (True, True)])
def test_hadamard_rotate_quant_parity(dtype, d, rot, trans, fmt):
    N = 304 if trans else 300            # ragged last block (transpose needs N % 16 == 0)
    inp = make_inputs(2, 3, N, d, dtype, seed=d + N)
    x = inp["q"]
    x[..., 3] *= 20                     # an outlier channel
    signs = random_signs(d, seed=d) if rot else None
    codes, scales = hadamard_rotate_quant(x.cuda(), None if signs is None else signs.cuda(),
                                          transpose_out=trans, fp8_format=fmt)
    torch.cuda.synchronize()
    c_ref, s_ref, y_ref = oracle.hadamard_rotate_quant(to_f64(x), None if signs is None else signs.numpy(),
                                                       128, transpose_out=trans, fmt=fmt)
    assert codes.shape == c_ref.shape
    np.testing.assert_allclose(scales.cpu().double().numpy(), s_ref, rtol=2e-6)
    flips = _codes_match(codes.cpu().numpy(), c_ref, y_ref, _band(y_ref, d, rot, oracle.FORMATS[fmt][2]),
                         f"{fmt} {dtype} d={d} rot={rot} trans={trans}", fmt=fmt)
    if not rot and dtype != "fp32":
        assert flips == 0, "16-bit inputs without rotation must give the oracle's codes exactly"


@pytest.mark.parametrize("N,rot,trans", [(N, r, t) for N in (300, 512)
                                          for r, t in ((True, False), (False, True), (False, False))
                                          if not (t and N % 16)])      # transposed output needs N % 16 == 0
@pytest.mark.parametrize("d", [64, 128, 256])
def test_per_tensor_quant_parity(d, rot, trans, N):
    """hadamard_rotate_quant_per_tensor: one scale per (b, h) over all N rows
    (the oracle's block quantisation with block_rows = N), replicated into
    every 128-row slot; codes as in the per-block test."""
    inp = make_inputs(2, 3, N, d, "bf16", seed=d + N + 5)
    x = inp["q"]
    x[..., 3] *= 20
    x[0, 1, 7:9] *= 4                     # one head with a larger maximum elsewhere
    signs = random_signs(d, seed=d + 1) if rot else None
    codes, scales = hadamard_rotate_quant(x.cuda(), None if signs is None else signs.cuda(), transpose_out=trans,
                                          per_tensor=True)
    torch.cuda.synchronize()
    c_ref, s_ref, y_ref = oracle.hadamard_rotate_quant(to_f64(x), None if signs is None else signs.numpy(), N,
                                                       transpose_out=trans)
    sc = scales.cpu().double().numpy()
    assert sc.shape == (2, 3, -(-N // 128))
    np.testing.assert_allclose(sc, np.broadcast_to(s_ref, sc.shape), rtol=2e-6)
    flips = _codes_match(codes.cpu().numpy(), c_ref, y_ref, _band(y_ref, d, rot), f"per-tensor d={d} rot={rot}")
    if not rot:
        assert flips == 0


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_per_tensor_attention_matches_simulation(d, causal):
    B, H, N = 1, 2, 512
    inp = _fp8_inputs(B, H, N, d, seed=d + 71, outliers=True)
    o, lse = attn_fwd_fp8_e2e(inp["q"].cuda(), inp["k"].cuda(), inp["v"].cuda(), inp["signs"].cuda(),
                              causal=causal, per_tensor=True)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_fp8_simulated(to_f64(inp["q"]), to_f64(inp["k"]), to_f64(inp["v"]),
                                                    inp["signs"].numpy(), 1 / math.sqrt(d), causal, block_rows=N,
                                                    quantize_p=True, p_block=p_block(d))
    _check_sim(o, lse, o_ref, lse_ref, f"per-tensor d={d} causal={causal}")


@pytest.mark.parametrize("d", [64, 128, 256])
def test_fp8_strided_inputs(d):
    """The FP8 entry points on [B, H, N, d] views of [B, N, H, d] tensors:
    the pre-pass (plain and with RoPE) and the attention with Q rotated in
    the kernel give bitwise the results of the same data laid out
    contiguously (the contiguous paths are checked against the oracle in
    the tests above)."""
    B, N, H = 2, 256, 3
    print(f"fp8 strided inputs d={d}", flush=True)
    g = torch.Generator().manual_seed(70 + d)
    base = [torch.randn(B, N, H, d, generator=g).to(torch.bfloat16).cuda() for _ in range(3)]
    view = [t.permute(0, 2, 1, 3) for t in base]
    cont = [t.contiguous() for t in view]
    assert not view[0].is_contiguous() and view[0].stride() == (N * H * d, d, H * d, 1)
    sg = random_signs(d, seed=71).cuda()
    for args in ((sg,), (None,)):
        c1, s1 = hadamard_rotate_quant(view[0], *args)
        c2, s2 = hadamard_rotate_quant(cont[0], *args)
        assert torch.equal(c1, c2) and torch.equal(s1, s2), f"pre-pass, signs={args[0] is not None}"
    for style in ("interleaved", "half"):
        c1, s1 = rope_hadamard_rotate_quant(view[1], sg, style=style, pos_offset=5)
        c2, s2 = rope_hadamard_rotate_quant(cont[1], sg, style=style, pos_offset=5)
        assert torch.equal(c1, c2) and torch.equal(s1, s2), f"rope pre-pass {style}"
    if d <= 128:
        k8, ks = hadamard_rotate_quant(cont[1], sg)
        v8, vs = hadamard_rotate_quant(cont[2], None, transpose_out=True)
        o1, l1 = attn_fwd_fp8_qrot(view[0], sg, k8, ks, v8, vs, causal=True)
        o2, l2 = attn_fwd_fp8_qrot(cont[0], sg, k8, ks, v8, vs, causal=True)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2), "attn_fwd_fp8_qrot"


def test_hadamard_block_max_encodes_to_448():
    inp = make_inputs(1, 2, 256, 128, "bf16", seed=3)
    signs = random_signs(128, 3)
    codes, _ = hadamard_rotate_quant(inp["k"].cuda(), signs.cuda())
    torch.cuda.synchronize()
    c = codes.cpu().numpy().reshape(2, 2, -1)       # (head, block, elements)
    assert np.all(np.max(c & 0x7F, axis=-1) == 0x7E)


def test_hadamard_zero_block_zero_scale():
    x = torch.zeros(1, 1, 256, 64, dtype=torch.bfloat16)
    x[0, 0, 200, 5] = -3.0
    codes, scales = hadamard_rotate_quant(x.cuda(), None)
    torch.cuda.synchronize()
    s = scales.cpu().numpy()[0, 0]
    assert s[0] == 0.0 and s[1] == np.float32(3.0 / 448)
    assert np.all(codes.cpu().numpy()[0, 0, :128] & 0x7F == 0)
    assert codes.cpu().numpy()[0, 0, 200, 5] == 0xFE


def _fp8_inputs(B, H, N, d, seed, outliers=True):
    inp = make_inputs(B, H, N, d, "fp8", seed=seed, outlier_frac=0.005 if outliers else 0.0)
    if "signs" not in inp:
        inp["signs"] = random_signs(d, seed)
    return inp


def p_block(d):
    """Keys per block of the kernels' online pass (the reference P is
    rounded against moves once per block): 128 for d <= 128, 64 for d = 256."""
    return 128 if d <= 128 else 64


def _sim_p(inp, causal, rotate=True, fmt="e4m3", v=None):
    """The oracle's FP8 simulation with rounded P (fp64 O, LSE) for all heads."""
    d = inp["q"].shape[-1]
    vv = to_f64(inp["v"] if v is None else v)
    return oracle.attention_fp8_simulated(to_f64(inp["q"]), to_f64(inp["k"]), vv,
                                          inp["signs"].numpy() if rotate else None, 1 / math.sqrt(d),
                                          causal, quantize_p=True, fmt=fmt, p_block=p_block(d))


def _check_sim(o, lse, o_ref, lse_ref, what):
    og = to_f64(o)
    assert np.all(np.isfinite(og)), what
    err = oracle.rel_rms(og, o_ref)
    ld = np.abs(lse.cpu().double().numpy() - lse_ref).ravel()
    p99 = float(np.quantile(ld, 0.99))
    print(f"[{what}] vs FP8 simulation: O rel RMS {err:.2e}, LSE mean {ld.mean():.2e} p99 {p99:.2e} "
          f"max {ld.max():.2e}", flush=True)
    assert err <= O_TOL, f"{what}: rel RMS vs FP8 simulation {err:.3e} > {O_TOL}"
    assert ld.mean() <= LSE_MEAN_TOL, f"{what}: mean |LSE err| vs FP8 simulation {ld.mean():.3e}"
    assert p99 <= LSE_TOL, f"{what}: 99th percentile |LSE err| vs FP8 simulation {p99:.3e} > {LSE_TOL}"
    return err, ld.max()


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("outliers", [False, True])
def test_fp8_attention_matches_simulation(d, causal, outliers, fmt):
    B, H, N = 1, 2, 384
    inp = _fp8_inputs(B, H, N, d, seed=d + 7, outliers=outliers)
    o, lse = attn_fwd_fp8_e2e(inp["q"].cuda(), inp["k"].cuda(), inp["v"].cuda(), inp["signs"].cuda(),
                              causal=causal, fp8_format=fmt)
    torch.cuda.synchronize()
    o_ref, lse_ref = _sim_p(inp, causal, fmt=fmt)
    _check_sim(o, lse, o_ref, lse_ref, f"{fmt} d={d} causal={causal} outliers={outliers}")
    # the quantisation error itself stays in the range E4M3 allows
    exact, _ = oracle.attention(to_f64(inp["q"]), to_f64(inp["k"]), to_f64(inp["v"]), 1 / math.sqrt(d), causal)
    assert oracle.rel_rms(to_f64(o), exact) < 0.5


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("outliers", [False, True])
@pytest.mark.parametrize("qdtype", ["bf16", "fp16"])
def test_fp8_q_in_kernel_matches_simulation(d, causal, outliers, fmt, qdtype):
    """attn_fwd_fp8_qrot: Q rotated and quantised by the attention kernel.
    Against the oracle's simulation at the kernel gates, and against the
    pre-pass path (hadamard_rotate_quant on Q, then attn_fwd_fp8), which it
    must reproduce up to Q codes that flip at a rounding midpoint: relative
    RMS between the two outputs <= 1e-3 (one flipped code moves a score by
    at most one E4M3 step of one Q element)."""
    B, H, N = 1, 2, 384
    inp = _fp8_inputs(B, H, N, d, seed=d + 11, outliers=outliers)
    if qdtype == "fp16":
        inp = dict(inp, q=inp["q"].to(torch.float16))
    q, k, v, sg = inp["q"].cuda(), inp["k"].cuda(), inp["v"].cuda(), inp["signs"].cuda()
    o, lse = attn_fwd_fp8_e2e(q, k, v, sg, causal=causal, fp8_format=fmt, q_in_kernel=True)
    o2, lse2 = attn_fwd_fp8_e2e(q, k, v, sg, causal=causal, fp8_format=fmt)
    torch.cuda.synchronize()
    sim_inp = dict(inp, q=inp["q"].to(torch.float32))
    o_ref, lse_ref = _sim_p(sim_inp, causal, fmt=fmt)
    _check_sim(o, lse, o_ref, lse_ref, f"q in kernel {qdtype} {fmt} d={d} causal={causal} outliers={outliers}")
    between = oracle.rel_rms(to_f64(o), to_f64(o2))
    print(f"  q in kernel vs pre-pass path: O rel RMS {between:.2e}", flush=True)
    assert between <= 1e-3


def test_fp8_q_in_kernel_workload(capsys):
    """The FP8 workload (B=2 H=16 N=8192 d=128, outlier channel) through
    attn_fwd_fp8_qrot, every head and row against the simulation at the
    kernel gates."""
    w = WORKLOADS["fp8_hadamard_8k"]
    inp = workload_inputs(w)
    q, k, v, sg = (inp[n].cuda() for n in ("q", "k", "v", "signs"))
    o, lse = attn_fwd_fp8_e2e(q, k, v, sg, q_in_kernel=True)
    torch.cuda.synchronize()
    o, lse = o.float().cpu().numpy(), lse.cpu().numpy()
    f32 = {n: inp[n].float().numpy() for n in ("q", "k", "v")}
    tasks = [(f32["q"][b, h], f32["k"][b, h], f32["v"][b, h], inp["signs"].numpy(), o[b, h], lse[b, h], w.scale,
              False) for b in range(w.B) for h in range(w.H)]
    r = reduce_fp8(map_heads(fp8_head_errors, tasks))
    with capsys.disabled():
        print(f"\n[fp8 workload full, q in kernel] {r['heads']} heads: GPU vs simulation {r['gpu_vs_simp']:.2e}, "
              f"|LSE err| mean {r['lse_simp_mean']:.2e} p99 {r['lse_simp_p99']:.2e}; vs exact "
              f"{r['gpu_vs_exact']:.4f}", flush=True)
    assert r["finite"] and r["heads"] == w.B * w.H
    assert r["gpu_vs_simp"] <= O_TOL and r["lse_simp_p99"] <= LSE_TOL and r["lse_simp_mean"] <= LSE_MEAN_TOL, r


def test_fp8_q_in_kernel_zero_q_block():
    """An all-zero 128-row block of Q (scale 0, codes 0): its rows see
    uniform weights, O is the mean of the visible V rows."""
    B, H, N, d = 1, 1, 256, 128
    inp = _fp8_inputs(B, H, N, d, seed=5, outliers=False)
    inp["q"][0, 0, 128:] = 0
    q, k, v, sg = inp["q"].cuda(), inp["k"].cuda(), inp["v"].cuda(), inp["signs"].cuda()
    o, lse = attn_fwd_fp8_e2e(q, k, v, sg, q_in_kernel=True)
    torch.cuda.synchronize()
    o_ref, lse_ref = _sim_p(inp, False)
    _check_sim(o, lse, o_ref, lse_ref, "q in kernel, zero Q block")


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("case", ["zero_block", "small_v", "zero_block_small_v", "uneven_blocks"])
def test_fp8_v_block_scales(d, case):
    """V blocks whose scales differ widely: an all-zero 128-row block (scale
    0, as padding to a multiple of 128 rows gives), V at 1e-3 of unit scale,
    both at once, and one block 100x larger than the rest.  The kernel must
    follow the simulation's reading (zero blocks take the largest scale's
    gain, the others 16 sV_j / sVmax) to the same tolerance."""
    B, H, N = 1, 2, 512
    inp = _fp8_inputs(B, H, N, d, seed=d + 51, outliers=False)
    v = inp["v"].float()
    if case in ("small_v", "zero_block_small_v"):
        v = v * 1e-3
    if case in ("zero_block", "zero_block_small_v"):
        v[:, :, 256:384] = 0
    if case == "uneven_blocks":
        v[:, :, 128:256] *= 100
    v = v.to(torch.bfloat16)
    for causal in (False, True):
        o, lse = attn_fwd_fp8_e2e(inp["q"].cuda(), inp["k"].cuda(), v.cuda(), inp["signs"].cuda(), causal=causal)
        torch.cuda.synchronize()
        o_ref, lse_ref = _sim_p(inp, causal, v=v)
        _check_sim(o, lse, o_ref, lse_ref, f"{case} d={d} causal={causal}")


def test_fp8_all_zero_v():
    B, H, N, d = 1, 2, 256, 128
    inp = _fp8_inputs(B, H, N, d, seed=5, outliers=False)
    v = torch.zeros(B, H, N, d, dtype=torch.bfloat16, device="cuda")
    for causal in (False, True):
        o, lse = attn_fwd_fp8_e2e(inp["q"].cuda(), inp["k"].cuda(), v, inp["signs"].cuda(), causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(o, torch.zeros_like(o))
        _, lse_ref = _sim_p(inp, causal, v=v.cpu())
        assert np.abs(lse.cpu().double().numpy() - lse_ref).max() <= 1e-3


def test_fp8_lse_close_to_simulated():
    B, H, N, d = 1, 1, 256, 128
    inp = _fp8_inputs(B, H, N, d, seed=21, outliers=False)
    o, lse = attn_fwd_fp8_e2e(inp["q"].cuda(), inp["k"].cuda(), inp["v"].cuda(), inp["signs"].cuda())
    torch.cuda.synchronize()
    signs = inp["signs"].numpy()
    qh = oracle.dequantize(*oracle.hadamard_rotate_quant(to_f64(inp["q"][0, 0]), signs, 128)[:2], 128)
    kh = oracle.dequantize(*oracle.hadamard_rotate_quant(to_f64(inp["k"][0, 0]), signs, 128)[:2], 128)
    vh = oracle.dequantize(*oracle.hadamard_rotate_quant(to_f64(inp["v"][0, 0]), None, 128)[:2], 128)
    _, lse_sim = oracle.attention_head(qh, kh, vh, 1 / math.sqrt(d))
    dl = np.abs(lse[0, 0].cpu().double().numpy() - lse_sim)
    # the row sums are those of the E4M3-rounded P: bounded by the relative
    # rounding of E4M3; many keys per row average the rounding out
    assert dl.max() <= math.log1p(2.0 ** -4)
    assert dl.mean() <= 1e-2


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_constant_v_is_returned_exactly(d, causal, fmt):
    # O is normalised by the sum of the weights its second product used, so a
    # constant V (codes all 448, one exact scale) comes back as that constant
    B, H, N = 1, 2, 384
    inp = _fp8_inputs(B, H, N, d, seed=d + 31)
    q, k = (inp[n].cuda() * 3 for n in ("q", "k"))
    v = torch.full((B, H, N, d), -1.75, dtype=torch.bfloat16, device="cuda")
    o, lse = attn_fwd_fp8_e2e(q, k, v, inp["signs"].cuda(), causal=causal, fp8_format=fmt)
    torch.cuda.synchronize()
    assert torch.equal(o, torch.full_like(o, -1.75)), (o.float() + 1.75).abs().max().item()
    assert torch.isfinite(lse).all()


def test_fp8_workload_sampled(capsys):
    """The FP8 workload at full size (the bench's launch configuration) on
    sampled heads: a fast variant of test_fp8_workload_full."""
    w = WORKLOADS["fp8_hadamard_8k"]
    inp = workload_inputs(w)
    q, k, v, sg = (inp[n].cuda() for n in ("q", "k", "v", "signs"))
    o, lse = attn_fwd_fp8_e2e(q, k, v, sg)
    torch.cuda.synchronize()
    o, lse = o.float().cpu().numpy(), lse.cpu().numpy()
    heads = [(0, 0), (1, 15), (0, 7), (1, 3)]
    tasks = [(inp["q"][b, h].float().numpy(), inp["k"][b, h].float().numpy(), inp["v"][b, h].float().numpy(),
              inp["signs"].numpy(), o[b, h], lse[b, h], w.scale, False) for b, h in heads]
    r = reduce_fp8(map_heads(fp8_head_errors, tasks))
    with capsys.disabled():
        print(f"\n[fp8 workload, 4 heads] vs simulation {r['gpu_vs_simp']:.2e}, LSE mean {r['lse_simp_mean']:.2e} "
              f"p99 {r['lse_simp_p99']:.2e} max {r['lse_simp_max']:.2e}; "
              f"vs exact {r['gpu_vs_exact']:.4f}", flush=True)
    assert r["finite"] and r["gpu_vs_simp"] <= O_TOL and r["lse_simp_p99"] <= LSE_TOL, r
    assert r["lse_simp_mean"] <= LSE_MEAN_TOL, r


@pytest.mark.parametrize("rotated", [True, False])
def test_fp8_workload_full(rotated, capsys):
    """Every head and row of the FP8 workload (B=2 H=16 N=8192 d=128, one
    outlier channel x20), rotated (the method) and unrotated (the comparison
    the pages make):
      * gate: the GPU against the oracle's simulation with rounded P over all
        B*H*N*d elements, at O_TOL / LSE_TOL / LSE_MEAN_TOL rotated and at
        UNROT_TOL unrotated (the FP8 MFMA's coarser sums; module docstring);
      * reported and checked for consistency: the error against exact
        attention, which must be the simulation's own error against exact
        attention (within 5 %): the kernel adds nothing of its own; and the
        floor of Q, K and V quantisation alone (P exact).
    The method's gate of relative RMS <= 3e-2 against exact attention is
    printed as met or NOT MET; on this workload E4M3 puts the result above it
    ("FlashAttention-3" page, section "FP8 路径与低精度误差", gives the
    direction of the rotation's effect, not a magnitude)."""
    w = WORKLOADS["fp8_hadamard_8k"]
    inp = workload_inputs(w)
    q, k, v, sg = (inp[n].cuda() for n in ("q", "k", "v", "signs"))
    if rotated:
        o, lse = attn_fwd_fp8_e2e(q, k, v, sg)
    else:
        q8, sq = hadamard_rotate_quant(q, None)
        k8, sk = hadamard_rotate_quant(k, None)
        v8, sv = hadamard_rotate_quant(v, None, transpose_out=True)
        o, lse = attn_fwd_fp8(q8, sq, k8, sk, v8, sv)
    torch.cuda.synchronize()
    o, lse = o.float().cpu().numpy(), lse.cpu().numpy()
    f32 = {n: inp[n].float().numpy() for n in ("q", "k", "v")}
    signs = inp["signs"].numpy() if rotated else None
    tasks = [(f32["q"][b, h], f32["k"][b, h], f32["v"][b, h], signs, o[b, h], lse[b, h], w.scale, False)
             for b in range(w.B) for h in range(w.H)]
    r = reduce_fp8(map_heads(fp8_head_errors, tasks))
    label = "rotated" if rotated else "unrotated"
    gate = "met" if r["gpu_vs_exact"] <= 3e-2 else "NOT MET"
    with capsys.disabled():
        print(f"\n[fp8 workload full, {label}] {r['heads']} heads: GPU vs simulation (rounded P) "
              f"{r['gpu_vs_simp']:.2e}, |LSE err| mean {r['lse_simp_mean']:.2e} p99 {r['lse_simp_p99']:.2e} "
              f"max {r['lse_simp_max']:.2e}; rel RMS vs exact: GPU "
              f"{r['gpu_vs_exact']:.4f}, simulation {r['simp_vs_exact']:.4f}, Q/K/V-only floor "
              f"{r['floor_vs_exact']:.4f}; gate rel-RMS <= 3e-2 vs exact: {gate}", flush=True)
    assert r["finite"] and r["heads"] == w.B * w.H
    if rotated:
        assert r["gpu_vs_simp"] <= O_TOL and r["lse_simp_p99"] <= LSE_TOL, r
        assert r["lse_simp_mean"] <= LSE_MEAN_TOL, r
    else:
        assert r["gpu_vs_simp"] <= UNROT_TOL and r["lse_simp_mean"] <= UNROT_TOL, r
    assert abs(r["gpu_vs_exact"] / r["simp_vs_exact"] - 1) <= 0.05, r


def test_fp8_outlier_sweep_rotation_on_gpu(capsys):
    """The GPU FP8 path against exact attention with and without the
    rotation, over outlier-channel rates 0, 0.5, 2 and 5 % of d (x20; 0, 1, 3
    and 6 channels at d = 128), with per-block (128 rows) and per-tensor (one
    per (b, h)) scales.  With three or more outlier channels the rotation
    must lower the error at least two-fold at both granularities (the
    direction of the pages' "about 2.6x" claim, "FlashAttention-3" page,
    section "FP8 路径与低精度误差"); with none it changes little.  A single
    outlier channel is reported only: whether it hurts the unrotated codes
    depends on the draw (the oracle's simulation shows both directions across
    seeds)."""
    B, H, N, d = 1, 4, 1024, 128
    rows = []
    for frac in (0.0, 0.005, 0.02, 0.05):
        inp = make_inputs(B, H, N, d, "fp8", seed=11, outlier_frac=frac)
        q, k, v, sg = (inp[n].cuda() for n in ("q", "k", "v", "signs"))
        exact, _ = oracle.attention(to_f64(inp["q"]), to_f64(inp["k"]), to_f64(inp["v"]), 1 / math.sqrt(d))
        res = {}
        for per_tensor in (False, True):
            o_rot, _ = attn_fwd_fp8_e2e(q, k, v, sg, per_tensor=per_tensor)
            o_plain, _ = attn_fwd_fp8_e2e(q, k, v, None, per_tensor=per_tensor)
            torch.cuda.synchronize()
            e_rot = oracle.rel_rms(to_f64(o_rot.cpu()), exact)
            e_plain = oracle.rel_rms(to_f64(o_plain.cpu()), exact)
            res[per_tensor] = (e_rot, e_plain)
            assert math.isfinite(e_rot) and math.isfinite(e_plain)
            if frac == 0.0:
                assert 0.8 <= e_plain / e_rot <= 1.25, (frac, per_tensor, e_rot, e_plain)
            elif frac >= 0.02:
                assert e_plain / e_rot >= 2.0, (frac, per_tensor, e_rot, e_plain)
        rows.append((frac, res))
    with capsys.disabled():
        print("\n[fp8 outlier sweep] rel RMS vs exact, rotated / unrotated / ratio, per-block | per-tensor: " +
              "; ".join(f"{f * 100:.1f}%: {r[False][0]:.4f} / {r[False][1]:.4f} / {r[False][1] / r[False][0]:.2f}x | "
                        f"{r[True][0]:.4f} / {r[True][1]:.4f} / {r[True][1] / r[True][0]:.2f}x" for f, r in rows),
              flush=True)


def test_fp8_e5m2_error_exceeds_e4m3(capsys):
    """E5M2 keeps 2 mantissa bits to E4M3's 3: on Gaussian inputs (no
    outliers, so range does not matter) its error against exact attention,
    through the GPU path, is the larger one, by about the factor its coarser
    rounding predicts (one bit: about 2x)."""
    B, H, N, d = 1, 4, 1024, 128
    inp = _fp8_inputs(B, H, N, d, seed=19, outliers=False)
    q, k, v, sg = (inp[n].cuda() for n in ("q", "k", "v", "signs"))
    exact, _ = oracle.attention(to_f64(inp["q"]), to_f64(inp["k"]), to_f64(inp["v"]), 1 / math.sqrt(d))
    err = {}
    for fmt in ("e4m3", "e5m2"):
        o, _ = attn_fwd_fp8_e2e(q, k, v, sg, fp8_format=fmt)
        torch.cuda.synchronize()
        err[fmt] = oracle.rel_rms(to_f64(o.cpu()), exact)
    assert 1.3 <= err["e5m2"] / err["e4m3"] <= 3.0, err
    with capsys.disabled():
        print(f"\n[fp8 formats] rel RMS vs exact: E4M3 {err['e4m3']:.4f}, E5M2 {err['e5m2']:.4f}", flush=True)
