"""GPU parity of split-KV attention (attn_fwd_splitkv) and of the partial
merge (attn_merge) against the fp64 oracle.

Tolerances: the merged O and LSE use attn_fwd's (bf16 / fp16 O: max |err|
<= 2e-2, mean <= 2e-3; LSE: max |err| <= 1e-3).  Each range's partial O is
fp32 (one rounding less than O) and is held to the same bar; a range a row
cannot see must come back exactly as O = 0, LSE = -inf.  attn_merge with
fp32 output on given partials: relative 1e-5 (fp32 exp and sums).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from exact_attention_forward_06_amd import attn_fwd, attn_fwd_splitkv, attn_merge, splitkv_chunk
from exact_attention_forward_06_amd.inputs import make_inputs, to_f64

pytestmark = pytest.mark.gpu

_DT = {"bf16": torch.bfloat16, "fp16": torch.float16}


def _check(o_gpu, lse_gpu, o_ref, lse_ref, what):
    err = np.abs(o_gpu - o_ref)
    assert np.all(np.isfinite(o_gpu)), what
    assert err.max() <= 2e-2, f"{what}: max |O err| {err.max():.3e}"
    assert err.mean() <= 2e-3, f"{what}: mean |O err| {err.mean():.3e}"
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lse_gpu), fin), f"{what}: -inf pattern of LSE"
    if fin.any():
        lerr = np.abs(lse_gpu[fin] - lse_ref[fin])
        assert lerr.max() <= 1e-3, f"{what}: max |LSE err| {lerr.max():.3e}"


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,S", [(300, 3), (512, 1), (1000, 7), (130, 2), (200, 64)])
def test_splitkv_matches_oracle(dtype, d, causal, N, S):
    """Merged output and every range's partial against the oracle; (200, 64)
    leaves most ranges past N (empty), (130, 2) has a ragged last range."""
    B, H = 1, 2
    print(f"\n[splitkv] {dtype} d={d} causal={causal} N={N} S={S}", flush=True)
    inp = make_inputs(B, H, N, d, dtype, seed=N + S + d)
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    o, lse, o_part, lse_part = attn_fwd_splitkv(q, k, v, S, causal=causal)
    torch.cuda.synchronize()
    scale = 1 / math.sqrt(d)
    qd, kd, vd = (to_f64(inp[n]) for n in ("q", "k", "v"))
    o_ref, lse_ref = oracle.attention(qd, kd, vd, scale, causal)
    _check(to_f64(o), lse.cpu().double().numpy(), o_ref, lse_ref, "merged")
    chunk = splitkv_chunk(N, S)
    op = o_part.cpu().double().numpy()
    lp = lse_part.cpu().double().numpy()
    for s in range(S):
        lo, hi = s * chunk, min(N, (s + 1) * chunk)
        for h in range(H):
            po, pl = oracle.attention_partial(qd[0, h], kd[0, h], vd[0, h], scale, min(lo, N), max(lo, hi), causal)
            _check(op[s, 0, h], lp[s, 0, h], po, pl, f"range {s} head {h}")
            unseen = ~np.isfinite(pl)
            assert np.all(op[s, 0, h][unseen] == 0.0), f"range {s}: O of unseen rows must be 0"


def test_splitkv_full_size_sampled_rows():
    """A few-heads, long-sequence shape where one Q block per CU is all the
    parallelism attn_fwd has (B=1, H=8, N=8192, d=128, 4 ranges): sampled
    rows of every head against the oracle."""
    B, H, N, d, S = 1, 8, 8192, 128, 4
    inp = make_inputs(B, H, N, d, "bf16", seed=7)
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    for causal in (False, True):
        print(f"\n[splitkv full] causal={causal}", flush=True)
        o, lse, _, _ = attn_fwd_splitkv(q, k, v, S, causal=causal)
        torch.cuda.synchronize()
        rng = np.random.default_rng(8)
        for h in range(H):
            rows = np.sort(rng.choice(N, 24, replace=False))
            rows = np.unique(np.concatenate([rows, [0, 2047, 2048, N - 1]]))
            o_ref, lse_ref = oracle.attention_rows(to_f64(inp["q"][0, h]), to_f64(inp["k"][0, h]),
                                                   to_f64(inp["v"][0, h]), rows, 1 / math.sqrt(d), causal)
            _check(to_f64(o[0, h].cpu())[rows], lse[0, h].cpu().double().numpy()[rows], o_ref, lse_ref,
                   f"head {h}")


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("out", ["fp32", "bf16"])
def test_merge_matches_oracle(d, out):
    """attn_merge on given partials, including a row no partial saw and
    partials of very different magnitude."""
    S, B, H, N = 5, 2, 3, 77
    rng = np.random.default_rng(d)
    o_parts = rng.standard_normal((S, B, H, N, d)).astype(np.float32)
    lse_parts = (rng.standard_normal((S, B, H, N)) * 30).astype(np.float32)
    lse_parts[:, 1, 2, 5] = -np.inf
    lse_parts[2, 0, 0, :] = -np.inf
    o_ref, lse_ref = oracle.merge_partials(o_parts.astype(np.float64), lse_parts.astype(np.float64))
    dt = torch.float32 if out == "fp32" else torch.bfloat16
    o, lse = attn_merge(torch.from_numpy(o_parts).cuda(), torch.from_numpy(lse_parts).cuda(), out_dtype=dt)
    torch.cuda.synchronize()
    og = o.float().cpu().double().numpy()
    lg = lse.cpu().double().numpy()
    assert lg[1, 2, 5] == -np.inf and np.all(og[1, 2, 5] == 0)
    fin = np.isfinite(lse_ref)
    np.testing.assert_allclose(lg[fin], lse_ref[fin], rtol=1e-6, atol=1e-5)
    if out == "fp32":
        np.testing.assert_allclose(og, o_ref, rtol=1e-5, atol=1e-5)
    else:
        np.testing.assert_allclose(og, o_ref, rtol=2 ** -8, atol=1e-3)


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_two_tilings_agree(dtype, d, causal):
    """Two tilings of one computation: attn_fwd (one pass over every K/V
    tile, one running max and sum) and attn_fwd_splitkv with 2 and 3 key
    ranges (a pass per range, each normalised on its own, merged through
    the LSEs in fp32).  Both accumulate in fp32 and round O once, so they
    must agree to within that rounding: at most 0.1 % of the elements more
    than one ulp of the 16-bit type apart, none by more than one ulp plus
    2^-8 max|V| (a weight rounded to the neighbouring 16-bit value moves its
    row by at most 2^-8 of |V_j - O_i|), and the LSE to fp32 precision.  Both round P to 16 bits against a whole-number
    running max, so P's rounding grid is the same whatever the tiling; what
    remains is the fp32 rounding of the exponent s c - m, whose m differs
    between the tilings, which flips the rounding of the rare weight that
    lies within ~1e-6 of a midpoint (a dominant one moves its row by up to
    two ulps).  A race or a tile-order
    dependence in either kernel breaks this without any oracle involved."""
    B, H, N = 2, 3, 1000
    print(f"two tilings {dtype} d={d} causal={causal}", flush=True)
    inp = make_inputs(B, H, N, d, dtype, seed=23 + d)
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    o1, l1 = attn_fwd(q, k, v, causal=causal)
    mant = 7 if dtype == "bf16" else 10
    for splits in (2, 3):
        o2, l2, _, _ = attn_fwd_splitkv(q, k, v, splits, causal=causal)
        torch.cuda.synchronize()
        a, b = o1.double(), o2.double()
        big = torch.maximum(a.abs(), b.abs()).clamp_min(2.0 ** -60)
        ulp = torch.exp2(torch.floor(torch.log2(big)) - mant)
        diff = (a - b).abs()
        over1 = (diff > ulp + 2.0 ** -20).double().mean().item()
        print(f"  splits={splits}: beyond 1 ulp {over1:.2e} of the elements, max {diff.max().item():.3e}", flush=True)
        vmax = v.abs().max().double().item()
        assert (diff <= ulp + 2.0 ** -8 * vmax).all(), f"splits={splits}: an element differs beyond one flipped weight"
        assert over1 <= 1e-3, f"splits={splits}: {over1:.2e} of the elements differ by more than 1 ulp"
        assert (diff > 0).double().mean().item() < 0.1, "the two tilings differ on many elements"
        assert (l1.double() - l2.double()).abs().max().item() <= 1e-5


@pytest.mark.parametrize("d", [64, 128, 256])
def test_splitkv_strided_inputs(d):
    """attn_fwd_splitkv on [B, H, N, d] views of [B, N, H, d] tensors gives
    bitwise the result of the same data laid out contiguously."""
    B, N, H = 1, 700, 3
    print(f"split-KV strided d={d}", flush=True)
    g = torch.Generator().manual_seed(80 + d)
    base = [torch.randn(B, N, H, d, generator=g).to(torch.bfloat16).cuda() for _ in range(3)]
    view = [t.permute(0, 2, 1, 3) for t in base]
    cont = [t.contiguous() for t in view]
    o1, l1, _, _ = attn_fwd_splitkv(*view, 3, causal=True)
    o2, l2, _, _ = attn_fwd_splitkv(*cont, 3, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_splitkv_long_sequence():
    """Split-KV over a 2^19-row head (4 key ranges of 2^17 keys): the merged
    output on sampled rows against the oracle."""
    N, d = 1 << 19, 128
    print(f"split-KV long sequence N={N}", flush=True)
    inp = make_inputs(1, 1, N, d, "bf16", seed=91)
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    o, lse, _, _ = attn_fwd_splitkv(q, k, v, 4, causal=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    rows = np.array(sorted({0, 1, N - 1, N // 4 - 1, N // 4, N // 2} | set(int(r) for r in rng.choice(N, 40, False))))
    o_r, l_r = oracle.attention_rows(to_f64(inp["q"][0, 0]), to_f64(inp["k"][0, 0]), to_f64(inp["v"][0, 0]),
                                     rows, 1 / math.sqrt(d), True)
    _check(to_f64(o[0, 0].cpu())[rows], lse[0, 0].cpu().double().numpy()[rows], o_r, l_r, "split-KV long")
