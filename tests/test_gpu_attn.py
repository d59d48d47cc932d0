"""GPU parity of attn_fwd (fp32 / fp16 / bf16) against the fp64 oracle.

Tolerances
  bf16 / fp16 O: max |err| <= 2e-2 and mean |err| <= 2e-3 (fp32 accumulation);
  fp32 O: max |err| <= 1e-4 (fp32 MFMA and exp2; errors ~1e-6 expected);
  LSE (all dtypes): max |err| <= 1e-3 against the oracle's fp64 value.
The oracle consumes the exact values the GPU receives (inputs upcast to fp64).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from exact_attention_forward_06_amd import attn_fwd
from exact_attention_forward_06_amd.inputs import WORKLOADS, make_inputs, to_f64, workload_inputs

from oracle_pool import head_errors, map_heads, reduce_errors

pytestmark = pytest.mark.gpu

TOL = {  # dtype -> (max abs O, mean abs O, max abs LSE)
    torch.bfloat16: (2e-2, 2e-3, 1e-3),
    torch.float16: (2e-2, 2e-3, 1e-3),
    torch.float32: (1e-4, 1e-5, 1e-4),
}


def _check(o_gpu, lse_gpu, o_ref, lse_ref, dtype, what=""):
    tmax, tmean, tlse = TOL[dtype]
    err = np.abs(o_gpu - o_ref)
    lerr = np.abs(lse_gpu - lse_ref)
    assert np.all(np.isfinite(o_gpu)) and np.all(np.isfinite(lse_gpu)), what
    assert err.max() <= tmax, f"{what}: max |O err| {err.max():.3e} > {tmax}"
    assert err.mean() <= tmean, f"{what}: mean |O err| {err.mean():.3e} > {tmean}"
    assert lerr.max() <= tlse, f"{what}: max |LSE err| {lerr.max():.3e} > {tlse}"
    return err.max(), err.mean(), lerr.max()


def _run(inp, causal, scale=None):
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    o, lse = attn_fwd(q, k, v, causal=causal, softmax_scale=scale)
    torch.cuda.synchronize()
    return o, lse


def _full_compare(inp, causal, dtype, what, scale=None):
    d = inp["q"].shape[-1]
    s = 1 / math.sqrt(d) if scale is None else scale
    o, lse = _run(inp, causal, scale)
    o_ref, lse_ref = oracle.attention(to_f64(inp["q"]), to_f64(inp["k"]), to_f64(inp["v"]), s, causal)
    return _check(to_f64(o), lse.cpu().double().numpy(), o_ref, lse_ref, dtype, what)


def _sample_rows(N, n_tiles_hint=128, seed=0, count=48):
    rng = np.random.default_rng(seed)
    edges = {0, 1, N - 1, N - 2}
    for t in range(n_tiles_hint, N, n_tiles_hint * 7):
        edges.update({t - 1, t})
    rows = set(int(r) for r in rng.choice(N, count, replace=False)) | {e for e in edges if 0 <= e < N}
    return np.array(sorted(rows))


def _sampled_compare(inp, o, lse, causal, dtype, what, heads):
    q, k, v = inp["q"], inp["k"], inp["v"]
    B, H, N, d = q.shape
    s = 1 / math.sqrt(d)
    og = []
    orf = []
    lg = []
    lrf = []
    for i, (b, h) in enumerate(heads):
        rows = _sample_rows(N, seed=i)
        o_r, l_r = oracle.attention_rows(to_f64(q[b, h]), to_f64(k[b, h]), to_f64(v[b, h]), rows, s, causal)
        og.append(to_f64(o[b, h][rows]))
        lg.append(lse[b, h][rows].double().cpu().numpy())
        orf.append(o_r)
        lrf.append(l_r)
    return _check(np.concatenate(og), np.concatenate(lg), np.concatenate(orf), np.concatenate(lrf),
                  dtype, what)


# ---------------------------------------------------------------- the workloads
def test_small_fp32_workload():
    w = WORKLOADS["small_fp32"]
    _full_compare(workload_inputs(w), w.causal, torch.float32, w.name)


def test_bf16_n2048_workload_full():
    w = WORKLOADS["bf16_n2048"]
    _full_compare(workload_inputs(w), w.causal, torch.bfloat16, w.name)


@pytest.mark.parametrize("name", ["bf16_causal_8k", "bf16_d64", "bf16_d256"])
def test_large_workload_sampled(name):
    w = WORKLOADS[name]
    inp = workload_inputs(w)
    o, lse = _run(inp, w.causal)
    o, lse = o.cpu(), lse.cpu()
    rng = np.random.default_rng(1)
    heads = [(0, 0), (w.B - 1, w.H - 1)] + [(int(rng.integers(w.B)), int(rng.integers(w.H))) for _ in range(4)]
    _sampled_compare(inp, o, lse, w.causal, torch.bfloat16, name, heads)
    # every row of every head: finite and LSE at least the largest single score term bound
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()


@pytest.mark.parametrize("N,d,causal", [(1 << 20, 64, True), (1 << 19, 128, False), (1 << 18, 256, True)])
def test_long_sequence_sampled(N, d, causal):
    """One head far longer than the workloads (up to 2^20 rows): every
    kernel's index and offset arithmetic at large N, on rows sampled across
    the whole sequence (the first and last rows, tile edges, random rows)
    against the oracle, which evaluates each sampled row in full."""
    print(f"attn_fwd long sequence N={N} d={d} causal={causal}", flush=True)
    inp = make_inputs(1, 1, N, d, "bf16", seed=N + d)
    o, lse = _run(inp, causal)
    o, lse = o.cpu(), lse.cpu()
    rng = np.random.default_rng(N)
    rows = {0, 1, 63, 64, 127, 128, 255, 256, N // 2 - 1, N // 2, N - 257, N - 256, N - 2, N - 1}
    rows = np.array(sorted(rows | set(int(r) for r in rng.choice(N, 40, replace=False))))
    q, k, v = (to_f64(inp[n][0, 0]) for n in ("q", "k", "v"))
    o_r, l_r = oracle.attention_rows(q, k, v, rows, 1 / math.sqrt(d), causal)
    _check(to_f64(o[0, 0])[rows], lse[0, 0].double().numpy()[rows], o_r, l_r, torch.bfloat16, f"long N={N} d={d}")
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()


@pytest.mark.parametrize("name", ["bf16_causal_8k", "bf16_d64", "bf16_d256"])
def test_large_workload_full(name, capsys):
    """Every head and every row of the large bf16 workloads (the bench's
    launch configuration) against the fp64 oracle, element by element, at
    the bf16 gates: max |O err| <= 2e-2, mean |O err| <= 2e-3 over all
    B*H*N*d elements, max |LSE err| <= 1e-3."""
    w = WORKLOADS[name]
    inp = workload_inputs(w)
    o, lse = _run(inp, w.causal)
    o, lse = o.float().cpu().numpy(), lse.cpu().numpy()
    f32 = {n: inp[n].float().numpy() for n in ("q", "k", "v")}
    tasks = [(f32["q"][b, h], f32["k"][b, h], f32["v"][b, h], o[b, h], lse[b, h], w.scale, w.causal)
             for b in range(w.B) for h in range(w.H)]
    r = reduce_errors(map_heads(head_errors, tasks))
    with capsys.disabled():
        print(f"\n[{name} full] {r['heads']} heads: max|O err| {r['max_abs']:.3e}, "
              f"mean|O err| {r['mean_abs']:.3e}, max|LSE err| {r['lse_max']:.3e}", flush=True)
    assert r["finite"] and r["heads"] == w.B * w.H
    assert r["max_abs"] <= 2e-2 and r["mean_abs"] <= 2e-3 and r["lse_max"] <= 1e-3, r


# ---------------------------------------------------------------- shapes and edges
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 77, 257, 300])
def test_small_shapes(dtype, d, causal, N):
    inp = make_inputs(1, 2, N, d, {torch.bfloat16: "bf16", torch.float16: "fp16",
                                    torch.float32: "fp32"}[dtype], seed=100 + N + d)
    _full_compare(inp, causal, dtype, f"{dtype} d={d} N={N} causal={causal}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "fp16"])
@pytest.mark.parametrize("d", [128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_multi_tile_ragged(causal, d, dtype):
    # several Q blocks and K/V tiles, ragged tail, B*H > 1
    sd = "bf16" if dtype == torch.bfloat16 else "fp16"
    inp = make_inputs(2, 3, 1000, d, sd, seed=7 if d == 128 else 8)
    _full_compare(inp, causal, dtype, f"N=1000 d={d} causal={causal} {sd}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "fp16"])
def test_causal_grid_more_items_than_cus(dtype):
    # causal d = 128 runs as a persistent grid, one workgroup per CU: 3 * 5
    # heads of 18 blocks of 256 rows are 270 items, more than the 256 CUs and
    # not a multiple of 8, so the XCDs' shares differ (34 or 33 items), the
    # workgroups of an XCD take two rounds and the second round is partial
    sd = "bf16" if dtype == torch.bfloat16 else "fp16"
    inp = make_inputs(3, 5, 4500, 128, sd, seed=11)
    _full_compare(inp, True, dtype, f"B=3 H=5 N=4500 d=128 causal (270 items) {sd}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_tile_sum_above_threshold(causal, d):
    """The forward takes P against the running max as it stands and takes a
    tile's exact max only when some lane's sum of P exceeds 2^8.  Scores
    here (log2 units, all queries alike): key 0 at 0 and the rest of keys
    0-127 at -10, so the running max starts at 0; keys 128-255 all at about
    7, so every lane's sum is far above 2^8 while no score is more than 8
    above the running max (the exact step runs and leaves the max alone);
    one key of 256-383 at about 9.5 (the exact step moves the max); random
    scores after that."""
    B, H, N = 1, 2, 700
    base = make_inputs(B, H, N, d, "bf16", seed=41 + d)
    q, k = base["q"].float(), base["k"].float()
    unit = 4.0 * (1 / math.sqrt(d)) * 1.4426950408889634   # score in log2 units per unit of k[..., 0]
    q[..., 0] = 4.0
    q[..., 1:] = 0.0
    k[..., 0] = -10.0 / unit
    k[:, :, 0, 0] = 0.0
    k[:, :, 128:256, 0] = 7.0 / unit
    k[:, :, 300, 0] = 9.5 / unit
    k[:, :, 384:, 0] = torch.randn(B, H, N - 384, generator=torch.Generator().manual_seed(3)) * 2.0 / unit
    inp = dict(q=q.to(torch.bfloat16), k=k.to(torch.bfloat16), v=base["v"])
    _full_compare(inp, causal, torch.bfloat16, f"tile sum above 2^8 d={d} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
def test_d256_split_tile_row_max(causal):
    """At d = 256 two waves share each 32-row query block, each taking half
    of the keys of every 64-key tile for S and half of d for O, and they
    agree on the row max of each tile through LDS.  Here every tile holds
    one dominant key, alternately in its first and its second 32 keys: in
    head 0 the peaks rise by about 10 (log2 units) per tile, so the running
    max moves -- and O is rescaled -- at every tile, from either half; in
    head 1 they fall, so the max stays with the first tile.  N = 340 leaves
    the second half of the last tile wholly past N."""
    B, H, N, d = 1, 2, 340, 256
    base = make_inputs(B, H, N, d, "bf16", seed=31)
    q, k = base["q"].float(), base["k"].float()
    q[..., 0] = 4.0
    k[..., 0] = 0.0
    n_t = (N + 63) // 64
    for t in range(n_t):
        pos = 64 * t + (40 if t % 2 else 10)
        pos = pos if pos < N else 64 * t + 5
        k[0, 0, pos, 0] = 28.0 * t
        k[0, 1, pos, 0] = 28.0 * (n_t - 1 - t)
    inp = dict(q=q.to(torch.bfloat16), k=k.to(torch.bfloat16), v=base["v"])
    _full_compare(inp, causal, torch.bfloat16, f"split-tile row max causal={causal}")


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_strided_bnhd_layout(d, causal):
    """q, k, v as [B, H, N, d] views of [B, N, H, d] tensors (n stride H*d),
    for every kernel (d = 256 is the wave-pair kernel)."""
    B, N, H = 2, 300, 4
    print(f"attn_fwd strided d={d} causal={causal}", flush=True)
    g = torch.Generator().manual_seed(3 + d)
    base = [torch.randn(B, N, H, d, generator=g).to(torch.bfloat16) for _ in range(3)]
    dev = [t.cuda().permute(0, 2, 1, 3) for t in base]       # [B, H, N, d] views, n stride H*d
    assert dev[0].stride() == (N * H * d, d, H * d, 1)
    o, lse = attn_fwd(*dev, causal=causal)
    torch.cuda.synchronize()
    ref = [to_f64(t.permute(0, 2, 1, 3)) for t in base]
    o_ref, lse_ref = oracle.attention(*ref, 1 / math.sqrt(d), causal)
    _check(to_f64(o), lse.cpu().double().numpy(), o_ref, lse_ref, torch.bfloat16, "strided")


def test_custom_scale_and_no_lse():
    inp = make_inputs(1, 2, 200, 64, "bf16", seed=9)
    _full_compare(inp, False, torch.bfloat16, "scale 0.3", scale=0.3)
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    o1, _ = attn_fwd(q, k, v, return_lse=False)
    o2, _ = attn_fwd(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


@pytest.mark.parametrize("d,shape", [(128, (2, 4, 1500)), (256, (2, 4, 1500)),
                                     (128, (2, 16, 4096))],   # 512 causal items: two rounds per CU
                         ids=["d128", "d256", "d128-512items"])
def test_bitwise_deterministic(d, shape):
    B, H, N = shape
    inp = make_inputs(B, H, N, d, "bf16", seed=11)
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    o1, l1 = attn_fwd(q, k, v, causal=True)
    o2, l2 = attn_fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_softmax_invariants_on_gpu():
    # constant V rows -> O equals that row; zero Q -> O is the (prefix) mean of V
    N, d = 333, 128
    g = torch.Generator().manual_seed(5)
    k = torch.randn(1, 1, N, d, generator=g).to(torch.bfloat16)
    row = torch.randn(d, generator=g).to(torch.bfloat16)
    v = row.expand(1, 1, N, d).contiguous()
    q = torch.randn(1, 1, N, d, generator=g).to(torch.bfloat16)
    o, _ = attn_fwd(q.cuda(), k.cuda(), v.cuda(), causal=True)
    torch.cuda.synchronize()
    assert np.abs(to_f64(o[0, 0]) - to_f64(row)[None, :]).max() <= 2e-2
    qz = torch.zeros_like(q)
    v2 = torch.randn(1, 1, N, d, generator=g).to(torch.bfloat16)
    o, lse = attn_fwd(qz.cuda(), k.cuda(), v2.cuda(), causal=True)
    torch.cuda.synchronize()
    pref = np.cumsum(to_f64(v2[0, 0]), 0) / np.arange(1, N + 1)[:, None]
    assert np.abs(to_f64(o[0, 0]) - pref).max() <= 2e-2
    np.testing.assert_allclose(lse[0, 0].cpu().double().numpy(), np.log(np.arange(1, N + 1)), atol=1e-4)


def test_lse_split_merge_on_gpu():
    # attention of N queries over key sets A and B (N keys each), merged
    # through the two LSEs, equals attention over the 2N keys [A; B] (run with
    # the queries repeated to 2N rows, as the API takes N_q = N_k): checks the
    # GPU's LSE as a quantity, not only against the oracle
    B, H, N, d = 1, 2, 500, 128
    inp_a = make_inputs(B, H, N, d, "bf16", seed=41)
    inp_b = make_inputs(B, H, N, d, "bf16", seed=42)
    q = inp_a["q"].cuda()
    ka, va = inp_a["k"].cuda(), inp_a["v"].cuda()
    kb, vb = inp_b["k"].cuda(), inp_b["v"].cuda()
    o1, l1 = attn_fwd(q, ka, va)
    o2, l2 = attn_fwd(q, kb, vb)
    o, lse = attn_fwd(torch.cat([q, q], 2), torch.cat([ka, kb], 2), torch.cat([va, vb], 2))
    torch.cuda.synchronize()
    l1, l2 = l1.double().cpu(), l2.double().cpu()
    lm = torch.logaddexp(l1, l2)
    om = torch.exp(l1 - lm)[..., None] * o1.double().cpu() + torch.exp(l2 - lm)[..., None] * o2.double().cpu()
    assert (lse[:, :, :N].double().cpu() - lm).abs().max().item() <= 1e-3
    assert (o[:, :, :N].double().cpu() - om).abs().max().item() <= 2e-2
    kk = np.concatenate([to_f64(inp_a["k"]), to_f64(inp_b["k"])], 2)
    vv = np.concatenate([to_f64(inp_a["v"]), to_f64(inp_b["v"])], 2)
    qq = np.concatenate([to_f64(inp_a["q"])] * 2, 2)
    _, lse_ref = oracle.attention(qq, kk, vv, 1 / math.sqrt(d), False)
    assert np.abs(lm.numpy() - lse_ref[:, :, :N]).max() <= 1e-3


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
def test_rising_scores_rescale_every_tile(dtype, causal):
    # scores grow steadily along the keys, so the running max moves by far more
    # than the lazy-rescale threshold at every tile (the rescale path runs
    # throughout); O and LSE must still match the oracle
    B, H, N, d = 1, 2, 700, 128
    g = torch.Generator().manual_seed(17)
    u = torch.randn(d, generator=g)
    u = u / u.norm()
    q = (u * 6.0 + 0.1 * torch.randn(B, H, N, d, generator=g))
    ramp = torch.linspace(0.0, 200.0, N)[None, None, :, None]   # ~14 log2 units of score per 64 keys
    k = ramp * u + 0.5 * torch.randn(B, H, N, d, generator=g)
    v = torch.randn(B, H, N, d, generator=g)
    tdt = {"bf16": torch.bfloat16, "fp16": torch.float16}[dtype]
    inp = {"q": q.to(tdt), "k": k.to(tdt), "v": v.to(tdt)}
    _full_compare(inp, causal, tdt, f"rising scores {dtype} causal={causal}")
