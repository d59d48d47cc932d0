"""Pins for the fp64 attention oracle: each test checks it against something
other than itself -- brute force, closed forms, invariants the definition
implies, the pages' tiled algorithm, and a library routine."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import attention, attention_head, attention_rows, row_softmax, scores


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# ---------------------------------------------------------------- brute force
def _brute_force_head(q, k, v, scale, causal):
    """Pure-Python loops with math.fsum: no numpy arithmetic at all."""
    n, d = len(q), len(q[0])
    dv = len(v[0])
    o, lse = [], []
    for i in range(n):
        keys = range(i + 1) if causal else range(len(k))
        s = [scale * math.fsum(q[i][c] * k[j][c] for c in range(d)) for j in keys]
        mx = max(s)
        w = [math.exp(x - mx) for x in s]
        tot = math.fsum(w)
        o.append([math.fsum(w[t] * v[j][c] for t, j in enumerate(keys)) / tot for c in range(dv)])
        lse.append(mx + math.log(tot))
    return np.array(o), np.array(lse)


@pytest.mark.parametrize("n,d,causal,seed", [(1, 1, False, 0), (5, 3, False, 1), (7, 8, True, 2),
                                             (16, 8, False, 3), (13, 4, True, 4)])
def test_matches_brute_force(n, d, causal, seed):
    q, k, v = _rand((n, d), seed), _rand((n, d), seed + 10), _rand((n, d), seed + 20)
    scale = 1 / math.sqrt(d)
    o, lse = attention_head(q, k, v, scale, causal)
    ob, lseb = _brute_force_head(q.tolist(), k.tolist(), v.tolist(), scale, causal)
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, lseb, rtol=0, atol=1e-13)


def test_nonsymmetric_operands_are_not_swapped():
    # Q K^T differs from K Q^T: with Nq != rows of K a transposed product
    # would not even have the right shape; with distinct q/k it has other values.
    q = np.array([[1.0, 0.0], [0.0, 2.0]])
    k = np.array([[0.0, 1.0], [3.0, 0.0]])
    s = scores(q, k, 1.0)
    np.testing.assert_array_equal(s, [[0.0, 3.0], [2.0, 0.0]])


# ---------------------------------------------------------------- closed forms
def test_two_key_closed_form():
    # d = 1, scale 1, q = 1, keys 0 and ln 3: softmax weights exactly 1/4, 3/4.
    q = np.array([[1.0]])
    k = np.array([[0.0], [math.log(3.0)]])
    v = np.array([[4.0, -8.0], [8.0, 4.0]])
    o, lse = attention_head(q, k, v, 1.0)
    np.testing.assert_allclose(o, [[0.25 * 4 + 0.75 * 8, 0.25 * -8 + 0.75 * 4]], atol=1e-15)
    np.testing.assert_allclose(lse, [math.log(4.0)], atol=1e-15)


def test_scale_is_applied():
    q = np.array([[2.0]])
    k = np.array([[1.0], [0.0]])
    v = np.array([[1.0], [0.0]])
    for scale in (1.0, 0.5, 0.125):
        o, lse = attention_head(q, k, v, scale)
        w = math.exp(2 * scale) / (math.exp(2 * scale) + 1)
        assert abs(o[0, 0] - w) < 1e-15
        assert abs(lse[0] - math.log(math.exp(2 * scale) + 1)) < 1e-14


# ---------------------------------------------------------------- mask
def test_causal_row0_sees_only_key0():
    q, k, v = _rand((9, 4), 5), _rand((9, 4), 6), _rand((9, 4), 7)
    o, lse, s, p = attention_head(q, k, v, 0.5, causal=True, return_sp=True)
    np.testing.assert_array_equal(o[0], v[0])
    assert lse[0] == pytest.approx(0.5 * float(q[0] @ k[0]), abs=1e-15)
    upper = np.triu(np.ones((9, 9), bool), 1)
    assert np.all(p[upper] == 0.0)
    assert np.all(np.isneginf(s[upper]))
    assert np.all(np.isfinite(s[~upper]))


def test_causal_prefix_means_with_zero_queries():
    n, d = 11, 3
    q = np.zeros((n, d))
    k, v = _rand((n, d), 8), _rand((n, d), 9)
    o, lse = attention_head(q, k, v, 1.0, causal=True)
    pref = np.cumsum(v, axis=0) / np.arange(1, n + 1)[:, None]
    np.testing.assert_allclose(o, pref, atol=1e-14)
    np.testing.assert_allclose(lse, np.log(np.arange(1, n + 1)), atol=1e-14)


# ---------------------------------------------------------------- softmax invariants
@pytest.mark.parametrize("causal", [False, True])
def test_rows_of_p_sum_to_one(causal):
    q, k = _rand((33, 16), 10) * 3, _rand((33, 16), 11) * 3
    p, m, l = row_softmax(scores(q, k, 0.25, causal))
    assert np.max(np.abs(p.sum(1) - 1)) <= 1e-12
    assert np.all(p >= 0)


def test_constant_v_gives_v():
    q, k = _rand((20, 8), 12), _rand((20, 8), 13)
    row = _rand((8,), 14)
    v = np.tile(row, (20, 1))
    for causal in (False, True):
        o, _ = attention_head(q, k, v, 0.3, causal)
        np.testing.assert_allclose(o, np.tile(row, (20, 1)), atol=1e-14)


def test_single_key_returns_its_row():
    q, k, v = _rand((1, 16), 15), _rand((1, 16), 16), _rand((1, 16), 17)
    o, lse = attention_head(q, k, v, 0.25)
    np.testing.assert_array_equal(o[0], v[0])
    assert lse[0] == pytest.approx(0.25 * float(q[0] @ k[0]), abs=1e-15)


def test_zero_queries_give_mean_and_log_n():
    n = 17
    q = np.zeros((n, 4))
    k, v = _rand((n, 4), 18), _rand((n, 4), 19)
    o, lse = attention_head(q, k, v, 1.0)
    np.testing.assert_allclose(o, np.tile(v.mean(0), (n, 1)), atol=1e-14)
    np.testing.assert_allclose(lse, np.full(n, math.log(n)), atol=1e-14)


def test_joint_permutation_of_keys_and_values():
    q, k, v = _rand((12, 8), 20), _rand((12, 8), 21), _rand((12, 8), 22)
    perm = np.random.default_rng(23).permutation(12)
    o1, l1 = attention_head(q, k, v, 0.4)
    o2, l2 = attention_head(q, k[perm], v[perm], 0.4)
    np.testing.assert_allclose(o1, o2, atol=1e-14)
    np.testing.assert_allclose(l1, l2, atol=1e-14)


def test_large_scores_stay_finite():
    # The max subtraction keeps exp in range even for scores ~1e3.
    q, k, v = _rand((6, 4), 24) * 40, _rand((6, 4), 25) * 40, _rand((6, 4), 26)
    o, lse = attention_head(q, k, v, 1.0)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    ob, lb = _brute_force_head(q.tolist(), k.tolist(), v.tolist(), 1.0, False)
    np.testing.assert_allclose(o, ob, atol=1e-12)


# ---------------------------------------------------------------- the pages' tiled algorithm
def _tiled_online_softmax(q, k, v, scale, causal, br, bc):
    """The blockwise forward of the "FlashAttention-2/3" page (section
    技术原理, the tiled pseudo-code, FA-2 loop order), in fp64, with the
    1/sqrt(d) scale applied and a single normalisation after the last K/V
    block (the page's deferred rescaling, FlashAttention-2 改进一)."""
    n, d = q.shape
    o = np.zeros((n, v.shape[1]))
    lse = np.zeros(n)
    for i0 in range(0, n, br):
        qi = q[i0:i0 + br]
        rows = np.arange(i0, min(n, i0 + br))
        acc = np.zeros((len(rows), v.shape[1]))
        l = np.zeros(len(rows))
        m = np.full(len(rows), -np.inf)
        for j0 in range(0, k.shape[0], bc):
            kj, vj = k[j0:j0 + bc], v[j0:j0 + bc]
            s = (qi @ kj.T) * scale
            if causal:
                cols = np.arange(j0, j0 + len(kj))
                s = np.where(cols[None, :] > rows[:, None], -np.inf, s)
            m_blk = s.max(1)
            m_new = np.maximum(m, m_blk)
            safe = np.where(np.isneginf(m_new), 0.0, m_new)
            p = np.exp(s - safe[:, None])
            alpha = np.exp(m - safe)
            l = alpha * l + p.sum(1)
            acc = alpha[:, None] * acc + p @ vj
            m = m_new
        o[rows] = acc / l[:, None]
        lse[rows] = m + np.log(l)
    return o, lse


@pytest.mark.parametrize("br,bc", [(1, 1), (3, 4), (4, 3), (16, 16), (5, 16), (16, 7)])
@pytest.mark.parametrize("causal", [False, True])
def test_blockwise_equals_two_pass(br, bc, causal):
    n, d = 29, 8
    q, k, v = _rand((n, d), 30) * 2, _rand((n, d), 31) * 2, _rand((n, d), 32)
    o, lse = attention_head(q, k, v, 1 / math.sqrt(d), causal)
    ot, lset = _tiled_online_softmax(q, k, v, 1 / math.sqrt(d), causal, br, bc)
    np.testing.assert_allclose(o, ot, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lset, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- library cross-check
@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_sdpa_fp64(causal):
    B, H, N, d = 2, 3, 37, 16
    q, k, v = _rand((B, H, N, d), 40), _rand((B, H, N, d), 41), _rand((B, H, N, d), 42)
    o, lse = attention(q, k, v, 1 / math.sqrt(d), causal)
    tq, tk, tv = (torch.from_numpy(a) for a in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal,
                                                           scale=1 / math.sqrt(d)).numpy()
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-13)
    s = torch.einsum("bhnd,bhmd->bhnm", tq, tk) / math.sqrt(d)
    if causal:
        s = s.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), rtol=0, atol=1e-13)


# ---------------------------------------------------------------- LSE
def test_lse_normalises_p():
    q, k = _rand((21, 8), 50), _rand((21, 8), 51)
    v = _rand((21, 8), 52)
    for causal in (False, True):
        o, lse, s, p = attention_head(q, k, v, 0.35, causal, return_sp=True)
        p2 = np.exp(s - lse[:, None])
        np.testing.assert_allclose(p2.sum(1), 1.0, atol=1e-13)
        np.testing.assert_allclose(p2, p, atol=1e-14)


def test_lse_split_merge():
    """Results over two halves of the keys merge to the full result through
    their LSEs (what makes partial results over K/V shards combinable)."""
    n, d = 40, 8
    q, k, v = _rand((n, d), 53), _rand((n, d), 54), _rand((n, d), 55)
    o, lse = attention_head(q, k, v, 0.3)
    o1, l1 = attention_head(q, k[:17], v[:17], 0.3)
    o2, l2 = attention_head(q, k[17:], v[17:], 0.3)
    lm = np.logaddexp(l1, l2)
    om = np.exp(l1 - lm)[:, None] * o1 + np.exp(l2 - lm)[:, None] * o2
    np.testing.assert_allclose(lm, lse, atol=1e-13)
    np.testing.assert_allclose(om, o, atol=1e-13)


# ------------------------------------------------------ key-range partials
def _brute_force_partial(q, k, v, scale, causal, k_begin, k_end):
    """Pure-Python loops: softmax over the keys of [k_begin, k_end) that a
    row sees; (0, -inf) for a row that sees none."""
    o, lse = [], []
    for i in range(len(q)):
        keys = [j for j in range(k_begin, k_end) if not (causal and j > i)]
        if not keys:
            o.append([0.0] * len(v[0]))
            lse.append(-math.inf)
            continue
        s = [scale * math.fsum(a * b for a, b in zip(q[i], k[j])) for j in keys]
        mx = max(s)
        w = [math.exp(x - mx) for x in s]
        tot = math.fsum(w)
        o.append([math.fsum(w[t] * v[j][c] for t, j in enumerate(keys)) / tot for c in range(len(v[0]))])
        lse.append(mx + math.log(tot))
    return np.array(o), np.array(lse)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("rng_", [(0, 5), (3, 9), (6, 11), (11, 11)])
def test_partial_matches_brute_force(causal, rng_):
    n, d = 11, 4
    q, k, v = _rand((n, d), 70), _rand((n, d), 71), _rand((n, d), 72)
    o, lse = oracle.attention_partial(q, k, v, 0.6, rng_[0], rng_[1], causal)
    ob, lb = _brute_force_partial(q.tolist(), k.tolist(), v.tolist(), 0.6, causal, *rng_)
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-13)
    assert np.array_equal(np.isinf(lse), np.isinf(lb))
    np.testing.assert_allclose(lse[np.isfinite(lb)], lb[np.isfinite(lb)], rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_partials_over_a_partition_merge_to_attention(causal):
    """Ranges that partition the keys (uneven, one past N, one empty) merge
    back to the full result; a range a row cannot see carries (0, -inf)."""
    n, d = 37, 6
    q, k, v = _rand((n, d), 73), _rand((n, d), 74), _rand((n, d), 75)
    cuts = [0, 5, 5, 19, 30, 40]
    parts = [oracle.attention_partial(q, k, v, 0.4, a, b, causal) for a, b in zip(cuts, cuts[1:])]
    o, lse = oracle.merge_partials(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
    oe, le = attention_head(q, k, v, 0.4, causal)
    np.testing.assert_allclose(o, oe, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, le, rtol=0, atol=1e-13)
    assert np.all(parts[1][1] == -np.inf) and np.all(parts[1][0] == 0)   # the empty range [5, 5)
    if causal:                                                            # rows 0..18 cannot see [19, 30)
        assert np.all(parts[3][1][:19] == -np.inf) and np.all(parts[3][0][:19] == 0)


def test_merge_is_associative_and_handles_all_empty_rows():
    rng = np.random.default_rng(76)
    o_parts = rng.standard_normal((3, 2, 5, 4))
    lse_parts = rng.standard_normal((3, 2, 5)) * 3
    lse_parts[:, 1, 2] = -np.inf          # a row no range saw
    lse_parts[0, 0, 0] = -np.inf          # a row one range did not see
    o, lse = oracle.merge_partials(o_parts, lse_parts)
    o12, l12 = oracle.merge_partials(o_parts[:2], lse_parts[:2])
    o3, l3 = oracle.merge_partials(np.stack([o12, o_parts[2]]), np.stack([l12, lse_parts[2]]))
    fin = np.isfinite(lse)
    np.testing.assert_allclose(o3, o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l3[fin], lse[fin], rtol=0, atol=1e-13)
    assert lse[1, 2] == -np.inf and np.all(o[1, 2] == 0)
    # a single partial merges to itself
    o1, l1 = oracle.merge_partials(o_parts[:1], lse_parts[:1])
    f1 = np.isfinite(lse_parts[0])
    np.testing.assert_allclose(o1[f1], o_parts[0][f1], atol=1e-15)
    assert np.all(o1[~f1] == 0) and np.all(l1[~f1] == -np.inf)


def test_rows_subset_equals_full():
    n, d = 50, 8
    q, k, v = _rand((n, d), 60), _rand((n, d), 61), _rand((n, d), 62)
    rows = np.array([0, 3, 17, 49])
    for causal in (False, True):
        o, lse = attention_head(q, k, v, 0.3, causal)
        orr, lr = attention_rows(q, k, v, rows, 0.3, causal)
        np.testing.assert_allclose(orr, o[rows], atol=1e-14)
        np.testing.assert_allclose(lr, lse[rows], atol=1e-14)


def test_batched_layout():
    B, H, N, d = 2, 2, 9, 4
    q, k, v = _rand((B, H, N, d), 70), _rand((B, H, N, d), 71), _rand((B, H, N, d), 72)
    o, lse = attention(q, k, v, 0.5, True)
    for b in range(B):
        for h in range(H):
            ob, lb = _brute_force_head(q[b, h].tolist(), k[b, h].tolist(), v[b, h].tolist(), 0.5, True)
            np.testing.assert_allclose(o[b, h], ob, atol=1e-13)
            np.testing.assert_allclose(lse[b, h], lb, atol=1e-13)


def test_credited_flops():
    assert oracle.credited_flops(2, 16, 8192, 128, True) == 549755813888.0
    assert oracle.credited_flops(4, 16, 2048, 128, False) == 137438953472.0


# ------------------------------------------------------------------ backward
def _loss(q, k, v, do, scale, causal):
    return float(np.sum(attention_head(q, k, v, scale, causal)[0] * do))


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_finite_differences(causal):
    """Central differences of L = sum(dO * O) in a few random directions of
    Q, K and V against the oracle's gradients (first-order identity)."""
    n, d = 9, 5
    q, k, v, do = (_rand((n, d), s) for s in (80, 81, 82, 83))
    scale = 0.7
    dq, dk, dv = oracle.attention_backward_head(q, k, v, do, scale, causal)
    rng = np.random.default_rng(84)
    eps = 1e-6
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        for _ in range(3):
            e = rng.standard_normal((n, d))
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p = [a + eps * e if i == which else a for i, a in enumerate(args_p)]
            args_m = [a - eps * e if i == which else a for i, a in enumerate(args_m)]
            fd = (_loss(*args_p, do, scale, causal) - _loss(*args_m, do, scale, causal)) / (2 * eps)
            assert abs(fd - float(np.sum(grad * e))) <= 1e-7 * max(1.0, abs(fd)), (which, fd)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_torch_autograd_fp64(causal):
    n, d = 40, 16
    q, k, v, do = (_rand((2, n, d), s) for s in (85, 86, 87, 88))
    dq, dk, dv = oracle.attention_backward(q, k, v, do, 0.25, causal)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=0.25)
    out.backward(torch.tensor(do))
    for ours, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        np.testing.assert_allclose(ours, ref.numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_invariants(causal):
    """Rows of dS sum to zero (so the key gradients sum to zero), and the
    value gradients sum to the summed upstream gradient (rows of P sum to 1)."""
    n, d = 30, 8
    q, k, v, do = (_rand((n, d), s) for s in (89, 90, 91, 92))
    dq, dk, dv = oracle.attention_backward_head(q, k, v, do, 0.5, causal)
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-12)
    np.testing.assert_allclose(dv.sum(axis=0), do.sum(axis=0), atol=1e-12)
    if causal:   # query 0 sees only key 0: its dS row is P_00 (dP_00 - D_0) = 0
        np.testing.assert_allclose(dq[0], 0.0, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_rows_match_finite_differences(causal):
    """attention_backward_rows against central differences of L = sum(dO * O)
    in random directions of one query row at a time (the first-order
    identity, independent of the full-head backward), and equal to the
    full-head backward's rows."""
    n, d = 11, 6
    q, k, v, do = (_rand((n, d), s) for s in (93, 94, 95, 96))
    scale = 0.6
    rows = [0, 3, 10]
    dq_rows = oracle.attention_backward_rows(q, k, v, do, rows, scale, causal)
    rng = np.random.default_rng(97)
    eps = 1e-6
    for r_i, r in enumerate(rows):
        for _ in range(3):
            e = np.zeros((n, d))
            e[r] = rng.standard_normal(d)
            fd = (_loss(q + eps * e, k, v, do, scale, causal) - _loss(q - eps * e, k, v, do, scale, causal)) / (2 * eps)
            assert abs(fd - float(np.dot(dq_rows[r_i], e[r]))) <= 1e-7 * max(1.0, abs(fd)), (r, fd)
    dq, _, _ = oracle.attention_backward_head(q, k, v, do, scale, causal)
    np.testing.assert_allclose(dq_rows, dq[rows], rtol=0, atol=1e-12)
