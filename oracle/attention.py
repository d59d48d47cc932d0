"""fp64 CPU oracle for the exact-attention forward.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import this module; the HIP path never does.  It
shares no code with the kernels or the C-ABI library.

What it computes is the plain definition, written out step by step with the
N x N score matrix S and probability matrix P materialised:

  * The attention definition O = softmax(Q K^T / sqrt(d)) V: the displayed
    equation at the top of the "FlashAttention-3" page (lyirs.cc), restated
    in its section "数学对象没变，执行图变了" (the maths is unchanged).
  * The three unfused steps S = Q K^T, P = softmax(S), O = P V: the
    "FlashAttention-2/3" page (compassingai.com), section "技术原理",
    block "标准注意力" (standard attention).  That block omits the 1/sqrt(d)
    factor; the oracle takes the scale as an argument (callers pass
    1/sqrt(d), as the FlashAttention-3 equation has it).
  * The row statistics m_i = max_j s_ij and l_i = sum_j exp(s_ij - m_i): the
    "FlashAttention-3" page, section "先回顾 FlashAttention 家族保留下来的部分".
  * The per-row logsumexp output (LSE): named in section 2.2 of the
    "Flash Attention V3" page (jsqmd.com) without a definition.  Reading
    adopted: LSE_i = m_i + ln l_i over the scaled, masked scores (natural
    log), i.e. ln sum_j exp(scale * q_i . k_j) over the keys row i sees.
  * The causal mask: section 2.2 of the "Flash Attention V3" page speaks of
    skipping fully masked blocks for autoregressive models.  Reading adopted:
    query i sees keys 0..i (top-left aligned, N_q = N_k), so no row is ever
    fully masked.

All arithmetic is float64 whatever the input dtype; inputs are upcast
exactly (bf16/fp16/fp32 values are representable in fp64).
"""
from __future__ import annotations

import numpy as np


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def scores(q, k, scale, causal=False):
    """S = (Q K^T) * scale for one head, with masked entries set to -inf.

    q: [Nq, d], k: [Nk, d].  Causal masking sets S_ij = -inf for j > i.
    """
    q = _f64(q)
    k = _f64(k)
    s = (q @ k.T) * float(scale)
    if causal:
        nq, nk = s.shape
        i = np.arange(nq)[:, None]
        j = np.arange(nk)[None, :]
        s = np.where(j > i, -np.inf, s)
    return s


def row_softmax(s):
    """Row softmax of a materialised score matrix.

    Returns (P, m, l) with m_i = max_j s_ij, l_i = sum_j exp(s_ij - m_i),
    P = exp(S - m) / l.  Masked entries (-inf) give exactly 0.
    """
    m = np.max(s, axis=1)
    e = np.exp(s - m[:, None])
    l = np.sum(e, axis=1)
    p = e / l[:, None]
    return p, m, l


def attention_head(q, k, v, scale, causal=False, return_sp=False):
    """One head: returns (O [N,d], LSE [N]) in fp64, optionally S and P."""
    s = scores(q, k, scale, causal)
    p, m, l = row_softmax(s)
    o = p @ _f64(v)
    lse = m + np.log(l)
    if return_sp:
        return o, lse, s, p
    return o, lse


def attention(q, k, v, scale, causal=False):
    """Batched [..., N, d] inputs; loops over the leading dims one head at a
    time so that only one N x N matrix is alive.  Returns fp64 (O, LSE)."""
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    lead = q.shape[:-2]
    n, d = q.shape[-2:]
    qf = q.reshape(-1, n, d)
    kf = k.reshape(-1, k.shape[-2], d)
    vf = v.reshape(-1, v.shape[-2], v.shape[-1])
    o = np.empty((qf.shape[0], n, vf.shape[-1]), np.float64)
    lse = np.empty((qf.shape[0], n), np.float64)
    for h in range(qf.shape[0]):
        o[h], lse[h] = attention_head(qf[h], kf[h], vf[h], scale, causal)
    return o.reshape(*lead, n, vf.shape[-1]), lse.reshape(*lead, n)


def attention_rows(q, k, v, rows, scale, causal=False):
    """The same definition evaluated for a subset of query rows of one head
    (q, k, v: [N, d]; rows: int indices).  Used where the full N x N matrix
    of a large workload would take too long: each output row depends only on
    its own query row and all keys."""
    rows = np.asarray(rows, dtype=np.int64)
    q = _f64(q)[rows]
    k = _f64(k)
    s = (q @ k.T) * float(scale)
    if causal:
        j = np.arange(k.shape[0])[None, :]
        s = np.where(j > rows[:, None], -np.inf, s)
    p, m, l = row_softmax(s)
    o = p @ _f64(v)
    return o, m + np.log(l)


def attention_partial(q, k, v, scale, k_begin, k_end, causal=False):
    """One head's attention restricted to the keys [k_begin, k_end): the
    definition above with the score matrix cut to those columns (the causal
    mask stays in global indices).  This is what a key range of split-KV
    computes -- the sequence-parallel split of the "FlashAttention-2/3" page
    (section "FlashAttention-2 的三大改进", 改进二), with the range's LSE as its
    state ("Flash Attention V3" page, section 2.2).

    Returns fp64 (O_part [N, d], LSE_part [N]); a row that sees no key of the
    range gets O_part = 0 and LSE_part = -inf.
    """
    s = scores(q, k, scale, causal)[:, k_begin:k_end]
    n = s.shape[0]
    vr = _f64(v)[k_begin:k_end]
    o = np.zeros((n, vr.shape[1]), np.float64)
    lse = np.full(n, -np.inf)
    seen = np.any(np.isfinite(s), axis=1) if s.shape[1] else np.zeros(n, bool)
    if np.any(seen):
        p, m, l = row_softmax(s[seen])
        o[seen] = p @ vr
        lse[seen] = m + np.log(l)
    return o, lse


def merge_partials(o_parts, lse_parts):
    """Combine partial results over disjoint key ranges:
    LSE = ln sum_s exp(LSE_s), O = sum_s exp(LSE_s - LSE) O_s (the online
    softmax update of the "FlashAttention-2/3" page, section "在线 Softmax",
    applied to whole ranges).  o_parts [S, ..., N, d], lse_parts [S, ..., N];
    rows whose partials are all -inf get O = 0 and LSE = -inf."""
    o_parts = _f64(o_parts)
    lse_parts = _f64(lse_parts)
    m = np.max(lse_parts, axis=0)
    seen = np.isfinite(m)
    msafe = np.where(seen, m, 0.0)
    w = np.exp(lse_parts - msafe[None])            # 0 for -inf partials
    tot = np.sum(w, axis=0)
    o = np.sum(w[..., None] * o_parts, axis=0) / np.where(seen, tot, 1.0)[..., None]
    o = np.where(seen[..., None], o, 0.0)
    lse = np.where(seen, msafe + np.log(np.where(seen, tot, 1.0)), -np.inf)
    return o, lse


def attention_backward_head(q, k, v, do, scale, causal=False):
    """Gradients of one head's attention output O = softmax(S) V, S = Q K^T *
    scale (masked entries -inf), with respect to Q, K and V for an upstream
    gradient dO: the chain rule through the three unfused steps, with S and P
    materialised.  The pages name the backward pass ("FlashAttention-3" page,
    section "适用范围和工程限制": fp16/bf16 forward and backward) and its
    recomputation of P from the stored logsumexp ("Flash Attention V3" page,
    sections 2.1 and 2.2) without a formula; this is the plain gradient:

        dV = P^T dO
        dP = dO V^T
        dS_ij = P_ij (dP_ij - D_i),   D_i = sum_j P_ij dP_ij = dO_i . O_i
        dQ = dS K * scale,   dK = dS^T Q * scale

    Returns fp64 (dQ, dK, dV).
    """
    q, k, v, do = (_f64(x) for x in (q, k, v, do))
    s = scores(q, k, scale, causal)
    p, _, _ = row_softmax(s)
    dv = p.T @ do
    dp = do @ v.T
    dsum = np.sum(p * dp, axis=1)
    ds = p * (dp - dsum[:, None])
    dq = ds @ k * float(scale)
    dk = ds.T @ q * float(scale)
    return dq, dk, dv


def attention_backward_rows(q, k, v, do, rows, scale, causal=False):
    """dQ of attention_backward_head for a subset of query rows of one head
    (q, k, v, do: [N, d]; rows: int indices).  Row i of dQ depends only on
    query row i, its upstream gradient row and all keys and values, so each
    sampled row is the gradient's definition evaluated for that row alone:

        s_i = q_i K^T * scale (masked -inf),   p_i = softmax(s_i)
        dp_i = dO_i V^T,   D_i = p_i . dp_i,   dq_i = (p_i o (dp_i - D_i)) K * scale

    Used where a whole head's N x N matrices would take too long.  Returns
    fp64 dQ[rows]."""
    rows = np.asarray(rows, dtype=np.int64)
    q, k, v, do = (_f64(x) for x in (q, k, v, do))
    s = (q[rows] @ k.T) * float(scale)
    if causal:
        j = np.arange(k.shape[0])[None, :]
        s = np.where(j > rows[:, None], -np.inf, s)
    p, _, _ = row_softmax(s)
    dp = do[rows] @ v.T
    dsum = np.sum(p * dp, axis=1)
    ds = p * (dp - dsum[:, None])
    return ds @ k * float(scale)


def attention_backward(q, k, v, do, scale, causal=False):
    """Batched [..., N, d] version of attention_backward_head (one head at a
    time).  Returns fp64 (dQ, dK, dV)."""
    q, k, v, do = (np.asarray(x) for x in (q, k, v, do))
    lead = q.shape[:-2]
    n, d = q.shape[-2:]
    outs = [np.empty((int(np.prod(lead)) if lead else 1, n, d), np.float64) for _ in range(3)]
    qf, kf, vf, df = (x.reshape(-1, n, d) for x in (q, k, v, do))
    for h in range(qf.shape[0]):
        for o, g in zip(outs, attention_backward_head(qf[h], kf[h], vf[h], df[h], scale, causal)):
            o[h] = g
    return tuple(o.reshape(*lead, n, d) for o in outs)


def credited_flops(B, H, N, d, causal):
    """Throughput convention: 4*B*H*N^2*d, halved under the causal mask."""
    f = 4.0 * B * H * N * N * d
    return f / 2 if causal else f
