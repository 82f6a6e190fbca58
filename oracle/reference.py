"""Plain fp64 definition of exact attention (the CPU oracle).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module; the product path never does.

Everything here is the textbook definition, written out with S and P
materialised in float64, one (batch, head) at a time:

    S = scale * Q K^T,   P = softmax(S) row-wise,   O = P V

(FlashAttention explainer, cztcode.com/2026/5368, §1 "the intermediate
matrices"; Flash Attention wiki note, astro-wiki, "bottleneck of standard
self-attention"; AI圣经13 FlashAttention review, chengyansuo.com, §02 on the
standard implementation).  The row max is subtracted before exponentiating
(safe softmax: wiki note, "Safe Softmax"; explainer §2), which leaves the
result unchanged and keeps exp finite for large scores.

Readings where the pages are silent (each listed in the design notes):
  * scale is an explicit argument, rounded to float32 first, because the
    library receives it as a float32;
  * causal masking is bottom-right aligned: query i sees key j iff
    j <= i + (Nk - Nq); for Nq == Nk this is the usual lower triangle;
  * a row with no visible key has O = 0 and LSE = -inf;
  * the saved statistic is LSE_i = ln sum_j exp(S_ij) over visible j
    (the "normalisation statistics" of explainer §3 / review §03).
"""
from __future__ import annotations

import numpy as np

NEG_INF = -np.inf


def _f64(x):
    """Exact upcast to a float64 array; accepts numpy arrays or (bf16, fp32,
    device) torch tensors without importing torch."""
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def f32_scale(scale: float) -> float:
    """The scale as the library sees it: rounded to float32, then widened."""
    return float(np.float32(scale))


def head_attention(Q, K, V, scale, causal=False, q_pos=None, nq_total=None):
    """Exact attention for one head.

    Q: [n, d] query rows, K: [Nk, d], V: [Nk, dv] (any real dtype; computed in
    float64).  q_pos: index of each query row within its length-nq_total query
    sequence (defaults to 0..n-1 with nq_total = n); only causal masking uses it.

    Returns (O [n, dv] float64, LSE [n] float64).
    """
    Q = _f64(Q)
    K = _f64(K)
    V = _f64(V)
    n = Q.shape[0]
    Nk = K.shape[0]
    if q_pos is None:
        q_pos = np.arange(n)
        nq_total = n
    q_pos = np.asarray(q_pos, dtype=np.int64)

    # Step 1: the full score matrix, materialised.
    S = f32_scale(scale) * (Q @ K.T)  # [n, Nk]

    # Step 2: causal mask, bottom-right aligned.
    if causal:
        last_visible = q_pos + (Nk - nq_total)  # key j visible iff j <= last_visible
        hidden = np.arange(Nk)[None, :] > last_visible[:, None]
        S = np.where(hidden, NEG_INF, S)

    # Step 3: safe softmax: row max, shifted exponentials, row sum, P.
    m = S.max(axis=1) if Nk > 0 else np.full(n, NEG_INF)
    empty = m == NEG_INF
    m_shift = np.where(empty, 0.0, m)
    E = np.exp(S - m_shift[:, None])  # exp(-inf) = 0 for hidden keys
    l = E.sum(axis=1)
    P = E / np.where(empty, 1.0, l)[:, None]  # materialised probabilities

    # Step 4: output and log-sum-exp.
    O = P @ V
    with np.errstate(divide="ignore"):
        lse = np.where(empty, NEG_INF, m_shift + np.log(np.where(empty, 1.0, l)))
    O[empty] = 0.0
    return O, lse


def attention(q, k, v, scale, causal=False):
    """Exact attention over [B, H, Nq, d] / [B, H, Nk, d] / [B, H, Nk, dv].

    Returns O [B, H, Nq, dv] and LSE [B, H, Nq], both float64."""
    B, H, Nq, _ = q.shape
    dv = v.shape[-1]
    O = np.zeros((B, H, Nq, dv))
    L = np.zeros((B, H, Nq))
    for b in range(B):
        for h in range(H):
            O[b, h], L[b, h] = head_attention(q[b, h], k[b, h], v[b, h], scale, causal)
    return O, L


def attention_rows(q, k, v, scale, causal, rows):
    """The same definition evaluated for selected output rows only.

    rows: iterable of (b, h, i).  Returns O [len(rows), dv] and LSE [len(rows)].
    Used at sizes where the full oracle would take too long."""
    rows = list(rows)
    Nq = q.shape[2]
    dv = v.shape[-1]
    O = np.zeros((len(rows), dv))
    L = np.zeros(len(rows))
    # group by head so K and V are converted once per head
    by_head: dict = {}
    for r, (b, h, i) in enumerate(rows):
        by_head.setdefault((b, h), []).append((r, i))
    for (b, h), items in by_head.items():
        idx = np.array([i for _, i in items])
        Kh = _f64(k[b, h])
        Vh = _f64(v[b, h])
        Qr = _f64(q[b, h])[idx]
        o, lse = head_attention(Qr, Kh, Vh, scale, causal, q_pos=idx, nq_total=Nq)
        for j, (r, _) in enumerate(items):
            O[r] = o[j]
            L[r] = lse[j]
    return O, L


def decode(q, kcache, vcache, seqlens, offsets, scale, heads=None, seqs=None):
    """Exact single-query attention over a packed token-major cache.

    q: [B, H, d]; kcache, vcache: [T, H, d]; sequence b owns cache rows
    offsets[b] .. offsets[b] + seqlens[b] - 1.  Every key of the sequence is
    visible (a single new query sees its whole history: explainer §6).
    `seqs` / `heads` restrict the evaluation to a subset (others stay NaN).

    Returns O [B, H, d] and LSE [B, H], float64."""
    B, H, d = q.shape
    O = np.full((B, H, vcache.shape[-1]), np.nan)
    L = np.full((B, H), np.nan)
    seqs = range(B) if seqs is None else seqs
    heads = range(H) if heads is None else heads
    for b in seqs:
        lo = int(offsets[b])
        n = int(seqlens[b])
        for h in heads:
            Kb = _f64(kcache[lo:lo + n, h])
            Vb = _f64(vcache[lo:lo + n, h])
            o, lse = head_attention(_f64(q[b, h])[None, :], Kb, Vb, scale)
            O[b, h] = o[0]
            L[b, h] = lse[0]
    return O, L


def decode_paged(q, kpages, vpages, block_table, seqlens, scale, heads=None, seqs=None):
    """Exact single-query attention over a paged cache.

    kpages, vpages: [num_pages, page_size, H, d]; block_table: [B, max_blocks].
    Key t of sequence b sits in page block_table[b, t // page_size] at slot
    t % page_size (the block table maps a sequence's logical blocks to the
    physical pages that hold them).  The sequence's keys are gathered in
    order and attended exactly as in `decode`.

    Returns O [B, H, d] and LSE [B, H], float64."""
    B, H, d = q.shape
    page_size = kpages.shape[1]
    bt = np.asarray(block_table.cpu() if hasattr(block_table, "cpu") else block_table)
    O = np.full((B, H, vpages.shape[-1]), np.nan)
    L = np.full((B, H), np.nan)
    seqs = range(B) if seqs is None else seqs
    heads = range(H) if heads is None else heads
    for b in seqs:
        n = int(seqlens[b])
        t = np.arange(n)
        page = bt[b, t // page_size]
        slot = t % page_size
        for h in heads:
            Kb = _f64(kpages[page, slot, h]) if n else np.zeros((0, d))
            Vb = _f64(vpages[page, slot, h]) if n else np.zeros((0, vpages.shape[-1]))
            o, lse = head_attention(_f64(q[b, h])[None, :], Kb, Vb, scale)
            O[b, h] = o[0]
            L[b, h] = lse[0]
    return O, L


def attention_varlen(q, k, v, cu_q, cu_k, scale, causal=False, seqs=None, heads=None):
    """Exact attention over a packed batch of sequences of different lengths.

    q: [Tq, H, d], k: [Tk, H, d], v: [Tk, H, dv], token-major; sequence b owns
    query rows cu_q[b] .. cu_q[b+1]-1 and key rows cu_k[b] .. cu_k[b+1]-1, and
    attends only within itself.  Causal masking is bottom-right aligned within
    each sequence (its queries are the last of its keys, as in a chunked
    prefill).  `seqs` / `heads` restrict the evaluation (others stay NaN).

    Returns O [Tq, H, dv] and LSE [H, Tq], float64."""
    cu_q = [int(x) for x in (cu_q.cpu() if hasattr(cu_q, "cpu") else cu_q)]
    cu_k = [int(x) for x in (cu_k.cpu() if hasattr(cu_k, "cpu") else cu_k)]
    Tq, H, _ = q.shape
    dv = v.shape[-1]
    O = np.full((Tq, H, dv), np.nan)
    L = np.full((H, Tq), np.nan)
    seqs = range(len(cu_q) - 1) if seqs is None else seqs
    heads = range(H) if heads is None else heads
    for b in seqs:
        qs, qe, ks, ke = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        if qe == qs:
            continue
        for h in heads:
            o, lse = head_attention(_f64(q[qs:qe, h]), _f64(k[ks:ke, h]), _f64(v[ks:ke, h]),
                                    scale, causal)
            O[qs:qe, h] = o
            L[h, qs:qe] = lse
    return O, L


def head_attention_grad(Q, K, V, dO, scale, causal=False):
    """Gradients of exact attention for one head, from the definition.

    With S = scale * Q K^T (hidden keys masked), P = softmax(S) row-wise and
    O = P V, the chain rule through O and through the row softmax gives

        dV = P^T dO
        dP = dO V^T
        dS = P * (dP - rowsum(P * dP))      (the softmax Jacobian, row by row)
        dQ = scale * dS K,   dK = scale * dS^T Q

    all materialised in float64.  A row with no visible key has P = 0 and
    contributes nothing.  The pages keep only O and the row statistics and
    recompute the needed blocks in the backward pass (AI圣经13 review §03,
    "recomputation"; explainer §3); this is the plain definition that such a
    backward must reproduce.

    Returns (dQ [n, d], dK [Nk, d], dV [Nk, dv]) float64."""
    Q, K, V, dO = _f64(Q), _f64(K), _f64(V), _f64(dO)
    n, Nk = Q.shape[0], K.shape[0]
    S = f32_scale(scale) * (Q @ K.T)
    if causal:
        hidden = np.arange(Nk)[None, :] > (np.arange(n) + (Nk - n))[:, None]
        S = np.where(hidden, NEG_INF, S)
    m = S.max(axis=1) if Nk > 0 else np.full(n, NEG_INF)
    empty = m == NEG_INF
    E = np.exp(S - np.where(empty, 0.0, m)[:, None])
    P = E / np.where(empty, 1.0, E.sum(axis=1))[:, None]
    P[empty] = 0.0
    dV = P.T @ dO
    dP = dO @ V.T
    dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
    sc = f32_scale(scale)
    return sc * (dS @ K), sc * (dS.T @ Q), dV


def attention_grad(q, k, v, do, scale, causal=False, heads=None):
    """head_attention_grad over [B, H, N, d] tensors; returns dQ, dK, dV
    (float64, same shapes as q, k, v).  `heads`: optional list of (b, h)
    pairs to evaluate (others stay NaN)."""
    B, H = q.shape[0], q.shape[1]
    dQ = np.full(q.shape, np.nan)
    dK = np.full(k.shape, np.nan)
    dV = np.full(v.shape, np.nan)
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    for b, h in pairs:
        dQ[b, h], dK[b, h], dV[b, h] = head_attention_grad(q[b, h], k[b, h], v[b, h], do[b, h],
                                                           scale, causal)
    return dQ, dK, dV


BLOCK = 64  # rows and keys per block of a block-sparse mask


def attention_block_sparse(q, k, v, block_mask, scale, causal=False, heads=None):
    """Exact attention in which key j is visible to query i only if the block
    mask admits the pair of 64-row / 64-key blocks (block_mask[h][i // 64]
    [j // 64] != 0) and, with causal, j <= i + Nk - Nq.  The pages' way of
    reaching long sequences skips whole tiles by a sparsity pattern (review
    §05) without giving one; here the pattern is an input.

    q: [B, H, Nq, d], k, v: [B, H, Nk, d]; block_mask [H, ceil(Nq/64),
    ceil(Nk/64)], shared by the batch.  Rows with no visible key: O = 0,
    LSE = -inf.  Returns O, LSE float64 (heads outside `heads`, a list of
    (b, h) pairs, stay NaN)."""
    B, H, Nq, _ = q.shape
    Nk = k.shape[2]
    M = np.asarray(block_mask.cpu() if hasattr(block_mask, "cpu") else block_mask) != 0
    O = np.full((B, H, Nq, v.shape[-1]), np.nan)
    L = np.full((B, H, Nq), np.nan)
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    ii, jj = np.arange(Nq)[:, None], np.arange(Nk)[None, :]
    for b, h in pairs:
        visible = M[h][ii // BLOCK, jj // BLOCK]
        if causal:
            visible = visible & (jj <= ii + (Nk - Nq))
        Q, K, V = _f64(q[b, h]), _f64(k[b, h]), _f64(v[b, h])
        S = np.where(visible, f32_scale(scale) * (Q @ K.T), NEG_INF)
        m = S.max(axis=1) if Nk > 0 else np.full(Nq, NEG_INF)
        empty = m == NEG_INF
        m_shift = np.where(empty, 0.0, m)
        E = np.exp(S - m_shift[:, None])
        l = E.sum(axis=1)
        P = E / np.where(empty, 1.0, l)[:, None]
        Ob = P @ V
        Ob[empty] = 0.0
        O[b, h] = Ob
        with np.errstate(divide="ignore"):
            L[b, h] = np.where(empty, NEG_INF, m_shift + np.log(np.where(empty, 1.0, l)))
    return O, L

