"""One-pass online attention and block-state merge, in float64 on the CPU.

TEST INFRASTRUCTURE ONLY (see oracle/reference.py).  These are the pages'
streaming formulation, kept as an independent cross-check of the materialising
definition in reference.py: the two reach the same result by different orders
of arithmetic, which is exactly the claim the method rests on.

Running state per query row, after seeing some keys (FlashAttention explainer,
cztcode.com/2026/5368, §2):
    m  largest score seen so far,
    l  sum of exp(s - m) over the keys seen,
    u  sum of exp(s - m) * v over the keys seen (a vector when v is one).
A new key with score s and value v moves the reference point to
m' = max(m, s); the old sums are rescaled by exp(m - m') (zero while m is
still -inf), the new key enters with weight exp(s - m').  The output is u / l.
This is the online-normaliser recurrence of the Flash Attention wiki note
("Online Softmax") carried through to the output ("online attention"), with
the division deferred to the end as the FlashAttention-2 note describes
("improvement two").

Two states over disjoint key sets combine by moving both to the larger
reference point and adding (explainer §3 and §7):
    m = max(mA, mB),  l = e^(mA-m) lA + e^(mB-m) lB,  u likewise.
"""
from __future__ import annotations

import math

import numpy as np


def _rescale(m_old: float, m_new: float) -> float:
    # exp(m_old - m_new), with the empty state (m_old = -inf) contributing 0
    if m_old == -math.inf:
        return 0.0
    return math.exp(m_old - m_new)


def online_row(scores, values):
    """Stream one query row's scores s_j and values v_j (scalar or vector).

    Returns the final state (m, l, u) without normalising."""
    m = -math.inf
    l = 0.0
    u = None
    for s, v in zip(scores, values):
        v = np.asarray(v, dtype=np.float64)
        if u is None:
            u = np.zeros_like(v)
        s = float(s)
        m_new = max(m, s)
        if m_new == -math.inf:  # still nothing visible
            continue
        alpha = _rescale(m, m_new)
        w = math.exp(s - m_new)
        l = alpha * l + w
        u = alpha * u + w * v
        m = m_new
    return m, l, u


def finish(state):
    """Output u / l and the log-sum-exp m + ln l of a state (empty -> 0, -inf)."""
    m, l, u = state
    if l == 0.0:
        return (np.zeros_like(u) if u is not None else 0.0), -math.inf
    return u / l, m + math.log(l)


def summarize(scores, values):
    """Block state from a whole block at once: its own max, sum and weighted sum."""
    scores = np.asarray(scores, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    m = float(scores.max())
    w = np.exp(scores - m)
    u = np.tensordot(w, values, axes=(0, 0))
    return m, float(w.sum()), u


def merge(a, b):
    """Combine the states of two disjoint key blocks."""
    ma, la, ua = a
    mb, lb, ub = b
    m = max(ma, mb)
    if m == -math.inf:
        return a
    fa = _rescale(ma, m)
    fb = _rescale(mb, m)
    return m, fa * la + fb * lb, fa * np.asarray(ua) + fb * np.asarray(ub)


def online_attention(q, k, v, scale, causal=False):
    """Whole-tensor attention through the online recurrence, row by row.

    Same conventions as reference.attention (fp32-rounded scale, bottom-right
    causal alignment, empty rows -> O = 0 and LSE = -inf)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, Nq, _ = q.shape
    Nk = k.shape[2]
    sc = float(np.float32(scale))
    O = np.zeros((B, H, Nq, v.shape[-1]))
    L = np.zeros((B, H, Nq))
    for b in range(B):
        for h in range(H):
            for i in range(Nq):
                n_vis = min(Nk, i + 1 + Nk - Nq) if causal else Nk
                n_vis = max(n_vis, 0)
                s = sc * (k[b, h, :n_vis] @ q[b, h, i])
                st = online_row(s, v[b, h, :n_vis])
                if st[2] is None:
                    O[b, h, i], L[b, h, i] = 0.0, -math.inf
                else:
                    O[b, h, i], L[b, h, i] = finish(st)
    return O, L
