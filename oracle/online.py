"""Streaming evaluation of exact attention by key blocks, float64, CPU.

TEST INFRASTRUCTURE ONLY (see oracle/reference.py).  An independent
cross-check of the materialising definition in reference.py: the same result
reached by a different order of arithmetic, which is the claim the method
rests on.

For a set of query rows and a block of keys, the partial state of every row
is a triple of arrays
    top   [n]      the largest score of the block (-inf if the row sees none),
    mass  [n]      the sum over the block of exp(score - top),
    acc   [n, dv]  the sum over the block of exp(score - top) * value.
The states of two disjoint key sets combine by referring both to the larger
top and adding; a set's output is acc / mass and its log-sum-exp is
top + ln(mass).  Scanning the keys one at a time is the per-key running
recurrence of the FlashAttention explainer (cztcode.com/2026/5368, §2; the
Flash Attention wiki note, "Online Softmax" and "online attention"); scanning
them in larger blocks is the tiled form with the block-merge rule of
explainer §3 and §7.  The division by mass happens once, at the end (wiki,
FlashAttention-2 notes, improvement two).

Everything is vectorised over rows; the block boundaries are arbitrary, so
tests can check that any partition of the keys gives the definition's result.
"""
from __future__ import annotations

import numpy as np

NEG_INF = -np.inf


def _as_values(values):
    """Values as a [keys, dv] float64 matrix (a vector is one column)."""
    values = np.asarray(values, dtype=np.float64)
    return values[:, None] if values.ndim == 1 else values


def _weight(x_top, new_top):
    """exp(x_top - new_top) per row, 0 where the row's old state is empty."""
    live = x_top != NEG_INF
    return np.where(live, np.exp(np.where(live, x_top, 0.0) - np.where(live, new_top, 0.0)), 0.0)


def block_state(scores, values):
    """Partial state of rows `scores` [n, kb] (-inf = hidden key) over the key
    block whose values are `values` [kb, dv]."""
    scores = np.atleast_2d(np.asarray(scores, dtype=np.float64))
    values = _as_values(values)
    n = scores.shape[0]
    if scores.shape[1] == 0:
        return np.full(n, NEG_INF), np.zeros(n), np.zeros((n, values.shape[1]))
    top = scores.max(axis=1)
    live = top != NEG_INF
    shifted = scores - np.where(live, top, 0.0)[:, None]
    w = np.exp(shifted)  # hidden keys -> exp(-inf) = 0
    return top, w.sum(axis=1), w @ values


def combine(x, y):
    """State over the union of the disjoint key sets of states x and y."""
    tx, mx, ax = x
    ty, my, ay = y
    t = np.maximum(tx, ty)
    fx = _weight(tx, t)
    fy = _weight(ty, t)
    return t, fx * mx + fy * my, fx[:, None] * ax + fy[:, None] * ay


def scan(scores, values, bounds):
    """Fold the state of a row set over consecutive key blocks.

    scores [n, Nk], values [Nk, dv]; bounds: increasing cut positions inside
    (0, Nk) -- block i holds keys bounds[i-1] .. bounds[i]-1.  Returns the
    state over all Nk keys."""
    scores = np.atleast_2d(np.asarray(scores, dtype=np.float64))
    values = _as_values(values)
    edges = [0] + [int(b) for b in bounds] + [scores.shape[1]]
    state = block_state(scores[:, :0], values[:0])  # the empty state
    for lo, hi in zip(edges[:-1], edges[1:]):
        state = combine(state, block_state(scores[:, lo:hi], values[lo:hi]))
    return state


def per_key(scores, values):
    """The state after scanning the keys one at a time (explainer §2)."""
    nk = np.atleast_2d(np.asarray(scores)).shape[1]
    return scan(scores, values, range(1, nk))


def normalise(state):
    """(O [n, dv], LSE [n]) of a state; rows that saw no key: O = 0, LSE = -inf."""
    top, mass, acc = state
    live = mass > 0
    safe = np.where(live, mass, 1.0)
    out = np.where(live[:, None], acc / safe[:, None], 0.0)
    with np.errstate(divide="ignore"):
        lse = np.where(live, top + np.log(safe), NEG_INF)
    return out, lse


def streamed_attention(q, k, v, scale, causal=False, block=1):
    """[B, H, N, d] attention through the block scan (keys in blocks of
    `block`), with the oracle's conventions: fp32-rounded scale, bottom-right
    causal alignment, empty rows O = 0 and LSE = -inf."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, Nq, _ = q.shape
    Nk = k.shape[2]
    sc = float(np.float32(scale))
    out = np.zeros((B, H, Nq, v.shape[-1]))
    lse = np.zeros((B, H, Nq))
    hidden = (np.arange(Nk)[None, :] > (np.arange(Nq) + (Nk - Nq))[:, None]) if causal else None
    for b in range(B):
        for h in range(H):
            s = sc * (q[b, h] @ k[b, h].T)
            if causal:
                s = np.where(hidden, NEG_INF, s)
            st = scan(s, v[b, h], range(block, Nk, block))
            out[b, h], lse[b, h] = normalise(st)
    return out, lse
