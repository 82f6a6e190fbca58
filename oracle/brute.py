"""Pure-Python brute force for tiny shapes (loops, math.exp, math.fsum).

TEST INFRASTRUCTURE ONLY (see oracle/reference.py).  No NumPy: every score,
weight and output element is computed by hand from the definition
softmax(scale * q . k) . v (FlashAttention explainer, cztcode.com/2026/5368,
§1), with the row max subtracted first (§2) and exactly rounded sums.
Nested lists in, nested lists out.
"""
from __future__ import annotations

import math


def attention(q, k, v, scale, causal=False):
    """q: [B][H][Nq][d], k: [B][H][Nk][d], v: [B][H][Nk][dv] as nested lists.

    Returns (O [B][H][Nq][dv], LSE [B][H][Nq])."""
    import struct

    sc = struct.unpack("f", struct.pack("f", float(scale)))[0]  # float32 rounding
    O, L = [], []
    for qb, kb, vb in zip(q, k, v):
        Ob, Lb = [], []
        for qh, kh, vh in zip(qb, kb, vb):
            Nq, Nk = len(qh), len(kh)
            dv = len(vh[0]) if Nk else 0
            Oh, Lh = [], []
            for i, qi in enumerate(qh):
                visible = [j for j in range(Nk) if (not causal) or j <= i + Nk - Nq]
                if not visible:
                    Oh.append([0.0] * dv)
                    Lh.append(-math.inf)
                    continue
                s = {j: sc * math.fsum(a * b for a, b in zip(qi, kh[j])) for j in visible}
                mx = max(s.values())
                w = {j: math.exp(s[j] - mx) for j in visible}
                den = math.fsum(w.values())
                Oh.append([math.fsum(w[j] * vh[j][c] for j in visible) / den for c in range(dv)])
                Lh.append(mx + math.log(den))
            Ob.append(Oh)
            Lb.append(Lh)
        O.append(Ob)
        L.append(Lb)
    return O, L
