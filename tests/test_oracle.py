"""Pins of the CPU oracle against what the pages and mathematics fix.

Each pin is a function of a per-head attention implementation, so the same
pins run against the oracle itself and against deliberately broken copies of
it (planted on the CPU, below): every plausible slip must fail at least one
pin.
"""
import inspect
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import brute, online
from oracle import reference as ref
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")
TOL = 1e-12


def attn(impl, q, k, v, scale, causal=False):
    B, H, Nq, _ = q.shape
    O = np.zeros((B, H, Nq, v.shape[-1]))
    L = np.zeros((B, H, Nq))
    for b in range(B):
        for h in range(H):
            O[b, h], L[b, h] = impl(q[b, h], k[b, h], v[b, h], scale, causal)
    return O, L


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def close(a, b, tol=TOL):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape
    both_inf = np.isneginf(a) & np.isneginf(b)
    diff = np.abs(np.where(both_inf, 0.0, a) - np.where(both_inf, 0.0, b))
    assert np.all(np.isfinite(diff)), "non-finite mismatch"
    assert diff.max(initial=0.0) <= tol, f"max diff {diff.max()}"


# ----------------------------------------------------------------- pins
def pin_worked_example(impl):
    """The scalar example of the explainer (§2) as d = 1 attention, scale 1."""
    g = json.load(open(GOLDEN))
    K = np.array(g["scores"], dtype=np.float64)[:, None]
    V = np.array(g["values"], dtype=np.float64)[:, None]
    O, L = impl(np.ones((1, 1)), K, V, 1.0, False)
    close(O[0, 0], float(g["O"]))
    close(L[0], float(g["LSE"]))
    # closed form, independent of the fixture
    e = math.exp
    closed = (2 * e(-2) - e(-3) + 4 + 3 * e(-4)) / (e(-2) + e(-3) + 1 + e(-4))
    close(O[0, 0], closed)


def pin_brute(impl):
    """Pure-Python brute force on tiny shapes, causal on and off, Nq != Nk."""
    for (B, H, Nq, Nk, d, dv, causal, seed) in [
        (2, 2, 5, 5, 4, 3, False, 1), (1, 2, 3, 7, 8, 8, True, 2),
        (2, 1, 7, 3, 2, 5, True, 3), (1, 1, 9, 9, 8, 4, True, 4),
        (1, 1, 4, 6, 3, 3, False, 5),
    ]:
        q, k, v = rand((B, H, Nq, d), seed), rand((B, H, Nk, d), seed + 10), rand((B, H, Nk, dv), seed + 20)
        scale = 1 / math.sqrt(d) if d != 4 else 0.7  # includes scales float32 cannot hold exactly
        Ob, Lb = brute.attention(q.tolist(), k.tolist(), v.tolist(), scale, causal)
        O, L = attn(impl, q, k, v, scale, causal)
        close(O, Ob)
        close(L, Lb)


def pin_constant_k(impl):
    """Every key equal -> equal scores -> uniform weights over the visible keys:
    O_i = mean of visible V rows, LSE_i = s + ln n_i with n_i = number visible."""
    for Nq, Nk, causal in [(6, 6, False), (6, 6, True), (4, 9, True), (9, 4, True), (5, 8, False)]:
        d = 5
        q = rand((1, 1, Nq, d), 11)
        krow = rand((d,), 12)
        k = np.broadcast_to(krow, (1, 1, Nk, d)).copy()
        v = rand((1, 1, Nk, 3), 13)
        scale = 0.3
        O, L = attn(impl, q, k, v, scale, causal)
        sc = float(np.float32(scale))
        for i in range(Nq):
            n = min(Nk, i + 1 + Nk - Nq) if causal else Nk
            if n <= 0:
                close(O[0, 0, i], np.zeros(3))
                assert L[0, 0, i] == -math.inf
                continue
            close(O[0, 0, i], v[0, 0, :n].mean(axis=0))
            close(L[0, 0, i], sc * float(q[0, 0, i] @ krow) + math.log(n))


def pin_scale_zero(impl):
    q, k, v = rand((1, 2, 5, 4), 21), rand((1, 2, 7, 4), 22), rand((1, 2, 7, 2), 23)
    O, L = attn(impl, q, k, v, 0.0, False)
    close(O, np.broadcast_to(v.mean(axis=2, keepdims=True), O.shape))
    close(L, np.full(L.shape, math.log(7)))


def pin_single_key(impl):
    """Nk = 1: the lone key gets all the weight; LSE is its score."""
    q, k, v = rand((1, 1, 4, 6), 31), rand((1, 1, 1, 6), 32), rand((1, 1, 1, 6), 33)
    O, L = attn(impl, q, k, v, 0.25, False)
    close(O[0, 0], np.broadcast_to(v[0, 0, 0], (4, 6)))
    close(L[0, 0], 0.25 * (q[0, 0] @ k[0, 0, 0]))


def pin_ones_v(impl):
    """Rows of P sum to 1, so V = 1 gives O = 1 on every non-empty row."""
    q, k = rand((1, 1, 6, 4), 41) * 5, rand((1, 1, 6, 4), 42) * 5
    v = np.ones((1, 1, 6, 3))
    O, _ = attn(impl, q, k, v, 0.5, True)
    close(O, np.ones_like(O))


def pin_shift(impl):
    """Adding c_i to every score of row i (via an extra q/k coordinate) leaves O
    unchanged and raises LSE_i by c_i."""
    Nq, Nk, d = 5, 8, 4
    q, k, v = rand((1, 1, Nq, d), 51), rand((1, 1, Nk, d), 52), rand((1, 1, Nk, 3), 53)
    scale = 0.5
    c = rand((Nq,), 54) * 40
    q2 = np.concatenate([q, (c / scale)[None, None, :, None]], axis=-1)
    k2 = np.concatenate([k, np.ones((1, 1, Nk, 1))], axis=-1)
    O1, L1 = attn(impl, q, k, v, scale, True)
    O2, L2 = attn(impl, q2, k2, v, scale, True)
    close(O2, O1, 1e-11)
    close(L2, L1 + c, 1e-11)


def pin_online(impl):
    """The streaming (m, l, u) evaluation of the pages reaches the same result,
    key by key (the running recurrence) and in blocks of 3 (tiles + merge)."""
    for Nq, Nk, causal in [(7, 7, True), (5, 11, True), (11, 5, True), (6, 9, False)]:
        q, k, v = rand((2, 2, Nq, 8), 61) * 3, rand((2, 2, Nk, 8), 62) * 3, rand((2, 2, Nk, 4), 63)
        O, L = attn(impl, q, k, v, 0.4, causal)
        for block in (1, 3):
            Oo, Lo = online.streamed_attention(q, k, v, 0.4, causal, block=block)
            close(O, Oo)
            close(L, Lo)


def pin_sdpa(impl):
    """torch's scaled_dot_product_attention in float64 on the CPU (tiny shapes).
    Its is_causal is top-left aligned, so Nq != Nk uses an explicit mask."""
    for Nq, Nk, causal in [(6, 6, False), (6, 6, True), (4, 7, True), (5, 9, False)]:
        q, k, v = rand((2, 3, Nq, 8), 71), rand((2, 3, Nk, 8), 72), rand((2, 3, Nk, 8), 73)
        scale = 1 / math.sqrt(8)
        mask = None
        if causal:
            i = torch.arange(Nq)[:, None]
            j = torch.arange(Nk)[None, :]
            mask = j <= i + (Nk - Nq)
        ref_o = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
            attn_mask=mask, scale=float(np.float32(scale))).numpy()
        O, _ = attn(impl, q, k, v, scale, causal)
        close(O, ref_o, 1e-12)


PINS = [pin_worked_example, pin_brute, pin_constant_k, pin_scale_zero, pin_single_key,
        pin_ones_v, pin_shift, pin_online, pin_sdpa]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin):
    pin(ref.head_attention)


# ------------------------------------------------- online / merge pins
def _row(x):
    return np.asarray(x, dtype=np.float64)[None, :]


def test_online_worked_example():
    g = json.load(open(GOLDEN))
    st = online.per_key(_row(g["scores"]), np.asarray(g["values"], dtype=np.float64))
    o, lse = online.normalise(st)
    close(o[0, 0], float(g["O"]))
    close(lse[0], float(g["LSE"]))
    # a naive exp without the max shift overflows, which is why the shift exists
    with np.errstate(over="ignore"):
        assert np.isinf(np.exp(np.float64(1000.0)))


def test_merge_worked_example():
    g = json.load(open(GOLDEN))
    s, v = _row(g["scores"]), np.asarray(g["values"], dtype=np.float64)

    def flat(st):
        return [st[0][0], st[1][0], st[2][0, 0]]

    left = online.block_state(s[:, :2], v[:2])
    right = online.block_state(s[:, 2:], v[2:])
    close(flat(left), [float(x) for x in g["left_state"]])
    close(flat(right), [float(x) for x in g["right_state"]])
    merged = online.combine(left, right)
    close(flat(merged), [float(x) for x in g["merged_state"]])
    close(merged[2][0, 0] / merged[1][0], float(g["merged_O"]))
    # the same split through the scan, and the per-key scan
    close(flat(online.scan(s, v, [2])), [float(x) for x in g["merged_state"]])
    close(online.normalise(online.per_key(s, v))[0][0, 0], float(g["merged_O"]))


def test_merge_invariance_every_split():
    """Splitting a row's keys anywhere (and in many pieces) and merging the
    block states reproduces the oracle row."""
    rng = np.random.default_rng(5)
    for trial in range(6):
        n, dv = int(rng.integers(2, 40)), int(rng.integers(1, 9))
        s = rng.standard_normal(n) * (1 + 300 * (trial % 2))
        v = rng.standard_normal((n, dv))
        O, L = ref.head_attention(np.ones((1, 1)), s[:, None], v, 1.0)
        sr = s[None, :]
        for cut in range(1, n):
            o, lse = online.normalise(online.scan(sr, v, [cut]))
            close(o[0], O[0], 1e-12 * max(1, np.abs(O).max()))
            close(lse[0], L[0], 1e-12 * max(1.0, abs(L[0])))
        for _ in range(5):
            k = int(rng.integers(2, min(n, 8) + 1))
            cuts = np.sort(rng.choice(np.arange(1, n), size=k - 1, replace=False))
            parts = np.split(np.arange(n), cuts)
            states = [online.block_state(sr[:, p], v[p]) for p in parts]
            order = rng.permutation(len(states))  # merge order must not matter
            st = states[order[0]]
            for j in order[1:]:
                st = online.combine(st, states[j])
            o, lse = online.normalise(st)
            close(o[0], O[0], 1e-12 * max(1, np.abs(O).max()))
            close(lse[0], L[0], 1e-12 * max(1.0, abs(L[0])))


# ---------------------------------------------------- conventions
def test_empty_rows_causal_more_queries_than_keys():
    q, k, v = rand((1, 1, 7, 4), 81), rand((1, 1, 3, 4), 82), rand((1, 1, 3, 4), 83)
    O, L = oracle.attention(q, k, v, 0.5, True)
    # bottom-right alignment: query i sees keys j <= i - 4, so rows 0..3 see none
    assert np.all(O[0, 0, :4] == 0) and np.all(np.isneginf(L[0, 0, :4]))
    assert np.all(np.isfinite(L[0, 0, 4:]))


def test_attention_rows_matches_full():
    q, k, v = rand((2, 3, 33, 8), 91), rand((2, 3, 40, 8), 92), rand((2, 3, 40, 8), 93)
    O, L = oracle.attention(q, k, v, 0.35, True)
    rows = [(1, 2, 0), (0, 0, 32), (1, 1, 17), (0, 2, 5), (1, 2, 31)]
    Or, Lr = oracle.attention_rows(q, k, v, 0.35, True, rows)
    for r, (b, h, i) in enumerate(rows):
        close(Or[r], O[b, h, i], 1e-13)
        close(Lr[r], L[b, h, i], 1e-13)


def test_decode_oracle_is_fwd_at_one_query():
    lens = torch.tensor([5, 1, 17, 9], dtype=torch.int32)
    q, kc, vc, sl, off = workloads.decode_inputs(4, 3, 8, lens, seed=3, dtype="f32")
    O, L = oracle.decode(q, kc, vc, sl, off, 0.3)
    for b in range(4):
        lo, n = int(off[b]), int(sl[b])
        qb = q[b][:, None, :].numpy()[None]                        # [1,H,1,d]
        kb = kc[lo:lo + n].permute(1, 0, 2).numpy()[None]           # [1,H,n,d]
        vb = vc[lo:lo + n].permute(1, 0, 2).numpy()[None]
        Of, Lf = oracle.attention(qb, kb, vb, 0.3, causal=True)     # Nq = 1 sees all keys
        close(O[b], Of[0, :, 0], 1e-13)
        close(L[b], Lf[0, :, 0], 1e-13)


def test_accepts_bf16_tensors_exactly():
    q, k, v = workloads.prefill_inputs(1, 2, 9, 9, 8, "bf16", seed=4)
    O1, L1 = oracle.attention(q, k, v, 0.2, True)
    O2, L2 = oracle.attention(q.double().numpy(), k.double().numpy(), v.double().numpy(), 0.2, True)
    close(O1, O2, 0.0)
    close(L1, L2, 0.0)


# ------------------------------------------- planted mistakes (CPU only)
MUTATIONS = {
    "dropped_scale": ("S = f32_scale(scale) * (Q @ K.T)", "S = (Q @ K.T)"),
    "top_left_causal": ("last_visible = q_pos + (Nk - nq_total)", "last_visible = q_pos"),
    "causal_off_by_one": ("hidden = np.arange(Nk)[None, :] > last_visible", "hidden = np.arange(Nk)[None, :] >= last_visible"),
    "no_max_shift": ("E = np.exp(S - m_shift[:, None])", "E = np.exp(S)"),
    "unnormalised_P": ("P = E / np.where(empty, 1.0, l)[:, None]", "P = E"),
    "lse_without_max": ("m_shift + np.log(", "0.0 + np.log("),
    "reversed_values": ("O = P @ V", "O = P @ V[::-1]"),
    "transposed_scores": ("(Q @ K.T)  #", "(K @ Q.T).T[:, ::-1]  #"),
    "max_over_wrong_axis": ("m = S.max(axis=1)", "m = S.max(axis=1) * 0 + S.max()"),
}


def _mutant(name):
    src = inspect.getsource(ref.head_attention)
    old, new = MUTATIONS[name]
    assert old in src, f"mutation anchor for {name} not found"
    ns = dict(ref.__dict__)
    exec(src.replace(old, new), ns)
    return ns["head_attention"]


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name):
    impl = _mutant(name)
    failed = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(impl)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            failed.append(pin.__name__)
    assert failed, f"mutation {name} slipped past every pin"


def _pages_by_hand(cache, lens, offs, bt, P, num_pages):
    """A page pool filled one token at a time from the block-table definition."""
    T, H, d = cache.shape
    pool = np.zeros((num_pages, P, H, d))
    for b, n in enumerate(lens):
        for t in range(n):
            pool[bt[b][t // P], t % P] = cache[offs[b] + t]
    return pool


@pytest.mark.parametrize("P", [1, 3, 16, 64])
def test_paged_decode_oracle_is_packed_decode(P):
    """Paging only moves keys around: gathering a sequence's keys through any
    block table gives the packed decode exactly (the packed oracle is pinned
    to the forward definition above)."""
    rng = np.random.default_rng(17 + P)
    lens = [0, 1, P, P + 1, 3 * P - 1, 40]
    B, H, d = len(lens), 2, 8
    offs = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(int)
    T = int(sum(lens))
    kc, vc = rng.standard_normal((T, H, d)), rng.standard_normal((T, H, d))
    q = rng.standard_normal((B, H, d))
    need = [-(-n // P) for n in lens]
    num_pages = sum(need) + 3
    order = rng.permutation(num_pages)
    bt = np.full((B, max(need)), -1)
    at = 0
    for b, n in enumerate(need):
        bt[b, :n] = order[at:at + n]
        at += n
    kp = _pages_by_hand(kc, lens, offs, bt, P, num_pages)
    vp = _pages_by_hand(vc, lens, offs, bt, P, num_pages)
    O1, L1 = oracle.decode(q, kc, vc, lens, offs, 0.3)
    O2, L2 = oracle.decode_paged(q, kp, vp, bt, lens, 0.3)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)
    # a block-table entry pointing at another sequence's page is noticed
    # (swapping two of a sequence's own pages would not be: with every key
    # visible, attention does not depend on key order)
    b, other = lens.index(3 * P - 1), lens.index(40)
    bad = bt.copy()
    bad[b, 0] = bt[other, 0]
    O3, _ = oracle.decode_paged(q, kp, vp, bad, lens, 0.3)
    assert not np.allclose(O3[b], O1[b])


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_oracle_against_brute_force(causal):
    """Packed sequences of different lengths (an empty one, queries fewer than
    keys as in a chunked prefill): every sequence attends only within itself,
    bottom-right aligned; checked against the pure-Python definition run per
    sequence."""
    rng = np.random.default_rng(5)
    lq, lk = [3, 0, 5, 1, 4], [3, 2, 9, 4, 0]
    cq = np.concatenate([[0], np.cumsum(lq)])
    ck = np.concatenate([[0], np.cumsum(lk)])
    H, d = 2, 4
    q = rng.standard_normal((cq[-1], H, d))
    k = rng.standard_normal((ck[-1], H, d))
    v = rng.standard_normal((ck[-1], H, 3))
    O, L = oracle.attention_varlen(q, k, v, cq, ck, 0.7, causal)
    for b in range(len(lq)):
        qb = [[q[cq[b]:cq[b + 1], h].tolist() for h in range(H)]]
        kb = [[k[ck[b]:ck[b + 1], h].tolist() for h in range(H)]]
        vb = [[v[ck[b]:ck[b + 1], h].tolist() for h in range(H)]]
        Ob, Lb = brute.attention(qb, kb, vb, 0.7, causal)
        for h in range(H):
            for i in range(lq[b]):
                r = cq[b] + i
                if lk[b] == 0 or (causal and i + lk[b] - lq[b] < 0):
                    assert np.all(O[r, h] == 0) and L[h, r] == -np.inf
                    continue
                close(O[r, h], np.array(Ob[0][h][i]), 1e-13)
                close(L[h, r], Lb[0][h][i], 1e-13)


# ------------------------------------------------------------- backward pass

def _torch_grads(Q, K, V, dO, scale, causal):
    q, k, v = (torch.tensor(x, requires_grad=True) for x in (Q, K, V))
    S = float(np.float32(scale)) * q @ k.T
    n, Nk = Q.shape[0], K.shape[0]
    if causal:
        S = S.masked_fill(torch.arange(Nk)[None, :] > (torch.arange(n) + (Nk - n))[:, None],
                          -float("inf"))
    P = torch.softmax(S, 1).nan_to_num(0.0)  # rows with no visible key: P = 0
    (P @ v * torch.tensor(dO)).sum().backward()
    return q.grad.numpy(), k.grad.numpy(), v.grad.numpy()


@pytest.mark.parametrize("causal,n,Nk", [(False, 6, 9), (True, 6, 9), (True, 9, 6), (False, 1, 1)])
def test_grad_oracle_matches_float64_autograd(causal, n, Nk):
    rng = np.random.default_rng(n * 10 + Nk)
    Q, K = rng.standard_normal((n, 5)), rng.standard_normal((Nk, 5))
    V, dO = rng.standard_normal((Nk, 3)), rng.standard_normal((n, 3))
    got = oracle.head_attention_grad(Q, K, V, dO, 0.4, causal)
    for g, t in zip(got, _torch_grads(Q, K, V, dO, 0.4, causal)):
        close(g, t, 1e-13)


def test_grad_oracle_matches_finite_differences():
    """Central differences of L = sum(O * dO) through the forward oracle."""
    rng = np.random.default_rng(3)
    Q, K, V = rng.standard_normal((3, 2)), rng.standard_normal((4, 2)), rng.standard_normal((4, 2))
    dO = rng.standard_normal((3, 2))
    for causal in (False, True):
        got = oracle.head_attention_grad(Q, K, V, dO, 0.7, causal)

        def loss(Qx, Kx, Vx):
            return float((ref.head_attention(Qx, Kx, Vx, 0.7, causal)[0] * dO).sum())

        for which, X in enumerate((Q, K, V)):
            num = np.zeros_like(X)
            for idx in np.ndindex(X.shape):
                args = [Q.copy(), K.copy(), V.copy()]
                h = 1e-6
                args[which][idx] += h
                up = loss(*args)
                args[which][idx] -= 2 * h
                num[idx] = (up - loss(*args)) / (2 * h)
            close(got[which], num, 1e-7)


def test_grad_closed_forms():
    rng = np.random.default_rng(4)
    n, d = 5, 4
    Q, dO = rng.standard_normal((n, d)), rng.standard_normal((n, 3))
    # one key: P = 1, so dS = 0 -> dQ = dK = 0 and dV = sum of dO
    K1, V1 = rng.standard_normal((1, d)), rng.standard_normal((1, 3))
    dQ, dK, dV = oracle.head_attention_grad(Q, K1, V1, dO, 0.3)
    assert np.abs(dQ).max() < 1e-15 and np.abs(dK).max() < 1e-15
    close(dV[0], dO.sum(axis=0), 1e-14)
    # identical keys: P uniform, each row of dS sums to zero -> dQ = 0
    K = np.repeat(rng.standard_normal((1, d)), 6, axis=0)
    V = rng.standard_normal((6, 3))
    dQ, _, dV = oracle.head_attention_grad(Q, K, V, dO, 0.3)
    assert np.abs(dQ).max() < 1e-14
    close(dV, np.repeat(dO.sum(axis=0, keepdims=True) / 6, 6, axis=0), 1e-14)
    # causal with more queries than keys: the first rows see no key and add nothing
    Q2, dO2 = rng.standard_normal((7, d)), rng.standard_normal((7, 3))
    dQ, dK, dV = oracle.head_attention_grad(Q2, K[:3], V[:3], dO2, 0.3, causal=True)
    assert np.all(dQ[:4] == 0)
    g2 = oracle.head_attention_grad(Q2[4:], K[:3], V[:3], dO2[4:], 0.3, causal=True)
    close(dK, g2[1], 1e-14)
    close(dV, g2[2], 1e-14)


def test_grad_row_term_equals_rowsum_do_o():
    """rowsum(P * dP) = rowsum(dO * O): the per-row term the backward can take
    from the saved output instead of from the scores."""
    rng = np.random.default_rng(6)
    Q, K, V = rng.standard_normal((8, 4)), rng.standard_normal((11, 4)), rng.standard_normal((11, 4))
    dO = rng.standard_normal((8, 4))
    O, _ = ref.head_attention(Q, K, V, 0.5, causal=True)
    S = float(np.float32(0.5)) * Q @ K.T
    S = np.where(np.arange(11)[None, :] > (np.arange(8) + 3)[:, None], -np.inf, S)
    P = np.exp(S - S.max(1, keepdims=True))
    P /= P.sum(1, keepdims=True)
    close((P * (dO @ V.T)).sum(1), (dO * O).sum(1), 1e-13)


def test_grad_planted_mistakes_are_caught():
    """Plausible slips in the gradient formulas fail the autograd pin."""
    rng = np.random.default_rng(8)
    Q, K, V, dO = (rng.standard_normal(s) for s in ((6, 4), (9, 4), (9, 4), (6, 4)))
    want = _torch_grads(Q, K, V, dO, 0.4, False)
    sc = float(np.float32(0.4))
    S = sc * Q @ K.T
    E = np.exp(S - S.max(1, keepdims=True))
    P = E / E.sum(1, keepdims=True)
    dP = dO @ V.T
    slips = {
        "no softmax Jacobian term": (sc * (P * dP) @ K, 0),
        "Jacobian term summed over the wrong axis": (sc * (P * (dP - (P * dP).sum(0))) @ K, 0),
        "dQ without the scale": ((P * (dP - (P * dP).sum(1, keepdims=True))) @ K, 0),
        "dK with the unnormalised weights": (sc * ((E * (dP - (P * dP).sum(1, keepdims=True))).T @ Q), 1),
        "dV with the unnormalised weights": (E.T @ dO, 2),
    }
    for name, (g, which) in slips.items():
        assert not np.allclose(g, want[which], atol=1e-6), name


def _torch_grads_batched(q, k, v, do, scale, causal):
    """dQ, dK, dV of sum(O * dO) for whole [B, H, N, d] tensors by float64
    torch autograd (batched products, no per-head loop)."""
    qt, kt, vt = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    S = float(np.float32(scale)) * qt @ kt.transpose(-1, -2)
    Nq, Nk = q.shape[2], k.shape[2]
    if causal:
        S = S.masked_fill(torch.arange(Nk)[None, :] > (torch.arange(Nq) + (Nk - Nq))[:, None],
                          -float("inf"))
    P = torch.softmax(S, -1).nan_to_num(0.0)
    (P @ vt * torch.tensor(do)).sum().backward()
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


def pin_attention_grad(impl):
    """The [B, H] gradient wrapper: every (b, h) slice against batched float64
    autograd, with heads that differ (distinct scales per head) so a mixed-up
    slice or a swapped dK / dV (d == dv here) cannot pass."""
    rng = np.random.default_rng(17)
    B, H, d = 2, 3, 5
    for causal, Nq, Nk in [(False, 6, 9), (True, 6, 9), (True, 9, 6), (False, 4, 4)]:
        spread = (1.0 + np.arange(B * H).reshape(B, H, 1, 1)) / 3
        q = rng.standard_normal((B, H, Nq, d)) * spread
        k = rng.standard_normal((B, H, Nk, d))
        v = rng.standard_normal((B, H, Nk, d)) + spread
        do = rng.standard_normal((B, H, Nq, d))
        want = _torch_grads_batched(q, k, v, do, 0.45, causal)
        got = impl(q, k, v, do, 0.45, causal)
        for g, w in zip(got, want):
            close(g, w, 1e-12)


def test_attention_grad_wrapper_pin():
    pin_attention_grad(oracle.attention_grad)


def test_attention_grad_wrapper_head_subset():
    """Only the listed (b, h) pairs are evaluated; they equal the full call."""
    rng = np.random.default_rng(18)
    q, k, v, do = (rng.standard_normal((2, 3, 5, 4)) for _ in range(4))
    full = oracle.attention_grad(q, k, v, do, 0.3, True)
    part = oracle.attention_grad(q, k, v, do, 0.3, True, heads=[(1, 2), (0, 1)])
    for f, g in zip(full, part):
        for b, h in [(1, 2), (0, 1)]:
            assert np.array_equal(f[b, h], g[b, h])
        assert np.isnan(g[0, 0]).all() and np.isnan(g[1, 1]).all()


def test_attention_grad_wrapper_planted_mistakes_are_caught():
    """Slips in the [B, H] wrapper (planted here, on the CPU) fail its pin."""
    def swapped_dk_dv(q, k, v, do, scale, causal):
        dq, dk, dv = oracle.attention_grad(q, k, v, do, scale, causal)
        return dq, dv, dk

    def next_head_keys(q, k, v, do, scale, causal):
        B, H = q.shape[:2]
        out = [np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape)]
        for b in range(B):
            for h in range(H):
                g = ref.head_attention_grad(q[b, h], k[b, (h + 1) % H], v[b, h], do[b, h], scale,
                                            causal)
                for o, x in zip(out, g):
                    o[b, h] = x
        return out

    def batch_index_mixed(q, k, v, do, scale, causal):
        B, H = q.shape[:2]
        out = [np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape)]
        for b in range(B):
            for h in range(H):
                g = ref.head_attention_grad(q[b, h], k[b, h], v[B - 1 - b, h], do[b, h], scale,
                                            causal)
                for o, x in zip(out, g):
                    o[b, h] = x
        return out

    for slip in (swapped_dk_dv, next_head_keys, batch_index_mixed):
        with pytest.raises(AssertionError):
            pin_attention_grad(slip)


# ---------------------------------------------------------- block sparsity

def _bs_inputs(B, H, Nq, Nk, d, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, H, Nq, d)), rng.standard_normal((B, H, Nk, d)),
            rng.standard_normal((B, H, Nk, d)))


@pytest.mark.parametrize("causal", [False, True])
def test_block_sparse_all_ones_is_dense(causal):
    q, k, v = _bs_inputs(1, 2, 130, 200, 8, 1)
    M = np.ones((2, 3, 4), dtype=np.uint8)
    O1, L1 = oracle.attention_block_sparse(q, k, v, M, 0.3, causal)
    O2, L2 = oracle.attention(q, k, v, 0.3, causal)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)


def test_block_sparse_lower_blocks_plus_diagonal_mask_is_causal():
    """Admitting exactly the blocks on and below the diagonal and masking
    inside them is causal attention (Nq = Nk)."""
    q, k, v = _bs_inputs(1, 1, 192, 192, 8, 2)
    M = np.tril(np.ones((3, 3), dtype=np.uint8))[None]
    O1, L1 = oracle.attention_block_sparse(q, k, v, M, 0.3, causal=True)
    O2, L2 = oracle.attention(q, k, v, 0.3, causal=True)
    close(O1, O2, 1e-14)
    close(L1, L2, 1e-14)


def test_block_sparse_against_brute_force():
    """A random block pattern (with an all-masked query block) against the
    pure-Python definition run on the visible keys of each row."""
    rng = np.random.default_rng(9)
    q, k, v = _bs_inputs(1, 2, 70, 150, 3, 3)
    M = (rng.random((2, 2, 3)) < 0.5).astype(np.uint8)
    M[1, 1, :] = 0  # a query block that sees nothing
    M[0, 0, 1] = 1
    for causal in (False, True):
        O, L = oracle.attention_block_sparse(q, k, v, M, 0.3, causal)
        for h in range(2):
            for i in range(70):
                keys = [j for j in range(150) if M[h, i // 64, j // 64] and (not causal or j <= i + 80)]
                if not keys:
                    assert np.all(O[0, h, i] == 0) and L[0, h, i] == -np.inf
                    continue
                Ob, Lb = brute.attention([[[q[0, h, i].tolist()]]], [[[k[0, h, j].tolist() for j in keys]]],
                                         [[[v[0, h, j].tolist() for j in keys]]], 0.3)
                close(O[0, h, i], np.array(Ob[0][0][0]), 1e-13)
                close(L[0, h, i], Lb[0][0][0], 1e-13)
