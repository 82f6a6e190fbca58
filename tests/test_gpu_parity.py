"""GPU parity: the HIP path, called through the C ABI, against the fp64 oracle.

Tolerances: max |O - O_oracle| <= 1e-5 for fp32 inputs and <= 2e-2 for bf16
inputs (fp32 accumulation); max |LSE - LSE_oracle| <= 1e-3 (-inf == -inf
counts as exact).  Inputs are the seeded workloads; the oracle reads host
copies of exactly the tensors the kernels read.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

TOL_F32, TOL_BF16, TOL_LSE = 1e-5, 2e-2, 1e-3


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def max_err(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    both = np.isneginf(a) & np.isneginf(b)
    d = np.abs(np.where(both, 0.0, a) - np.where(both, 0.0, b))
    return float(np.nan_to_num(d, nan=np.inf).max(initial=0.0))


def check(o, lse, O, L, tol, what):
    eo = max_err(W.to_f64(o), O)
    el = max_err(W.to_f64(lse), L)
    log(f"  {what}: err_O={eo:.3e} err_LSE={el:.3e}")
    assert eo <= tol, f"{what}: err_O {eo}"
    assert el <= TOL_LSE, f"{what}: err_LSE {el}"
    return eo, el


def run_fwd(fa, q, k, v, scale, causal):
    f = fa.fa_fwd_f32 if q.dtype == torch.float32 else fa.fa_fwd
    o, lse = f(q, k, v, scale, causal)
    torch.cuda.synchronize()
    return o, lse


# ------------------------------------------------------------- configs
def test_tiny_f32(fa):
    s = W.TINY_F32
    log(f"case {s.name}")
    q, k, v = W.prefill_spec_inputs(s, "cuda")
    o, lse = run_fwd(fa, q, k, v, s.scale, s.causal)
    O, L = oracle.attention(q, k, v, s.scale, s.causal)
    check(o, lse, O, L, TOL_F32, s.name)


def _sampled_rows(B, H, Nq, n_heads, n_rows, seed):
    rng = np.random.default_rng(seed)
    rows = []
    heads = [(int(rng.integers(B)), int(rng.integers(H))) for _ in range(n_heads)]
    heads += [(0, 0), (B - 1, H - 1)]
    for b, h in heads:
        idx = set(rng.integers(0, Nq, n_rows).tolist()) | {0, 1, 127, 128, Nq - 1}
        rows += [(b, h, i) for i in sorted(i for i in idx if i < Nq)]
    return rows


@pytest.mark.parametrize("spec", [W.GPT2M, W.GPT2M_CAUSAL, W.LONG_PREFILL], ids=lambda s: s.name)
def test_prefill_full_size_sampled(fa, spec):
    """The benchmark shapes, in the launch configuration the benchmark times;
    the oracle evaluates sampled rows one by one."""
    log(f"case {spec.name}")
    q, k, v = W.prefill_spec_inputs(spec, "cuda")
    o, lse = run_fwd(fa, q, k, v, spec.scale, spec.causal)
    rows = _sampled_rows(spec.B, spec.H, spec.Nq, 6, 48, spec.seed)
    O, L = oracle.attention_rows(q, k, v, spec.scale, spec.causal, rows)
    idx = tuple(torch.as_tensor(a, device=o.device) for a in np.array(rows).T)
    og = o[idx].cpu()
    lg = lse[idx].cpu()
    check(og, lg, O, L, TOL_BF16, spec.name)
    # every output is finite, every LSE finite (no empty rows in these shapes)
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()


@pytest.mark.parametrize("d", [128, 64])
def test_prefill_very_long_sampled(fa, d):
    """A sequence eight times the long prefill's (N = 65536, causal, two
    heads): 256 query tiles per head and walks of up to 1024 key tiles, in
    the streaming launch; sampled rows against the oracle."""
    B, H, N = 1, 2, 65536
    log(f"case very long prefill N={N} d={d}")
    q, k, v = W.prefill_inputs(B, H, N, N, d, "bf16", seed=4242 + d, device="cuda")
    scale = d ** -0.5
    o, lse = run_fwd(fa, q, k, v, scale, True)
    rows = _sampled_rows(B, H, N, 1, 24, 4242 + d) + [(0, 1, N - 2), (0, 0, N // 2)]
    O, L = oracle.attention_rows(q, k, v, scale, True, rows)
    idx = tuple(torch.as_tensor(a, device=o.device) for a in np.array(rows).T)
    check(o[idx].cpu(), lse[idx].cpu(), O, L, TOL_BF16, f"N={N} d={d}")
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()


def test_long_prefill_whole_output(fa):
    """The long causal prefill (B=1, H=32, N=8192, d=128) in the launch the
    benchmark times: every element of O and LSE of all 32 heads against the
    oracle, head by head."""
    s = W.LONG_PREFILL
    log(f"case {s.name} whole output")
    q, k, v = W.prefill_spec_inputs(s, "cuda")
    o, lse = run_fwd(fa, q, k, v, s.scale, s.causal)
    oh, lh = o.cpu(), lse.cpu()
    qh, kh, vh = q.cpu(), k.cpu(), v.cpu()
    worst_o = worst_l = 0.0
    for h in range(s.H):
        O, L = oracle.head_attention(qh[0, h], kh[0, h], vh[0, h], s.scale, s.causal)
        worst_o = max(worst_o, max_err(W.to_f64(oh[0, h]), O))
        worst_l = max(worst_l, max_err(W.to_f64(lh[0, h]), L))
    log(f"  all {s.H} heads: err_O={worst_o:.3e} err_LSE={worst_l:.3e}")
    assert worst_o <= TOL_BF16 and worst_l <= TOL_LSE


def test_prefill_gpt2m_whole_heads(fa):
    """Complete heads of the GPT-2-medium shape, every row, causal and not."""
    for spec in (W.GPT2M, W.GPT2M_CAUSAL):
        log(f"case {spec.name} whole heads")
        q, k, v = W.prefill_spec_inputs(spec, "cuda")
        o, lse = run_fwd(fa, q, k, v, spec.scale, spec.causal)
        for b, h in [(0, 0), (17, 5), (63, 15)]:
            O, L = oracle.head_attention(q[b, h], k[b, h], v[b, h], spec.scale, spec.causal)
            check(o[b, h], lse[b, h], O, L, TOL_BF16, f"{spec.name} b={b} h={h}")


# ------------------------------------------------------------- edge shapes
EDGE = [
    # B, H, Nq, Nk, d, causal
    (1, 2, 200, 200, 128, False), (1, 2, 200, 200, 128, True),
    (2, 1, 200, 200, 64, False), (2, 1, 200, 200, 64, True),
    (1, 2, 100, 300, 128, True), (1, 2, 300, 100, 128, True),
    (1, 1, 300, 100, 64, True), (1, 3, 1, 777, 128, False), (1, 1, 1, 1, 64, False),
    (1, 1, 129, 65, 128, False), (1, 1, 64, 64, 128, True), (1, 1, 4, 1000, 64, True),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", EDGE, ids=lambda s: "x".join(map(str, s)))
def test_edge_shapes(fa, shape, dtype):
    B, H, Nq, Nk, d, causal = shape
    log(f"case edge {shape} {dtype}")
    q, k, v = W.prefill_inputs(B, H, Nq, Nk, d, dtype, seed=Nq * 7 + Nk + d, device="cuda")
    scale = 1 / math.sqrt(d)
    o, lse = run_fwd(fa, q, k, v, scale, causal)
    O, L = oracle.attention(q, k, v, scale, causal)
    check(o, lse, O, L, TOL_F32 if dtype == "f32" else TOL_BF16, f"{shape} {dtype}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("scale", [0.0, -0.09, 0.5])
@pytest.mark.parametrize("d", [64, 128])
def test_unusual_scales(fa, dtype, scale, d):
    log(f"case scale {scale} {dtype} d={d}")
    # bf16 d = 64 with 200 heads x 2 query tiles: more tiles than CUs, so the
    # sign flip and the zero-scale path also run inside a stream of tiles.
    H, Nq = (200, 300) if (d == 64 and dtype == "bf16") else (2, 150)
    q, k, v = W.prefill_inputs(1, H, Nq, 170, d, dtype, seed=5 + d, device="cuda")
    o, lse = run_fwd(fa, q, k, v, scale, True)
    O, L = oracle.attention(q, k, v, scale, True)
    check(o, lse, O, L, TOL_F32 if dtype == "f32" else TOL_BF16, f"scale={scale} {dtype} d={d}")


@pytest.mark.parametrize("d", [64, 128])
def test_large_scores(fa, d):
    """Scores near 1000 (the explainer's §2 example magnitude): the running
    maximum keeps exp finite."""
    log(f"case large scores d={d}")
    g = torch.Generator(device="cuda").manual_seed(11)
    B, H, N = 1, 2, 256
    scale = 1 / math.sqrt(d)
    e = torch.randn(d, generator=g, device="cuda")
    e = e / e.norm() * math.sqrt(1000 / scale)          # scale * |e|^2 = 1000
    q = (torch.randn(B, H, N, d, generator=g, device="cuda") + e).to(torch.bfloat16)
    k = (torch.randn(B, H, N, d, generator=g, device="cuda") + e).to(torch.bfloat16)
    v = torch.randn(B, H, N, d, generator=g, device="cuda").to(torch.bfloat16)
    for causal in (False, True):
        o, lse = run_fwd(fa, q, k, v, scale, causal)
        O, L = oracle.attention(q, k, v, scale, causal)
        assert L.min() > 900
        check(o, lse, O, L, TOL_BF16, f"large scores d={d} causal={causal}")


@pytest.mark.parametrize("d,B,H,N", [(128, 2, 4, 520), (64, 3, 200, 600)])
def test_deterministic(fa, d, B, H, N):
    """Run-to-run bit-identical prefill (d = 64: a stream with more query tiles
    than CUs)."""
    log(f"case determinism d={d}")
    q, k, v = W.prefill_inputs(B, H, N, N, d, "bf16", seed=9, device="cuda")
    for causal in (True, False):
        o1, l1 = run_fwd(fa, q, k, v, 0.088, causal)
        o2, l2 = run_fwd(fa, q, k, v, 0.088, causal)
        assert torch.equal(o1, o2) and torch.equal(l1, l2), causal


def test_binding_refuses_wrong_buffers(fa):
    """Caller-supplied outputs, gradients and workspaces of the wrong shape,
    dtype or device are refused by the binding before anything is launched."""
    log("case binding validation")
    dev = "cuda"
    q, k, v = W.prefill_inputs(1, 2, 64, 80, 128, "bf16", seed=3, device=dev)
    bad_out = torch.empty(1, 2, 63, 128, dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError):
        fa.fa_fwd(q, k, v, out=bad_out)
    with pytest.raises(ValueError):
        fa.fa_fwd(q, k, v, lse=torch.empty(1, 2, 65, device=dev))
    with pytest.raises(ValueError):
        fa.fa_fwd(q, k.cpu(), v)
    with pytest.raises(ValueError):
        fa.fa_fwd(q, k[:, :, :40].contiguous(), v)  # k and v lengths differ
    o, lse = fa.fa_fwd(q, k, v)
    do = torch.randn_like(q)
    for kw in ({"dq": torch.empty(1, 2, 64, 127, device=dev)},
               {"dk": torch.empty(1, 2, 64, 128, device=dev)},
               {"dv": torch.empty(1, 2, 80, 128, dtype=torch.bfloat16, device=dev)},
               {"workspace": torch.empty(8, dtype=torch.uint8, device=dev)}):
        with pytest.raises(ValueError):
            fa.fa_bwd(q, k, v, o, do, lse, **kw)
    m = W.block_mask("ones", 2, 64, 80).to(dev)
    with pytest.raises(ValueError):
        fa.fa_fwd_block_sparse(q, k, v, m, out=bad_out)
    lens = [5, 9]
    dq_, dkc, dvc, sl, off = W.decode_inputs(2, 2, 128, lens, seed=1, device=dev)
    with pytest.raises(ValueError):
        fa.fa_decode_varlen(dq_, dkc, dvc, sl, off, 9, out=torch.empty(2, 2, 64, dtype=torch.bfloat16,
                                                                        device=dev))
    with pytest.raises(ValueError):
        fa.fa_decode_varlen(dq_, dkc, dvc, sl, off, 9, lse=torch.empty(2, 3, device=dev))
    with pytest.raises(ValueError):
        fa.fa_decode_varlen(dq_, dkc, dvc, sl, off, 9,
                            workspace=torch.zeros(16, dtype=torch.uint8, device=dev))
    with pytest.raises(ValueError):
        fa.fa_decode_varlen(dq_, dkc, dvc, sl[:1].contiguous(), off, 9)
    lq = [30, 10]
    vq, vk, vv, cq, ck = W.varlen_inputs(lq, lq, 2, 128, seed=2, device=dev)
    with pytest.raises(ValueError):
        fa.fa_fwd_varlen(vq, vk, vv, cq, ck, 30, lse=torch.empty(2, 39, device=dev))
    with pytest.raises(ValueError):
        fa.fa_fwd_varlen(vq, vk, vv, cq, ck[:2].contiguous(), 30)
    torch.cuda.synchronize()


# ------------------------------------------------------------- decode
def run_decode(fa, q, kc, vc, sl, off, max_len, scale, split_keys=0, workspace=None):
    if split_keys:
        o, lse = fa.fa_decode_varlen_split(q, kc, vc, sl, off, max_len, split_keys, scale,
                                           workspace=workspace)
    else:
        o, lse = fa.fa_decode_varlen(q, kc, vc, sl, off, max_len, scale, workspace=workspace)
    torch.cuda.synchronize()
    return o, lse


def test_decode_single_full(fa):
    s = W.DECODE_SINGLE
    log(f"case {s.name}")
    q, kc, vc, sl, off = W.decode_spec_inputs(s, "cuda")
    o, lse = run_decode(fa, q, kc, vc, sl, off, s.max_len, s.scale)
    O, L = oracle.decode(q, kc, vc, sl.cpu(), off.cpu(), s.scale)
    check(o, lse, O, L, TOL_BF16, s.name)


def test_decode_batched_full_size(fa):
    """The batched decode workload in the benchmark's launch: all 64 sequences
    against the oracle on three heads (first, a middle one, last), and the
    whole output twice over for run-to-run equality."""
    s = W.DECODE_BATCHED
    log(f"case {s.name}")
    q, kc, vc, sl, off = W.decode_spec_inputs(s, "cuda")
    log(f"  T={kc.shape[0]} tokens, {kc.numel() * 4 / 1e9:.2f} GB of K+V")
    o, lse = run_decode(fa, q, kc, vc, sl, off, s.max_len, s.scale)
    slh, offh = sl.cpu(), off.cpu()
    heads = [0, 13, s.H - 1]
    O, L = oracle.decode(q, kc, vc, slh, offh, s.scale, heads=heads)
    check(o[:, heads], lse[:, heads], O[:, heads], L[:, heads], TOL_BF16,
          s.name + " all sequences, heads 0/13/31")
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    o2, lse2 = run_decode(fa, q, kc, vc, sl, off, s.max_len, s.scale)
    assert torch.equal(o, o2) and torch.equal(lse, lse2), "batched decode not deterministic"


@pytest.mark.parametrize("d", [64, 128])
def test_decode_edge_lengths(fa, d):
    lens = [1, 0, 128, 16384, 63, 65, 257, 5000]
    log(f"case decode edge lengths d={d}")
    q, kc, vc, sl, off = W.decode_inputs(len(lens), 4, d, lens, seed=17, device="cuda")
    scale = 1 / math.sqrt(d)
    for sk in (0, 64, 1024):
        o, lse = run_decode(fa, q, kc, vc, sl, off, max(lens), scale, sk)
        O, L = oracle.decode(q, kc, vc, sl.cpu(), off.cpu(), scale)
        check(o, lse, O, L, TOL_BF16, f"d={d} split_keys={sk}")
        assert (o[1] == 0).all() and torch.isneginf(lse[1]).all()


@pytest.mark.parametrize("d", [128, 64])
def test_decode_very_long(fa, d):
    """Decode over 262144 cached tokens (with a shorter sequence beside it):
    256 chunks of 1024 keys for one (sequence, head), merged across XCDs,
    and the merge kernel path for a finer split; every output against the
    oracle."""
    lens = [262144, 100003]
    log(f"case decode very long d={d}")
    q, kc, vc, sl, off = W.decode_inputs(len(lens), 4, d, lens, seed=23 + d, device="cuda")
    scale = 1 / math.sqrt(d)
    O, L = oracle.decode(q, kc, vc, sl.cpu(), off.cpu(), scale)
    for sk in (0, 256):
        o, lse = run_decode(fa, q, kc, vc, sl, off, max(lens), scale, sk)
        check(o, lse, O, L, TOL_BF16, f"d={d} split_keys={sk}")


def test_decode_split_invariance(fa):
    s = W.DECODE_SINGLE
    log("case decode split invariance")
    q, kc, vc, sl, off = W.decode_spec_inputs(s, "cuda")
    ref_o, ref_l = run_decode(fa, q, kc, vc, sl, off, s.max_len, s.scale, 8192)
    for sk in (64, 128, 256, 512, 2048):
        o, lse = run_decode(fa, q, kc, vc, sl, off, s.max_len, s.scale, sk)
        el = (lse - ref_l).abs().max().item()
        eo = (o.float() - ref_o.float()).abs().max().item()
        log(f"  split_keys={sk}: dLSE={el:.2e} dO={eo:.2e}")
        assert el <= 1e-5 and eo <= 2 ** -7


def test_decode_matches_fwd_single_query(fa):
    log("case decode vs fwd Nq=1")
    lens = [300, 1000, 77]
    q, kc, vc, sl, off = W.decode_inputs(3, 2, 128, lens, seed=23, device="cuda")
    o, lse = run_decode(fa, q, kc, vc, sl, off, 1000, 0.088)
    for b, n in enumerate(lens):
        lo = int(off[b])
        qb = q[b][None, :, None, :].contiguous()
        kb = kc[lo:lo + n].permute(1, 0, 2)[None].contiguous()
        vb = vc[lo:lo + n].permute(1, 0, 2)[None].contiguous()
        of, lf = run_fwd(fa, qb, kb, vb, 0.088, False)
        assert (lf[0, :, 0] - lse[b]).abs().max().item() <= 1e-4
        assert (of[0, :, 0].float() - o[b].float()).abs().max().item() <= 2e-2


COUNTER_BYTES = 65536  # arrival counters at the start of every decode workspace


def test_decode_workspace_reused_across_calls(fa):
    """One zero-filled workspace serves consecutive calls of different shapes
    and chunk sizes (the chunk states of one call land where another call's
    would not); the arrival counters are zero again after every call."""
    log("case decode workspace reuse")
    cases = [([700, 64, 3000, 1], 4, 256), ([5000] * 9, 7, 64), ([700, 64, 3000, 1], 4, 0),
             ([1, 2, 3], 40, 64), ([8192], 32, 0)]
    need = max(fa.fa_decode_split_workspace_bytes(len(l), H, 128, max(l), sk or 256)
               for l, H, sk in cases)
    need = max(need, max(fa.fa_decode_workspace_bytes(len(l), H, 128, max(l)) for l, H, _ in cases))
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for call, (lens, H, sk) in enumerate(cases):
        q, kc, vc, sl, off = W.decode_inputs(len(lens), H, 128, lens, seed=100 + call, device="cuda")
        o, lse = run_decode(fa, q, kc, vc, sl, off, max(lens), 0.088, sk, workspace=ws)
        O, L = oracle.decode(q, kc, vc, sl.cpu(), off.cpu(), 0.088)
        check(o, lse, O, L, TOL_BF16, f"reuse call {call} B={len(lens)} H={H} split_keys={sk}")
        assert int(ws[:COUNTER_BYTES].count_nonzero()) == 0, "arrival counters left nonzero"


def test_decode_merge_paths_agree(fa):
    """The merge by the last chunk to finish (counters) and the separate merge
    kernel (beyond 1024 chunks per sequence, 4096 chunk workgroups in all, or
    16384 sequence-head pairs) against the oracle."""
    log("case decode merge paths")
    lens = [64 * 1100, 3000, 1]
    q, kc, vc, sl, off = W.decode_inputs(len(lens), 2, 128, lens, seed=41, device="cuda")
    O, L = oracle.decode(q, kc, vc, sl.cpu(), off.cpu(), 0.088)
    o1, l1 = run_decode(fa, q, kc, vc, sl, off, max(lens), 0.088, 64)     # 1100 chunks: kernel
    o2, l2 = run_decode(fa, q, kc, vc, sl, off, max(lens), 0.088, 128)    # 550 chunks, 3300 workgroups: fused
    check(o1, l1, O, L, TOL_BF16, "merge kernel")
    check(o2, l2, O, L, TOL_BF16, "fused merge")
    # many (sequence, head) pairs: 4100 x 4 > 16384 counters -> merge kernel
    lens2 = [(i * 37) % 900 for i in range(4100)]
    q, kc, vc, sl, off = W.decode_inputs(len(lens2), 4, 64, lens2, seed=43, device="cuda")
    o3, l3 = run_decode(fa, q, kc, vc, sl, off, max(lens2), 0.125, 256)
    seqs = [0, 1, 25, 1000, 4099]
    O3, L3 = oracle.decode(q, kc, vc, sl.cpu(), off.cpu(), 0.125, seqs=seqs)
    check(o3[seqs], l3[seqs], O3[seqs], L3[seqs], TOL_BF16, "16400 sequence-head pairs")


def test_decode_deterministic(fa):
    """Decode is run-to-run bit-identical: single request (fused merge) and an
    explicit chunking that takes the merge kernel."""
    log("case decode determinism")
    s = W.DECODE_SINGLE
    q, kc, vc, sl, off = W.decode_spec_inputs(s, "cuda")
    for sk in (0, 64):
        a = run_decode(fa, q, kc, vc, sl, off, s.max_len, s.scale, sk)
        b = run_decode(fa, q, kc, vc, sl, off, s.max_len, s.scale, sk)
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]), sk


VARLEN_CASES = [
    # (d, causal, query lengths, key lengths)
    (128, True, [1, 255, 256, 257, 600, 0, 1000], [1, 255, 256, 257, 600, 0, 1000]),
    (128, True, [100, 300, 1], [900, 300, 4000]),     # chunked prefill: keys before the queries
    (128, True, [300, 70], [64, 0]),                  # more queries than keys: empty rows
    (128, False, [513, 7, 64], [1025, 33, 64]),
    (64, True, [1, 129, 500], [1, 700, 500]),
    (64, False, [200, 40], [77, 3000]),
    (64, True, [300, 0, 70, 5], [64, 5, 0, 700]),     # empty sequence, keyless rows
]
# Many short sequences of seeded random lengths (empty ones among them): a
# grid of hundreds of sequences, most a single query tile.
_MANY = [int(x) for x in np.random.default_rng(5).integers(0, 300, 400)]
VARLEN_CASES += [
    (128, True, _MANY, _MANY),
    (64, False, _MANY, _MANY[::-1]),
]


@pytest.mark.parametrize("d,causal,lq,lk", VARLEN_CASES)
def test_fwd_varlen(fa, d, causal, lq, lk):
    log(f"case varlen d={d} causal={causal} lq={lq[:8]} ({len(lq)} sequences) lk={lk[:8]}")
    H = 3
    q, k, v, cq, ck = W.varlen_inputs(lq, lk, H, d, seed=61 + d + len(lq), device="cuda")
    o, lse = fa.fa_fwd_varlen(q, k, v, cq, ck, max(lq), 1 / math.sqrt(d), causal)
    torch.cuda.synchronize()
    O, L = oracle.attention_varlen(q, k, v, cq, ck, 1 / math.sqrt(d), causal)
    check(o, lse, O, L, TOL_BF16, "varlen")


@pytest.mark.parametrize("d,causal", [(128, True), (128, False), (64, True)])
def test_fwd_varlen_equals_dense(fa, d, causal):
    """Sequences of one length packed token-major give exactly the dense
    kernel's result on the [B, H, N, d] layout (same tiles, same arithmetic)."""
    log(f"case varlen vs dense d={d} causal={causal}")
    B, H, N = 3, 4, 700
    q, k, v = W.prefill_inputs(B, H, N, N, d, "bf16", seed=71, device="cuda")
    o, lse = fa.fa_fwd(q, k, v, 0.09, causal)
    pack = lambda t: t.permute(0, 2, 1, 3).reshape(B * N, H, d).contiguous()  # noqa: E731
    cu = torch.arange(0, (B + 1) * N, N, dtype=torch.int32, device="cuda")
    o2, lse2 = fa.fa_fwd_varlen(pack(q), pack(k), pack(v), cu, cu, N, 0.09, causal)
    torch.cuda.synchronize()
    assert torch.equal(pack(o), o2)
    assert torch.equal(lse.permute(1, 0, 2).reshape(H, B * N), lse2)


# Dense prefill (d = 64 and d = 128) runs as a stream: one workgroup per CU
# walks every G-th query tile (G = CU count), carrying its tile pipeline
# across query tiles.  These shapes have more query tiles than CUs, partial
# last rounds, mixed tile counts and, causally with Nq > Nk, query tiles that
# see no key at all; the last two (non-causal, whole rounds) take the d = 64
# path that deals all query tiles of a head to one XCD in one round.
STREAM = [
    # B, H, Nq, Nk, causal
    (1, 128, 600, 100, True),
    (2, 100, 300, 333, False),
    (1, 96, 1000, 1000, True),
    (5, 67, 600, 600, True),   # B*H = 335, odd: 1005 query tiles, no head-to-XCD alignment
    (2, 128, 1024, 1024, False),
    (1, 64, 2048, 1500, False),
]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("shape", STREAM, ids=lambda s: "x".join(map(str, s)))
def test_fwd_stream(fa, shape, d):
    B, H, Nq, Nk, causal = shape
    log(f"case d{d} stream {shape}")
    q, k, v = W.prefill_inputs(B, H, Nq, Nk, d, "bf16", seed=Nq + Nk + H, device="cuda")
    o, lse = run_fwd(fa, q, k, v, 0.125, causal)
    heads = [(0, 0), (B - 1, H // 2), (B - 1, H - 1), (B // 2, H // 3)]
    for b, h in heads:
        O, L = oracle.head_attention(q[b, h], k[b, h], v[b, h], 0.125, causal)
        check(o[b, h], lse[b, h], O, L, TOL_BF16, f"d{d} stream {shape} b={b} h={h}")
    # A head computed alone (a single item) is bit-identical to the same head
    # inside the stream: nothing carries over between query tiles.
    for b, h in heads:
        o1, lse1 = run_fwd(fa, q[b:b + 1, h:h + 1].contiguous(), k[b:b + 1, h:h + 1].contiguous(),
                           v[b:b + 1, h:h + 1].contiguous(), 0.125, causal)
        assert torch.equal(o1[0, 0], o[b, h]) and torch.equal(lse1[0, 0], lse[b, h]), (b, h)


def test_fwd_varlen_full_size_sampled(fa):
    """The packed causal workload (8 sequences, lengths U[512, 8192], H=32):
    shortest and longest sequence, two heads each, against the oracle."""
    s = W.VARLEN_PREFILL
    lens, q, k, v, cq, ck = W.varlen_spec_inputs(s, "cuda")
    log(f"case {s.name} lens={lens.tolist()}")
    o, lse = fa.fa_fwd_varlen(q, k, v, cq, ck, int(lens.max()), s.scale, s.causal)
    torch.cuda.synchronize()
    seqs = [int(torch.argmin(lens)), int(torch.argmax(lens))]
    heads = [0, s.H - 1]
    O, L = oracle.attention_varlen(q, k, v, cq, ck, s.scale, s.causal, seqs=seqs, heads=heads)
    cqh = cq.cpu().tolist()
    for b in seqs:
        r = slice(cqh[b], cqh[b + 1])
        for h in heads:
            check(o[r, h], lse[h, r], O[r, h], L[h, r], TOL_BF16, f"seq {b} head {h}")


# The gradients have no unit scale, so the bf16 tolerance applies relative to
# the largest reference magnitude: P, dS and (through D = rowsum(dO * O)) O
# enter the products in bf16, each with relative rounding 2^-9.
TOL_GRAD_REL, TOL_GRAD_ABS = 2e-2, 1e-5


def check_grads(got, want, what):
    for name, a, b in zip(("dq", "dk", "dv"), got, want):
        a = W.to_f64(a)
        assert a.shape == b.shape, (name, a.shape, b.shape)
        err = float(np.abs(a - b).max(initial=0.0))
        ref = float(np.abs(b).max(initial=0.0))
        log(f"  {what} {name}: err={err:.3e} max|ref|={ref:.3e}")
        assert np.isfinite(a).all(), f"{what} {name}: non-finite"
        assert err <= TOL_GRAD_REL * ref + TOL_GRAD_ABS, f"{what} {name}: {err} vs {ref}"


BWD_SHAPES = [(1, 2, 1, 1), (2, 2, 33, 33), (1, 2, 100, 300), (1, 2, 300, 100), (1, 1, 129, 129),
              (1, 2, 512, 512)]


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,Nq,Nk", BWD_SHAPES)
def test_bwd(fa, d, causal, B, H, Nq, Nk):
    log(f"case bwd d={d} causal={causal} B={B} H={H} Nq={Nq} Nk={Nk}")
    q, k, v = W.prefill_inputs(B, H, Nq, Nk, d, "bf16", seed=Nq + Nk + d, device="cuda")
    do = W.prefill_inputs(B, H, Nq, 1, d, "bf16", seed=900 + Nq, device="cuda")[0]
    sc = 1 / math.sqrt(d)
    o, lse = fa.fa_fwd(q, k, v, sc, causal)
    grads = fa.fa_bwd(q, k, v, o, do, lse, sc, causal)
    torch.cuda.synchronize()
    check_grads(grads, oracle.attention_grad(q, k, v, do, sc, causal), "bwd")


@pytest.mark.parametrize("d", [128, 64])
def test_bwd_deterministic(fa, d):
    """The backward is run-to-run bit-identical: no atomics, every gradient
    element accumulated in a fixed order by one wave."""
    log(f"case bwd determinism d={d}")
    B, H, N = 2, 3, 777
    q, k, v = W.prefill_inputs(B, H, N, N, d, "bf16", seed=31 + d, device="cuda")
    do = W.prefill_inputs(B, H, N, 1, d, "bf16", seed=32 + d, device="cuda")[0]
    sc = 1 / math.sqrt(d)
    for causal in (True, False):
        o, lse = fa.fa_fwd(q, k, v, sc, causal)
        g1 = fa.fa_bwd(q, k, v, o, do, lse, sc, causal)
        g2 = fa.fa_bwd(q, k, v, o, do, lse, sc, causal)
        torch.cuda.synchronize()
        for a, b in zip(g1, g2):
            assert torch.equal(a, b), causal


def test_bwd_full_size_one_head(fa):
    """The long causal shape (B=1, H=32, N=8192, d=128) through forward and
    backward on the GPU; one whole head's three gradients against the oracle."""
    s = W.LONG_PREFILL
    log(f"case bwd {s.name}")
    q, k, v = W.prefill_spec_inputs(s, "cuda")
    do = W.prefill_inputs(s.B, s.H, s.Nq, 1, s.d, "bf16", seed=s.seed + 1, device="cuda")[0]
    o, lse = fa.fa_fwd(q, k, v, s.scale, s.causal)
    dq, dk, dv = fa.fa_bwd(q, k, v, o, do, lse, s.scale, s.causal)
    torch.cuda.synchronize()
    h = 17
    want = oracle.head_attention_grad(q[0, h], k[0, h], v[0, h], do[0, h], s.scale, s.causal)
    check_grads((dq[0, h], dk[0, h], dv[0, h]), want, f"head {h}")


SPARSE_CASES = [
    # (kind, causal, Nq, Nk)
    ("random", False, 300, 300),
    ("random", True, 300, 300),
    ("random", True, 200, 700),
    ("random", False, 700, 130),
    ("local_global", True, 1024, 1024),
    ("local_global", False, 520, 900),
    ("zeros", False, 256, 256),
]


@pytest.mark.parametrize("kind,causal,Nq,Nk", SPARSE_CASES)
def test_fwd_block_sparse(fa, kind, causal, Nq, Nk):
    log(f"case block sparse {kind} causal={causal} Nq={Nq} Nk={Nk}")
    B, H, d = 2, 3, 128
    q, k, v = W.prefill_inputs(B, H, Nq, Nk, d, "bf16", seed=Nq + 3 * Nk, device="cuda")
    m = W.block_mask(kind, H, Nq, Nk, seed=Nq)
    o, lse = fa.fa_fwd_block_sparse(q, k, v, m.to("cuda"), 0.088, causal)
    torch.cuda.synchronize()
    O, L = oracle.attention_block_sparse(q, k, v, m, 0.088, causal)
    check(o, lse, O, L, TOL_BF16, f"block sparse {kind}")


@pytest.mark.parametrize("causal", [False, True])
def test_fwd_block_sparse_all_ones_equals_dense(fa, causal):
    """Every block admitted: the same tiles in the same order as the dense
    kernel, so the results are identical."""
    B, H, N, d = 1, 4, 777, 128
    q, k, v = W.prefill_inputs(B, H, N, N, d, "bf16", seed=31, device="cuda")
    o, lse = fa.fa_fwd(q, k, v, 0.088, causal)
    o2, lse2 = fa.fa_fwd_block_sparse(q, k, v, W.block_mask("ones", H, N, N).to("cuda"), 0.088,
                                      causal)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


def test_fwd_block_sparse_full_size_one_head(fa):
    """N=8192, H=32, causal, local window of 2 blocks each side plus the first
    key block: one head against the oracle."""
    s = W.LONG_PREFILL
    log(f"case block sparse {s.name} local_global")
    q, k, v = W.prefill_spec_inputs(s, "cuda")
    m = W.block_mask("local_global", s.H, s.Nq, s.Nk)
    o, lse = fa.fa_fwd_block_sparse(q, k, v, m.to("cuda"), s.scale, s.causal)
    torch.cuda.synchronize()
    h = 5
    O, L = oracle.attention_block_sparse(q, k, v, m, s.scale, s.causal, heads=[(0, h)])
    check(o[0, h], lse[0, h], O[0, h], L[0, h], TOL_BF16, f"head {h}")


def paged_copy(kc, vc, sl, off, page_size, seed, spare=3, max_len=None):
    bt, npg = W.paged_layout(sl, page_size, seed=seed, spare_pages=spare, max_len=max_len)
    kp = W.to_pages(kc, sl, off, bt, page_size, npg)
    vp = W.to_pages(vc, sl, off, bt, page_size, npg)
    return bt, kp, vp


@pytest.mark.parametrize("d,P,sk", [(128, 1, 64), (128, 16, 0), (128, 16, 256), (128, 64, 128),
                                    (128, 256, 0), (128, 4096, 0), (64, 32, 0)])
def test_decode_paged(fa, d, P, sk):
    """Paged cache, pages in random order: against the oracle, and identical
    to the packed kernel run with the same chunks (same arithmetic, only the
    addresses differ)."""
    lens = [0, 1, max(P - 1, 2), P, P + 1, 700, 3000]
    B, H = len(lens), 4
    log(f"case decode paged d={d} page={P} split_keys={sk}")
    q, kc, vc, sl, off = W.decode_inputs(B, H, d, lens, seed=50 + P, device="cuda")
    bt, kp, vp = paged_copy(kc, vc, sl, off, P, seed=P)
    o, lse = fa.fa_decode_paged(q, kp, vp, bt.to("cuda"), sl, max(lens), 0.088, sk)
    sk_used = sk or fa.fa_decode_paged_split_keys(B, H, d, max(lens), P)
    o2, lse2 = fa.fa_decode_varlen_split(q, kc, vc, sl, off, max(lens), sk_used, 0.088)
    torch.cuda.synchronize()
    O, L = oracle.decode_paged(q, kp, vp, bt, sl.cpu(), 0.088)
    check(o, lse, O, L, TOL_BF16, f"paged page={P}")
    assert torch.equal(o, o2), "paged and packed outputs differ"
    assert torch.equal(lse.isneginf(), lse2.isneginf())
    fin = ~lse.isneginf()
    assert torch.equal(lse[fin], lse2[fin]), "paged and packed LSE differ"


def test_decode_paged_batched_full_size(fa):
    """The batched decode workload (64 sequences, lengths U[128, 16384]) with
    16-token pages in random order: whole output identical to the packed
    kernel, sampled (sequence, head) pairs against the oracle."""
    s = W.DECODE_BATCHED
    log(f"case {s.name} paged 16")
    q, kc, vc, sl, off = W.decode_spec_inputs(s, "cuda")
    bt, kp, vp = paged_copy(kc, vc, sl, off, 16, seed=s.seed, max_len=s.max_len)
    del kc, vc
    o, lse = fa.fa_decode_paged(q, kp, vp, bt.to("cuda"), sl, s.max_len, s.scale, 0)
    torch.cuda.synchronize()
    seqs, heads = [0, 7, 31, 63], [0, 13, 31]
    O, L = oracle.decode_paged(q, kp, vp, bt, sl.cpu(), s.scale, heads=heads, seqs=seqs)
    idx = np.ix_(seqs, heads)
    check(o[seqs][:, heads], lse[seqs][:, heads], O[idx], L[idx], TOL_BF16, "paged batched sampled")
    del kp, vp
    q2, kc, vc, sl2, off2 = W.decode_spec_inputs(s, "cuda")
    sk = fa.fa_decode_paged_split_keys(s.B, s.H, s.d, s.max_len, 16)
    o2, lse2 = fa.fa_decode_varlen_split(q2, kc, vc, sl2, off2, s.max_len, sk, s.scale)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


def test_probe_read_runs(fa):
    """The read probe (a measurement aid) streams a buffer and leaves the sink
    alone unless the data's XOR hits its fixed constant (zeros never do)."""
    log("case probe read")
    buf = torch.zeros(3 << 20, dtype=torch.uint8, device="cuda")
    sink = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    fa.fa_probe_read(buf, sink=sink)
    fa.fa_probe_read(buf, nbytes=4096 + 16, sink=sink)  # a ragged last workgroup
    torch.cuda.synchronize()
    assert sink.item() == 7


def test_probe_issue_runs(fa):
    """The issue probe (a measurement aid) times every role on a few
    workgroups: positive cycle counts, and a product alone costs at least its
    32 pipeline cycles (8 passes of 4) and not absurdly more."""
    log("case probe issue")
    for ra, rb, na, nb in (("products", "none", 64, 0), ("lds_tr8", "lds16", 64, 64),
                           ("product_softmax", "product_8fma", 64, 64), ("fma", "exp", 64, 64)):
        out = fa.fa_probe_issue(ra, rb, na, nb, grid=4)
        cyc = out[:, :, 0]
        assert bool((cyc[:, :4] > 0).all()), (ra, rb)
        if nb:
            assert bool((cyc[:, 4:] > 0).all()), (ra, rb)
    out = fa.fa_probe_issue("products", "none", 1024, 0, grid=4)
    per_op = float(out[:, :4, 0].double().mean()) / 1024
    assert 28.0 <= per_op <= 200.0, per_op
