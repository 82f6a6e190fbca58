"""fa_decode_varlen_noalloc, the decode entry point that allocates nothing
(its chunk states live in the library's fixed per-device scratch), against
fa_decode_varlen with a caller workspace, through the C ABI, on two calls in
a row: the batched decode workload, then a smaller one."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

TOL_BF16, TOL_LSE = 2e-2, 1e-3


def _max_err(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    both = np.isneginf(a) & np.isneginf(b)
    return float(np.abs(np.where(both, 0.0, a) - np.where(both, 0.0, b)).max(initial=0.0))


def test_noalloc_decode_matches_workspace_decode(fa):
    s = W.DECODE_BATCHED
    small = ([5000, 0, 1, 300, 2049], 8, 64)  # second call: fewer sequences, heads, keys; d = 64
    cases = [("batched workload", None), ("smaller", small)]
    for name, spec in cases:
        print(f"case noalloc {name}", flush=True)
        if spec is None:
            q, kc, vc, sl, off = W.decode_spec_inputs(s, "cuda")
            max_len, scale, heads = s.max_len, s.scale, [0, 31]
        else:
            lens, H, d = spec
            q, kc, vc, sl, off = W.decode_inputs(len(lens), H, d, lens, seed=77, device="cuda")
            max_len, scale, heads = max(lens), 1 / math.sqrt(d), list(range(H))
        o1, l1 = fa.fa_decode_varlen_noalloc(q, kc, vc, sl, off, max_len, scale)
        o2, l2 = fa.fa_decode_varlen(q, kc, vc, sl, off, max_len, scale)
        torch.cuda.synchronize()
        # the two entry points differ only in the order of the fp32 merge
        eo = _max_err(o1.float().cpu(), o2.float().cpu())
        el = _max_err(l1.cpu(), l2.cpu())
        print(f"  vs fa_decode_varlen: dO={eo:.3e} dLSE={el:.3e}", flush=True)
        assert eo <= 2 ** -7 and el <= 1e-5
        assert torch.equal(torch.isneginf(l1), torch.isneginf(l2))
        O, L = oracle.decode(q, kc, vc, sl.cpu(), off.cpu(), scale, heads=heads)
        eo = _max_err(o1[:, heads].float().cpu(), O[:, heads])
        el = _max_err(l1[:, heads].cpu(), L[:, heads])
        print(f"  vs oracle: err_O={eo:.3e} err_LSE={el:.3e}", flush=True)
        assert eo <= TOL_BF16 and el <= TOL_LSE


def test_noalloc_decode_rejects_oversized_call(fa):
    """More chunk state than the fixed scratch: refused before any launch."""
    q, kc, vc, sl, off = W.decode_inputs(2, 2, 128, [3, 4], seed=1, device="cuda")
    B, H = 2048, 128  # 2048 x 128 heads x 2 chunks x 130 x 4 B > 16 MiB
    qb = torch.zeros(B, H, 128, dtype=torch.bfloat16, device="cuda")
    kb = torch.zeros(8, H, 128, dtype=torch.bfloat16, device="cuda")
    slb = torch.full((B,), 8, dtype=torch.int32, device="cuda")
    offb = torch.zeros(B, dtype=torch.int32, device="cuda")
    with pytest.raises(fa.FAError) as e:
        fa.fa_decode_varlen_noalloc(qb, kb, kb, slb, offb, 100000, 0.088)
    assert e.value.status == fa.FA_ERR_SCRATCH
    # the library still works afterwards
    o, lse = fa.fa_decode_varlen_noalloc(q, kc, vc, sl, off, 4, 0.088)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()
