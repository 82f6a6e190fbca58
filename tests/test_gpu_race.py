"""Race check: the library against its race-check build (libfa_paranoid.so,
FA_PARANOID_SYNC: every memory operation drained at a barrier at each LDS
stage boundary of the hand-pipelined kernels, full device-scope fences around
the decode arrival counters).  The two builds do the same arithmetic in the
same order, so their outputs must be bit-identical; a missing or miscounted
wait in the library (a tile read before its copy lands, a buffer overwritten
while still read, a chunk state read before it is visible) would show up
as a difference."""
import math
import os

import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu

PARANOID = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "io_aware_exact_17_amd", "libfa_paranoid.so")


@pytest.fixture(scope="module")
def paranoid(fa):
    return fa.load_library(PARANOID)


def both(fa, paranoid, fn):
    a = fn()
    torch.cuda.synchronize()
    with fa.using_library(paranoid):
        b = fn()
        torch.cuda.synchronize()
    return a, b


def same(a, b, what):
    for x, y in zip(a, b):
        assert torch.equal(x, y), f"{what}: the race-check build differs"


@pytest.mark.parametrize("d,B,H,N", [(128, 2, 4, 700), (128, 1, 32, 8192), (64, 2, 100, 600)])
@pytest.mark.parametrize("causal", [True, False])
def test_prefill_matches_race_check_build(fa, paranoid, d, B, H, N, causal):
    print(f"case race prefill d={d} B={B} H={H} N={N} causal={causal}", flush=True)
    q, k, v = W.prefill_inputs(B, H, N, N, d, "bf16", seed=N + d, device="cuda")
    a, b = both(fa, paranoid, lambda: fa.fa_fwd(q, k, v, 1 / math.sqrt(d), causal))
    same(a, b, f"prefill d={d}")


def test_decode_matches_race_check_build(fa, paranoid):
    print("case race decode", flush=True)
    s = W.DECODE_BATCHED
    q, kc, vc, sl, off = W.decode_spec_inputs(s, "cuda")
    a, b = both(fa, paranoid, lambda: fa.fa_decode_varlen(q, kc, vc, sl, off, s.max_len, s.scale))
    same(a, b, "batched decode")
    a, b = both(fa, paranoid, lambda: fa.fa_decode_varlen_split(q, kc, vc, sl, off, s.max_len, 256,
                                                                s.scale))
    same(a, b, "batched decode, 256-key chunks")
    s = W.DECODE_SINGLE
    q, kc, vc, sl, off = W.decode_spec_inputs(s, "cuda")
    a, b = both(fa, paranoid, lambda: fa.fa_decode_varlen(q, kc, vc, sl, off, s.max_len, s.scale))
    same(a, b, "single decode")


@pytest.mark.parametrize("d", [128, 64])
def test_backward_matches_race_check_build(fa, paranoid, d):
    print(f"case race backward d={d}", flush=True)
    q, k, v = W.prefill_inputs(1, 4, 700, 700, d, "bf16", seed=3, device="cuda")
    do = W.prefill_inputs(1, 4, 700, 1, d, "bf16", seed=4, device="cuda")[0]
    o, lse = fa.fa_fwd(q, k, v, 1 / math.sqrt(d), True)
    a, b = both(fa, paranoid, lambda: fa.fa_bwd(q, k, v, o, do, lse, 1 / math.sqrt(d), True))
    same(a, b, f"backward d={d}")
