"""Benchmark of the exact-attention forward path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--cpu-budget SECONDS]
    python bench.py --sweep-seqlen

One step is one pass of the whole hot path over resident synthetic inputs:
  1. fa_fwd      causal prefill, B=1, H=32, Nq=Nk=8192, d=128, bf16
  2. fa_decode_varlen  batched decode, 64 sequences x 32 heads, d=128, history
                 lengths uniform in [128, 16384] (packed bf16 K/V cache)
  3. fa_decode_varlen  single-request decode, 32 heads, 8192-token history
  4. fa_decode_paged   the batched decode's cache as 16-token pages in seeded
                 random order (block table per sequence)
  5. fa_fwd_varlen     packed causal prefill of 8 sequences, lengths U[512, 8192],
                 H=32, d=128 (token-major [T, H, d], cu_seqlens)
  6. fa_bwd            backward of call 1 (its O and LSE, a seeded dO), fp32
                 gradients, by recomputation
  7. fa_fwd_block_sparse  call 1's inputs under a 64x64 block mask: a window of
                 two blocks either side of the diagonal plus the first key block
  8. fa_fwd      GPT-2-medium-shaped attention, B=64, H=16, N=1024, d=64, bf16,
                 non-causal, then the same inputs causal
The batched decode streams ~8.7 GB, far more than the 256 MB last-level
cache, so the single-request decode that follows reads its 128 MiB of K/V
from HBM.  Every call is bracketed by HIP events on the stream it runs on.

Prints one JSON line: `value` is the prefill rate in TFLOP/s (4*B*H*N^2*d/2
algorithmic FLOPs over the prefill kernel's event time); the decode KV-read
rates (GB/s) ride along in `decode`, beside the read rate a plain streaming
read kernel reaches on the same byte counts (the empirical ceiling); `roofline` describes the prefill kernel
against the bf16 dense matrix-core peak; `cpu_baseline` times the fp64 oracle
on a bounded sample of the prefill on the host.

`--sweep-seqlen` instead times the prefill (d=128 with H=32, d=64 with H=16,
non-causal and causal) and the d=128 backward at sequence lengths 512 ..
32768 with the batch chosen so that every launch holds 32768 tokens, and
prints one JSON line per shape.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fwd TFLOP/s @ causal N=8192 d=128 bf16; decode KV-read GB/s"
PEAK_BF16_TFLOPS = 2516.6   # 256 CUs x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU
PEAK_HBM_GBPS = 8000.0      # HBM3E
# HBM bytes per prefill launch from rocprofv3 FETCH_SIZE + WRITE_SIZE at this
# workload, each scaled by what the counter reads for a plain 1 GiB copy
# (FETCH x2.0, WRITE x1.0): 215595.2 KiB x 2 + 66560 KiB.  None whenever the
# prefill kernel has changed since the counters were taken.
PREFILL_TRAFFIC_BYTES = 509696410


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=30)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--cpu-budget", type=float, default=12.0,
                   help="seconds of host time for the oracle baseline sample")
    p.add_argument("--sweep-seqlen", action="store_true",
                   help="time prefill and backward against sequence length instead")
    p.add_argument("--probe-issue", action="store_true",
                   help="print what one SIMD overlaps (products, vector work, LDS reads) instead")
    return p.parse_args()


# (role of waves 0-3, role of waves 4-7, operations each): a role alone, then
# beside another role on the same SIMDs.
PROBE_CASES = (
    ("products", "none", 1024, 0), ("fma", "none", 8192, 0), ("exp", "none", 4096, 0),
    ("lds16", "none", 2048, 0), ("lds_tr8", "none", 2048, 0),
    ("product_softmax", "none", 1024, 0), ("product_8fma", "none", 1024, 0),
    ("products", "fma", 1024, 8192), ("products", "exp", 1024, 4096),
    ("products", "lds16", 1024, 2048), ("products", "lds_tr8", 1024, 2048),
    ("products", "products", 1024, 1024), ("product_softmax", "product_softmax", 1024, 1024),
    ("lds16", "lds16", 2048, 2048), ("lds_tr8", "lds_tr8", 2048, 2048),
    ("products", "product_softmax", 1024, 1024), ("products", "product_8fma", 1024, 1024),
    ("products", "product_8fma", 2048, 1024),
)


def probe_issue(fa):
    """Shader-clock cycles per operation of each wave group (mean over all
    workgroups, second of two runs), one 8-wave workgroup per CU."""
    rows = []
    for ra, rb, na, nb in PROBE_CASES:
        for _ in range(2):
            out = fa.fa_probe_issue(ra, rb, na, nb)
        cyc = out[:, :, 0].double()
        simd = (out[:, :, 1] >> 4) & 3  # HW_ID bits 5:4
        simd_ok = bool(simd[:, :4].eq(simd[:, 4:]).all()) and all(
            len(set(row)) == 4 for row in simd[:, :4].tolist())
        a = float(cyc[:, :4].mean())
        b = float(cyc[:, 4:].mean())
        rows.append((ra, rb, na, nb, a, b, simd_ok))
        line = f"A={ra:<16} x{na:<5} B={rb:<16} x{nb:<5}  A {a:9.0f} cyc ({a / na:6.2f}/op)"
        if nb:
            line += f"  B {b:9.0f} cyc ({b / nb:6.2f}/op)"
        line += f"  waves w, w+4 share a SIMD: {simd_ok}"
        print(line, flush=True)
    simd = ((out[0, :, 1] >> 4) & 3).tolist()
    print(f"SIMD of waves 0-7 in workgroup 0 (HW_ID bits 5:4): {simd}; HW_ID: "
          + " ".join(f"{int(x):#010x}" for x in out[0, :, 1]), flush=True)
    return rows


SWEEP_TOKENS = 32768
SWEEP_LENGTHS = (512, 1024, 2048, 4096, 8192, 16384, 32768)


def sweep_seqlen(fa, W, dev):
    """TFLOP/s of the prefill and the d=128 backward against sequence length
    at a fixed 32768 tokens per launch (B = 32768 / N), seeded N(0,1) inputs,
    the mean of HIP-event times on the launch stream after warm-up calls."""
    import torch

    stream = torch.cuda.current_stream(dev)

    def mean_ms(fn, reps, skip):
        ts = []
        for i in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            e1.synchronize()
            if i >= skip:
                ts.append(e0.elapsed_time(e1))
        return statistics.mean(ts)

    for d, H in ((128, 32), (64, 16)):
        for N in SWEEP_LENGTHS:
            B = SWEEP_TOKENS // N
            scale = d ** -0.5
            q, k, v = W.prefill_inputs(B, H, N, N, d, "bf16", seed=7, device=dev)
            o = torch.empty_like(q)
            lse = torch.empty(B, H, N, dtype=torch.float32, device=dev)
            rec = {"d": d, "H": H, "B": B, "N": N, "unit": "TFLOP/s"}
            for causal in (False, True):
                ms = mean_ms(lambda: fa.fa_fwd(q, k, v, scale, causal, out=o, lse=lse), 20, 5)
                flops = 4 * B * H * N * N * d / (2 if causal else 1)
                rec["fwd_causal" if causal else "fwd"] = round(flops / (ms * 1e-3) / 1e12, 1)
            if d == 128:
                dout = W.prefill_inputs(B, H, N, N, d, "bf16", seed=8, device=dev)[0]
                ws = torch.empty(fa.fa_bwd_workspace_bytes(B, H, N), dtype=torch.uint8, device=dev)
                dq = torch.empty(B, H, N, d, dtype=torch.float32, device=dev)
                dk, dv = torch.empty_like(dq), torch.empty_like(dq)
                for causal in (False, True):
                    fa.fa_fwd(q, k, v, scale, causal, out=o, lse=lse)
                    ms = mean_ms(lambda: fa.fa_bwd(q, k, v, o, dout, lse, scale, causal, dq=dq,
                                                   dk=dk, dv=dv, workspace=ws), 12, 3)
                    flops = 2.5 * 4 * B * H * N * N * d / (2 if causal else 1)
                    rec["bwd_causal" if causal else "bwd"] = round(flops / (ms * 1e-3) / 1e12, 1)
                del dout, ws, dq, dk, dv
            print(json.dumps(rec), flush=True)
            del q, k, v, o, lse
            torch.cuda.empty_cache()


def blas_threads():
    """Threads of the BLAS library NumPy calls (the oracle's products)."""
    try:
        from threadpoolctl import threadpool_info

        return max(i.get("num_threads", 1) for i in threadpool_info())
    except Exception:
        import torch

        return torch.get_num_threads()


def oracle_per_config(budget_s: float, dev, decode_batched):
    """The oracle timed on bounded samples of the other workloads, on the
    host, after the GPU timing: the tiny fp32 case whole, whole heads of the
    GPT-2-medium shape (non-causal) until the budget, the single decode whole,
    and whole sequences (all heads) of the batched decode until the budget.
    Inputs are copied to the host before the clock starts."""
    import torch

    import oracle
    import workloads as W

    out = {}
    s = W.TINY_F32
    q, k, v = W.prefill_spec_inputs(s, "cpu")
    t0 = time.perf_counter()
    oracle.attention(q, k, v, s.scale, s.causal)
    dt = time.perf_counter() - t0
    out["tiny_f32"] = {"s": round(dt, 4), "GFLOP/s": round(s.flops() / dt / 1e9, 3)}

    G = W.GPT2M
    g = torch.Generator().manual_seed(G.seed)
    heads, t_tot = 0, 0.0
    while heads == 0 or t_tot < budget_s:
        qh, kh, vh = (torch.randn(G.Nq, G.d, generator=g).to(torch.bfloat16) for _ in range(3))
        t0 = time.perf_counter()
        oracle.head_attention(qh, kh, vh, G.scale, causal=False)
        t_tot += time.perf_counter() - t0
        heads += 1
    out["gpt2_medium_noncausal"] = {
        "GFLOP/s": round(heads * 4.0 * G.Nq * G.Nk * G.d / t_tot / 1e9, 2),
        "sample": f"{heads} whole heads of {G.B * G.H}, {t_tot:.2f} s"}

    S = W.DECODE_SINGLE
    q, kc, vc, sl, off = W.decode_spec_inputs(S, "cpu")
    t0 = time.perf_counter()
    oracle.decode(q, kc, vc, sl, off, S.scale)
    dt = time.perf_counter() - t0
    out["decode_single"] = {"GB/s": round(W.decode_kv_bytes(sl, S.H, S.d) / dt / 1e9, 3),
                            "s": round(dt, 3), "sample": "whole workload"}

    D = W.DECODE_BATCHED
    dq, dk, dv, dl, do = decode_batched
    lens = dl.cpu()
    offs = do.cpu()
    seqs, t_tot, nbytes = 0, 0.0, 0
    while seqs < D.B and (seqs == 0 or t_tot < budget_s):
        lo, n = int(offs[seqs]), int(lens[seqs])
        kh, vh = dk[lo:lo + n].cpu(), dv[lo:lo + n].cpu()
        qh = dq[seqs:seqs + 1].cpu()
        one = torch.tensor([n], dtype=torch.int32)
        zero = torch.zeros(1, dtype=torch.int32)
        t0 = time.perf_counter()
        oracle.decode(qh, kh, vh, one, zero, D.scale)
        t_tot += time.perf_counter() - t0
        nbytes += W.decode_kv_bytes(one, D.H, D.d)
        seqs += 1
    out["decode_batched"] = {"GB/s": round(nbytes / t_tot / 1e9, 3),
                             "sample": f"{seqs} of {D.B} whole sequences, all heads, {t_tot:.2f} s"}
    out["cores"] = len(os.sched_getaffinity(0))
    out["blas_threads"] = blas_threads()
    return out


def sclk_mhz():
    """The current shader clock level from sysfs (None where not readable)."""
    import glob

    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            for line in open(path):
                if line.strip().endswith("*"):
                    return int(line.split(":")[1].strip().split("Mhz")[0].split("MHz")[0])
        except (OSError, ValueError, IndexError):
            continue
    return None


def cpu_baseline(budget_s: float):
    """The fp64 oracle (as it stands) on whole heads of the causal prefill
    workload, one head at a time until the budget is spent (at least one)."""
    import numpy as np
    import torch

    import oracle
    import workloads as W

    threads = blas_threads()
    s = W.LONG_PREFILL
    g = torch.Generator().manual_seed(s.seed)
    heads = 0
    flops = 0.0
    t_total = 0.0
    while heads == 0 or t_total < budget_s:
        q = torch.randn(s.Nq, s.d, generator=g).to(torch.bfloat16).double().numpy()
        k = torch.randn(s.Nk, s.d, generator=g).to(torch.bfloat16).double().numpy()
        v = torch.randn(s.Nk, s.d, generator=g).to(torch.bfloat16).double().numpy()
        t0 = time.perf_counter()
        oracle.head_attention(q, k, v, s.scale, causal=True)
        t_total += time.perf_counter() - t0
        heads += 1
        flops += 4.0 * s.Nq * s.Nk * s.d / 2
        if heads >= s.H:
            break
    return {"value": flops / t_total / 1e12, "unit": "TFLOP/s",
            "cores": len(os.sched_getaffinity(0)), "blas_threads": int(threads),
            "kind": "oracle",
            "sample": f"{heads} of {s.H} heads of the causal N=8192 d=128 prefill, whole heads, "
                      f"fp64 NumPy with S and P materialised; {t_total:.1f} s"}


def read_ceiling(torch, fa, dev, stream, small_bytes):
    """Empirical read bandwidth (GB/s) of a plain streaming-read kernel
    (fa_probe_read) for the single decode's byte count and for 8 GiB, each
    repetition on a region no earlier repetition touched (cold, clean cache).
    Each timed read is queued behind an untimed 1 GiB read of another region,
    so the GPU reaches the start event with the timed launch already
    submitted, as in the bench step (an idle GPU would add the host's launch
    latency, several microseconds, to a 25 us read)."""
    big = torch.empty(8 << 30, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    filler = big[7 << 30:]  # never timed

    def timed(nbytes, offsets, skip, fill):
        ts = []
        for i, off in enumerate(offsets):
            e0, e1 = ev(), ev()
            if fill:
                fa.fa_probe_read(filler, sink=sink, stream=stream)
            e0.record(stream)
            fa.fa_probe_read(big[off:off + nbytes], sink=sink, stream=stream)
            e1.record(stream)
            e1.synchronize()
            if i >= skip:
                ts.append(e0.elapsed_time(e1))
        return nbytes / (statistics.mean(ts) * 1e-3) / 1e9

    small = timed(small_bytes, [i * small_bytes for i in range(12)], 2, True)
    full = timed(big.numel(), [0, 0, 0], 1, False)
    del big
    return small, full


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU "
              "sharding of this path is a design note, not a measured configuration.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import io_aware_exact_17_amd as fa
    import workloads as W

    fa.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)
    if args.sweep_seqlen:
        sweep_seqlen(fa, W, dev)
        return
    if args.probe_issue:
        probe_issue(fa)
        return

    P = W.LONG_PREFILL
    DB = W.DECODE_BATCHED
    DS = W.DECODE_SINGLE
    q, k, v = W.prefill_spec_inputs(P, dev)
    o = torch.empty_like(q)
    lse = torch.empty(P.B, P.H, P.Nq, dtype=torch.float32, device=dev)

    dbq, dbk, dbv, dbl, dbo = W.decode_spec_inputs(DB, dev)
    lens_b = dbl.cpu()
    db_out = torch.empty_like(dbq)
    db_lse = torch.empty(DB.B, DB.H, dtype=torch.float32, device=dev)
    db_sk = fa.fa_decode_split_keys(DB.B, DB.H, DB.d, DB.max_len)
    # decode workspaces: zero-filled once (their arrival counters start at 0
    # and every call leaves them at 0)
    db_ws = torch.zeros(fa.fa_decode_workspace_bytes(DB.B, DB.H, DB.d, DB.max_len),
                        dtype=torch.uint8, device=dev)

    dsq, dsk, dsv, dsl, dso = W.decode_spec_inputs(DS, dev)
    ds_out = torch.empty_like(dsq)
    ds_lse = torch.empty(DS.B, DS.H, dtype=torch.float32, device=dev)
    ds_sk = fa.fa_decode_split_keys(DS.B, DS.H, DS.d, DS.max_len)
    ds_ws = torch.zeros(fa.fa_decode_workspace_bytes(DS.B, DS.H, DS.d, DS.max_len),
                        dtype=torch.uint8, device=dev)

    # The batched workload again as a paged cache (16-token pages, random order).
    PAGE = 16
    pg_bt, pg_pages = W.paged_layout(dbl.cpu(), PAGE, seed=DB.seed, max_len=DB.max_len)
    pg_k = W.to_pages(dbk, dbl, dbo, pg_bt, PAGE, pg_pages)
    pg_v = W.to_pages(dbv, dbl, dbo, pg_bt, PAGE, pg_pages)
    pg_bt = pg_bt.to(dev)
    pg_sk = fa.fa_decode_paged_split_keys(DB.B, DB.H, DB.d, DB.max_len, PAGE)
    pg_ws = torch.zeros(fa.fa_decode_split_workspace_bytes(DB.B, DB.H, DB.d, DB.max_len, pg_sk),
                        dtype=torch.uint8, device=dev)
    pg_out = torch.empty_like(dbq)
    pg_lse = torch.empty(DB.B, DB.H, dtype=torch.float32, device=dev)

    # Packed variable-length causal prefill.
    VL = W.VARLEN_PREFILL
    vl_lens, vlq, vlk, vlv, vlcq, vlck = W.varlen_spec_inputs(VL, dev)
    vl_max = int(vl_lens.max())
    vl_out = torch.empty_like(vlq)
    vl_lse = torch.empty(VL.H, vlq.shape[0], dtype=torch.float32, device=dev)
    vl_flops = VL.flops(vl_lens)

    # Backward of the long prefill: dO seeded, O and LSE from call 1.
    bw_do = W.prefill_inputs(P.B, P.H, P.Nq, 1, P.d, "bf16", seed=P.seed + 1, device=dev)[0]
    bw_dq = torch.empty(q.shape, dtype=torch.float32, device=dev)
    bw_dk = torch.empty(k.shape, dtype=torch.float32, device=dev)
    bw_dv = torch.empty(v.shape, dtype=torch.float32, device=dev)
    bw_ws = torch.empty(fa.fa_bwd_workspace_bytes(P.B, P.H, P.Nq), dtype=torch.uint8, device=dev)
    bw_flops = 2.5 * P.flops()

    # Block-sparse forward of the long prefill's inputs (local window + global block).
    bs_mask_h = W.block_mask("local_global", P.H, P.Nq, P.Nk)
    bs_mask = bs_mask_h.to(dev)
    bs_out = torch.empty_like(q)
    bs_lse = torch.empty_like(lse)
    bs_pairs = W.block_mask_pairs(bs_mask_h[:1], P.Nq, P.Nk, True) * P.H * P.B  # same pattern per head
    bs_flops = 4.0 * P.d * bs_pairs

    # GPT-2-medium-shaped attention (d = 64), non-causal and causal.
    G = W.GPT2M
    gq, gk, gv = W.prefill_spec_inputs(G, dev)
    g_out = torch.empty_like(gq)
    g_lse = torch.empty(G.B, G.H, G.Nq, dtype=torch.float32, device=dev)

    # A plain copy of known size, untimed: its HBM counters calibrate the
    # prefill kernel's FETCH_SIZE / WRITE_SIZE when this script runs under
    # rocprofv3 --pmc.
    cal_src = torch.empty(1 << 29, dtype=torch.bfloat16, device=dev).fill_(1.0)
    cal_dst = torch.empty_like(cal_src)
    cal_dst.copy_(cal_src)
    del cal_src, cal_dst
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def step(rec):
        e0, e1, e2, e3, e4, e5, e6, e7, e8, e9 = (ev() for _ in range(10))
        e0.record(stream)
        fa.fa_fwd(q, k, v, P.scale, True, out=o, lse=lse)
        e1.record(stream)
        fa.fa_decode_varlen(dbq, dbk, dbv, dbl, dbo, DB.max_len, DB.scale, out=db_out,
                            lse=db_lse, workspace=db_ws)
        e2.record(stream)
        fa.fa_decode_varlen(dsq, dsk, dsv, dsl, dso, DS.max_len, DS.scale, out=ds_out,
                            lse=ds_lse, workspace=ds_ws)
        e3.record(stream)
        fa.fa_decode_paged(dbq, pg_k, pg_v, pg_bt, dbl, DB.max_len, DB.scale, 0, out=pg_out,
                           lse=pg_lse, workspace=pg_ws)
        e4.record(stream)
        fa.fa_fwd_varlen(vlq, vlk, vlv, vlcq, vlck, vl_max, VL.scale, VL.causal, out=vl_out,
                         lse=vl_lse)
        e5.record(stream)
        fa.fa_bwd(q, k, v, o, bw_do, lse, P.scale, True, dq=bw_dq, dk=bw_dk, dv=bw_dv,
                  workspace=bw_ws)
        e6.record(stream)
        fa.fa_fwd_block_sparse(q, k, v, bs_mask, P.scale, True, out=bs_out, lse=bs_lse)
        e7.record(stream)
        fa.fa_fwd(gq, gk, gv, G.scale, False, out=g_out, lse=g_lse)
        e8.record(stream)
        fa.fa_fwd(gq, gk, gv, G.scale, True, out=g_out, lse=g_lse)
        e9.record(stream)
        if rec is not None:
            rec.append((e0, e1, e2, e3, e4, e5, e6, e7, e8, e9))

    for _ in range(args.warmup):
        step(None)
    torch.cuda.synchronize()

    recs = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(recs)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    t_pre = [r[0].elapsed_time(r[1]) for r in recs]
    t_db = [r[1].elapsed_time(r[2]) for r in recs]
    t_ds = [r[2].elapsed_time(r[3]) for r in recs]
    t_pg = [r[3].elapsed_time(r[4]) for r in recs]
    t_vl = [r[4].elapsed_time(r[5]) for r in recs]
    t_bw = [r[5].elapsed_time(r[6]) for r in recs]
    t_bs = [r[6].elapsed_time(r[7]) for r in recs]
    t_gn = [r[7].elapsed_time(r[8]) for r in recs]
    t_gc = [r[8].elapsed_time(r[9]) for r in recs]
    ms_step = wall * 1e3 / args.steps

    flops = P.flops()
    pre_ms = statistics.mean(t_pre)
    tflops = flops / (pre_ms * 1e-3) / 1e12
    db_bytes = W.decode_kv_bytes(lens_b, DB.H, DB.d)
    ds_bytes = W.decode_kv_bytes(dsl.cpu(), DS.H, DS.d)
    db_gbps = db_bytes / (statistics.mean(t_db) * 1e-3) / 1e9
    ds_gbps = ds_bytes / (statistics.mean(t_ds) * 1e-3) / 1e9
    pg_gbps = db_bytes / (statistics.mean(t_pg) * 1e-3) / 1e9
    vl_tflops = vl_flops / (statistics.mean(t_vl) * 1e-3) / 1e12
    bw_tflops = bw_flops / (statistics.mean(t_bw) * 1e-3) / 1e12
    bs_tflops = bs_flops / (statistics.mean(t_bs) * 1e-3) / 1e12
    g_flops, gc_flops = W.GPT2M.flops(), W.GPT2M_CAUSAL.flops()
    gn_tflops = g_flops / (statistics.mean(t_gn) * 1e-3) / 1e12
    gc_tflops = gc_flops / (statistics.mean(t_gc) * 1e-3) / 1e12

    ceil_small, ceil_big = read_ceiling(torch, fa, dev, stream, ds_bytes)

    max_alloc = torch.cuda.max_memory_allocated(dev)
    cpu = cpu_baseline(args.cpu_budget)
    per_cfg = oracle_per_config(min(3.0, args.cpu_budget / 4), dev, (dbq, dbk, dbv, dbl, dbo))

    line = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "causal prefill B=1 H=32 N=8192 d=128 + batched varlen decode "
                        "64 seqs x 32 heads d=128 len U[128,16384] + single decode H=32 N=8192 d=128 "
                        "+ the batched decode over a paged cache (16-token pages) "
                        "+ packed causal prefill 8 seqs x 32 heads d=128 len U[512,8192] "
                        "+ backward of the causal prefill + block-sparse causal prefill "
                        "(local window of 2 blocks + first block, 64x64 blocks) "
                        "+ GPT-2-medium-shaped prefill B=64 H=16 N=1024 d=64, non-causal and causal",
            "prefill": {"B": P.B, "H": P.H, "Nq": P.Nq, "Nk": P.Nk, "d": P.d, "causal": True,
                        "seed": P.seed, "flops": flops, "ms_mean": round(pre_ms, 4),
                        "ms_median": round(statistics.median(t_pre), 4),
                        "ms_min": round(min(t_pre), 4)},
            "decode_batched": {"B": DB.B, "H": DB.H, "d": DB.d, "seed": DB.seed,
                               "tokens": int(lens_b.sum()), "kv_bytes": db_bytes,
                               "split_keys": db_sk, "ms_mean": round(statistics.mean(t_db), 4)},
            "decode_single": {"B": DS.B, "H": DS.H, "Nk": DS.fixed_len, "d": DS.d,
                              "kv_bytes": ds_bytes, "split_keys": ds_sk,
                              "ms_mean": round(statistics.mean(t_ds), 4)},
            "decode_paged": {"page_size": PAGE, "pages": pg_pages, "split_keys": pg_sk,
                             "kv_bytes": db_bytes, "ms_mean": round(statistics.mean(t_pg), 4)},
            "block_sparse": {"B": P.B, "H": P.H, "N": P.Nq, "d": P.d, "causal": True,
                             "mask": "local_global window 2", "block": 64,
                             "admitted_blocks": int(bs_mask_h.sum()),
                             "visible_pairs": bs_pairs, "flops": bs_flops,
                             "ms_mean": round(statistics.mean(t_bs), 4)},
            "backward": {"B": P.B, "H": P.H, "N": P.Nq, "d": P.d, "causal": True,
                         "flops": bw_flops, "ms_mean": round(statistics.mean(t_bw), 4)},
            "gpt2_medium": {"B": G.B, "H": G.H, "N": G.Nq, "d": G.d, "seed": G.seed,
                            "flops_noncausal": g_flops, "flops_causal": gc_flops,
                            "ms_mean_noncausal": round(statistics.mean(t_gn), 4),
                            "ms_mean_causal": round(statistics.mean(t_gc), 4)},
            "prefill_varlen": {"B": VL.B, "H": VL.H, "d": VL.d, "causal": VL.causal,
                               "seed": VL.seed, "lengths": [int(x) for x in vl_lens],
                               "flops": vl_flops, "ms_mean": round(statistics.mean(t_vl), 4)},
        },
        "decode": {"unit": "GB/s",
                   "batched_kv_read": round(db_gbps, 1),
                   "single_kv_read": round(ds_gbps, 1),
                   "paged_batched_kv_read": round(pg_gbps, 1),
                   "frac_of_hbm_peak": {"batched": round(db_gbps / PEAK_HBM_GBPS, 4),
                                        "single": round(ds_gbps / PEAK_HBM_GBPS, 4),
                                        "paged_batched": round(pg_gbps / PEAK_HBM_GBPS, 4)},
                   "read_ceiling": {"128MiB": round(ceil_small, 1), "8GiB": round(ceil_big, 1),
                                    "kind": "plain non-temporal 16-byte-load read kernel, cold clean cache"},
                   "frac_of_read_ceiling": {"batched": round(db_gbps / ceil_big, 4),
                                            "single": round(ds_gbps / ceil_small, 4),
                                            "paged_batched": round(pg_gbps / ceil_big, 4)}},
        "roofline": {
            "kernel": "fwd_bf16_kernel<128, causal>",
            "bound": "mfma",
            "achieved": round(tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": PREFILL_TRAFFIC_BYTES,
        },
        "varlen": {"unit": "TFLOP/s", "prefill_varlen": round(vl_tflops, 2),
                   "frac_of_bf16_peak": round(vl_tflops / PEAK_BF16_TFLOPS, 4)},
        "gpt2_medium": {"unit": "TFLOP/s", "noncausal": round(gn_tflops, 2),
                        "causal": round(gc_tflops, 2),
                        "frac_of_bf16_peak": {"noncausal": round(gn_tflops / PEAK_BF16_TFLOPS, 4),
                                              "causal": round(gc_tflops / PEAK_BF16_TFLOPS, 4)}},
        "block_sparse": {"unit": "TFLOP/s", "value": round(bs_tflops, 2),
                         "flops_convention": "4 * d * visible (query, key) pairs"},
        "backward": {"unit": "TFLOP/s", "value": round(bw_tflops, 2),
                     "frac_of_bf16_peak": round(bw_tflops / PEAK_BF16_TFLOPS, 4),
                     "flops_convention": "2.5 x forward (five products of 2*N*N*d, halved causal)"},
        "cpu_baseline": cpu,
        "oracle_per_config": per_cfg,
        "memory": {"max_allocated_bytes": int(max_alloc),
                   "workspace_bytes": {"decode_batched": db_ws.numel(),
                                       "decode_single": ds_ws.numel(),
                                       "decode_paged": pg_ws.numel(),
                                       "backward": bw_ws.numel()},
                   "note": "every buffer is allocated by the caller (torch); the library "
                           "allocates no device memory"},
        "dispatch": {"fa_fwd d=128 causal": "fwd_bf16_kernel<128, true, false, false>",
                     "fa_fwd d=64": "fwd_bf16_kernel<64, causal, false> (fwd_bf16_d64.hip)",
                     "fa_decode_varlen / fa_decode_paged": "single request: decode_split_kernel<128, packed, fused=true>; batched: decode_split_kernel<128, packed|paged, fused=false> + decode_merge_kernel<128>",
                     "fa_fwd_varlen": "fwd_bf16_kernel<128, true, true, false>",
                     "fa_fwd_block_sparse": "fwd_bf16_kernel<128, true, false, true>",
                     "fa_bwd": "bwd_rows_kernel, bwd_dkdv_kernel, bwd_dq_kernel",
                     "library": fa.LIB_PATH.replace(ROOT + os.sep, ""),
                     "fallback": "none (the binding raises if the library is missing)"},
        "device": {"name": props.name, "gcn_arch": getattr(props, "gcnArchName", ""),
                   "cus": props.multi_processor_count, "torch": torch.__version__,
                   "hip": torch.version.hip, "sclk_mhz_at_end": sclk_mhz()},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
