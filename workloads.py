"""Seeded synthetic inputs for the exact-attention forward path.

This module only draws random tensors and lays them out; it holds none of the
attention arithmetic.  Both the HIP path (through its tests and the benchmark)
and the CPU oracle take their inputs from here, so neither has to trust the
other's data.

Shapes follow the scenarios the pages name:
  * GPT-2-medium attention: batch 64, 16 heads, N = 1024
    (AI圣经13 FlashAttention review, chengyansuo.com, §02);
  * long prefill 8192/8192, single-request decode 1/8192 and batched decode
    with mixed history lengths (FlashAttention explainer, cztcode.com/2026/5368,
    §6 table);
  * head dimension 64 to 128 (AI圣经13 review, §03).

Recipe: a torch.Generator on the device the tensors are made on, seeded per
workload, draws N(0, 1) in float32; bf16 workloads round those draws to bf16
(round-to-nearest-even).  Draw order: lengths (batched decode only), then q,
then k, then v.  The host copy of the rounded tensors is what the oracle reads.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class PrefillSpec:
    name: str
    B: int
    H: int
    Nq: int
    Nk: int
    d: int
    dtype: str  # "bf16" | "f32"
    causal: bool
    seed: int

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def flops(self) -> float:
        """Algorithmic FLOPs: two Nq x Nk x d contractions (QK^T and PV).

        Causal work is counted as half of the dense work (the 4*B*H*N^2*d/2
        convention)."""
        f = 4.0 * self.B * self.H * self.Nq * self.Nk * self.d
        return f / 2 if self.causal else f


@dataclass(frozen=True)
class DecodeSpec:
    name: str
    B: int
    H: int
    d: int
    min_len: int
    max_len: int
    seed: int
    fixed_len: int | None = None  # single-request decode uses one fixed length

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


# Tiny fp32 non-causal case the oracle finishes instantly.
TINY_F32 = PrefillSpec("tiny_f32_n128_d64", 1, 1, 128, 128, 64, "f32", False, 1701)
# GPT-2-medium-shaped attention, non-causal and causal.
GPT2M = PrefillSpec("gpt2m_b64_h16_n1024_d64", 64, 16, 1024, 1024, 64, "bf16", False, 1702)
GPT2M_CAUSAL = PrefillSpec("gpt2m_b64_h16_n1024_d64_causal", 64, 16, 1024, 1024, 64, "bf16", True, 1702)
# Single-request decode over an 8192-token history.
DECODE_SINGLE = DecodeSpec("decode_single_h32_n8192_d128", 1, 32, 128, 8192, 8192, 1703, fixed_len=8192)
# Batched decode, 64 sequences with history lengths uniform in [128, 16384].
DECODE_BATCHED = DecodeSpec("decode_batched_b64_h32_len128-16384_d128", 64, 32, 128, 128, 16384, 1704)
# Long causal prefill 8192/8192.
LONG_PREFILL = PrefillSpec("prefill_causal_h32_n8192_d128", 1, 32, 8192, 8192, 128, "bf16", True, 1705)


@dataclass(frozen=True)
class VarlenSpec:
    name: str
    B: int
    H: int
    d: int
    min_len: int
    max_len: int
    seed: int
    causal: bool

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def flops(self, lens) -> float:
        """4*H*d*Lq*Lk per sequence, halved when causal (the dense convention)."""
        tot = sum(int(x) * int(x) for x in lens)
        return 4.0 * self.H * self.d * tot / (2.0 if self.causal else 1.0)


# Packed variable-length causal prefill: 8 sequences, lengths uniform in
# [512, 8192] (queries = keys per sequence).
VARLEN_PREFILL = VarlenSpec("prefill_varlen_b8_h32_len512-8192_d128_causal", 8, 32, 128, 512, 8192,
                            1706, True)


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _normal(shape, g, device, dtype):
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    return x.to(dtype) if dtype != torch.float32 else x


def prefill_inputs(B, H, Nq, Nk, d, dtype="bf16", seed=0, device="cpu"):
    """q [B,H,Nq,d], k [B,H,Nk,d], v [B,H,Nk,d], contiguous, N(0,1)."""
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    g = _gen(device, seed)
    q = _normal((B, H, Nq, d), g, device, tdt)
    k = _normal((B, H, Nk, d), g, device, tdt)
    v = _normal((B, H, Nk, d), g, device, tdt)
    return q, k, v


def prefill_spec_inputs(spec: PrefillSpec, device="cpu"):
    return prefill_inputs(spec.B, spec.H, spec.Nq, spec.Nk, spec.d, spec.dtype, spec.seed, device)


def decode_lengths(B, min_len, max_len, seed, fixed_len=None):
    """Per-sequence history lengths (int32, host), drawn first from the seed."""
    if fixed_len is not None:
        return torch.full((B,), fixed_len, dtype=torch.int32)
    g = _gen("cpu", seed)
    return torch.randint(min_len, max_len + 1, (B,), generator=g, dtype=torch.int64).to(torch.int32)


def decode_inputs(B, H, d, seqlens, seed=0, device="cpu", dtype="bf16"):
    """Packed token-major cache for decode.

    Returns q [B,H,d], kcache [T,H,d], vcache [T,H,d] with T = sum(seqlens),
    seqlens int32 [B] and offsets int32 [B] (exclusive prefix sums), all on
    `device`.  Sequence b owns cache rows offsets[b] .. offsets[b]+seqlens[b]-1.
    """
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    seqlens = torch.as_tensor(seqlens, dtype=torch.int32).cpu()
    offs = torch.zeros(B, dtype=torch.int64)
    if B > 1:
        offs[1:] = torch.cumsum(seqlens.to(torch.int64), 0)[:-1]
    T = int(seqlens.to(torch.int64).sum())
    g = _gen(device, seed + 7919)  # lengths use the plain seed on the host
    q = _normal((B, H, d), g, device, tdt)
    k = _normal((max(T, 1), H, d), g, device, tdt)[:T]
    v = _normal((max(T, 1), H, d), g, device, tdt)[:T]
    return (q, k.contiguous(), v.contiguous(), seqlens.to(device),
            offs.to(torch.int32).to(device))


def decode_spec_inputs(spec: DecodeSpec, device="cpu"):
    lens = decode_lengths(spec.B, spec.min_len, spec.max_len, spec.seed, spec.fixed_len)
    return decode_inputs(spec.B, spec.H, spec.d, lens, spec.seed, device)


def paged_layout(seqlens, page_size, seed=0, spare_pages=0, max_len=None):
    """A block table for a paged cache: sequence b needs ceil(len_b / page_size)
    pages, and all pages (plus `spare_pages` never referenced) are handed out
    in a seeded random order.  The table has room for `max_len` keys per
    sequence (default: the longest).  Returns (block_table int32
    [B, max_blocks] on the host, unreferenced entries -1, and num_pages)."""
    lens = [int(x) for x in torch.as_tensor(seqlens).cpu()]
    need = [-(-n // page_size) for n in lens]
    num_pages = max(sum(need) + spare_pages, 1)
    perm = torch.randperm(num_pages, generator=_gen("cpu", seed + 104729)).to(torch.int32)
    cols = max(max(need), -(-int(max_len) // page_size) if max_len else 0, 1)
    bt = torch.full((len(lens), cols), -1, dtype=torch.int32)
    at = 0
    for b, n in enumerate(need):
        bt[b, :n] = perm[at:at + n]
        at += n
    return bt, num_pages


def to_pages(cache, seqlens, offsets, block_table, page_size, num_pages):
    """Copy a packed token-major cache [T, H, d] into a page pool
    [num_pages, page_size, H, d] laid out by `block_table` (slots no sequence
    uses stay zero).  Runs on the cache's device."""
    dev = cache.device
    T, H, d = cache.shape
    pool = torch.zeros((num_pages * page_size, H, d), dtype=cache.dtype, device=dev)
    lens = torch.as_tensor(seqlens).cpu().to(torch.int64)
    offs = torch.as_tensor(offsets).cpu().to(torch.int64)
    bt = torch.as_tensor(block_table).cpu().to(torch.int64)
    src, dst = [], []
    for b in range(len(lens)):
        n = int(lens[b])
        if n == 0:
            continue
        t = torch.arange(n)
        src.append(offs[b] + t)
        dst.append(bt[b, t // page_size] * page_size + t % page_size)
    if src:
        pool[torch.cat(dst).to(dev)] = cache[torch.cat(src).to(dev)]
    return pool.view(num_pages, page_size, H, d)


def varlen_inputs(lens_q, lens_k, H, d, seed=0, device="cpu", dtype="bf16"):
    """Packed token-major batch: q [sum Lq, H, d], k, v [sum Lk, H, d] N(0,1),
    and int32 cu_seqlens_q / cu_seqlens_k [B+1] (exclusive prefix sums with the
    total appended), all on `device`."""
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    lq = torch.as_tensor(lens_q, dtype=torch.int64).cpu()
    lk = torch.as_tensor(lens_k, dtype=torch.int64).cpu()
    cq = torch.zeros(len(lq) + 1, dtype=torch.int64)
    ck = torch.zeros(len(lk) + 1, dtype=torch.int64)
    cq[1:] = torch.cumsum(lq, 0)
    ck[1:] = torch.cumsum(lk, 0)
    g = _gen(device, seed + 7919)
    Tq, Tk = int(cq[-1]), int(ck[-1])
    q = _normal((max(Tq, 1), H, d), g, device, tdt)[:Tq].contiguous()
    k = _normal((max(Tk, 1), H, d), g, device, tdt)[:Tk].contiguous()
    v = _normal((max(Tk, 1), H, d), g, device, tdt)[:Tk].contiguous()
    return q, k, v, cq.to(torch.int32).to(device), ck.to(torch.int32).to(device)


def varlen_spec_inputs(spec: VarlenSpec, device="cpu"):
    """The spec's lengths (drawn first, on the host) and its packed inputs."""
    lens = decode_lengths(spec.B, spec.min_len, spec.max_len, spec.seed)
    return (lens,) + varlen_inputs(lens, lens, spec.H, spec.d, spec.seed, device)


def block_mask(kind, H, Nq, Nk, seed=0, window=2, density=0.5):
    """A uint8 block mask [H, ceil(Nq/64), ceil(Nk/64)] over 64 x 64 blocks:
    "ones", "zeros", "random" (each block admitted with `density`), or
    "local_global" (query block i admits key blocks i-window .. i+window
    after aligning the ends, plus key block 0 for every query block)."""
    nqb, nkb = -(-Nq // 64), -(-Nk // 64)
    if kind == "ones":
        return torch.ones((H, nqb, nkb), dtype=torch.uint8)
    if kind == "zeros":
        return torch.zeros((H, nqb, nkb), dtype=torch.uint8)
    if kind == "random":
        g = _gen("cpu", seed)
        return (torch.rand((H, nqb, nkb), generator=g) < density).to(torch.uint8)
    if kind == "local_global":
        i = torch.arange(nqb)[:, None] + (nkb - nqb)
        j = torch.arange(nkb)[None, :]
        m = ((j - i).abs() <= window) | (j == 0)
        return m.to(torch.uint8)[None].expand(H, nqb, nkb).contiguous()
    raise ValueError(kind)


def block_mask_pairs(mask, Nq, Nk, causal):
    """Visible (query, key) pairs of a block mask (summed over heads): the
    algorithmic work of a block-sparse pass is 4 * d * pairs FLOPs per batch."""
    M = torch.as_tensor(mask).to(torch.bool)
    H, nqb, nkb = M.shape
    rows = torch.arange(Nq)
    cols = torch.arange(Nk)
    total = 0
    for h in range(H):
        vis = M[h][rows[:, None] // 64, cols[None, :] // 64]
        if causal:
            vis = vis & (cols[None, :] <= rows[:, None] + (Nk - Nq))
        total += int(vis.sum())
    return total


def decode_kv_bytes(seqlens, H, d, elem_bytes=2) -> int:
    """Bytes of K plus V history the decode step must read."""
    T = int(torch.as_tensor(seqlens).to(torch.int64).sum())
    return 2 * T * H * d * elem_bytes


def to_f64(t: torch.Tensor):
    """Exact upcast of a (possibly bf16, possibly device) tensor to a float64 numpy array."""
    return t.detach().to("cpu").to(torch.float64).numpy()
