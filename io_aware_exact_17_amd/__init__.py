"""Python binding of libfa.so, the MI355X exact-attention forward library.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI (include/fa.h).  torch supplies device memory and
the current stream.  The functions carry the C entry points' names.  There is
no fallback: if the shared library is missing, or a call is rejected, an
exception is raised.

    o, lse = fa_fwd(q, k, v, scale, causal)            # bf16 [B,H,N,d]
    o, lse = fa_fwd_f32(q, k, v, scale, causal)        # fp32 [B,H,N,d]
    o, lse = fa_fwd_varlen(q, k, v, cu_q, cu_k, max_q, scale, causal)  # packed [T,H,d]
    dq, dk, dv = fa_bwd(q, k, v, o, dout, lse, scale, causal)          # fp32 gradients
    o, lse = fa_fwd_block_sparse(q, k, v, block_mask, scale, causal)   # 64x64 block mask
    o, lse = fa_decode_varlen(q, kcache, vcache, seqlens, offsets, max_seqlen, scale)
    o, lse = fa_decode_paged(q, kpages, vpages, block_table, seqlens, max_seqlen, scale)
"""
from __future__ import annotations

import ctypes
import math
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

FA_OK = 0
FA_ERR_INVALID_ARG = -1
FA_ERR_UNSUPPORTED = -2
FA_ERR_WORKSPACE = -3
FA_ERR_HIP = -4

# Every symbol the C ABI exports, with (restype, argtypes).
_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_Z = ctypes.c_size_t
SIGNATURES = {
    "fa_fwd": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P]),
    "fa_fwd_f32": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P]),
    "fa_fwd_block_sparse": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P]),
    "fa_bwd_workspace_bytes": (_Z, [_I, _I, _I]),
    "fa_bwd": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P, _Z, _P]),
    "fa_fwd_varlen": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P]),
    "fa_decode_split_keys": (_I, [_I, _I, _I, _I]),
    "fa_decode_workspace_bytes": (_Z, [_I, _I, _I, _I, _I]),
    "fa_decode_varlen": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _P, _Z, _P]),
    "fa_status_string": (ctypes.c_char_p, [_I]),
    "fa_decode_paged_split_keys": (_I, [_I, _I, _I, _I, _I]),
    "fa_decode_paged": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I, _P,
                             _Z, _P]),
    "fa_probe_read": (_I, [_P, _Z, _P, _P]),
}

_lib = None


class FAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {fa_status_string(status)}")


def load():
    """Load libfa.so (after torch, so both share torch's HIP runtime)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run io_aware_exact_17_amd/build.py")
        import torch  # noqa: F401  (maps torch's libamdhip64 first)

        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def fa_status_string(status: int) -> str:
    return load().fa_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != FA_OK:
        raise FAError(status, where)


def _on_device(t):
    """Make t's device current for the call: kernels launched on the default
    (null) stream go to the current device."""
    import torch

    return torch.cuda.device(t.device)


def _stream(t, stream):
    import torch

    s = stream if stream is not None else torch.cuda.current_stream(t.device)
    return ctypes.c_void_p(s.cuda_stream)


def _dev(t, name, dtype, ndim):
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a HIP device, got {t.device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _fwd(entry, dtype, q, k, v, scale, causal, out, lse, stream):
    import torch

    lib = load()
    pq, pk, pv = _dev(q, "q", dtype, 4), _dev(k, "k", dtype, 4), _dev(v, "v", dtype, 4)
    B, H, Nq, d = q.shape
    if k.shape[:2] != (B, H) or k.shape[3] != d or v.shape != k.shape:
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on one device")
    Nk = k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    po = _dev(out, "out", dtype, 4)
    pl = _dev(lse, "lse", torch.float32, 3)
    if tuple(out.shape) != tuple(q.shape) or tuple(lse.shape) != (B, H, Nq):
        raise ValueError("out / lse shape mismatch")
    with _on_device(q):
        st = getattr(lib, entry)(pq, pk, pv, po, pl, B, H, Nq, Nk, d, float(scale), int(bool(causal)),
                                 _stream(q, stream))
    _check(st, entry)
    return out, lse


def fa_fwd(q, k, v, scale=None, causal=False, out=None, lse=None, stream=None):
    """bf16 forward pass; q [B,H,Nq,d], k/v [B,H,Nk,d] -> (O bf16, LSE fp32 [B,H,Nq])."""
    import torch

    return _fwd("fa_fwd", torch.bfloat16, q, k, v, scale, causal, out, lse, stream)


def fa_fwd_f32(q, k, v, scale=None, causal=False, out=None, lse=None, stream=None):
    """fp32 forward pass with the same contract as fa_fwd."""
    import torch

    return _fwd("fa_fwd_f32", torch.float32, q, k, v, scale, causal, out, lse, stream)


def fa_decode_split_keys(B, H, d, max_seqlen) -> int:
    return int(load().fa_decode_split_keys(B, H, d, max_seqlen))


def fa_fwd_block_sparse(q, k, v, block_mask, scale=None, causal=False, out=None, lse=None,
                        stream=None):
    """Block-sparse forward: q [B,H,Nq,128], k/v [B,H,Nk,128] bf16; block_mask
    uint8 [H, ceil(Nq/64), ceil(Nk/64)] on the device (nonzero = admitted).
    Returns (O bf16 [B,H,Nq,128], LSE fp32 [B,H,Nq])."""
    import torch

    lib = load()
    pq = _dev(q, "q", torch.bfloat16, 4)
    pk = _dev(k, "k", torch.bfloat16, 4)
    pv = _dev(v, "v", torch.bfloat16, 4)
    pm = _dev(block_mask, "block_mask", torch.uint8, 3)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if k.shape != (B, H, Nk, d) or v.shape != k.shape:
        raise ValueError("q, k, v shapes disagree")
    if tuple(block_mask.shape) != (H, -(-Nq // 64), -(-Nk // 64)):
        raise ValueError("block_mask must be [H, ceil(Nq/64), ceil(Nk/64)]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    po = _dev(out, "out", torch.bfloat16, 4)
    pl = _dev(lse, "lse", torch.float32, 3)
    with _on_device(q):
        st = lib.fa_fwd_block_sparse(pq, pk, pv, po, pl, pm, B, H, Nq, Nk, d, float(scale),
                                     1 if causal else 0, _stream(q, stream))
    _check(st, "fa_fwd_block_sparse")
    return out, lse


def fa_bwd_workspace_bytes(B, H, Nq) -> int:
    return int(load().fa_bwd_workspace_bytes(B, H, Nq))


def fa_bwd(q, k, v, o, dout, lse, scale=None, causal=False, dq=None, dk=None, dv=None,
           workspace=None, stream=None):
    """Backward of fa_fwd: q, k, v, o, dout bf16 [B,H,N,d] and lse fp32 [B,H,Nq]
    (o and lse from the forward).  Returns (dq, dk, dv) fp32."""
    import torch

    lib = load()
    ptrs = [_dev(t, n, torch.bfloat16, 4) for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"),
                                                       (dout, "dout"))]
    pl = _dev(lse, "lse", torch.float32, 3)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if k.shape != (B, H, Nk, d) or v.shape != k.shape or o.shape != q.shape or dout.shape != q.shape:
        raise ValueError("q, k, v, o, dout shapes disagree")
    if tuple(lse.shape) != (B, H, Nq):
        raise ValueError("lse must be [B, H, Nq]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty(q.shape, dtype=torch.float32, device=q.device) if dq is None else dq
    dk = torch.empty(k.shape, dtype=torch.float32, device=q.device) if dk is None else dk
    dv = torch.empty(v.shape, dtype=torch.float32, device=q.device) if dv is None else dv
    gp = [_dev(t, n, torch.float32, 4) for t, n in ((dq, "dq"), (dk, "dk"), (dv, "dv"))]
    if workspace is None:
        workspace = torch.empty(max(fa_bwd_workspace_bytes(B, H, Nq), 16), dtype=torch.uint8,
                                device=q.device)
    pw = _dev(workspace, "workspace", torch.uint8, 1)
    with _on_device(q):
        st = lib.fa_bwd(*ptrs, pl, *gp, B, H, Nq, Nk, d, float(scale), 1 if causal else 0, pw,
                        workspace.numel(), _stream(q, stream))
    _check(st, "fa_bwd")
    return dq, dk, dv


def fa_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, scale=None, causal=False,
                  out=None, lse=None, stream=None):
    """Packed variable-length forward: q [total_q,H,d], k/v [total_k,H,d] bf16,
    cu_seqlens_q/k int32 [B+1] on the device, max_seqlen_q a host int >= every
    query count.  Returns (O bf16 [total_q,H,d], LSE fp32 [H,total_q])."""
    import torch

    lib = load()
    pq = _dev(q, "q", torch.bfloat16, 3)
    pk = _dev(k, "k", torch.bfloat16, 3)
    pv = _dev(v, "v", torch.bfloat16, 3)
    pcq = _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32, 1)
    pck = _dev(cu_seqlens_k, "cu_seqlens_k", torch.int32, 1)
    Tq, H, d = q.shape
    if k.shape[1:] != (H, d) or v.shape != k.shape:
        raise ValueError("q, k, v shapes disagree")
    if cu_seqlens_k.shape != cu_seqlens_q.shape:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both have B+1 entries")
    B = cu_seqlens_q.shape[0] - 1
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((H, Tq), dtype=torch.float32, device=q.device)
    po = _dev(out, "out", torch.bfloat16, 3)
    pl = _dev(lse, "lse", torch.float32, 2)
    with _on_device(q):
        st = lib.fa_fwd_varlen(pq, pk, pv, po, pl, pcq, pck, B, H, d, Tq, int(max_seqlen_q),
                               float(scale), 1 if causal else 0, _stream(q, stream))
    _check(st, "fa_fwd_varlen")
    return out, lse


def fa_decode_workspace_bytes(B, H, d, max_seqlen, split_keys=0) -> int:
    return int(load().fa_decode_workspace_bytes(B, H, d, max_seqlen, split_keys))


def fa_decode_varlen(q, kcache, vcache, seqlens, offsets, max_seqlen, scale=None, split_keys=0,
                     out=None, lse=None, workspace=None, stream=None):
    """Decode over a packed cache: q [B,H,d], kcache/vcache [T,H,d] bf16,
    seqlens/offsets int32 [B] on the device; max_seqlen a host int >= every
    seqlens[b].  A caller-provided workspace is a uint8 tensor of at least
    fa_decode_workspace_bytes bytes.  Returns (O bf16 [B,H,d], LSE fp32 [B,H])."""
    import torch

    lib = load()
    pq = _dev(q, "q", torch.bfloat16, 3)
    pk = _dev(kcache, "kcache", torch.bfloat16, 3)
    pv = _dev(vcache, "vcache", torch.bfloat16, 3)
    ps = _dev(seqlens, "seqlens", torch.int32, 1)
    po_ = _dev(offsets, "offsets", torch.int32, 1)
    B, H, d = q.shape
    if kcache.shape[1:] != (H, d) or vcache.shape != kcache.shape:
        raise ValueError("cache shape mismatch")
    if seqlens.shape[0] != B or offsets.shape[0] != B:
        raise ValueError("seqlens / offsets must have B entries")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    po = _dev(out, "out", torch.bfloat16, 3)
    pl = _dev(lse, "lse", torch.float32, 2)
    need = fa_decode_workspace_bytes(B, H, d, int(max_seqlen), int(split_keys))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    pw = _dev(workspace, "workspace", torch.uint8, 1)
    with _on_device(q):
        st = lib.fa_decode_varlen(pq, pk, pv, ps, po_, po, pl, B, H, d, int(max_seqlen), float(scale),
                                  int(split_keys), pw, workspace.numel(), _stream(q, stream))
    _check(st, "fa_decode_varlen")
    return out, lse


def fa_decode_paged_split_keys(B, H, d, max_seqlen, page_size) -> int:
    return int(load().fa_decode_paged_split_keys(B, H, d, max_seqlen, page_size))


def fa_decode_paged(q, kpages, vpages, block_table, seqlens, max_seqlen, scale=None, split_keys=0,
                    out=None, lse=None, workspace=None, stream=None):
    """Decode over a paged cache: q [B,H,d], kpages/vpages [num_pages,page_size,H,d]
    bf16, block_table int32 [B,max_blocks] and seqlens int32 [B] on the device;
    max_seqlen a host int >= every seqlens[b].  Returns (O bf16 [B,H,d], LSE
    fp32 [B,H])."""
    import torch

    lib = load()
    pq = _dev(q, "q", torch.bfloat16, 3)
    pk = _dev(kpages, "kpages", torch.bfloat16, 4)
    pv = _dev(vpages, "vpages", torch.bfloat16, 4)
    pb = _dev(block_table, "block_table", torch.int32, 2)
    ps = _dev(seqlens, "seqlens", torch.int32, 1)
    B, H, d = q.shape
    num_pages, page_size = kpages.shape[0], kpages.shape[1]
    if kpages.shape[2:] != (H, d) or vpages.shape != kpages.shape:
        raise ValueError("page pool shape mismatch")
    if block_table.shape[0] != B or seqlens.shape[0] != B:
        raise ValueError("block_table / seqlens must have B rows")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    po = _dev(out, "out", torch.bfloat16, 3)
    pl = _dev(lse, "lse", torch.float32, 2)
    sk = int(split_keys) or fa_decode_paged_split_keys(B, H, d, int(max_seqlen), int(page_size))
    need = fa_decode_workspace_bytes(B, H, d, int(max_seqlen), sk)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    pw = _dev(workspace, "workspace", torch.uint8, 1)
    with _on_device(q):
        st = lib.fa_decode_paged(pq, pk, pv, pb, ps, po, pl, B, H, d, int(page_size), int(num_pages),
                                 int(block_table.shape[1]), int(max_seqlen), float(scale),
                                 int(split_keys), pw, workspace.numel(), _stream(q, stream))
    _check(st, "fa_decode_paged")
    return out, lse


def fa_probe_read(buf, nbytes=None, sink=None, stream=None):
    """Measurement aid (include/fa_probe.h): a plain streaming read of the first
    `nbytes` bytes (default: all) of the contiguous device tensor `buf`."""
    import torch

    if not isinstance(buf, torch.Tensor) or buf.device.type != "cuda" or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    total = buf.numel() * buf.element_size()
    n = total if nbytes is None else int(nbytes)
    if n > total:
        raise ValueError("nbytes exceeds the buffer")
    if sink is None:
        sink = torch.empty(1, dtype=torch.int32, device=buf.device)
    with _on_device(buf):
        st = load().fa_probe_read(ctypes.c_void_p(buf.data_ptr()), n, ctypes.c_void_p(sink.data_ptr()),
                                  _stream(buf, stream))
    _check(st, "fa_probe_read")
