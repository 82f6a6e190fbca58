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
    o, lse = fa_decode_varlen_split(q, kcache, vcache, seqlens, offsets, max_seqlen, split_keys)
    o, lse = fa_decode_paged(q, kpages, vpages, block_table, seqlens, max_seqlen, scale)

Every tensor the caller passes (inputs, and outputs or workspaces given in
place of the ones the binding would allocate) is checked for dtype, shape,
contiguity and device before the library is called: a wrong-sized buffer is
refused here, never handed to a kernel.
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
FA_ERR_SCRATCH = -5

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
    "fa_decode_workspace_bytes": (_Z, [_I, _I, _I, _I]),
    "fa_decode_varlen": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _P, _Z, _P]),
    "fa_decode_split_workspace_bytes": (_Z, [_I, _I, _I, _I, _I]),
    "fa_decode_varlen_split": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _P, _Z,
                                    _P]),
    "fa_status_string": (ctypes.c_char_p, [_I]),
    "fa_decode_paged_split_keys": (_I, [_I, _I, _I, _I, _I]),
    "fa_decode_paged": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I, _P,
                             _Z, _P]),
    "fa_probe_read": (_I, [_P, _Z, _P, _P]),
    "fa_probe_issue": (_I, [_I, _I, _I, _I, _I, _P, _P]),
    "fa_decode_varlen_noalloc": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _P]),
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


def load_library(path):
    """Another build of the library (e.g. the race-check build
    libfa_paranoid.so), loaded beside the default one with the same
    signatures; use it through `using_library`."""
    import torch  # noqa: F401

    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


class using_library:
    """Context manager: the functions of this module call `lib` inside it."""

    def __init__(self, lib):
        self.lib = lib

    def __enter__(self):
        global _lib
        self.saved = load()
        _lib = self.lib
        return self.lib

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


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


def _dev(t, name, dtype, ndim, shape=None, device=None):
    """Check a tensor handed to the library and return its device address.

    shape: the exact shape required (None: any of `ndim` dims); device: the
    device every tensor of the call must share (None: any HIP device)."""
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a HIP device, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the call's other tensors on {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _extent(t, i, ndim):
    """t.shape[i] when t is a tensor of ndim dims, else -1 (so that _dev then
    reports what is wrong with t)."""
    import torch

    return t.shape[i] if isinstance(t, torch.Tensor) and t.dim() == ndim else -1


def _workspace(ws, need, device, zero):
    """A caller's workspace (uint8, >= need bytes, on `device`) or a new one;
    decode workspaces are zero-filled (their arrival counters start at 0)."""
    import torch

    if ws is None:
        alloc = torch.zeros if zero else torch.empty
        ws = alloc(max(need, 16), dtype=torch.uint8, device=device)
    _dev(ws, "workspace", torch.uint8, 1, device=device)
    if ws.numel() < need:
        raise ValueError(f"workspace has {ws.numel()} bytes, the call needs {need}")
    return ws


def _fwd(entry, dtype, q, k, v, scale, causal, out, lse, stream):
    import torch

    lib = load()
    pq = _dev(q, "q", dtype, 4)
    dev = q.device
    B, H, Nq, d = q.shape
    Nk = _extent(k, 2, 4)
    pk = _dev(k, "k", dtype, 4, (B, H, Nk, d), dev)
    pv = _dev(v, "v", dtype, 4, (B, H, Nk, d), dev)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=dev)
    po = _dev(out, "out", dtype, 4, q.shape, dev)
    pl = _dev(lse, "lse", torch.float32, 3, (B, H, Nq), dev)
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
    dev = q.device
    B, H, Nq, d = q.shape
    Nk = _extent(k, 2, 4)
    pk = _dev(k, "k", torch.bfloat16, 4, (B, H, Nk, d), dev)
    pv = _dev(v, "v", torch.bfloat16, 4, (B, H, Nk, d), dev)
    pm = _dev(block_mask, "block_mask", torch.uint8, 3, (H, -(-Nq // 64), -(-Nk // 64)), dev)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=dev)
    po = _dev(out, "out", torch.bfloat16, 4, q.shape, dev)
    pl = _dev(lse, "lse", torch.float32, 3, (B, H, Nq), dev)
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
    pq = _dev(q, "q", torch.bfloat16, 4)
    dev = q.device
    B, H, Nq, d = q.shape
    Nk = _extent(k, 2, 4)
    kshape = (B, H, Nk, d)
    ptrs = [pq] + [_dev(t, n, torch.bfloat16, 4, shp, dev)
                   for t, n, shp in ((k, "k", kshape), (v, "v", kshape), (o, "o", q.shape),
                                     (dout, "dout", q.shape))]
    pl = _dev(lse, "lse", torch.float32, 3, (B, H, Nq), dev)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty(q.shape, dtype=torch.float32, device=dev) if dq is None else dq
    dk = torch.empty(kshape, dtype=torch.float32, device=dev) if dk is None else dk
    dv = torch.empty(kshape, dtype=torch.float32, device=dev) if dv is None else dv
    gp = [_dev(t, n, torch.float32, 4, shp, dev)
          for t, n, shp in ((dq, "dq", q.shape), (dk, "dk", kshape), (dv, "dv", kshape))]
    workspace = _workspace(workspace, fa_bwd_workspace_bytes(B, H, Nq), dev, zero=False)
    pw = ctypes.c_void_p(workspace.data_ptr())
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
    dev = q.device
    Tq, H, d = q.shape
    Tk = _extent(k, 0, 3)
    pk = _dev(k, "k", torch.bfloat16, 3, (Tk, H, d), dev)
    pv = _dev(v, "v", torch.bfloat16, 3, (Tk, H, d), dev)
    pcq = _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32, 1, device=dev)
    B = cu_seqlens_q.shape[0] - 1
    pck = _dev(cu_seqlens_k, "cu_seqlens_k", torch.int32, 1, (B + 1,), dev)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((H, Tq), dtype=torch.float32, device=dev)
    po = _dev(out, "out", torch.bfloat16, 3, q.shape, dev)
    pl = _dev(lse, "lse", torch.float32, 2, (H, Tq), dev)
    with _on_device(q):
        st = lib.fa_fwd_varlen(pq, pk, pv, po, pl, pcq, pck, B, H, d, Tq, int(max_seqlen_q),
                               float(scale), 1 if causal else 0, _stream(q, stream))
    _check(st, "fa_fwd_varlen")
    return out, lse


def fa_decode_workspace_bytes(B, H, d, max_seqlen) -> int:
    return int(load().fa_decode_workspace_bytes(B, H, d, max_seqlen))


def fa_decode_split_workspace_bytes(B, H, d, max_seqlen, split_keys) -> int:
    return int(load().fa_decode_split_workspace_bytes(B, H, d, max_seqlen, split_keys))


def _decode_packed(split_keys, q, kcache, vcache, seqlens, offsets, max_seqlen, scale, out, lse,
                   workspace, stream):
    import torch

    lib = load()
    pq = _dev(q, "q", torch.bfloat16, 3)
    dev = q.device
    B, H, d = q.shape
    T = _extent(kcache, 0, 3)
    pk = _dev(kcache, "kcache", torch.bfloat16, 3, (T, H, d), dev)
    pv = _dev(vcache, "vcache", torch.bfloat16, 3, (T, H, d), dev)
    ps = _dev(seqlens, "seqlens", torch.int32, 1, (B,), dev)
    po_ = _dev(offsets, "offsets", torch.int32, 1, (B,), dev)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    po = _dev(out, "out", torch.bfloat16, 3, q.shape, dev)
    pl = _dev(lse, "lse", torch.float32, 2, (B, H), dev)
    if split_keys:
        need = fa_decode_split_workspace_bytes(B, H, d, int(max_seqlen), int(split_keys))
    else:
        need = fa_decode_workspace_bytes(B, H, d, int(max_seqlen))
    workspace = _workspace(workspace, need, dev, zero=True)
    pw = ctypes.c_void_p(workspace.data_ptr())
    with _on_device(q):
        if split_keys:
            entry = "fa_decode_varlen_split"
            st = lib.fa_decode_varlen_split(pq, pk, pv, ps, po_, po, pl, B, H, d, int(max_seqlen),
                                            float(scale), int(split_keys), pw, workspace.numel(),
                                            _stream(q, stream))
        else:
            entry = "fa_decode_varlen"
            st = lib.fa_decode_varlen(pq, pk, pv, ps, po_, po, pl, B, H, d, int(max_seqlen),
                                      float(scale), pw, workspace.numel(), _stream(q, stream))
    _check(st, entry)
    return out, lse


def fa_decode_varlen(q, kcache, vcache, seqlens, offsets, max_seqlen, scale=None, out=None,
                     lse=None, workspace=None, stream=None):
    """Decode over a packed cache: q [B,H,d], kcache/vcache [T,H,d] bf16,
    seqlens/offsets int32 [B] on the device; max_seqlen a host int >= every
    seqlens[b].  A caller-provided workspace is a uint8 tensor of at least
    fa_decode_workspace_bytes bytes whose first 64 KiB were zero-filled once
    (torch.zeros); the library leaves them zero.  Without one, a zero-filled
    workspace is allocated for the call.  Returns (O bf16 [B,H,d], LSE fp32
    [B,H])."""
    return _decode_packed(0, q, kcache, vcache, seqlens, offsets, max_seqlen, scale, out, lse,
                          workspace, stream)


def fa_decode_varlen_split(q, kcache, vcache, seqlens, offsets, max_seqlen, split_keys, scale=None,
                           out=None, lse=None, workspace=None, stream=None):
    """fa_decode_varlen with an explicit chunk size (a positive multiple of 64);
    the workspace is sized by fa_decode_split_workspace_bytes."""
    if int(split_keys) < 1:
        raise ValueError("split_keys must be positive (fa_decode_varlen picks its own)")
    return _decode_packed(int(split_keys), q, kcache, vcache, seqlens, offsets, max_seqlen, scale,
                          out, lse, workspace, stream)


def fa_decode_varlen_noalloc(q, kcache, vcache, seqlens, offsets, max_seqlen, scale=None, out=None,
                             lse=None, stream=None):
    """fa_decode_varlen without a workspace: the library's fixed per-device
    scratch holds the chunk states (include/fa.h states the size limit and
    that calls overlapping on one device race).  The C call allocates
    nothing; pass `out` and `lse` to keep this wrapper from allocating them."""
    import torch

    lib = load()
    pq = _dev(q, "q", torch.bfloat16, 3)
    dev = q.device
    B, H, d = q.shape
    T = _extent(kcache, 0, 3)
    pk = _dev(kcache, "kcache", torch.bfloat16, 3, (T, H, d), dev)
    pv = _dev(vcache, "vcache", torch.bfloat16, 3, (T, H, d), dev)
    ps = _dev(seqlens, "seqlens", torch.int32, 1, (B,), dev)
    po_ = _dev(offsets, "offsets", torch.int32, 1, (B,), dev)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    po = _dev(out, "out", torch.bfloat16, 3, q.shape, dev)
    pl = _dev(lse, "lse", torch.float32, 2, (B, H), dev)
    with _on_device(q):
        st = lib.fa_decode_varlen_noalloc(pq, pk, pv, ps, po_, po, pl, B, H, d, int(max_seqlen),
                                          float(scale), _stream(q, stream))
    _check(st, "fa_decode_varlen_noalloc")
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
    dev = q.device
    B, H, d = q.shape
    num_pages, page_size = _extent(kpages, 0, 4), _extent(kpages, 1, 4)
    pk = _dev(kpages, "kpages", torch.bfloat16, 4, (num_pages, page_size, H, d), dev)
    pv = _dev(vpages, "vpages", torch.bfloat16, 4, (num_pages, page_size, H, d), dev)
    max_blocks = _extent(block_table, 1, 2)
    pb = _dev(block_table, "block_table", torch.int32, 2, (B, max_blocks), dev)
    ps = _dev(seqlens, "seqlens", torch.int32, 1, (B,), dev)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    po = _dev(out, "out", torch.bfloat16, 3, q.shape, dev)
    pl = _dev(lse, "lse", torch.float32, 2, (B, H), dev)
    sk = int(split_keys) or fa_decode_paged_split_keys(B, H, d, int(max_seqlen), int(page_size))
    need = fa_decode_split_workspace_bytes(B, H, d, int(max_seqlen), sk) if sk > 0 else 16
    workspace = _workspace(workspace, need, dev, zero=True)
    pw = ctypes.c_void_p(workspace.data_ptr())
    with _on_device(q):
        st = lib.fa_decode_paged(pq, pk, pv, pb, ps, po, pl, B, H, d, int(page_size), int(num_pages),
                                 int(block_table.shape[1]), int(max_seqlen), float(scale),
                                 int(split_keys), pw, workspace.numel(), _stream(q, stream))
    _check(st, "fa_decode_paged")
    return out, lse


PROBE_ROLES = {"none": 0, "products": 1, "fma": 2, "exp": 3, "lds16": 4, "lds_tr8": 5,
               "product_softmax": 6, "product_8fma": 7}


def fa_probe_issue(role_a, role_b, n_a, n_b, grid=None, device=None, stream=None):
    """Measurement aid (include/fa_probe.h): waves 0-3 of each 8-wave
    workgroup run `role_a` n_a times, waves 4-7 `role_b` n_b times (roles by
    name, PROBE_ROLES).  Returns a host int64 tensor [grid, 8, 2]: per wave,
    shader-clock cycles and the HW_ID register.  `grid` defaults to the
    device's CU count (one workgroup per CU)."""
    import torch

    dev = torch.device("cuda" if device is None else device)
    if grid is None:
        grid = torch.cuda.get_device_properties(dev).multi_processor_count
    out = torch.zeros(int(grid), 8, 2, dtype=torch.int64, device=dev)
    with _on_device(out):
        st = load().fa_probe_issue(PROBE_ROLES[role_a], PROBE_ROLES[role_b], int(n_a), int(n_b), int(grid),
                                   ctypes.c_void_p(out.data_ptr()), _stream(out, stream))
    _check(st, "fa_probe_issue")
    return out.cpu()


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
