"""The C ABI without a GPU: the library loads, exports every symbol the header
declares, and rejects every invalid call before touching the HIP runtime."""
import ctypes
import os
import re
import subprocess

import pytest

import io_aware_exact_17_amd as fa
from conftest import ROOT, gpu_available

HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]
OK, INVALID, UNSUPPORTED, WORKSPACE, HIPERR, SCRATCH = 0, -1, -2, -3, -4, -5

# Fake, suitably aligned device addresses: never dereferenced, because every
# call below is rejected by the host-side checks (or, without a GPU, by the
# runtime) before anything runs.
A = 0x10000
A2 = 0x20000


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_library_exists_and_loads():
    assert os.path.exists(fa.LIB_PATH), "run io_aware_exact_17_amd/build.py first"
    fa.load()


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(fa.SIGNATURES), "binding and header disagree"
    out = subprocess.run(["nm", "-D", "--defined-only", fa.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (fa_[a-z0-9_]+)$", out, flags=re.M))
    missing = set(names) - exported
    assert not missing, f"not exported: {missing}"
    lib = fa.load()
    for n in names:
        assert getattr(lib, n) is not None


def test_status_strings():
    for s in (OK, INVALID, UNSUPPORTED, WORKSPACE, HIPERR, SCRATCH):
        assert fa.fa_status_string(s).startswith("FA_")
    assert "unknown" in fa.fa_status_string(12345)


def fwd_call(entry="fa_fwd", q=A, k=A, v=A, o=A2, lse=A2, B=1, H=1, Nq=8, Nk=8, d=64,
             scale=0.125, causal=0):
    lib = fa.load()
    return getattr(lib, entry)(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, None)


@pytest.mark.parametrize("entry", ["fa_fwd", "fa_fwd_f32"])
def test_fwd_rejects_invalid_arguments(entry):
    assert fwd_call(entry, q=None) == INVALID
    assert fwd_call(entry, k=None) == INVALID
    assert fwd_call(entry, v=None) == INVALID
    assert fwd_call(entry, o=None) == INVALID
    assert fwd_call(entry, lse=None) == INVALID
    assert fwd_call(entry, q=A + 8) == INVALID      # not 16-byte aligned
    assert fwd_call(entry, lse=A2 + 2) == INVALID
    for bad in ({"B": 0}, {"H": 0}, {"Nq": 0}, {"Nk": 0}, {"B": -3}, {"Nq": -1}):
        assert fwd_call(entry, **bad) == INVALID
    assert fwd_call(entry, B=1 << 16, H=1 << 16) == INVALID  # B*H overflows int
    assert fwd_call(entry, scale=float("nan")) == INVALID
    assert fwd_call(entry, scale=float("inf")) == INVALID
    for d in (0, 32, 63, 96, 256):
        assert fwd_call(entry, d=d) == UNSUPPORTED
    # grid of more than 2^31 - 1 workgroups
    assert fwd_call(entry, B=65535, H=65535 // 2, Nq=1 << 20) == INVALID
    # sequences longer than 2^30 (kernel index arithmetic is 32-bit)
    assert fwd_call(entry, Nq=(1 << 30) + 1) == INVALID
    assert fwd_call(entry, Nk=(1 << 30) + 1) == INVALID
    assert fwd_call(entry, Nq=2**31 - 1, Nk=2**31 - 1) == INVALID


def varlen_call(q=A, k=A, v=A, o=A2, lse=A2, cq=A2, ck=A2, B=2, H=4, d=64, total_q=100,
                max_seqlen_q=60, scale=0.125, causal=1):
    lib = fa.load()
    return lib.fa_fwd_varlen(q, k, v, o, lse, cq, ck, B, H, d, total_q, max_seqlen_q, scale,
                             causal, None)


def test_varlen_rejects_bad_arguments():
    for kw in ("q", "k", "v", "o", "lse", "cq", "ck"):
        assert varlen_call(**{kw: None}) == INVALID
    assert varlen_call(q=A + 8) == INVALID
    assert varlen_call(cq=A2 + 2) == INVALID
    for bad in ({"B": 0}, {"B": 65536}, {"H": 0}, {"total_q": 0}, {"max_seqlen_q": 0},
                {"max_seqlen_q": 101}, {"scale": float("nan")}):
        assert varlen_call(**bad) == INVALID
    for d in (0, 32, 96, 256):
        assert varlen_call(d=d) == UNSUPPORTED
    # d = 64 counts one workgroup per (sequence, query tile, head) over the
    # whole batch: 600 tiles x 65535 sequences x 64 heads > 2^31 - 1.
    assert varlen_call(B=65535, H=64, total_q=600 * 256, max_seqlen_q=600 * 256) == INVALID


def dec_call(q=A, kc=A, vc=A, sl=A2, off=A2, o=A2, lse=A2, B=2, H=4, d=128, max_seqlen=100,
             scale=0.1, ws=A, ws_bytes=1 << 30):
    """fa_decode_varlen with exactly the parameters of the boundary's signature."""
    lib = fa.load()
    return lib.fa_decode_varlen(q, kc, vc, sl, off, o, lse, B, H, d, max_seqlen, scale, ws,
                                ws_bytes, None)


def dec_split_call(split_keys=64, **kw):
    lib = fa.load()
    a = dict(q=A, kc=A, vc=A, sl=A2, off=A2, o=A2, lse=A2, B=2, H=4, d=128, max_seqlen=100,
             scale=0.1, ws=A, ws_bytes=1 << 30)
    a.update(kw)
    return lib.fa_decode_varlen_split(a["q"], a["kc"], a["vc"], a["sl"], a["off"], a["o"], a["lse"],
                                      a["B"], a["H"], a["d"], a["max_seqlen"], a["scale"], split_keys,
                                      a["ws"], a["ws_bytes"], None)


def test_decode_signature_is_the_boundary():
    """fa_decode_varlen / fa_decode_workspace_bytes take exactly the boundary's
    parameters (q, kcache, vcache, seqlens, offsets, o, lse, B, H, d,
    max_seqlen, scale, workspace, workspace_bytes, stream)."""
    header = open(os.path.join(ROOT, "include", "fa.h")).read()
    flat = re.sub(r"\s+", " ", header)
    assert ("int fa_decode_varlen(const void* q, const void* kcache, const void* vcache, "
            "const int32_t* seqlens, const int32_t* offsets, void* o, float* lse, int B, int H, "
            "int d, int max_seqlen, float scale, void* workspace, size_t workspace_bytes, "
            "hipStream_t stream);") in flat
    assert "size_t fa_decode_workspace_bytes(int B, int H, int d, int max_seqlen);" in flat
    assert len(fa.SIGNATURES["fa_decode_varlen"][1]) == 15
    assert len(fa.SIGNATURES["fa_decode_workspace_bytes"][1]) == 4


def test_decode_rejects_invalid_arguments():
    for kw in ("q", "kc", "vc", "sl", "off", "o", "lse"):
        assert dec_call(**{kw: None}) == INVALID
        assert dec_split_call(**{kw: None}) == INVALID
    assert dec_call(kc=A + 4) == INVALID
    assert dec_call(sl=A2 + 1) == INVALID
    for bad in ({"B": 0}, {"H": 0}, {"max_seqlen": 0}, {"B": 70000}, {"H": 70000}):
        assert dec_call(**bad) == INVALID
        assert dec_split_call(**bad) == INVALID
    assert dec_call(scale=float("nan")) == INVALID
    assert dec_call(max_seqlen=(1 << 30) + 1) == INVALID
    assert fa.fa_decode_split_keys(1, 1, 128, (1 << 30) + 1) == 0
    assert fa.fa_decode_workspace_bytes(65536, 1, 128, 100) == 0
    assert fa.fa_decode_split_keys(2**31 - 1, 2**31 - 1, 128, 1 << 20) == 0
    assert dec_split_call(split_keys=0) == INVALID     # the split entry needs an explicit size
    assert dec_split_call(split_keys=-64) == INVALID
    assert dec_split_call(split_keys=100) == INVALID   # not a multiple of 64
    assert dec_split_call(split_keys=64, max_seqlen=64 * 4097, ws_bytes=1 << 40) == INVALID  # > 4096 chunks
    assert dec_call(d=96) == UNSUPPORTED
    assert dec_split_call(d=96) == UNSUPPORTED
    assert dec_call(ws=None) == WORKSPACE
    assert dec_call(ws=A + 8) == WORKSPACE
    need = fa.fa_decode_workspace_bytes(2, 4, 128, 100)
    assert dec_call(ws_bytes=need - 1) == WORKSPACE
    need64 = fa.fa_decode_split_workspace_bytes(2, 4, 128, 100, 64)
    assert dec_split_call(ws_bytes=need64 - 1) == WORKSPACE


COUNTER_BYTES = 65536  # arrival counters at the start of every decode workspace


def test_workspace_and_split_plan():
    # with fewer (sequence, head) pairs than CUs, chunks as long as still give
    # every CU a workgroup: 32 heads x 8192 keys -> 8 chunks of 1024
    assert fa.fa_decode_split_keys(1, 32, 128, 8192) == 1024
    assert fa.fa_decode_workspace_bytes(1, 32, 128, 8192) == COUNTER_BYTES + 1 * 32 * 8 * 130 * 4
    assert fa.fa_decode_split_keys(4, 32, 128, 8192) == 4096   # 128 pairs x 2 chunks
    assert fa.fa_decode_split_keys(1, 1, 128, 65536) == 256    # one pair: 256 chunks
    assert fa.fa_decode_split_keys(1, 32, 128, 100) == 256
    assert fa.fa_decode_split_workspace_bytes(1, 32, 128, 8192, 0) == fa.fa_decode_workspace_bytes(
        1, 32, 128, 8192)
    # a large batch gets longer chunks, keeping the grid <= 16384 workgroups
    sk = fa.fa_decode_split_keys(64, 32, 128, 16384)
    assert sk == 2048 and 64 * 32 * -(-16384 // sk) <= 16384
    assert fa.fa_decode_split_workspace_bytes(3, 5, 64, 1000, 128) == COUNTER_BYTES + 3 * 5 * 8 * 66 * 4
    # the automatic plan keeps at most 256 chunks per sequence
    assert -(-(1 << 24) // fa.fa_decode_split_keys(1, 1, 128, 1 << 24)) <= 256
    assert fa.fa_decode_split_workspace_bytes(0, 5, 64, 1000, 128) == 0
    assert fa.fa_decode_split_workspace_bytes(3, 5, 96, 1000, 128) == 0
    assert fa.fa_decode_split_workspace_bytes(3, 5, 64, 1000, 100) == 0      # not a multiple of 64
    assert fa.fa_decode_split_workspace_bytes(1, 1, 64, 64 * 4097, 64) == 0  # > 4096 chunks
    assert fa.fa_decode_workspace_bytes(0, 5, 64, 1000) == 0


def noalloc_call(q=A, kc=A, vc=A, sl=A2, off=A2, o=A2, lse=A2, B=2, H=4, d=128, max_seqlen=100,
                 scale=0.1):
    lib = fa.load()
    return lib.fa_decode_varlen_noalloc(q, kc, vc, sl, off, o, lse, B, H, d, max_seqlen, scale, None)


def test_noalloc_decode_rejects_invalid_arguments():
    for kw in ("q", "kc", "vc", "sl", "off", "o", "lse"):
        assert noalloc_call(**{kw: None}) == INVALID
    assert noalloc_call(kc=A + 4) == INVALID
    for bad in ({"B": 0}, {"H": 0}, {"max_seqlen": 0}, {"B": 70000}, {"scale": float("inf")}):
        assert noalloc_call(**bad) == INVALID
    assert noalloc_call(d=96) == UNSUPPORTED
    # the fixed scratch is 16 MiB of chunk states: 64 sequences x 32 heads of
    # 16384 keys fit (8 chunks of 2048 keys), 2048 x 128 heads do not
    assert 64 * 32 * 8 * 130 * 4 <= 16 << 20
    assert noalloc_call(B=2048, H=128, max_seqlen=100000) == SCRATCH
    assert noalloc_call(B=1024, H=64, d=64, max_seqlen=1 << 20) == SCRATCH


@pytest.mark.skipif(gpu_available(), reason="uses fake device pointers; only safe with no GPU")
def test_valid_call_without_gpu_reports_hip_error():
    # All checks pass, so the launch reaches the HIP runtime, which has no
    # device here: the status must be FA_ERR_HIP, not a crash.
    assert fwd_call() == HIPERR
    assert fwd_call("fa_fwd_f32", d=128, causal=1) == HIPERR
    assert dec_call() == HIPERR
    assert dec_split_call(split_keys=128) == HIPERR
    assert noalloc_call(B=64, H=32, max_seqlen=16384) == HIPERR


def test_binding_validates_tensors():
    import torch

    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.fa_fwd(q, q, q)  # host tensors are refused
    with pytest.raises(TypeError):
        fa.fa_fwd(None, q, q)


def test_probe_rejects_invalid_arguments():
    lib = fa.load()
    assert lib.fa_probe_read(None, 1024, A2, None) == INVALID
    assert lib.fa_probe_read(A, 1024, None, None) == INVALID
    assert lib.fa_probe_read(A, 0, A2, None) == INVALID
    assert lib.fa_probe_read(A, 1000, A2, None) == INVALID  # not a multiple of 16
    assert lib.fa_probe_read(A + 8, 1024, A2, None) == INVALID


def test_probe_issue_rejects_invalid_arguments():
    lib = fa.load()
    P = fa.PROBE_ROLES
    ok = (P["products"], P["fma"], 64, 64, 4, A, None)
    for i, badv in ((0, -1), (0, 8), (1, 8), (2, 12), (3, -8), (2, 1 << 21), (2, 0), (4, 0), (4, 65536),
                    (5, None), (5, A + 4)):
        args = list(ok)
        args[i] = badv
        assert lib.fa_probe_issue(*args) == INVALID, (i, badv)
    # a role of none takes no operations
    assert lib.fa_probe_issue(P["none"], P["none"], 0, 0, 0, A, None) == INVALID  # grid 0


def paged_call(q=A, kp=A, vp=A, bt=A2, sl=A2, o=A2, lse=A2, B=2, H=4, d=128, page=16,
               num_pages=100, max_blocks=8, max_seqlen=100, scale=0.1, split_keys=0,
               ws=A, ws_bytes=1 << 30):
    lib = fa.load()
    return lib.fa_decode_paged(q, kp, vp, bt, sl, o, lse, B, H, d, page, num_pages, max_blocks,
                               max_seqlen, scale, split_keys, ws, ws_bytes, None)


def test_decode_paged_rejects_invalid_arguments():
    assert paged_call(bt=None) == INVALID
    assert paged_call(kp=A + 4) == INVALID
    assert paged_call(bt=A2 + 2) == INVALID
    for page in (0, 3, 48, 1 << 17):
        assert paged_call(page=page) == INVALID, page
    assert paged_call(num_pages=0) == INVALID
    assert paged_call(max_blocks=6) == INVALID           # 6 * 16 < 100 keys
    assert paged_call(page=1, max_blocks=100, split_keys=2048) == INVALID  # 2049 pages per chunk
    assert paged_call(split_keys=96) == INVALID
    assert paged_call(d=96) == UNSUPPORTED
    assert paged_call(ws=None) == WORKSPACE
    need = fa.fa_decode_split_workspace_bytes(2, 4, 128, 100,
                                              fa.fa_decode_paged_split_keys(2, 4, 128, 100, 16))
    assert paged_call(ws_bytes=need - 1) == WORKSPACE


def test_decode_paged_split_plan():
    # pages of 16 keep the packed plan; single-key pages shrink the chunk to fit 1024 pages
    assert fa.fa_decode_paged_split_keys(1, 32, 128, 8192, 16) == fa.fa_decode_split_keys(1, 32, 128, 8192)
    sk = fa.fa_decode_paged_split_keys(1, 1, 128, 1 << 20, 1)
    assert sk % 64 == 0 and sk + 1 <= 1024
    assert fa.fa_decode_paged_split_keys(1, 1, 128, 100, 3) == 0
    # no chunk size meets both the 1024-page and the 4096-chunk limits
    assert fa.fa_decode_paged_split_keys(1, 1, 128, 1 << 23, 1) == 0
    assert paged_call(page=1, max_blocks=1 << 23, max_seqlen=1 << 23) == INVALID


@pytest.mark.skipif(gpu_available(), reason="uses fake device pointers; only safe with no GPU")
@pytest.mark.parametrize("B,H,max_seqlen,page", [
    (1, 32, 8192, 16), (64, 32, 16384, 16), (1, 1, 200000, 1), (1, 8, 1 << 22, 2),
    (3, 5, 1000, 1024), (2, 2, (1 << 23) - 1, 4), (1, 1, 1, 1), (1, 1, 65536 * 8, 65536)])
def test_every_paged_plan_is_accepted(B, H, max_seqlen, page):
    """Whatever nonzero chunk size fa_decode_paged_split_keys reports, fa_decode_paged
    accepts: its checks pass and the call reaches the (absent) HIP runtime."""
    sk = fa.fa_decode_paged_split_keys(B, H, 128, max_seqlen, page)
    if sk == 0:
        return
    need = fa.fa_decode_split_workspace_bytes(B, H, 128, max_seqlen, sk)
    assert need > 0
    mb = -(-max_seqlen // page)
    for split in (0, sk):
        assert paged_call(B=B, H=H, page=page, max_blocks=mb, max_seqlen=max_seqlen,
                          split_keys=split, ws_bytes=need) == HIPERR



def test_block_sparse_rejects_invalid_arguments():
    lib = fa.load()
    call = lambda **kw: lib.fa_fwd_block_sparse(  # noqa: E731
        kw.get("q", A), A, A, A2, A2, kw.get("m", A2), 1, 2, kw.get("Nq", 64), kw.get("Nk", 64),
        kw.get("d", 128), 0.1, 0, None)
    assert call(m=None) == INVALID
    assert call(q=A + 8) == INVALID
    assert call(d=64) == UNSUPPORTED
    assert call(Nk=64 * 1024 + 1) == INVALID  # more than 1024 key blocks
