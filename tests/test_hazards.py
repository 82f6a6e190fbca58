"""Static check of the hand-scheduled matrix products in the generated gfx950
assembly (CPU only: hipcc cross-compiles).

Several kernels issue v_mfma_f32_32x32x16_bf16 as inline assembly, which the
compiler does not guard with wait states, and read the products with vector
instructions after explicit pauses.  For every product that writes vector
registers, the check walks forward through straight-line code and counts wait
states (1 per instruction, N+1 per s_nop N, 4 per further product); any
vector, LDS or memory instruction touching the product's registers before 18
wait states (more than an 8-pass product needs) is a finding.  It also flags
a vector write to a register that a product reads as its A or B operand within
the two instructions before it.
"""
import os
import re
import shutil
import subprocess

import pytest

from conftest import ROOT

CSRC = os.path.join(ROOT, "io_aware_exact_17_amd", "csrc")
NEED = 18
REG = re.compile(r"\b([va])(?:\[(\d+):(\d+)\]|(\d+)\b)")
STOP = (".LBB", "s_branch", "s_cbranch", "s_endpgm", "s_setpc")


def _regs(text):
    out = set()
    for m in REG.finditer(text):
        if m.group(4) is not None:
            out.add((m.group(1), int(m.group(4))))
        else:
            out.update((m.group(1), r) for r in range(int(m.group(2)), int(m.group(3)) + 1))
    return out


def findings(asm: str, name_filter: str = ""):
    """(function, products, [findings]) for every function in `asm`."""
    result = []
    for name, body in re.findall(r"^(_Z\S+):[^\n]*\n(.*?)\.Lfunc_end", asm, flags=re.S | re.M):
        if name_filter not in name:
            continue
        ins = [l.strip() for l in body.splitlines()]
        ins = [l for l in ins if l.startswith(".LBB") or
               (l and not l.startswith((";", ".", "//")) and not l.endswith(":"))]
        bad, n_products = [], 0
        for i, line in enumerate(ins):
            if not line.startswith("v_mfma"):
                continue
            n_products += 1
            ops = line.split(None, 1)[1].split(",")
            dst, ab = _regs(ops[0]), _regs(",".join(ops[1:3]))
            ws = 0
            for nxt in ins[i + 1:]:
                if nxt.startswith(STOP):
                    break
                op = nxt.split()[0]
                if op == "s_nop":
                    ws += int(nxt.split()[1]) + 1
                    continue
                if op.startswith("v_mfma"):
                    ws += 4
                    continue
                if ws >= NEED:
                    break
                if op.startswith(("v_", "ds_", "global_", "buffer_")) and _regs(nxt) & dst:
                    bad.append(f"{ws} wait states after `{line}`: `{nxt}`")
                    break
                ws += 1
            for prev in ins[max(0, i - 2):i]:
                if prev.startswith("v_") and not prev.startswith("v_mfma") and "," in prev:
                    if _regs(prev.split(None, 1)[1].split(",")[0]) & ab:
                        bad.append(f"vector write right before `{line}`: `{prev}`")
        result.append((name, n_products, bad))
    return result


SYNTH = """\
_Z4earlyv:                               ; @_Z4earlyv
\tv_mfma_f32_32x32x16_bf16 v[96:111], v[2:5], a[0:3], 0
\tv_fma_f32 v1, v96, s15, -v234
\ts_endpgm
.Lfunc_end0:
_Z6pausedv:                              ; @_Z6pausedv
\tv_mfma_f32_32x32x16_bf16 v[96:111], v[2:5], a[0:3], 0
\ts_nop 15
\ts_nop 3
\tv_fma_f32 v1, v96, s15, -v234
\ts_endpgm
.Lfunc_end1:
_Z7operandv:                             ; @_Z7operandv
\tv_mov_b32 v3, 0
\tv_mfma_f32_32x32x16_bf16 v[16:31], v[2:5], a[0:3], 0
\ts_endpgm
.Lfunc_end2:
"""


def test_check_catches_planted_hazards():
    got = {name: len(bad) for name, _, bad in findings(SYNTH)}
    assert got == {"_Z4earlyv": 1, "_Z6pausedv": 0, "_Z7operandv": 1}


def _device_asm(src, tmp_path):
    from io_aware_exact_17_amd import build as b

    hipcc = shutil.which("hipcc") or os.path.join(b.ROCM, "bin", "hipcc")
    out = tmp_path / (os.path.basename(src) + ".s")
    flags = [f for f in b.HIP_FLAGS if f != "-fPIC"]
    subprocess.run([hipcc, *flags, f"-I{b.INCLUDE}", f"-I{CSRC}", f"-I{b.ROCM}/include",
                    "--cuda-device-only", "-S", src, "-o", str(out)],
                   check=True, capture_output=True)
    return out.read_text()


@pytest.mark.parametrize("src,kernel", [("fwd_bf16.hip", "fwd_bf16_kernel"),
                                        ("fwd_bf16_d64.hip", "fwd_bf16_kernel"),
                                        ("bwd_bf16.hip", "_kernel")])
def test_no_product_hazards(src, kernel, tmp_path):
    if not (shutil.which("hipcc") or os.path.exists("/opt/rocm/bin/hipcc")):
        pytest.skip("hipcc not available")
    res = findings(_device_asm(os.path.join(CSRC, src), tmp_path), kernel)
    assert res and sum(n for _, n, _ in res) > 0, "no products found: the parser lost the kernels"
    bad = [(name, b) for name, _, bl in res for b in bl]
    assert not bad, bad[:5]
