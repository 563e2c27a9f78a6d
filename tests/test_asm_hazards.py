"""The AGPR-accumulator MFMAs of the one-wave dK/dV kernel are inline assembly,
so the compiler inserts no wait states before them. A VALU write of one of their
A/B operand registers needs two wait states before the MFMA reads it. This test
compiles bwd_kernels.hip for gfx950 to assembly and checks, for every such MFMA
of bwd_dkdv64_kernel, that neither of the two instructions before it is a VALU
instruction writing one of its operand registers."""
import os
import re
import shutil
import subprocess

import pytest

from scaled_dot_product_04_amd import _build

CSRC = os.path.join(os.path.dirname(_build.__file__), "csrc")


def _regs(tok: str) -> set:
    m = re.match(r"v\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _kernel_lines(asm: str, name_re: str) -> list:
    lines = asm.splitlines()
    st = next(k for k, l in enumerate(lines) if re.match(r"^_ZN4sdpa\w+:", l) and re.search(name_re, l))
    en = next(k for k in range(st, len(lines)) if lines[k].startswith(".Lfunc_end"))
    return [l.strip() for l in lines[st:en] if l.strip() and not l.strip().startswith((";", "."))]


def find_hazards(ins: list) -> tuple:
    n, bad = 0, []
    for i, l in enumerate(ins):
        if not (l.startswith("v_mfma") and " a[" in l):
            continue
        n += 1
        ops = [x.strip() for x in l.split(None, 1)[1].split(",")]
        src = _regs(ops[1]) | _regs(ops[2])
        for p in ins[max(0, i - 2):i]:
            if p.startswith("v_") and not p.startswith("v_mfma"):
                if _regs(p.split(None, 1)[1].split(",")[0].strip()) & src:
                    bad.append((p, l))
    return n, bad


def test_scanner_flags_a_planted_hazard():
    ins = ["v_mov_b32_e32 v5, 0", "v_mfma_f32_32x32x16_bf16 a[0:15], v[4:7], v[8:11], a[0:15]"]
    assert find_hazards(ins) == (1, [(ins[0], ins[1])])
    ins = ["v_mov_b32_e32 v5, 0", "s_nop 0", "s_nop 0", "v_mfma_f32_32x32x16_bf16 a[0:15], v[4:7], v[8:11], a[0:15]"]
    assert find_hazards(ins) == (1, [])


@pytest.mark.skipif(shutil.which(_build.HIPCC) is None and not os.path.exists(_build.HIPCC), reason="hipcc not found")
@pytest.mark.parametrize("src,kernel", [("bwd_kernels.hip", "bwd_dkdv64_kernel")])
def test_asm_mfma_operands_have_wait_states(tmp_path, src, kernel):
    out = tmp_path / "k.s"
    cmd = [_build.HIPCC, *_build.FLAGS, "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    asm = out.read_text()
    for name in [kernel + "INS_5Bf16TELb1E", kernel + "INS_5Bf16TELb0E", kernel + "INS_4F16TELb1E", kernel + "INS_4F16TELb0E"]:
        n, bad = find_hazards(_kernel_lines(asm, name))
        assert n > 0, name
        assert not bad, (name, bad[:3])
