"""The scaled fp8 MFMA (v_mfma_scale_f32_32x32x64_f8f6f4) reads its 8-register
operands over several cycles after it issues, which the compiler's hazard
model does not cover: a VALU write into a dead operand register one
instruction after the MFMA was seen to corrupt the product.  gmm_mx.hip fences
every such MFMA; this test compiles it to gfx950 assembly and checks that no
VALU instruction writes an operand register (sources, block scales) of a
scaled MFMA within 16 wait states of it."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "combine_router_gating_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
WINDOW = 16


def _regs(tok):
    m = re.match(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _vdst(line):
    op = line.split()[0]
    if not op.startswith("v_") or op.startswith(("v_cmp", "v_readfirstlane", "v_readlane")):
        return set()
    return _regs(line[len(op):].split(",")[0].strip())


def _violations(asm):
    lines = [l.strip() for l in asm.split("\n")]
    bad, n = [], 0
    for i, l in enumerate(lines):
        if not l.startswith("v_mfma_scale"):
            continue
        n += 1
        toks = [t.strip() for t in l[len(l.split()[0]):].split(",")]
        ops = _regs(toks[1]) | _regs(toks[2]) | _regs(toks[4]) | _regs(toks[5].split()[0])
        ws = 0
        for t in lines[i + 1:]:
            if ws >= WINDOW:
                break
            if not t or t.startswith(";") or t.endswith(":") or t.startswith("."):
                continue
            m = re.match(r"s_nop (\d+)", t)
            if m:
                ws += int(m.group(1)) + 1
                continue
            ws += 1
            if _vdst(t) & ops:
                bad.append((ws, l, t))
    return n, bad


def test_parser_sees_a_planted_hazard():
    asm = ("v_mfma_scale_f32_32x32x64_f8f6f4 v[0:15], v[16:23], v[24:31], v[0:15], v40, v41 op_sel_hi:[0,0,0]\n"
           "s_nop 3\n v_add_u32_e32 v18, v1, v2\n")
    n, bad = _violations(asm)
    assert n == 1 and len(bad) == 1 and bad[0][0] == 5
    n, bad = _violations(asm.replace("s_nop 3", "s_nop 7\ns_nop 7"))
    assert n == 1 and not bad


@pytest.mark.skipif(not shutil.which(HIPCC) and not os.path.exists(HIPCC), reason="hipcc not found")
def test_scaled_mfma_operands_are_fenced(tmp_path):
    out = tmp_path / "gmm_mx.s"
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature",
                    "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-S",
                    "--cuda-device-only", os.path.join(CSRC, "gmm_mx.hip"), "-o", str(out)],
                   check=True, capture_output=True)
    n, bad = _violations(out.read_text())
    assert n > 0
    assert not bad, bad[:5]
