"""Checks on the gfx950 assembly of the kernels (CPU only: hipcc cross-compiles).

Some matrix products are written as single inline-asm instructions so that
their operands stay in fixed register files; the compiler's hazard
recognizer does not see those as MFMAs.  The one hazard they leave to the
code around them is a VALU write of a register followed, within two wait
states, by an MFMA that reads it (the hardware does not interlock it).  This
test compiles every kernel source to assembly and checks that no MFMA has a
VALU write of one of its source registers among the two instructions before
it (an s_nop N counts N + 1).
"""
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "exact_attention_50_amd"))
import build  # noqa: E402

REG = re.compile(r"\b([va])(?:\[(\d+):(\d+)\]|(\d+)\b)")


def regs(text):
    out = set()
    for m in REG.finditer(text):
        kind = m.group(1)
        if m.group(4) is not None:
            out.add((kind, int(m.group(4))))
        else:
            out.update((kind, r) for r in range(int(m.group(2)), int(m.group(3)) + 1))
    return out


def assembly(src):
    cmd = [build.HIPCC, *build.CFLAGS, "--cuda-device-only", "-S", src, "-o", "-"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        pytest.skip(f"hipcc unavailable or failed: {r.stderr[-500:]}")
    return r.stdout


def instructions(asm):
    """(text, is_label) per line of code, comments and directives dropped."""
    out = []
    for line in asm.splitlines():
        s = line.split(";")[0].strip()
        if not s or s.startswith("."):
            if s.endswith(":"):
                out.append((s, True))
            continue
        if s.endswith(":"):
            out.append((s, True))
            continue
        out.append((s, False))
    return out


def wait_states(ins):
    m = re.match(r"s_nop\s+(\d+)", ins)
    return int(m.group(1)) + 1 if m else 1


def valu_def(ins):
    op = ins.split()[0]
    if not op.startswith("v_") or op.startswith("v_mfma") or op.startswith("v_cmp") or op.startswith("v_readfirstlane") \
            or op.startswith("v_readlane"):
        return set()
    dst = ins.split(None, 1)[1].split(",")[0] if " " in ins else ""
    return regs(dst)


def hazards(asm):
    ins = instructions(asm)
    bad = []
    for i, (text, is_label) in enumerate(ins):
        if is_label or not text.startswith("v_mfma"):
            continue
        operands = text.split(None, 1)[1].split(",")
        srcs = regs(",".join(operands[1:]))
        ws, j = 0, i - 1
        while j >= 0 and ws < 2:
            t, lab = ins[j]
            if lab:
                break
            hit = valu_def(t) & srcs
            if hit:
                bad.append(f"{t}  ->  {text}")
            ws += wait_states(t)
            j -= 1
        if j >= 0 and ins[j][1] and ws < 2:
            bad.append(f"block start {ins[j][0]} within two wait states of {text}")
    return bad


def test_scanner_finds_a_planted_hazard():
    snippet = """
    v_cvt_pk_bf16_f32 v3, v10, v11
    v_mfma_f32_32x32x16_bf16 a[0:15], v[20:23], v[0:3], a[0:15]
    v_add_u32_e32 v40, v41, v42
    s_nop 1
    v_mfma_f32_32x32x16_bf16 a[0:15], v[40:43], v[0:3], a[0:15]
    v_add_u32_e32 v50, v41, v42
    s_nop 0
    ds_read_b128 v[60:63], v1
    v_mfma_f32_32x32x16_bf16 a[0:15], v[48:51], v[0:3], a[0:15]
    """
    bad = hazards(snippet)
    assert len(bad) == 1 and "v_cvt_pk_bf16_f32 v3" in bad[0]


@pytest.mark.parametrize("src", [s for s in build.sources() if s.endswith(("fa_bwd.hip", "fa_fwd.hip"))])
def test_no_valu_write_right_before_mfma_read(src):
    bad = hazards(assembly(src))
    assert not bad, "VALU write then MFMA read without two wait states:\n" + "\n".join(bad[:20])
