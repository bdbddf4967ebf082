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


BRANCH = re.compile(r"^s_(?:cbranch_\w+|branch)\s+(\S+)")


def hazards(asm):
    """VALU writes of an MFMA's source registers fewer than two wait states
    before it, on any path into the MFMA (fall-through and branches)."""
    ins = instructions(asm)
    preds = {}   # label -> indices of the branches that jump to it
    for i, (text, is_label) in enumerate(ins):
        m = None if is_label else BRANCH.match(text)
        if m:
            preds.setdefault(m.group(1), []).append(i)
    bad = []

    def scan(j, budget, srcs, mfma, seen):
        # walk back from instruction j with `budget` wait states left
        while j >= 0 and budget > 0:
            t, lab = ins[j]
            if lab:
                name = t.rstrip(":")
                for bi in preds.get(name, []):
                    if (bi, budget) not in seen:
                        seen.add((bi, budget))
                        scan(bi - 1, budget - 1, srcs, mfma, seen)   # the branch itself issues
                j -= 1
                if j >= 0 and not ins[j][1] and ins[j][0].startswith("s_branch"):
                    return   # no fall-through into the label
                continue
            hit = valu_def(t) & srcs
            if hit:
                bad.append(f"{t}  ->  {mfma}")
            budget -= wait_states(t)
            j -= 1

    for i, (text, is_label) in enumerate(ins):
        if is_label or not text.startswith("v_mfma"):
            continue
        operands = text.split(None, 1)[1].split(",")
        scan(i - 1, 2, regs(",".join(operands[1:])), text, set())
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
    # a write on a branch path into the MFMA's block is found too
    branchy = """
    v_cvt_pk_bf16_f32 v7, v10, v11
    s_cbranch_scc1 .LBB0_5
    v_add_u32_e32 v40, v41, v42
    s_nop 3
    .LBB0_5:
    v_mfma_f32_32x32x16_bf16 a[0:15], v[4:7], v[0:3], a[0:15]
    """
    bad = hazards(branchy)
    assert len(bad) == 1 and "v_cvt_pk_bf16_f32 v7" in bad[0], bad


KERNEL_SOURCES = [s for s in build.sources() if os.path.basename(s).startswith(("fa_bwd", "fa_fwd"))]


@pytest.fixture(scope="module")
def kernel_assembly():
    import concurrent.futures as cf
    with cf.ThreadPoolExecutor(max_workers=min(8, len(KERNEL_SOURCES))) as ex:
        return dict(zip(KERNEL_SOURCES, ex.map(assembly, KERNEL_SOURCES)))


def test_kernel_sources_found():
    names = {os.path.basename(s) for s in KERNEL_SOURCES}
    assert "fa_bwd.hip" in names and any(n.startswith("fa_fwd") for n in names)


@pytest.mark.parametrize("src", KERNEL_SOURCES, ids=os.path.basename)
def test_no_valu_write_right_before_mfma_read(src, kernel_assembly):
    bad = hazards(kernel_assembly[src])
    assert not bad, "VALU write then MFMA read without two wait states:\n" + "\n".join(bad[:20])


def early_accumulator_reads(asm, mnemonic="v_mfma_f32_32x32x64_f8f6f4", drain_nops=3):
    """For every `mnemonic` product written as inline asm, the instructions up
    to the next drain (drain_nops consecutive `s_nop 7`, 24 wait states) that
    read or write its accumulator other than further products.  The compiler
    does not know these are MFMAs, so such an instruction -- typically a
    register-allocation copy -- would read a result that is not yet written.
    Straight-line scan per code path (labels end nothing: a product is always
    drained in its own block in the kernels checked)."""
    ins = [t for t, lab in instructions(asm) if not lab]
    bad = []
    for k, t in enumerate(ins):
        if not t.startswith(mnemonic):
            continue
        dst = regs(t.split(",")[0])
        nops = 0
        for u in ins[k + 1:]:
            if u.startswith("s_nop 7"):
                nops += 1
                if nops == drain_nops:
                    break
                continue
            nops = 0
            if u.startswith(mnemonic) or u.startswith("s_"):
                continue
            if regs(u) & dst:
                bad.append(f"{t}  ->  {u}")
                break
    return bad


@pytest.mark.parametrize("src", [s for s in KERNEL_SOURCES if os.path.basename(s) == "fa_fwd8.hip"],
                         ids=os.path.basename)
def test_fp8_products_drained_before_any_other_use(src, kernel_assembly):
    asm = kernel_assembly[src]
    assert asm.count("v_mfma_f32_32x32x64_f8f6f4") >= 16
    bad = early_accumulator_reads(asm)
    assert not bad, "accumulator used before the drain:\n" + "\n".join(bad[:20])


@pytest.mark.parametrize("src", [s for s in KERNEL_SOURCES if os.path.basename(s) == "fa_fwd8.hip"],
                         ids=os.path.basename)
def test_mxfp4_products_drained_before_any_other_use(src, kernel_assembly):
    """The scaled fp4 products of the MXFP4 forward are inline asm too."""
    asm = kernel_assembly[src]
    assert asm.count("v_mfma_scale_f32_32x32x64_f8f6f4") >= 8
    bad = early_accumulator_reads(asm, mnemonic="v_mfma_scale_f32_32x32x64_f8f6f4")
    assert not bad, "accumulator used before the drain:\n" + "\n".join(bad[:20])


def test_drain_scanner_finds_a_planted_copy():
    planted = "\n".join([
        "\tv_mfma_f32_32x32x64_f8f6f4 v[0:15], v[16:23], v[24:31], v[0:15]",
        "\tv_mfma_f32_32x32x64_f8f6f4 v[32:47], v[16:23], v[24:31], v[32:47]",
        "\tv_mov_b64_e32 v[50:51], v[14:15]",
        "\ts_nop 7", "\ts_nop 7", "\ts_nop 7",
        "\tv_mov_b64_e32 v[52:53], v[46:47]",
    ])
    bad = early_accumulator_reads(planted)
    assert len(bad) == 1 and "v[50:51], v[14:15]" in bad[0], bad
