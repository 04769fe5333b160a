"""Wait states around the instructions the kernels issue from inline asm.

The compiler's hazard recognizer does not look inside inline asm, so these
instructions carry their own waits; this test compiles the device code with
the library's flags and checks the result.

LDS DMA (`buffer_load_dword[x4] ... lds`): each asm block writes M0 and then
waits with its own `s_nop`: 4 (five wait states) where the buffer descriptor
may just have been written by a VALU instruction (the `v_readfirstlane`s that
build it), 0 where the same descriptor was used by an earlier DMA. gfx9's rule
is that a VMEM instruction reading an SGPR needs five wait states after a VALU
write of that SGPR, and one after an SALU write of M0 for an LDS DMA. Walking
back from every DMA: within the five wait states before it, no VALU
instruction may write its descriptor or soffset SGPRs, and no label or branch
may intervene (a path from elsewhere could not be checked).

MFMA (the backward's S and dP products, `v_mfma_f32_32x32x16_bf16` into VGPRs):
an operand written by a VALU instruction needs two wait states before the
MFMA reads it (each asm block starts with `s_nop 1`), and the 8-pass result
is not readable by other instructions for 12 wait states on gfx950 (what the
compiler itself leaves after such an MFMA). Walking forward from
every asm MFMA, nothing but the next MFMA of the same accumulation chain
(same registers as destination and accumulator input) may touch its
destination registers within 12 wait states, and no label or branch may
intervene.
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess

import pytest

from tiled_attention_fa2_amd import build as fabuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCES = [
    os.path.join(ROOT, "tiled_attention_fa2_amd", "csrc", "fa_api.hip"),
    os.path.join(ROOT, "tiled_attention_fa2_amd", "csrc", "fa_bwd_api.hip"),
    os.path.join(ROOT, "tiled_attention_fa2_amd", "csrc", "fa_quant_api.hip"),
    os.path.join(ROOT, "tests", "hip", "stage_variants.hip"),
]
NEED_WAIT = 5


def _sgprs(tok: str) -> set[int]:
    tok = tok.strip()
    m = re.fullmatch(r"s\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.fullmatch(r"s(\d+)", tok)
    return {int(m.group(1))} if m else set()


def _operands(line: str) -> list[str]:
    parts = line.split(None, 1)
    if len(parts) < 2:
        return []
    return [t.strip() for t in re.split(r",(?![^\[]*\])", parts[1].split(";")[0])]


def check_asm(text: str):
    """Returns (number of DMAs checked, list of violations)."""
    lines = [l.strip() for l in text.split("\n")]
    checked, bad = 0, []
    for i, l in enumerate(lines):
        if not (l.startswith("buffer_load_dword") and re.search(r"\blds\b", l)):
            continue
        checked += 1
        ops = _operands(l)
        need = _sgprs(ops[1]) | (_sgprs(ops[2].split()[0]) if len(ops) > 2 else set())
        waits, j = 0, i - 1
        while waits < NEED_WAIT:
            if j < 0:
                bad.append((i, l, "start of file"))
                break
            t = lines[j]
            j -= 1
            if not t or t.startswith(";") or t.startswith("."):
                if t.startswith(".LBB") or (t.startswith(".") and t.endswith(":")):
                    bad.append((i, l, "label " + t))
                    break
                continue
            if t.endswith(":"):
                bad.append((i, l, "label " + t))
                break
            op = t.split()[0]
            if op.startswith("s_cbranch") or op == "s_branch" or op.startswith("s_setpc") or op.startswith("s_swappc"):
                bad.append((i, l, "branch " + t))
                break
            if op == "s_nop":
                waits += int(_operands(t)[0], 0) + 1
                continue
            if op.startswith("v_"):
                dst = _operands(t)
                if dst and _sgprs(dst[0]) & need:
                    bad.append((i, l, "VALU write " + t))
                    break
            waits += 1
    return checked, bad


MFMA_WAIT = 12


def _vgprs(tok: str) -> set[int]:
    tok = tok.strip().split()[0] if tok.strip() else ""
    m = re.fullmatch(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.fullmatch(r"v(\d+)", tok)
    return {int(m.group(1))} if m else set()


def check_asm_mfma(text: str):
    """Returns (number of asm MFMAs checked, list of violations)."""
    lines = [l.strip() for l in text.split("\n")]
    checked, bad, in_asm, prev = 0, [], False, None
    for i, l in enumerate(lines):
        if l.startswith(";;#ASMSTART"):
            in_asm, prev = True, None
            continue
        if l.startswith(";;#ASMEND"):
            in_asm = False
            continue
        if not in_asm or not l or l.startswith(";"):
            continue
        if not l.startswith("v_mfma"):
            prev = l
            continue
        checked += 1
        if prev is None or not prev.startswith("s_nop") or int(_operands(prev)[0], 0) < 1:
            bad.append((i, l, "no s_nop >= 1 before it in its asm block"))
        prev = l
        dst = _vgprs(_operands(l)[0])
        waits, j = 0, i + 1
        while waits < MFMA_WAIT:
            if j >= len(lines):
                bad.append((i, l, "end of file"))
                break
            t = lines[j]
            j += 1
            if not t or t.startswith(";") or t.startswith("."):
                if t.startswith(".LBB") or (t.startswith(".") and t.endswith(":")):
                    bad.append((i, l, "label " + t))
                    break
                continue
            if t.endswith(":"):
                bad.append((i, l, "label " + t))
                break
            op = t.split()[0]
            if op.startswith("s_cbranch") or op == "s_branch" or op.startswith("s_setpc"):
                bad.append((i, l, "branch " + t))
                break
            if op == "s_nop":
                waits += int(_operands(t)[0], 0) + 1
                continue
            ops = _operands(t)
            if op.startswith("v_mfma") and len(ops) > 3 and _vgprs(ops[0]) == dst and _vgprs(ops[3]) == dst:
                break   # the chain goes on: the next MFMA accumulates into the same registers
            touched = set()
            for x in ops:
                touched |= _vgprs(x)
            if touched & dst:
                bad.append((i, l, f"after {waits} wait states: " + t))
                break
            waits += 1
    return checked, bad


@pytest.mark.skipif(shutil.which(fabuild.HIPCC) is None and not os.path.exists(fabuild.HIPCC),
                    reason="hipcc not available")
@pytest.mark.parametrize("src", SOURCES, ids=lambda p: os.path.basename(p))
def test_asm_wait_states(src, tmp_path):
    flags = [f for f in fabuild.FLAGS if f not in ("-shared", "-fPIC")]
    out = tmp_path / "dev.s"
    r = subprocess.run([fabuild.HIPCC, *flags, "--cuda-device-only", "-S", src, "-o", str(out)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    text = out.read_text()
    checked, bad = check_asm(text)
    if os.path.basename(src) != "fa_quant_api.hip":
        assert checked > 0, "no LDS DMA found: the check would be vacuous"
    assert not bad, "\n".join(f"line {i}: {l}  <- {why}" for i, l, why in bad[:20])
    n_mfma, bad = check_asm_mfma(text)
    if os.path.basename(src) == "fa_bwd_api.hip":
        assert n_mfma > 0, "no asm MFMA found: the check would be vacuous"
    assert not bad, "\n".join(f"line {i}: {l}  <- {why}" for i, l, why in bad[:20])


def test_checker_flags_a_planted_hazard():
    good = """
\tv_readfirstlane_b32 s7, v3
\ts_mov_b32 s6, s1
\t;;#ASMSTART
\ts_mov_b32 m0, s9
\ts_nop 4
\tbuffer_load_dwordx4 v1, s[4:7], 0 offen lds
\t;;#ASMEND
\t;;#ASMSTART
\ts_mov_b32 m0, s10
\ts_nop 0
\tbuffer_load_dwordx4 v2, s[4:7], 0 offen lds
\t;;#ASMEND
"""
    assert check_asm(good) == (2, [])
    # the descriptor rewritten by a VALU right before a nop-0 DMA
    bad = good.replace("\ts_mov_b32 m0, s10\n", "\tv_readfirstlane_b32 s6, v4\n\ts_mov_b32 m0, s10\n")
    n, found = check_asm(bad)
    assert n == 2 and len(found) == 1 and "VALU write" in found[0][2]
    # a VALU write of soffset counts too
    soff = bad.replace("v_readfirstlane_b32 s6, v4", "v_readfirstlane_b32 s12, v4").replace(
        "v2, s[4:7], 0 offen", "v2, s[4:7], s12 offen")
    assert len(check_asm(soff)[1]) == 1
    # a label inside the window cannot be checked
    lab = good.replace("\t;;#ASMSTART\n\ts_mov_b32 m0, s10", ".LBB0_3:\n\t;;#ASMSTART\n\ts_mov_b32 m0, s10")
    assert "label" in check_asm(lab)[1][0][2]


def test_mfma_checker_flags_planted_hazards():
    good = """
\t;;#ASMSTART
\ts_nop 1
\tv_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], 0
\t;;#ASMEND
\t;;#ASMSTART
\ts_nop 1
\tv_mfma_f32_32x32x16_bf16 v[0:15], v[24:27], v[28:31], v[0:15]
\t;;#ASMEND
\tv_add_u32_e32 v40, 4, v41
\t;;#ASMSTART
\ts_nop 7
\ts_nop 7
\t;;#ASMEND
\tv_exp_f32_e32 v1, v0
"""
    assert check_asm_mfma(good) == (2, [])
    # the result read before the drain
    early = good.replace("\tv_add_u32_e32 v40, 4, v41", "\tv_mov_b32_e32 v40, v3")
    n, found = check_asm_mfma(early)
    assert n == 2 and len(found) == 1 and "v_mov_b32" in found[0][2]
    # an asm MFMA without its leading wait
    nowait = good.replace("\ts_nop 1\n\tv_mfma_f32_32x32x16_bf16 v[0:15], v[24:27]",
                          "\tv_mfma_f32_32x32x16_bf16 v[0:15], v[24:27]")
    assert any("no s_nop" in why for _, _, why in check_asm_mfma(nowait)[1])
    # a chain into other registers is no chain
    other = good.replace("v[28:31], v[0:15]", "v[28:31], v[32:47]")
    assert len(check_asm_mfma(other)[1]) == 1
