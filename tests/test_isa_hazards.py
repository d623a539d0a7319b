"""The decode kernel's multiply-adds take their first operand from another
lane through a DPP row broadcast written as inline assembly, which the
compiler's hazard recognizer does not see.  gfx9 requires two wait states
between a VALU write of a VGPR and a DPP read of it.  This compiles the kernel
file to gfx950 assembly (no GPU needed) and checks every DPP instruction in it.
"""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _regs(tok):
    tok = tok.strip().rstrip(",")
    m = re.match(r"v\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _vgpr_writes(inst):
    op = inst.split()[0]
    if not op.startswith("v_") or op.startswith(("v_cmp", "v_readlane", "v_readfirstlane")):
        return set()
    return _regs(inst[len(op):].split(",")[0])


def _wait_states(inst):
    op = inst.split()[0]
    return int(inst.split()[1], 0) + 1 if op == "s_nop" else 1


def dpp_hazards(asm_text):
    """(checked, violations): for each *_dpp instruction, a VALU write of its
    DPP source within the two preceding wait states, following fall-through
    and every branch into a label."""
    insts, labels, branches = [], {}, {}
    for line in asm_text.split("\n"):
        t = line.split(";")[0].strip()
        if not t:
            continue
        if re.match(r"^[\w.$]+:$", t):
            labels[t[:-1]] = len(insts)
            insts.append(("label", t[:-1]))
            continue
        if t.startswith("."):
            continue
        insts.append(("inst", t))
    for k, (kind, t) in enumerate(insts):
        if kind == "inst":
            m = re.match(r"s_(?:cbranch_\w+|branch)\s+([\w.$]+)", t)
            if m:
                branches.setdefault(m.group(1), []).append(k)

    def back(k, src, need):
        j, ws = k - 1, 0
        while j >= 0 and ws < need:
            kind, t = insts[j]
            if kind == "label":
                for b in branches.get(t, []):
                    hit = back(b, src, need - ws)
                    if hit:
                        return hit
            elif t.startswith("s_endpgm"):
                return None
            else:
                if src & _vgpr_writes(t):
                    return t
                ws += _wait_states(t)
            j -= 1
        return None

    checked, bad = 0, []
    for k, (kind, t) in enumerate(insts):
        if kind == "inst" and "_dpp" in t.split()[0]:
            checked += 1
            src = _regs(t[len(t.split()[0]):].split(",")[1])
            hit = back(k, src, 2)
            if hit:
                bad.append((t, hit))
    return checked, bad


def test_checker_finds_a_planted_hazard():
    asm = "\n".join(["f:", "\tv_mul_f32_e32 v5, v1, v2",
                     "\tv_fmac_f32_dpp v6, v5, v7 row_newbcast:0 row_mask:0xf bank_mask:0xf",
                     "\tv_mul_f32_e32 v8, v1, v2", "\ts_nop 0",
                     "\tv_fmac_f32_dpp v6, v8, v7 row_newbcast:0 row_mask:0xf bank_mask:0xf",
                     "\tv_mul_f32_e32 v9, v1, v2", "\ts_nop 1",
                     "\tv_fmac_f32_dpp v6, v9, v7 row_newbcast:0 row_mask:0xf bank_mask:0xf", "\ts_endpgm"])
    checked, bad = dpp_hazards(asm)
    assert checked == 3 and len(bad) == 2


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_decode_kernels_have_no_dpp_source_hazard(tmp_path):
    from decode_attention_offloaded_amd import build as kb
    out = tmp_path / "kvd_attend.s"
    cmd = ([HIPCC] + kb.COMMON + ["--offload-arch=" + kb.ARCH] + kb.CODE_OBJECT + kb.NO_PACKED_FP32 +
           kb.KERNARG_PRELOAD + ["--cuda-device-only", "-S", "-o", str(out),
                                 os.path.join(kb.CSRC, "kvd_attend.hip")])
    subprocess.run(cmd, check=True, capture_output=True)
    text = out.read_text()
    checked, bad = dpp_hazards(text)
    assert checked > 1000, "expected the broadcast multiply-adds in the assembly"
    assert "row_newbcast" in text
    assert not bad, bad[:5]
