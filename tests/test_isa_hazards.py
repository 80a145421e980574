"""Wait states around the attention kernel's inline-assembly MFMAs.

The PV accumulation is issued as inline assembly (a scaled FP8 MFMA), which
the compiler does not look into: it inserts no wait states between that
instruction and the VALU code around it. The kernel separates them by hand.
This test compiles the kernels for gfx950 and checks every instantiation's
machine code, following branches (accumulators may be VGPRs or AGPRs):
  - after an inline-assembly MFMA, no other instruction reads or writes its
    accumulator registers within AFTER wait states (an 8-pass XDL result
    needs 12 before VALU may read it; 24 are given),
  - before it, no VALU instruction writes its source registers within
    BEFORE wait states (2 are needed; 4 are given).
Wait states are counted as one per instruction and n+1 per s_nop n, which
undercounts (an MFMA issue takes several cycles), so the check is
conservative. The scanner itself is checked on small listings with a planted
hazard.
"""
import importlib.util
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
AFTER = 16
BEFORE = 2
ASM_MFMA = "v_mfma_scale_f32_16x16x128_f8f6f4"


def _build_module():
    spec = importlib.util.spec_from_file_location(
        "oc_build", os.path.join(ROOT, "bit_fp8_attention_block_amd", "build.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def _regs(text):
    """VGPRs and AGPRs named in an operand list, as ('v', n) / ('a', n)."""
    out = set()
    for m in re.finditer(r"\b([va])\[(\d+):(\d+)\]|\b([va])(\d+)\b", text):
        if m.group(4):
            out.add((m.group(4), int(m.group(5))))
        else:
            out.update((m.group(1), r) for r in range(int(m.group(2)), int(m.group(3)) + 1))
    return out


def _parse(body):
    """Instructions of one function as (is_inline_asm, opcode, operands) and
    the index of each label."""
    ins, labels, in_asm = [], {}, False
    for line in body.split("\n"):
        t = line.strip()
        if t.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if t.startswith(";;#ASMEND"):
            in_asm = False
            continue
        m = re.match(r"^(\.LBB\w+):", line)
        if m:
            labels[m.group(1)] = len(ins)
            continue
        if line.startswith("\t") and t and not t.startswith((".", ";")):
            parts = t.split(None, 1)
            ins.append((in_asm, parts[0], parts[1] if len(parts) > 1 else ""))
    return ins, labels


def _waits(op, args):
    return int(args.split()[0]) + 1 if op == "s_nop" else 1


def scan(body):
    """Hazards around inline-assembly MFMAs in one function's assembly."""
    ins, labels = _parse(body)
    found = []
    for k, (is_asm, op, args) in enumerate(ins):
        if not (is_asm and op == ASM_MFMA):
            continue
        ops = [x.strip() for x in args.split(",")]
        acc = _regs(ops[0])
        srcs = _regs(ops[1]) | _regs(ops[2]) | _regs(ops[4]) | _regs(ops[5].split()[0])
        # forward, along every path, until AFTER wait states have passed
        todo, seen = [(k + 1, 0)], set()
        while todo:
            i, w = todo.pop()
            while i < len(ins) and w < AFTER:
                if (i, w) in seen:
                    break
                seen.add((i, w))
                a2, op2, args2 = ins[i]
                if op2 == "s_endpgm":
                    break
                if op2.startswith("s_cbranch") or op2 == "s_branch":
                    tgt = args2.split()[0]
                    if tgt in labels:
                        todo.append((labels[tgt], w + 1))
                    if op2 == "s_branch":
                        break
                    i, w = i + 1, w + 1
                    continue
                chained = a2 and op2 == ASM_MFMA and args2.split(",")[3].strip() == args2.split(",")[0].strip()
                if _regs(args2) & acc and not chained:
                    found.append(f"after +{w}: {op} {args} | {op2} {args2}")
                w += _waits(op2, args2)
                i += 1
        # backward, in program order, over BEFORE wait states
        w = 0
        for i in range(k - 1, -1, -1):
            a2, op2, args2 = ins[i]
            w += _waits(op2, args2)
            if w > BEFORE:
                break
            if op2.startswith("v_") and not op2.startswith("v_mfma") and _regs(args2.split(",")[0]) & srcs:
                found.append(f"before -{w}: {op2} {args2} | {op} {args}")
    return found


def _functions(asm):
    for m in re.finditer(r"^(_ZN2oc1\d+attn_kernel\w*):", asm, re.M):
        end = asm.index(".Lfunc_end", m.end())
        yield m.group(1), asm[m.end():end]


LISTING = """\t;;#ASMSTART
\tv_mfma_scale_f32_16x16x128_f8f6f4 v[10:13], v[20:27], v[30:37], v[10:13], v1, v2 op_sel_hi:[0,0,0]
\t;;#ASMEND
{between}
\tv_add_f32_e32 v40, v11, v40
\ts_endpgm
"""


def test_scanner_flags_a_read_of_the_accumulator_right_after_the_mfma():
    assert len(scan(LISTING.format(between="\tv_mov_b32_e32 v50, 0"))) == 1
    fenced = "\t;;#ASMSTART\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\t;;#ASMEND"
    assert scan(LISTING.format(between=fenced)) == []


def test_scanner_flags_a_read_on_a_branch_target():
    body = ("\t;;#ASMSTART\n\tv_mfma_scale_f32_16x16x128_f8f6f4 v[10:13], v[20:27], v[30:37], v[10:13], v1, v2 "
            "op_sel_hi:[0,0,0]\n\t;;#ASMEND\n\ts_cbranch_scc1 .LBB0_2\n\ts_nop 7\n\ts_nop 7\n\ts_endpgm\n"
            ".LBB0_2:\n\tv_mul_f32_e32 v12, 2.0, v12\n\ts_endpgm\n")
    assert len(scan(body)) == 1


def test_scanner_flags_a_valu_write_of_the_p_operand_right_before_the_mfma():
    body = ("\tv_perm_b32 v37, v5, v6, s0\n\t;;#ASMSTART\n\tv_mfma_scale_f32_16x16x128_f8f6f4 v[10:13], v[20:27], "
            "v[30:37], v[10:13], v1, v2 op_sel_hi:[0,0,0]\n\t;;#ASMEND\n\ts_nop 7\n\ts_nop 7\n\ts_endpgm\n")
    assert len(scan(body)) == 1
    fenced = body.replace("\t;;#ASMSTART\n\tv_mfma", "\t;;#ASMSTART\n\ts_nop 3\n\t;;#ASMEND\n\t;;#ASMSTART\n\tv_mfma")
    assert scan(fenced) == []


def test_attention_kernels_keep_their_wait_states(tmp_path):
    b = _build_module()
    try:
        hipcc = b._hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    out = tmp_path / "attention.s"
    cmd = [hipcc, *b.FLAGS, "--cuda-device-only", "-S", "-o", str(out),
           os.path.join(b.CSRC, "attention.hip")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    asm = out.read_text()
    n_fn = n_mfma = 0
    problems = []
    for name, body in _functions(asm):
        n_fn += 1
        n_mfma += body.count(ASM_MFMA)
        problems += [f"{name}: {p}" for p in scan(body)]
    assert n_fn >= 8 and n_mfma > 0
    assert problems == [], "\n".join(problems[:20])
