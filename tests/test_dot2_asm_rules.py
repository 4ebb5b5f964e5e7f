"""The hand-scheduled dot2 blocks (dot2_asm.h) against gfx950's software-managed
VALU hazards, checked on the CPU.

The compiler inserts the wait states its hazard recognizer knows about, but it
does not look inside inline asm, so the generated blocks must hold them by
construction. This test rebuilds every block from gen_dot2_asm.py, checks that
dot2_asm.h is exactly the generator's output, and then walks each block's
instruction list with a model of the hazards that apply to it:

  * DPP: an instruction with a DPP operand reads VGPRs early, so every VGPR it
    reads (the broadcast x, the weight pair and the accumulator) needs 2 wait
    states after a VALU instruction wrote it;
  * DOT results: a v_dot2c result needs 3 wait states before any VALU
    instruction other than a DOT that takes it as its accumulator reads it;
  * block edges: inputs may have been written by the instruction just before
    the block, and outputs may be read by the instruction just after it.

`s_nop n` supplies n + 1 wait states and every other instruction one. The same
model gives the wait states the compiler itself inserts for these instruction
pairs on gfx950 (2 before a DPP read of a VALU result, 3 between a DOT and an
ordinary VALU reader, none between chained DOTs). It also explains the
variant that builds the weight pairs of two words with one 64-bit shift: with
the generator's accumulator rotation its pair order puts two DPP dots on one
accumulator back to back at M = 1 and 2.
"""
import importlib.util
import io
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "spec_verify_amd", "csrc")

SGPR_OPERANDS = {"mask"}


def _generator():
    spec = importlib.util.spec_from_file_location("gen_dot2_asm", os.path.join(CSRC, "gen_dot2_asm.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


GEN = _generator()


def _asm_lines(block_text):
    body = re.search(r'asm volatile\("(.*?)"\n', block_text, re.S).group(1)
    return body.split("\\n\\t")


def _regs(tok):
    """VGPR names of one operand (a %[name] token; pairs are listed as name.lo/.hi)."""
    m = re.fullmatch(r"%\[(\w+)(\.lo|\.hi)?\]", tok)
    if not m or m.group(1) in SGPR_OPERANDS:
        return []
    name = m.group(1)
    if m.group(2):
        return [name + m.group(2)]
    if name.endswith("_64"):
        return [name + ".lo", name + ".hi"]
    return [name]


def _parse(line):
    """(opcode, written VGPRs, read VGPRs, wait states it supplies, is DPP, is DOT)."""
    parts = line.split(None, 1)
    op = parts[0]
    if op == "s_nop":
        return op, [], [], int(parts[1]) + 1, False, False
    ops = [t.strip() for t in parts[1].split(",")]
    ops = [t.split()[0] for t in ops]          # drop modifiers (row_newbcast:..., op_sel:...)
    dst = _regs(ops[0])
    srcs = [r for t in ops[1:] for r in _regs(t)]
    dot = op.startswith("v_dot2c")
    dpp = op.endswith("_dpp")
    if dot:
        srcs = dst + srcs                       # the accumulator is read as well
    return op, dst, srcs, 1, dpp, dot


def check_block(lines, inputs, outputs):
    """Return the list of hazard violations of one block (empty if none)."""
    bad = []
    last = {r: ("valu", 0) for r in inputs}      # writer kind, position in wait states
    pos = 1                                      # wait states elapsed since the block began
    written = set(inputs)
    for i, line in enumerate(lines):
        op, dst, srcs, ws, dpp, dot = _parse(line)
        if op == "s_nop":
            pos += ws
            continue
        for r in srcs:
            if r not in written:
                bad.append(f"{i}: {line}: reads {r} before it is written")
                continue
            kind, at = last[r]
            gap = pos - at - 1
            if dpp and gap < 2:
                bad.append(f"{i}: {line}: DPP reads {r} {gap} wait states after a VALU write")
            is_acc = dot and r in dst
            if kind == "dot" and not is_acc and gap < 3:
                bad.append(f"{i}: {line}: reads DOT result {r} after {gap} wait states")
        for r in dst:
            last[r] = ("dot" if dot else "valu", pos)
            written.add(r)
        pos += ws
    for r in outputs:
        kind, at = last.get(r, ("none", 0))
        if kind == "dot" and pos - at - 1 < 3:
            bad.append(f"block end: DOT result {r} has only {pos - at - 1} wait states")
    return bad


def _io(M, R, words):
    inputs = [f"p{m}" for m in range(M)] + [f"x{m}" for m in range(M)] + [f"w{j}" for j in range(words)]
    inputs += ["magic", "sc"]
    return inputs, [f"p{m}" for m in range(M)]


def test_header_is_the_generators_output():
    buf = io.StringIO()
    GEN.main(buf)
    with open(os.path.join(CSRC, "dot2_asm.h")) as f:
        assert f.read() == buf.getvalue(), "dot2_asm.h differs from gen_dot2_asm.py's output"


@pytest.mark.parametrize("M", range(1, 9))
@pytest.mark.parametrize("fmt", ["w4a16", "mxfp8"])
def test_generated_blocks_are_hazard_free(fmt, M):
    text = GEN.w4a16_block(M) if fmt == "w4a16" else GEN.mxfp8_block(M)
    inputs, outputs = _io(M, GEN._sets(M), 4 if fmt == "w4a16" else 8)
    assert check_block(_asm_lines(text), inputs, outputs) == []


def test_checker_catches_planted_hazards():
    """The model is not vacuous: a DPP dot on the block's inputs without the
    leading s_nop, a block without the trailing s_nop, a weight pair built next
    to its DPP dot and a DOT result read early are each reported."""
    dot = "v_dot2c_f32_bf16_dpp %[p0], %[x0], %[w0] row_newbcast:0 row_mask:0xf bank_mask:0xf"
    assert check_block(["s_nop 1", dot, "s_nop 2"], ["p0", "x0", "w0"], ["p0"]) == []
    assert check_block([dot, "s_nop 2"], ["p0", "x0", "w0"], ["p0"])   # inputs read at once
    assert check_block(["s_nop 1", dot], ["p0", "x0", "w0"], ["p0"])   # no trailing s_nop
    lines = _asm_lines(GEN.w4a16_block(3))
    inputs, outputs = _io(3, 1, 4)
    assert check_block(lines, inputs, outputs) == []
    assert check_block(lines[:-1], inputs, outputs)                    # no s_nop 2 last
    i = next(k for k, l in enumerate(lines) if l.startswith("v_dot2c"))
    early = lines[:i] + ["v_and_or_b32 %[t0], %[w0], %[mask], %[magic]"] + lines[i:]
    assert check_block(early, inputs, outputs)                         # pair built right before its dot
    peek = lines[:i + 1] + ["v_add_f32 %[t1], %[p0], %[p0]"] + lines[i + 1:]
    assert check_block(peek, inputs, outputs)                          # DOT result read by a VALU at once


def _w4a16_block_shift64(M, rotate_by_issue):
    """Instruction list of the 64-bit-shift variant: the pairs of words j and
    j + 1 come from one v_lshrrev_b64 per shift (11 instead of 14 instructions
    per two words). Built like the kept blocks, four temporaries at a time, so
    each group of four dots takes shifts s and s + 1 of both words: the pairs
    enter the accumulators in the order 4j+s, 4j+4+s, 4j+s+1, 4j+5+s, ...
    The accumulator set of a dot is its pair index mod R (the generator's rule,
    which assumes pairs in index order) or its issue position mod R."""
    R = GEN._sets(M)
    lines = []
    GEN._prologue(M, R, lines)
    name = GEN._acc_name(M)
    order = []
    for j in (0, 2):
        for s0 in (0, 2):
            pairs = []
            for s, (ta, tb) in ((s0, (0, 1)), (s0 + 1, (2, 3))):
                if s == 0:
                    lines.append(f"v_and_or_b32 %[t{ta}], %[w{j}], %[mask], %[magic]")
                    lines.append(f"v_and_or_b32 %[t{tb}], %[w{j + 1}], %[mask], %[magic]")
                else:
                    lines.append(f"v_lshrrev_b64 %[s_64], {4 * s}, %[w{j}{j + 1}_64]")
                    lines.append(f"v_and_or_b32 %[t{ta}], %[s_64.lo], %[mask], %[magic]")
                    lines.append(f"v_and_or_b32 %[t{tb}], %[s_64.hi], %[mask], %[magic]")
                pairs += [(4 * j + s, ta), (4 * (j + 1) + s, tb)]
            for p, t in pairs:
                r = (len(order) if rotate_by_issue else p) % R
                for m in range(M):
                    lines.append(f"v_dot2c_f32_bf16_dpp {name(m, r)}, %[x{m}], %[t{t}] "
                                 f"row_newbcast:{p} row_mask:0xf bank_mask:0xf")
                order.append(p)
    GEN._epilogue(M, R, lines)
    return lines, order


def test_shift64_variant_root_cause():
    """The 64-bit-shift variant once gave last-bit differences in two outputs of
    the M = 1 decode GEMV. Taken with the generator's accumulator rotation (set
    = pair index mod R), its pair order puts two DPP dots on one accumulator
    back to back for M = 1 and 2 (pairs 4 and 1 both land in set 1 at M = 1;
    pairs 0 and 4 in set 0 at M = 2): a DPP read of a VALU result with fewer
    than 2 wait states, which the hardware does not interlock. For M >= 3 the
    M dots of a pair separate them and the schedule is clean. Rotating by issue
    position instead removes the hazard at every M, and what is left is a
    different (equally valid) order of the fp32 additions."""
    inputs_extra = ["w01_64.lo", "w01_64.hi", "w23_64.lo", "w23_64.hi"]
    for M in range(1, 9):
        inputs, outputs = _io(M, GEN._sets(M), 4)
        lines, order = _w4a16_block_shift64(M, rotate_by_issue=False)
        bad = check_block(lines, inputs + inputs_extra, outputs)
        if M <= 2:
            early = [re.search(r"DPP reads (\w+) ", b) for b in bad]
            assert bad and all(e and e.group(1)[0] in "pe" for e in early), (M, bad)  # accumulators only
        else:
            assert bad == [], (M, bad)
        lines, order = _w4a16_block_shift64(M, rotate_by_issue=True)
        assert check_block(lines, inputs + inputs_extra, outputs) == [], M
        assert sorted(order) == list(range(16)) and order != list(range(16))
