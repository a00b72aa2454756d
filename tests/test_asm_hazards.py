"""CPU check of the inline assembly in the HIP sources.

The compiler's hazard recognizer does not look inside inline assembly.  A
vector-memory instruction whose scalar base register was written by a VALU
instruction (v_readlane / v_readfirstlane, e.g. when the compiler reloads a
spilled SGPR from a lane) needs 5 wait states before it reads that base, and
an SALU write of M0 needs 1 before an LDS DMA.  With fewer, the load can use a
stale base and fault.  Every inline-asm block that issues a vector-memory or
LDS-DMA instruction must therefore open with `s_nop 4` (5 wait states) or
more.  A DPP read after a VALU write needs 2 wait states (`s_nop 1`).
"""
import glob
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "quantized_kv_cache_row_amd", "csrc")

VMEM = re.compile(r"\b(global_(load|store|atomic)\w*|buffer_(load|store|atomic)\w*|flat_\w+|scratch_\w+)")
DPP = re.compile(r"\b\w+_dpp\b|\b(quad_perm|row_ror|row_mirror|row_half_mirror|row_bcast\w*)\b")


def _asm_blocks(text):
    """(line, template) for every asm statement: the adjacent string literals
    that open its argument list (a macro parameter spliced between literals,
    as in `"... " PAT " ..."`, stands in as its name)."""
    out = []
    for m in re.finditer(r"\basm\s*(?:volatile\s*)?\(", text):
        i = m.end()
        parts = []
        while True:
            s = re.match(r"(?:\s|\\\n)*\"((?:[^\"\\]|\\.)*)\"", text[i:])
            if s:
                parts.append(s.group(1))
                i += s.end()
                continue
            s = re.match(r"(?:\s|\\\n)*([A-Z_][A-Z0-9_]*)(?=(?:\s|\\\n)*\")", text[i:])
            if s and parts:
                parts.append(s.group(1))
                i += s.end()
                continue
            break
        out.append((text.count("\n", 0, m.start()) + 1, "".join(parts).replace("\\n", "\n").replace("\\t", " ")))
    return out


def _leading_nop(template):
    first = template.strip().split("\n")[0].strip()
    m = re.match(r"s_nop\s+(\d+)$", first)
    return int(m.group(1)) if m else -1


def _sources():
    files = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.h")))
    assert files
    return files


def test_vmem_asm_blocks_open_with_five_wait_states():
    seen = 0
    for path in _sources():
        for line, tpl in _asm_blocks(open(path).read()):
            if VMEM.search(tpl):
                seen += 1
                assert _leading_nop(tpl) >= 4, f"{os.path.basename(path)}:{line}: VMEM asm without s_nop 4: {tpl!r}"
    assert seen >= 2  # the fp8 decode's LDS DMA blocks


def test_dpp_asm_blocks_open_with_two_wait_states():
    seen = 0
    for path in _sources():
        for line, tpl in _asm_blocks(open(path).read()):
            if DPP.search(tpl) and not VMEM.search(tpl):
                seen += 1
                assert _leading_nop(tpl) >= 1, f"{os.path.basename(path)}:{line}: DPP asm without s_nop 1: {tpl!r}"
    assert seen >= 1  # the TQ4 encoder's and q4_0 append's DPP butterflies


def test_the_checker_sees_a_missing_preamble():
    bad = 'asm volatile("global_load_lds_dwordx4 %0, %1" :: "v"(o), "s"(b));'
    (line, tpl), = _asm_blocks(bad)
    assert VMEM.search(tpl) and _leading_nop(tpl) < 4
    good = 'asm volatile("s_nop 4\\n\\tglobal_load_lds_dword %0, %1" :: "v"(o), "s"(b));'
    (line, tpl), = _asm_blocks(good)
    assert _leading_nop(tpl) == 4
