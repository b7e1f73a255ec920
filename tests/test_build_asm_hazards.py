"""Inline assembly must declare what it overwrites (CPU only: scans the
gfx950 assembly the compiler writes for each kernel source).

The K/V descriptor size of the forward kernel is clamped with scalar
instructions in an asm statement; s_min / s_max write SCC. Without "scc" in
its clobbers the compiler once placed that statement between the two halves
of a 64-bit address add (s_add_u32 ... s_addc_u32), so the carry the second
half read was the clamp's SCC: the tile address gained 4 GiB and the GPU took
a memory fault. This test scans every kernel for an SCC read that follows an
SCC-writing asm block with no SCC write in between."""

import re

import pytest

from tiled_attention_amd import build

SCC_WRITERS = ("s_cmp", "s_min_", "s_max_", "s_add_u32", "s_sub_u32", "s_add_i32", "s_sub_i32", "s_and_",
               "s_or_", "s_xor_", "s_andn2_", "s_orn2_", "s_nand_", "s_nor_", "s_xnor_", "s_lshl", "s_lshr",
               "s_ashr", "s_bfe_", "s_not_", "s_abs_", "s_bitcmp", "s_addc_u32", "s_subb_u32", "s_absdiff")
SCC_READERS = ("s_cbranch_scc", "s_cselect_", "s_addc_u32", "s_subb_u32", "s_cmov")
BLOCK_END = re.compile(r"^(\.LBB\d+_\d+:|s_branch|s_cbranch_|s_endpgm|s_setpc)")


def scc_hazards(asm_text):
    """(function, line) of each SCC read reached from an SCC-writing inline asm
    block with no intervening SCC write, within its basic block."""
    found = []
    func = None
    lines = [l.strip() for l in asm_text.splitlines()]
    k = 0
    while k < len(lines):
        l = lines[k]
        m = re.match(r"^([A-Za-z_][\w.$]*):", l)
        if m and not l.startswith(".L"):
            func = m.group(1)
        if l == ";;#ASMSTART":
            j = k + 1
            writes = False
            while j < len(lines) and lines[j] != ";;#ASMEND":
                if lines[j].startswith(SCC_WRITERS):
                    writes = True
                j += 1
            if writes:
                for q in range(j + 1, len(lines)):
                    t = lines[q]
                    if t == ";;#ASMSTART" or not t or t.startswith((";", ".")) and not t.startswith(".LBB"):
                        continue
                    if t.startswith(SCC_READERS):
                        found.append((func, t))
                        break
                    if t.startswith(SCC_WRITERS) or BLOCK_END.match(t):
                        break
            k = j
        k += 1
    return found


def test_scanner_finds_the_hazard_it_is_for():
    bad = "\n".join(["k:", "s_add_u32 s4, s4, 0x2000", ";;#ASMSTART", "s_max_i32 s6, s7, 0", "s_min_i32 s6, s6, 9",
                     ";;#ASMEND", "s_addc_u32 s5, s5, 0"])
    good = bad.replace(";;#ASMSTART", "s_addc_u32 s5, s5, 0\n;;#ASMSTART").replace("\ns_addc_u32 s5, s5, 0", "", 1)
    assert scc_hazards(bad) == [("k", "s_addc_u32 s5, s5, 0")]
    assert scc_hazards(good.replace(";;#ASMEND\ns_addc_u32 s5, s5, 0", ";;#ASMEND")) == []


@pytest.mark.parametrize("src", [s for s in build.SOURCES if s.endswith(".hip")])
def test_no_scc_read_after_scc_writing_asm(src):
    assert scc_hazards(build.assembly(src)) == []
