"""Inline assembly must declare what it overwrites (CPU only: scans the
gfx950 assembly the compiler writes for each kernel source).

The K/V descriptor size of the forward kernel is clamped with scalar
instructions in an asm statement; s_min / s_max write SCC. Without "scc" in
its clobbers the compiler once placed that statement between the two halves
of a 64-bit address add (s_add_u32 ... s_addc_u32), so the carry the second
half read was the clamp's SCC: the tile address gained 4 GiB and the GPU took
a memory fault. This test scans every kernel for an SCC read that follows an
SCC-writing asm block with no SCC write in between."""

import functools
import re

import pytest

from tiled_attention_amd import build


@functools.lru_cache(maxsize=None)
def _assembly(src):
    # one compile per source for all the scans of this module
    return build.assembly(src)

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
    assert scc_hazards(_assembly(src)) == []


# The Q tile is loaded with inline-asm global loads that the compiler does not
# track, so the K/V DMAs can stream behind them; the compiler takes the
# destination registers as written when the asm statement ends. Until the
# inline-asm vmcnt wait that follows, no instruction may read those registers
# (a copy would take the value before the data lands) or write them (the load
# would later overwrite that value).
def _vregs(text):
    out = set()
    for m in re.finditer(r"\bv\[(\d+):(\d+)\]", text):
        out |= set(range(int(m.group(1)), int(m.group(2)) + 1))
    for m in re.finditer(r"\bv(\d+)\b", text):
        out.add(int(m.group(1)))
    return out


def _functions(asm_text):
    """{name: [(instruction, inside an asm block)]} with labels kept as
    instructions of their own ("LABEL:name")."""
    funcs, cur, in_asm = {}, None, False
    for raw in asm_text.splitlines():
        t = raw.strip()
        if t == ";;#ASMSTART":
            in_asm = True
            continue
        if t == ";;#ASMEND":
            in_asm = False
            continue
        t = t.split(";")[0].strip()
        if not t:
            continue
        m = re.match(r"^([A-Za-z_.$][\w.$]*):$", t)
        if m:
            if not t.startswith(".L"):
                cur = funcs.setdefault(m.group(1), [])
            elif cur is not None:
                cur.append(("LABEL:" + m.group(1), False))
            continue
        if cur is not None and not t.startswith("."):
            cur.append((t, in_asm))
    return funcs


def asm_load_hazards(asm_text):
    """(function, instruction) of each instruction that touches the
    destination registers of an inline-asm global load on some path from the
    load to the next inline-asm vmcnt wait (branches followed both ways)."""
    found = []
    for func, ins in _functions(asm_text).items():
        labels = {t[6:]: k for k, (t, _) in enumerate(ins) if t.startswith("LABEL:")}
        for k0, (t0, a0) in enumerate(ins):
            if not (a0 and t0.startswith("global_load")):
                continue
            dst = _vregs(t0.split(None, 1)[1].split(",")[0])
            seen, todo = set(), [k0 + 1]
            while todo:
                k = todo.pop()
                if k >= len(ins) or k in seen:
                    continue
                seen.add(k)
                t, in_asm = ins[k]
                if t.startswith("LABEL:"):
                    todo.append(k + 1)
                    continue
                op = t.split(None, 1)
                args = op[1] if len(op) > 1 else ""
                if in_asm and op[0].startswith("s_waitcnt") and "vmcnt" in args:
                    continue
                if _vregs(args) & dst and not (in_asm and op[0].startswith("global_load") and
                                                  _vregs(args.split(",")[0]) == dst and
                                                  not _vregs(",".join(args.split(",")[1:])) & dst):
                    found.append((func, t))
                if op[0] in ("s_endpgm", "s_setpc_b64"):
                    continue
                if op[0].startswith("s_branch") or op[0].startswith("s_cbranch"):
                    tgt = args.strip()
                    if tgt in labels:
                        todo.append(labels[tgt])
                    if op[0].startswith("s_branch"):
                        continue
                todo.append(k + 1)
    return found


def test_load_scanner_finds_a_copy_before_the_wait():
    load = [";;#ASMSTART", "global_load_dwordx4 v[8:11], v[2:3], off", ";;#ASMEND"]
    wait = [";;#ASMSTART", "s_waitcnt vmcnt(3)", "s_barrier", ";;#ASMEND"]
    ok = "\n".join(["k:"] + load + ["v_add_u32_e32 v2, 32, v2"] + wait + ["v_mov_b32_e32 v20, v9"])
    assert asm_load_hazards(ok) == []
    bad = "\n".join(["k:"] + load + ["v_mov_b32_e32 v20, v9"] + wait)
    assert asm_load_hazards(bad) == [("k", "v_mov_b32_e32 v20, v9")]
    bad = "\n".join(["k:"] + load + ["v_mov_b32_e32 v10, 0"] + wait)
    assert asm_load_hazards(bad) == [("k", "v_mov_b32_e32 v10, 0")]


def test_q_registers_untouched_until_their_wait():
    assert asm_load_hazards(_assembly("fwd_mfma.hip")) == []
