"""The build's scan for spill stores placed under a narrowed exec mask at a join block
(gated_delta_rule_log2_amd/codecheck.py): hand-made listings with and without the
placement, and the built library itself."""
import os
import shutil

import pytest

from gated_delta_rule_log2_amd import codecheck

LIB = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "gated_delta_rule_log2_amd",
                   "libkda.so")


def listing(body):
    """An llvm-objdump style listing of one kernel, every instruction 4 bytes from 0x1000;
    'B<label>' in a branch is replaced by the word offset to the line tagged '<label>:'."""
    index, out, addr = {}, [], 0x1000
    for text in body:
        if text.endswith(":"):
            index[text[:-1]] = addr
        else:
            addr += 4
    addr = 0x1000
    for text in body:
        if text.endswith(":"):
            continue
        for tag, target in index.items():
            if f"B{tag}" in text:
                off = (target - (addr + 4)) // 4
                text = text.replace(f"B{tag}", str(off & 0xFFFF))
        out.append(f"\t{text}  // {addr:012X}: 00000000")
        addr += 4
    return "0000000000001000 <kern>:\n" + "\n".join(out) + "\n"


REGION = ["v_cmp_gt_u32_e64 s[96:97], 0x80, v0", "s_and_saveexec_b64 s[2:3], s[96:97]", "s_cbranch_execz Bjoin",
          "v_add_u32_e32 v1, 1, v1"]


def test_flags_live_in_spill_at_join_head():
    asm = listing(REGION + ["join:", "scratch_store_dwordx2 off, v[146:147], off offset:40",
                            "s_or_b64 exec, exec, s[2:3]", "scratch_load_dwordx2 v[8:9], off, off offset:40"])
    found = codecheck.scan(asm)
    assert len(found) == 1 and "offset:40" in found[0]


def test_flags_loop_exit_join():
    asm = listing(["v_cmp_gt_u32_e64 s[96:97], 0x80, v0", "s_and_saveexec_b64 s[2:3], s[96:97]",
                   "s_cbranch_execz Bexit", "loop:", "v_add_u32_e32 v9, 64, v9", "s_andn2_b64 exec, exec, s[4:5]",
                   "s_cbranch_execnz Bloop", "exit:", "scratch_store_dword off, v98, off",
                   "s_or_b64 exec, exec, s[2:3]"])
    assert len(codecheck.scan(asm)) == 1


def test_ignores_value_written_in_the_join_block():
    # a spill slot updated in the region's lanes only: read, modified and written back
    asm = listing(REGION + ["join:", "scratch_load_dwordx4 v[2:5], off, off", "global_load_dword v5, v[0:1], off",
                            "scratch_store_dwordx4 off, v[2:5], off", "s_or_b64 exec, exec, s[2:3]"])
    assert codecheck.scan(asm) == []


def test_ignores_spill_after_the_restore_and_inside_the_region():
    asm = listing(REGION + ["scratch_store_dword off, v1, off offset:8", "join:", "s_or_b64 exec, exec, s[2:3]",
                            "scratch_store_dword off, v98, off"])
    assert codecheck.scan(asm) == []


@pytest.mark.skipif(not os.path.exists(LIB), reason="library not built")
@pytest.mark.skipif(not shutil.which(os.path.join(codecheck.LLVM_BIN, "llvm-objdump")), reason="no llvm-objdump")
def test_built_library_has_no_misplaced_spills():
    assert codecheck.check_library(LIB) == []
