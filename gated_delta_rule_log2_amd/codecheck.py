"""Static check of the built gfx950 kernels: spill slots written under a narrower exec mask
than the one they are read back under.

The compiler can place the stores of VGPR spills at the head of the block that joins a
divergent region (a branch on a lane condition, or the exit of a loop whose trip count
differs between lanes), before the instruction that restores the exec mask
(``s_or_b64 exec, exec, s[..]``).  Lanes that were inactive in the region, which at a
loop exit is every lane, then never write their spill slot, and a reload after the join,
under the full mask, returns whatever the scratch memory held.  A per-chunk backward
kernel built that way reloaded a 64-bit address from such a slot and ended in a memory
aperture fault.

The scan disassembles every gfx950 code object in the library (the ``.hip_fatbin``
section holds one offload bundle per translation unit) and looks for that placement: a
scratch store at the head of a branch-target block, before the block's exec restore, of
a register the block has not written (see `scan`).  It is a pattern match on the
listing, not a control-flow analysis: a guard against this one compiler behaviour, not a
proof that every spill is correct.

    python -m gated_delta_rule_log2_amd.codecheck [library]
"""
from __future__ import annotations

import os
import re
import struct
import subprocess
import sys
import tempfile

LLVM_BIN = os.environ.get("KDA_LLVM_BIN", "/opt/rocm/llvm/bin")
_MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"

_FUNC = re.compile(r"^[0-9a-f]+ <([^>]+)>:$")


def code_objects(library: str, arch: str = "gfx950") -> list[bytes]:
    """The device code objects for `arch` inside `library`'s offload bundles."""
    with tempfile.TemporaryDirectory() as tmp:
        sec = os.path.join(tmp, "fatbin")
        out = os.path.join(tmp, "lib")
        subprocess.run([os.path.join(LLVM_BIN, "llvm-objcopy"), f"--dump-section=.hip_fatbin={sec}", library, out],
                       check=True, capture_output=True)
        with open(sec, "rb") as f:
            data = f.read()
    objs = []
    pos = data.find(_MAGIC)
    while pos >= 0:
        (entries,) = struct.unpack_from("<Q", data, pos + len(_MAGIC))
        p = pos + len(_MAGIC) + 8
        for _ in range(entries):
            off, size, tlen = struct.unpack_from("<QQQ", data, p)
            p += 24
            triple = data[p:p + tlen].decode()
            p += tlen
            if triple.endswith(arch):
                objs.append(data[pos + off:pos + off + size])
        pos = data.find(_MAGIC, pos + 1)
    return objs


def disassemble(code_object: bytes) -> str:
    with tempfile.NamedTemporaryFile(suffix=".elf") as f:
        f.write(code_object)
        f.flush()
        r = subprocess.run([os.path.join(LLVM_BIN, "llvm-objdump"), "-d", "--no-show-raw-insn", f.name],
                           check=True, capture_output=True, text=True)
    return r.stdout


_ADDR = re.compile(r"//\s*([0-9A-Fa-f]+):")
_BRANCH = re.compile(r"s_(cbranch_\w+|branch)\s+(\d+)$")


def _regs(operand: str) -> set[str]:
    """The 32-bit VGPR/AGPR names an operand covers ('v[4:5]' -> {'v4', 'v5'})."""
    m = re.fullmatch(r"([av])\[(\d+):(\d+)\]", operand)
    if m:
        return {f"{m.group(1)}{i}" for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    return {operand} if re.fullmatch(r"[av]\d+", operand) else set()


def _kernels(asm: str) -> list[tuple[str, list[tuple[int, str]]]]:
    """(symbol, [(address, instruction text)]) per function of an llvm-objdump listing."""
    out = []
    for line in asm.splitlines():
        m = _FUNC.match(line.strip())
        if m:
            out.append((m.group(1), []))
            continue
        ins = line.split("//")[0].strip()
        a = _ADDR.search(line)
        if out and ins and a:
            out[-1][1].append((int(a.group(1), 16), ins))
    return out


def scan(asm: str) -> list[str]:
    """Spill stores at the head of a join block, before its exec restore.

    For every `s_or_b64 exec, exec, s[..]` the straight-line run before it is walked back
    to the start of its block (a branch target; the walk stops at a branch or another
    write of exec, which mark a fall-through from inside the region).  A scratch store in
    that run whose source register is not written earlier in the run stores a value that
    was live into the join, under the mask of the region being left; those are reported."""
    findings = []
    for name, insts in _kernels(asm):
        targets = set()
        for addr, ins in insts:
            m = _BRANCH.match(ins)
            if m:
                off = int(m.group(2))
                off = off - 65536 if off >= 32768 else off
                targets.add(addr + 4 + 4 * off)
        for k, (addr, ins) in enumerate(insts):
            if not ins.startswith("s_or_b64 exec, exec,"):
                continue
            for j in range(k - 1, -1, -1):
                a2, i2 = insts[j]
                dst = i2.split(" ", 1)[1].split(",")[0].strip() if " " in i2 else ""
                if re.match(r"s_(cbranch|branch|setpc)", i2) or dst == "exec":
                    break
                if a2 in targets:
                    written: set[str] = set()
                    for a3, i3 in insts[j:k]:
                        if i3.startswith("scratch_store"):
                            src = i3.split(",")[1].strip()
                            if not (_regs(src) & written):
                                findings.append(f"{name}: `{i3}` at 0x{a3:x}, head of the join block at "
                                                f"0x{a2:x}, before the exec restore at 0x{addr:x}")
                        elif not i3.startswith(("s_", "global_store", "ds_write", "buffer_store")):
                            d3 = i3.split(" ", 1)[1].split(",")[0].strip() if " " in i3 else ""
                            written |= _regs(d3)
                    break
    return findings


def check_library(library: str) -> list[str]:
    findings = []
    for obj in code_objects(library):
        findings += scan(disassemble(obj))
    return findings


def main(argv: list[str]) -> int:
    here = os.path.dirname(os.path.abspath(__file__))
    library = argv[1] if len(argv) > 1 else os.path.join(here, "libkda.so")
    findings = check_library(library)
    for f in findings:
        print(f)
    print(f"{len(findings)} finding(s) in {library}")
    return 1 if findings else 0


if __name__ == "__main__":
    sys.exit(main(sys.argv))
