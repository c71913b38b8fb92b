"""The gate's FMAs read their weight operand through DPP (a row broadcast)
written as inline asm, which the compiler's hazard checker does not look
inside. gfx950 needs two wait states between a VALU write of a VGPR and a
DPP read of it. This test disassembles the gfx950 code objects of the built
library (LLVM's own tools, on code built here) and checks every DPP
instruction against that rule, treating branch targets as unknown history."""

import os
import re
import struct
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "mixture_experts_routing_gemm_amd", "libmoe_mi355x.so")
LLVM = os.environ.get("ROCM_LLVM_BIN", "/opt/rocm/llvm/bin")
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"

_REG = re.compile(r"^v(?:(\d+)|\[(\d+):(\d+)\])$")
_SYM = re.compile(r"^([0-9a-f]+) <(.+)>:$")
_INS = re.compile(r"^\s+(\S+)\s*(.*?)\s*//\s*([0-9A-Fa-f]+):[^<]*(?:<(.+)\+0x([0-9a-f]+)>)?\s*$")


def vgprs(operand):
    """VGPR numbers named by an operand such as v7 or v[4:7] (empty if none)."""
    m = _REG.match(operand.strip())
    if not m:
        return set()
    if m.group(1) is not None:
        return {int(m.group(1))}
    return set(range(int(m.group(2)), int(m.group(3)) + 1))


def parse(disasm):
    """[(address, mnemonic, operands)] and the set of branch-target addresses."""
    syms, ins, targets = {}, [], set()
    for line in disasm.splitlines():
        m = _SYM.match(line.strip())
        if m:
            syms[m.group(2)] = int(m.group(1), 16)
            targets.add(int(m.group(1), 16))
            continue
        m = _INS.match(line)
        if not m:
            continue
        ops = [o.strip() for o in m.group(2).split(",")] if m.group(2) else []
        ins.append((int(m.group(3), 16), m.group(1), ops))
        if m.group(4) is not None:
            targets.add((m.group(4), int(m.group(5), 16)))
    resolved = set()
    for t in targets:
        resolved.add(syms[t[0]] + t[1] if isinstance(t, tuple) else t)
    return ins, resolved


def dpp_hazards(ins, targets):
    """DPP reads of a VGPR written by VALU within the two wait states before
    (an instruction that is a branch target ends the look-back: flagged)."""
    bad = []
    for i, (addr, mn, ops) in enumerate(ins):
        if "_dpp" not in mn or len(ops) < 2:
            continue
        src = vgprs(ops[1].split()[0])
        states, j = 0, i
        while states < 2:
            if ins[j][0] in targets or j == 0:
                bad.append((hex(addr), mn, "branch target within two wait states"))
                break
            j -= 1
            pmn, pops = ins[j][1], ins[j][2]
            if pmn == "s_nop":
                states += (int(pops[0], 0) if pops else 0) + 1
                continue
            if pmn.startswith("v_") and pops and vgprs(pops[0]) & src:
                bad.append((hex(addr), mn, f"{pmn} {pops[0]}, {2 - states} wait state(s) before"))
                break
            states += 1
    return bad


def gfx950_objects(lib):
    """The gfx950 code objects of every offload bundle in the library."""
    with tempfile.TemporaryDirectory() as tmp:
        fat = os.path.join(tmp, "fat.bin")
        subprocess.run([os.path.join(LLVM, "llvm-objcopy"), "--dump-section",
                        f".hip_fatbin={fat}", lib], check=True, capture_output=True)
        data = open(fat, "rb").read()
    objs = []
    for m in re.finditer(re.escape(MAGIC), data):
        st = m.start()
        off = st + len(MAGIC)
        (n,) = struct.unpack_from("<Q", data, off)
        off += 8
        for _ in range(n):
            eo, es, ts = struct.unpack_from("<QQQ", data, off)
            off += 24
            triple = data[off:off + ts].decode()
            off += ts
            if triple.endswith("gfx950"):
                objs.append(data[st + eo:st + eo + es])
    return objs


def disassemble(obj):
    with tempfile.TemporaryDirectory() as tmp:
        path = os.path.join(tmp, "co.o")
        open(path, "wb").write(obj)
        res = subprocess.run([os.path.join(LLVM, "llvm-objdump"), "-d", "--mcpu=gfx950", path],
                             check=True, capture_output=True, text=True)
    return res.stdout


PLANTED = """0000000000001000 <k>:
	v_lshlrev_b32_e32 v15, 16, v18                             // 000000001000: 00000000
	v_add_u32_e32 v9, v1, v2                                   // 000000001004: 00000000
	v_fmac_f32_dpp v14, v15, v10 row_newbcast:0 row_mask:0xf bank_mask:0xf// 000000001008: 00000000 00000000
	v_mov_b64_e32 v[20:21], v[2:3]                             // 000000001010: 00000000
	s_nop 1                                                    // 000000001014: 00000000
	v_fmac_f32_dpp v14, v21, v10 row_newbcast:1 row_mask:0xf bank_mask:0xf// 000000001018: 00000000 00000000
	s_cbranch_scc1 1                                           // 000000001020: 00000000 <k+0x28>
	v_add_u32_e32 v9, v1, v2                                   // 000000001024: 00000000
	v_fmac_f32_dpp v14, v30, v10 row_newbcast:2 row_mask:0xf bank_mask:0xf// 000000001028: 00000000 00000000
"""


def test_checker_finds_planted_hazards():
    ins, targets = parse(PLANTED)
    bad = dpp_hazards(ins, targets)
    # the first DPP reads v15 one wait state after its write; the second is
    # spaced by s_nop 1; the third is a branch target
    assert [b[0] for b in bad] == ["0x1008", "0x1028"]


@pytest.mark.skipif(not os.path.exists(LIB), reason="library not built")
def test_built_gate_code_has_no_dpp_read_hazard():
    objs = gfx950_objects(LIB)
    assert objs
    n_dpp, bad = 0, []
    for obj in objs:
        ins, targets = parse(disassemble(obj))
        n_dpp += sum("_dpp" in mn for _, mn, _ in ins)
        bad += dpp_hazards(ins, targets)
    assert n_dpp > 1000  # the row-broadcast gate kernels are in the build
    assert bad == [], bad[:10]
