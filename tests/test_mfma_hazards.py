"""Matrix-instruction operand hazards in the built library (no GPU).

The P.V and row-sum MFMAs are inline asm, which the compiler's hazard recognizer does
not see: it inserts no wait states between a vector instruction that writes a VGPR and
an inline-asm MFMA that reads it.  The CDNA3/CDNA4 ISA reference guides' table of
required independent instructions asks for two wait states there (a VALU write of a
VGPR followed by an XDL/SMFMA read of it as SrcA, SrcB, SrcC or a scale operand).  A
register copy or a rematerialised constant placed by the compiler just ahead of such
an MFMA makes it read the old register contents: rows of the output then change with
the register allocation of the kernel variant.

Results: an XDL MFMA's destination registers may be read or written by a non-matrix
instruction only after a number of wait states that grows with its passes.  The compiler
inserts, for its own builtin MFMAs on gfx950 (compiling a builtin followed by a vector
read shows it), 20 wait states after a 16-pass v_mfma(_scale)_f32_32x32x64_f8f6f4 and 12
after an 8-pass v_mfma_f32_32x32x16_bf16; after the inline-asm ones, vacc_settle's three
s_nop 7 give 24.

This test disassembles the gfx950 code objects of libattnfwd.so (llvm-objdump) and
checks, for every MFMA of every kernel, that no vector instruction within the two
wait states before it writes one of its source registers, and that no non-matrix
instruction touches its destination registers within the wait states above (s_nop N
counts N+1 wait states, any other instruction one).  The scans follow the code layout
and stop at a branch, so they see fall-through neighbours only.
"""
import os
import re
import shutil
import subprocess

import pytest

from fp8_causal_prefill_tiled_amd import build
from test_kernel_resources import _code_objects, _fatbin

VALU_TO_MFMA_WAIT_STATES = 2


def _objdump():
    for p in (shutil.which("llvm-objdump"), "/opt/rocm/llvm/bin/llvm-objdump",
              "/opt/rocm/lib/llvm/bin/llvm-objdump"):
        if p and os.path.exists(p):
            return p
    return None


def _vgprs(op):
    op = op.strip()
    m = re.fullmatch(r"v\[(\d+):(\d+)\]", op)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.fullmatch(r"v(\d+)", op)
    return {int(m.group(1))} if m else set()


def _functions(disassembly):
    """{function name: [(mnemonic, [operands])]} from llvm-objdump -d output."""
    parts = re.split(r"\n[0-9a-fA-F]+ <([^>]+)>:\n", "\n" + disassembly)
    out = {}
    for k in range(1, len(parts), 2):
        ins = []
        for line in parts[k + 1].split("\n"):
            line = line.split("//")[0].strip()
            if not line or line.endswith(":"):
                continue
            fields = line.split(None, 1)
            ins.append((fields[0], [o.strip() for o in fields[1].split(",")] if len(fields) > 1 else []))
        out[parts[k]] = ins
    return out


def _wait_states(mnemonic, ops):
    return int(ops[0], 0) + 1 if mnemonic == "s_nop" else 1


def find_hazards(functions, need=VALU_TO_MFMA_WAIT_STATES):
    """(number of MFMAs checked, [(function, writer, mfma, wait states between)])."""
    checked, bad = 0, []
    for name, ins in functions.items():
        for i, (mn, ops) in enumerate(ins):
            if not mn.startswith("v_mfma") or not ops:
                continue
            checked += 1
            srcs = set().union(*(_vgprs(o) for o in ops[1:]))
            w, j = 0, i - 1
            while j >= 0 and w < need:
                m2, o2 = ins[j]
                if m2.startswith(("s_branch", "s_cbranch", "s_setpc", "s_endpgm")):
                    break
                if m2.startswith("v_") and not m2.startswith("v_mfma") and o2 and _vgprs(o2[0]) & srcs:
                    bad.append((name, f"{m2} {', '.join(o2)}", f"{mn} {', '.join(ops)}", w))
                    break
                w += _wait_states(m2, o2)
                j -= 1
    return checked, bad


RESULT_WAIT_STATES = {"v_mfma_scale_f32_32x32x64_f8f6f4": 20, "v_mfma_f32_32x32x64_f8f6f4": 20,
                      "v_mfma_f32_32x32x16_bf16": 12}


def find_result_hazards(functions):
    """(number of MFMAs checked, [(function, mfma, toucher, wait states between)])."""
    checked, bad = 0, []
    for name, ins in functions.items():
        for i, (mn, ops) in enumerate(ins):
            need = RESULT_WAIT_STATES.get(mn)
            if need is None or not ops:
                continue
            checked += 1
            dst = _vgprs(ops[0])
            w, j = 0, i + 1
            while j < len(ins) and w < need:
                m2, o2 = ins[j]
                if m2.startswith(("s_branch", "s_cbranch", "s_setpc", "s_endpgm")):
                    break
                if not m2.startswith(("v_mfma", "s_")) and set().union(set(), *(_vgprs(o) for o in o2)) & dst:
                    bad.append((name, f"{mn} {', '.join(ops)}", f"{m2} {', '.join(o2)}", w))
                    break
                w += _wait_states(m2, o2)
                j += 1
    return checked, bad


def test_checker_flags_a_planted_hazard():
    # the checker itself: a vector move into an A-operand register right ahead of the MFMA
    # is flagged; the same move two wait states earlier (s_nop 1) is not
    dis = """
0000000000001000 <k>:
	v_mov_b64_e32 v[96:97], s[4:5]                             // 000000001000: 00000000
	v_mfma_scale_f32_32x32x64_f8f6f4 v[16:31], v[96:103], v[80:87], v[16:31], v188, v146 // 000000001004: 00000000
	v_mov_b64_e32 v[96:97], s[4:5]                             // 000000001010: 00000000
	s_nop 1                                                    // 000000001014: 00000000
	v_mfma_scale_f32_32x32x64_f8f6f4 v[16:31], v[96:103], v[80:87], v[16:31], v188, v146 // 000000001018: 00000000
	v_add_u32_e32 v146, 1, v146                                // 000000001020: 00000000
	v_mfma_scale_f32_32x32x64_f8f6f4 v[16:31], v[96:103], v[80:87], v[16:31], v188, v146 // 000000001024: 00000000
"""
    checked, bad = find_hazards(_functions(dis))
    assert checked == 3
    assert [b[3] for b in bad] == [0, 0]            # the first and the third (scale operand)
    assert "v[96:97]" in bad[0][1] and "v146" in bad[1][1]
    # a result read 19 wait states after a 16-pass MFMA is flagged, 20 is not
    dis2 = """
0000000000002000 <k2>:
	v_mfma_f32_32x32x64_f8f6f4 v[2:17], v[18:25], v[26:33], 0 // 000000002000: 00000000
	s_nop 15                                                   // 000000002008: 00000000
	s_nop 2                                                    // 00000000200c: 00000000
	v_add_f32_e32 v1, v2, v7                                   // 000000002010: 00000000
	v_mfma_f32_32x32x64_f8f6f4 v[2:17], v[18:25], v[26:33], 0 // 000000002014: 00000000
	s_nop 15                                                   // 00000000201c: 00000000
	s_nop 3                                                    // 000000002020: 00000000
	v_add_f32_e32 v1, v2, v7                                   // 000000002024: 00000000
"""
    checked, bad = find_result_hazards(_functions(dis2))
    assert checked == 2 and len(bad) == 1 and bad[0][3] == 19


def test_no_vector_write_just_ahead_of_an_mfma(tmp_path):
    if not os.path.exists(build.LIB):
        pytest.skip("libattnfwd.so is not built")
    objdump = _objdump()
    if objdump is None:
        pytest.skip("llvm-objdump not found")
    functions = {}
    for i, co in enumerate(_code_objects(_fatbin(build.LIB))):
        path = tmp_path / f"co{i}.elf"
        path.write_bytes(co)
        dis = subprocess.run([objdump, "-d", "--no-show-raw-insn", "--mcpu=gfx950", str(path)],
                             capture_output=True, text=True, check=True).stdout
        functions.update(_functions(dis))
    checked, bad = find_hazards(functions)
    assert checked > 1000, checked                  # every attention kernel's MFMAs were seen
    assert not bad, bad[:5]
    checked, bad = find_result_hazards(functions)
    assert checked > 1000, checked
    assert not bad, bad[:5]
