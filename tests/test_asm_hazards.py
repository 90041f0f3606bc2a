"""Checks on the gfx950 assembly of the kernels (CPU only: hipcc cross-compiles).

The streamed tile loads are inline assembly (``global_load_lds_dwordx4``), which the
compiler does not know to be a vector memory instruction, so it inserts none of the
wait states such an instruction needs before it:
  * 5 after a vector-ALU instruction that writes an SGPR the load reads (its scalar
    base); the compiler writes SGPRs from the vector ALU when it reloads spilled
    scalars (``v_readlane``) or moves a uniform value (``v_readfirstlane``);
  * 1 after a write of M0, which holds the load's LDS address.
The assembly supplies them itself (``s_nop 4``).  These tests compile the kernels
with the library's own flags and check every such load in program order, and that
no kernel spills registers to scratch memory.
"""
import os
import re
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from causal_attention_fa_amd import build as B

KERNEL_SOURCES = ["fa_fwd.hip", "fa_bwd.hip", "fa_decode.hip"]
VMEM_SGPR_WAIT = 5
M0_WAIT = 1

_INSTR = re.compile(r"^\s+([a-z_0-9]+)(.*)$")
_SREG = re.compile(r"\bs\[(\d+):(\d+)\]|\bs(\d+)\b")


def _sgprs(text):
    """The SGPR numbers an operand string names."""
    out = set()
    for m in _SREG.finditer(text):
        if m.group(3) is not None:
            out.add(int(m.group(3)))
        else:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return out


def _instructions(asm):
    """(opcode, operands) in program order; labels and branches appear as None."""
    out = []
    for line in asm.splitlines():
        s = line.split(";", 1)[0].rstrip()
        if not s:
            continue
        if not s[0].isspace():
            out.append(None)  # a label: other paths join here
            continue
        m = _INSTR.match(s)
        if m is None or m.group(1).startswith("."):
            continue
        op, args = m.group(1), m.group(2).strip()
        out.append((op, args))
        if op.startswith("s_cbranch") or op == "s_branch":
            out.append(None)
    return out


def _wait_states(op, args):
    if op == "s_nop":
        return int(args, 0) + 1
    return 1


def hazards(asm):
    """Direct loads whose scalar base or M0 was written too few wait states before.
    Returns a list of (index, reason).  Walks back in program order within a basic
    block (a label or branch ends the walk: the loads this guards are straight-line
    sequences of assembly statements)."""
    ins = _instructions(asm)
    found = []
    for i, x in enumerate(ins):
        if x is None or x[0] != "global_load_lds_dwordx4":
            continue
        operands = [a.strip() for a in x[1].split(",")]
        base = _sgprs(operands[1]) if len(operands) > 1 and operands[1] != "off" else set()
        waited = 0
        j = i - 1
        while j >= 0 and ins[j] is not None and waited < VMEM_SGPR_WAIT:
            op, args = ins[j]
            dst = args.split(",", 1)[0]
            if op.startswith("v_") and base & _sgprs(dst):
                found.append((i, f"{op} writes the base {dst} {waited} wait states before the load"))
            if dst.strip() == "m0" and waited < M0_WAIT:
                found.append((i, f"{op} writes M0 {waited} wait states before the load"))
            waited += _wait_states(op, args)
            j -= 1
    return found


def test_hazard_check_finds_planted_hazards():
    """The checker itself, on hand-written sequences: a v_readlane of the base two
    instructions before the load, and an M0 write right before it, are reported; the
    same with s_nop 4 in between is not."""
    bad = """
\tv_readlane_b32 s5, v255, 8
\ts_add_i32 m0, s82, 0x1000
\tglobal_load_lds_dwordx4 v217, s[4:5]
"""
    good = """
\tv_readlane_b32 s5, v255, 8
\ts_add_i32 m0, s82, 0x1000
\ts_nop 4
\tglobal_load_lds_dwordx4 v217, s[4:5]
"""
    reasons = [r for _, r in hazards(bad)]
    assert any("v_readlane_b32 writes the base s5" in r for r in reasons), reasons
    assert any("writes M0 0 wait states" in r for r in reasons), reasons
    assert hazards(good) == []
    # a register the load does not read is no hazard
    assert hazards("\tv_readfirstlane_b32 s9, v1\n\tglobal_load_lds_dwordx4 v2, s[4:5]\n") == []


@pytest.fixture(scope="module")
def kernel_asm():
    """gfx950 device assembly of every kernel source, compiled with the library's flags."""
    flags = [f for f in B.HIP_FLAGS if f != "-fPIC"]
    tmp = tempfile.mkdtemp(prefix="fa_asm_")

    def one(src):
        out = os.path.join(tmp, src + ".s")
        cmd = [B.hipcc()] + flags + ["-x", "hip", "--cuda-device-only", "-S", os.path.join(B.CSRC, src), "-o", out]
        subprocess.run(cmd, check=True, stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
        with open(out) as f:
            return src, f.read()

    with ThreadPoolExecutor(max_workers=len(KERNEL_SOURCES)) as ex:
        return dict(ex.map(one, KERNEL_SOURCES))


@pytest.mark.parametrize("src", KERNEL_SOURCES)
def test_direct_loads_have_their_wait_states(kernel_asm, src):
    asm = kernel_asm[src]
    n = asm.count("global_load_lds_dwordx4")
    assert n > 0, "no direct loads found: the check would prove nothing"
    found = hazards(asm)
    assert not found, f"{src}: {len(found)} loads without their wait states, e.g. {found[:3]}"


@pytest.mark.parametrize("src", KERNEL_SOURCES)
def test_no_kernel_spills(kernel_asm, src):
    sizes = re.findall(r"\.amdhsa_kernel (\S+)[\s\S]*?\.amdhsa_private_segment_fixed_size (\d+)", kernel_asm[src])
    assert sizes, "no kernel descriptors found"
    spilling = [(k, int(n)) for k, n in sizes if int(n) != 0]
    assert not spilling, f"{src}: kernels using scratch memory: {spilling[:3]}"


def _two_wave_kernels(asm):
    """(name, registers) of the 16-bit gradient kernels meant to run two waves per
    SIMD: every dQ and dK/dV instance except the dK/dV read-ahead form, which runs
    one wave per SIMD by design.  `.amdhsa_next_free_vgpr` counts the vector and
    accumulation registers together; above 256 a SIMD holds only one such wave."""
    out = []
    for name, n in re.findall(r"\.amdhsa_kernel (\S+)[\s\S]*?\.amdhsa_next_free_vgpr (\d+)", asm):
        if not ("DF16_" in name or "DF16b" in name):
            continue
        if "dq_kernel" in name:
            out.append((name, int(n)))
        elif "dkdv_kernel" in name:
            flags = re.findall(r"ELb([01])", name)
            if len(flags) == 4 and flags[3] == "0":
                out.append((name, int(n)))
    return out


def test_two_wave_gradient_kernels_fit_256_registers(kernel_asm):
    found = _two_wave_kernels(kernel_asm["fa_bwd.hip"])
    assert len(found) >= 40, f"only {len(found)} gradient kernels found: the check would prove little"
    over = [(k, n) for k, n in found if n > 256]
    assert not over, f"kernels past 256 registers (one wave per SIMD): {over[:3]}"
