"""Host-side check of the inline-asm contract of the GEMM main loop (no GPU needed).

The slice blocks in gemm_slice_asm.inc are pasted into asm statements in gemm.hip.  The
compiler trusts what those statements declare, so a register that a block writes without
declaring it can silently hold a value of the compiler's (a wrong result that depends on
register allocation, not a fault).  Checked here, for every asm statement of gemm.hip that
uses a slice or tail macro:
  - every VGPR the block writes is one of the statement's outputs or declared clobbers;
  - a block with scalar ALU instructions (they set SCC) declares "scc";
  - a block that writes M0 declares "m0".
"""
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "blockwise_scaled_fp8_quant_amd", "csrc")

# instructions that leave their first operand untouched (stores, copies into LDS, waits)
NO_VGPR_DEST = ("global_load_lds", "global_store", "ds_write", "s_", "buffer_store")
SCC_WRITERS = re.compile(r"^(s_add_|s_sub_|s_cmp|s_and_|s_or_|s_xor_|s_andn2|s_orn2|s_lshl|s_lshr|s_ashr|s_bfe|"
                         r"s_min_|s_max_|s_abs|s_not_|s_mul_hi|s_addk|s_bcnt|s_bitcmp)")


def macros():
    text = open(os.path.join(CSRC, "gemm_slice_asm.inc")).read()
    out = {}
    for m in re.finditer(r"#define (PURO_SLICE_ASM_\w+) \\\n((?:.*\\\n)*.*)", text):
        out[m.group(1)] = [ln.strip() for ln in re.findall(r'"([^"]*)\\n\\t"', m.group(2))]
    for m in re.finditer(r"#define (PURO_SLICE_ASM_\w*CLOBBERS) (.*)", text):
        out[m.group(1)] = re.findall(r'"([^"]*)"', m.group(2))
    return out


def regs(spec):
    """Register numbers named by a v[a:b] or vN operand (a string)."""
    m = re.fullmatch(r"v\[(\d+):(\d+)\]", spec)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.fullmatch(r"v(\d+)", spec)
    return {int(m.group(1))} if m else set()


def written_vgprs(lines):
    out = set()
    for ln in lines:
        parts = ln.replace(",", " ").split()
        if not parts or parts[0].startswith(NO_VGPR_DEST):
            continue
        out |= regs(parts[1]) if len(parts) > 1 else set()
    return out


def asm_statements():
    """(macro name, statement text) for every asm volatile(PURO_SLICE_ASM_...) in gemm.hip."""
    src = open(os.path.join(CSRC, "gemm.hip")).read()
    out = []
    for m in re.finditer(r"asm volatile\((PURO_SLICE_ASM_\w+)", src):
        depth, i = 1, m.end()
        while depth:
            depth += {"(": 1, ")": -1}.get(src[i], 0)
            i += 1
        out.append((m.group(1), src[m.start():i]))
    return out


def declared(stmt, mac):
    """VGPRs named by the statement's operand constraints and clobbers (clobber macros expanded)."""
    got = set()
    for a, b in re.findall(r'\{v\[(\d+):(\d+)\]\}', stmt):
        got |= set(range(int(a), int(b) + 1))
    for name in re.findall(r"(PURO_SLICE_ASM_\w*CLOBBERS)", stmt):
        for item in mac[name]:
            got |= regs(item)
    return got


STATEMENTS = asm_statements()


def test_every_slice_block_is_used():
    used = {name for name, _ in STATEMENTS}
    mac = macros()
    blocks = {n for n in mac if not n.endswith("CLOBBERS")}
    assert blocks == used, f"blocks without an asm statement or vice versa: {blocks ^ used}"


@pytest.mark.parametrize("name,stmt", STATEMENTS, ids=[n for n, _ in STATEMENTS])
def test_block_declares_what_it_writes(name, stmt):
    mac = macros()
    lines = mac[name]
    missing = written_vgprs(lines) - declared(stmt, mac)
    assert not missing, f"{name} writes VGPRs it does not declare: {sorted(missing)}"
    ops = [ln.split()[0] for ln in lines if ln.split()]
    if any(SCC_WRITERS.match(op) for op in ops):
        assert '"scc"' in stmt, f"{name} sets SCC (scalar ALU) but does not declare \"scc\""
    if any(ln.replace(",", " ").split()[1:2] == ["m0"] for ln in lines if ln.split()):
        assert '"m0"' in stmt, f"{name} writes M0 but does not declare \"m0\""
