"""Host-side checks of the four-wave GEMM's K loop (gemm_w4_asm.inc), no GPU needed.

The loop is one inline-asm statement whose text comes from gen_w4_asm.py.  The compiler trusts what
the statement declares and inserts no waits or hazard padding inside it, so the properties it relies
on are checked here on the generated text itself, by replaying the statement's control flow for
1 .. 6 slices (every path: the paired loop, the one- and two-slice remainders) as a straight
instruction trace:
  - the committed text is what the generator writes;
  - a VALU read of an MFMA result comes at least 12 wait states after the MFMA (the gfx950 figure
    for v_mfma_f32_16x16x128_f8f6f4) and an LDS-DMA load at least one after an SALU write of M0;
  - no register an LDS read writes is read or rewritten before an lgkmcnt wait covers that read
    (LDS reads complete in order);
  - at every s_barrier the only loads still in flight are the L2 prefetches (which land in an LDS
    area nothing reads): the copies of the stage the next slice multiplies have landed;
  - every register the statement writes is one of its outputs or declared clobbers (VGPRs, AGPRs,
    SGPR operands), and SCC and M0 are declared.
"""
import importlib.util
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "blockwise_scaled_fp8_quant_amd", "csrc")
INC = os.path.join(CSRC, "gemm_w4_asm.inc")
MFMA_VALU_WAIT = 12
PF_LDS = "135168"


def load_generator():
    spec = importlib.util.spec_from_file_location("gen_w4_asm", os.path.join(CSRC, "gen_w4_asm.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def mainloop(text=None):
    text = text if text is not None else open(INC).read()
    m = re.search(r"#define PURO_W4_MAINLOOP \\\n((?:.*\\\n)*.*)", text)
    return [ln.strip() for ln in re.findall(r'"([^"]*)\\n\\t"', m.group(1))]


def clobber_agprs(text=None):
    text = text if text is not None else open(INC).read()
    m = re.search(r"#define PURO_W4_CLOBBERS (.*)", text)
    return {int(x) for x in re.findall(r'"a(\d+)"', m.group(1))}


def trace(lines, pairs, rem):
    """The instructions executed for `pairs` loop iterations and `rem` remaining slices."""
    labels = {ln[:-1]: i for i, ln in enumerate(lines) if ln.endswith(":")}
    regs = {"%[pairs]": pairs, "%[rem]": rem}
    scc, i, out = False, 0, []
    while i < len(lines):
        ln = lines[i]
        op = ln.split()[0] if ln else ""
        i += 1
        if ln.endswith(":"):
            continue
        args = [a.strip() for a in ln[len(op):].split(",")]
        if op == "s_cmp_le_i32":
            scc = regs[args[0]] <= int(args[1])
        elif op == "s_cmp_gt_i32":
            scc = regs[args[0]] > int(args[1])
        elif op == "s_cmp_eq_i32":
            scc = regs[args[0]] == int(args[1])
        elif op == "s_sub_i32" and args[0] == "%[pairs]":
            regs["%[pairs]"] -= int(args[2])
        elif op == "s_cbranch_scc1":
            i = labels[args[0]] if scc else i
        elif op == "s_cbranch_scc0":
            i = labels[args[0]] if not scc else i
        elif op == "s_branch":
            i = labels[args[0]]
        else:
            out.append(ln)
    return out


def reg_set(spec):
    """Registers ('v', n) / ('a', n) named by one operand, or an empty set."""
    spec = spec.strip()
    m = re.fullmatch(r"([va])\[(\d+):(\d+)\]", spec)
    if m:
        return {(m.group(1), r) for r in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.fullmatch(r"([va])(\d+)", spec)
    return {(m.group(1), int(m.group(2)))} if m else set()


def operands(ln):
    op = ln.split()[0]
    rest = ln[len(op):]
    rest = re.sub(r"\boffset:\d+", "", rest)
    return op, [a.strip() for a in rest.split(",") if a.strip()]


def is_valu(op):
    return op.startswith("v_") and not op.startswith("v_mfma")


def wait_states(ln):
    op = ln.split()[0]
    return int(ln.split()[1]) + 1 if op == "s_nop" else 1


def replay(tr):
    """Check hazards, LDS-read waits and barrier-time loads along one trace; returns the number of
    MFMAs issued."""
    ws = 0
    mfma_dst = {}                 # register -> wait-state count right after the MFMA that wrote it
    lds_pending = []              # register sets of outstanding LDS reads, oldest first
    vm_pending = []               # True for each outstanding prefetch, False for a copy
    m0_at, m0_val = None, None
    n_mfma = 0
    for ln in tr:
        op, args = operands(ln)
        if op == "s_waitcnt":
            m = re.search(r"lgkmcnt\((\d+)\)", ln)
            if m:
                keep = int(m.group(1))
                lds_pending = lds_pending[len(lds_pending) - keep:] if keep else []
            m = re.search(r"vmcnt\((\d+)\)", ln)
            if m:
                keep = int(m.group(1))
                vm_pending = vm_pending[len(vm_pending) - keep:] if keep else []
        elif op == "s_barrier":
            assert all(vm_pending), f"barrier with a copy in flight: {ln}"
            assert not lds_pending, "barrier with an LDS read in flight"
        reads, writes = set(), set()
        if op.startswith("v_mfma"):
            writes = reg_set(args[0])
            reads = reg_set(args[1]) | reg_set(args[2])
            n_mfma += 1
        elif op.startswith("ds_read"):
            writes = reg_set(args[0])
        elif op.startswith("buffer_load") and ln.endswith("lds"):
            reads = reg_set(args[0])
            assert m0_at is not None and ws - m0_at >= 1, f"LDS-DMA load right after the M0 write: {ln}"
            vm_pending.append(m0_val == PF_LDS)
        elif is_valu(op):
            writes = reg_set(args[0])
            for a in args[1:]:
                reads |= reg_set(a)
            if op.startswith("v_fmac"):
                reads |= writes
            for r in reads:
                if r in mfma_dst:
                    gap = ws - mfma_dst[r]
                    assert gap >= MFMA_VALU_WAIT, f"VALU reads {r} {gap} wait states after its MFMA: {ln}"
        elif op.startswith("s_") and args and args[0] == "m0":
            m0_at = ws + 1                              # wait states are counted after the write
            m0_val = args[-1] if op == "s_mov_b32" else None
        for p in lds_pending:
            assert not (p & (reads | writes)), f"register of a pending LDS read used: {ln}"
        if op.startswith("ds_read"):
            lds_pending.append(writes)
            assert len(lds_pending) <= 15
        for r in writes:
            mfma_dst.pop(r, None)
        ws += wait_states(ln)
        if op.startswith("v_mfma"):
            for r in writes:
                mfma_dst[r] = ws                        # wait states are counted after the MFMA
    return n_mfma


def test_generated_text_is_committed(tmp_path):
    gen = load_generator()
    out = tmp_path / "gemm_w4_asm.inc"
    gen.main(str(out))
    assert out.read_text() == open(INC).read(), "gemm_w4_asm.inc differs from what gen_w4_asm.py writes"


@pytest.mark.parametrize("slices", [1, 2, 3, 4, 5, 6])
def test_trace(slices):
    lines = mainloop()
    pairs = (slices - 1) // 2
    rem = slices - 2 * pairs
    tr = trace(lines, pairs, rem)
    assert replay(tr) == 64 * slices
    assert tr.count("s_barrier") == slices + 1          # the prologue's and one per slice


def statement():
    src = open(os.path.join(CSRC, "gemm_w4.hip")).read()
    outs = re.search(r"#define PURO_W4_OUTS((?:.*\\\n)*.*)", src).group(1)
    ins = re.search(r"#define PURO_W4_INS((?:.*\\\n)*.*)", src).group(1)
    clob = re.search(r"#define PURO_W4_CLOB (.*)", src).group(1)
    return outs, ins, clob


def test_declared_writes():
    lines = [ln for ln in mainloop() if not ln.endswith(":")]
    outs, ins, clob = statement()
    declared = set()
    for kind, a, b in re.findall(r"\{([va])\[(\d+):(\d+)\]\}", outs):
        declared |= {(kind, r) for r in range(int(a), int(b) + 1)}
    for kind, a in re.findall(r"\{([va])(\d+)\}", outs):
        declared.add((kind, int(a)))
    declared |= {("a", r) for r in clobber_agprs()}
    declared |= {("v", int(r)) for r in re.findall(r'"v(\d+)"', clob)}
    sgpr_outs = set(re.findall(r"\[(\w+)\] \"(?:\+|=&)s\"", outs))
    assert '"m0"' in clob and '"scc"' in clob
    for ln in lines:
        op, args = operands(ln)
        if op in ("s_waitcnt", "s_barrier", "s_nop") or op.startswith(("s_cmp", "s_cbranch", "s_branch")):
            continue
        if op.startswith("buffer_load"):
            continue                                     # its first operand is an address
        if op.startswith("s_"):
            dst = args[0]
            m = re.fullmatch(r"%\[(\w+)\]", dst)
            assert dst == "m0" or (m and m.group(1) in sgpr_outs), f"undeclared SGPR write: {ln}"
            continue
        for r in reg_set(args[0]):
            assert r in declared, f"undeclared register write {r}: {ln}"
    # the pinned SGPR inputs (the copy groups' row offsets) are never written
    for ln in lines:
        op, args = operands(ln)
        if op.startswith("s_") and args and re.fullmatch(r"s\d+", args[0]):
            pytest.fail(f"write of a pinned input SGPR: {ln}")


def test_copies_cover_both_operands():
    """Each copying slice moves 8 + 8 row groups of A and B, the row scales and the weight scale,
    plus the three prefetches."""
    lines = mainloop()
    tr = trace(lines, 1, 1)                              # prologue + 3 slices
    loads = [ln for ln in tr if ln.startswith("buffer_load")]
    assert len(loads) == 3 * (16 + 2 + 3)
    assert sum(" %[rA], " in ln and "dwordx4" in ln for ln in loads) == 3 * 8
    assert sum(" %[rB], " in ln and "dwordx4" in ln for ln in loads) == 3 * 8


def _mutants(lines):
    """Copies of the loop with one planted scheduling mistake each."""
    out = {}
    i = next(i for i, ln in enumerate(lines) if ln.startswith("s_waitcnt vmcnt(3)"))
    out["barrier before the copies land"] = lines[:i] + ["s_waitcnt vmcnt(4) lgkmcnt(0)"] + lines[i + 1:]
    i = next(i for i, ln in enumerate(lines) if ln.startswith("s_waitcnt lgkmcnt(") and not ln.endswith("(0)"))
    out["fragment read not waited for"] = lines[:i] + lines[i + 1:]
    j = next(i for i, ln in enumerate(lines) if ln.startswith("v_mfma"))
    p = lines[j].split()[1].rstrip(",")
    first = int(re.match(r"v\[(\d+)", p).group(1))
    out["promotion right behind its MFMA"] = lines[:j + 1] + [f"v_fmac_f32 v0, v{first}, v236"] + lines[j + 1:]
    i = next(i for i, ln in enumerate(lines) if ln.startswith("buffer_load") and i > 100)
    out["M0 written right before the load"] = lines[:i] + ["s_mov_b32 m0, 0"] + lines[i:]
    return out


@pytest.mark.parametrize("name", ["barrier before the copies land", "fragment read not waited for",
                                  "promotion right behind its MFMA", "M0 written right before the load"])
def test_replay_rejects_planted_mistakes(name):
    bad = _mutants(mainloop())[name]
    with pytest.raises(AssertionError):
        for slices in (1, 2, 3, 4):
            pairs = (slices - 1) // 2
            replay(trace(bad, pairs, slices - 2 * pairs))
