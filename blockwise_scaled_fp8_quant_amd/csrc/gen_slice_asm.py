"""Generate gemm_slice_asm.inc: the hand-scheduled gfx950 instruction sequences for one
128-deep slice of the blockwise-scaled FP8 GEMM.

    python blockwise_scaled_fp8_quant_amd/csrc/gen_slice_asm.py   # rewrites gemm_slice_asm.inc

The generated text is committed; the library build does not run this script.

Three variants.  Two differ in how the slice product of a tile is promoted:
  ROWSCALE (FWD / DGRAD)  one scale per lane and row group: sA(i,kb) * sB(block,kb) is the
                          same for the 16 columns a lane owns (they sit in one 128x128
                          weight block), so the promotion is 16 FMAs:  C += P * sc.
  COLSCALE (WGRAD)        sB(j,kb) differs per column: 16 multiplies by the lane's 16 column
                          scales (read from LDS) and 16 FMAs by its row scale:
                          P *= sB(j);  C += P * sA(i).

The third, MXSCALE (the MXFP8 GEMM), promotes nothing: every operand block of 32 elements
carries an E8M0 scale that the scaled MFMA (v_mfma_scale_f32_32x32x64_f8f6f4) applies itself,
so both MFMAs of a tile accumulate straight into the tile's accumulator.  In that instruction
a scale block is the 16-byte group g of both lane halves, scaled by lane half g's scale byte
(op_sel picks the byte); the kernel feeds lane half h chunks h, h+4 / h+2, h+6 so that these
groups are the MX blocks 0, 2 / 1, 3 of the slice, and each lane's scale operand is one 16-bit
LDS read holding MX blocks 2h (byte 0, first MFMA) and 2h + 1 (byte 1, second MFMA).

Register map (per lane; pinned by the asm statement's constraints and clobbers):
  v[0:127]    accumulators: output tile T = 2*ni + mi (32 x 32, 16 fp32 per lane) in v[16T:16T+15]
  v[128:143]  slice product P of even tiles (clobbered)
  v[144:159]  slice product P of odd tiles; tile 7's product is carried out of the block and
              promoted at the start of the next block (or by the tail block after the loop)
  v[160:175]  A fragment, row group mi = 0 (4 x 16-byte LDS chunks per lane)
  v[176:191]  A fragment, row group mi = 1
  ROWSCALE:   v[192:207] B fragment buffer 0 (column tiles ni = 0, 2), v[208:223] buffer 1 (ni = 1, 3)
  COLSCALE:   v[192:207] B fragment (one buffer), v[208:223] the 16 column scales of the current
              column tile (column tile 3's are carried out of the block with tile 7's product)
  MXSCALE:    v[192:223] as ROWSCALE; v128, v129 the A scale pairs of row groups 0 / 1,
              v130 .. v133 the B scale pairs of column tiles 0 .. 3 (P registers are unused)
Operands: %[aj0..3] / %[bj0..3] LDS byte addresses of this lane's 4 swizzled 16-byte chunks in
its A / B row (row group / column tile offsets are 4096-byte immediates); ROWSCALE: %[sc0],
%[sc1] the promotion scale of row group 0 / 1 for this slice, %[scp] the scale of the carried
product; COLSCALE: %[sa0], %[sa1], %[sap] the row scales likewise and %[sbj] the LDS address
of the lane's first column-scale quad (column tile / quad offsets are immediates); MXSCALE:
%[xaj] / %[xbj] the LDS addresses of the lane's A / B scale pair (row group / column tile
offsets are immediates); for the copy
of the next slice into the other LDS stage: %[ga0..3] / %[gb0..3] the (wave-uniform) global
addresses of the wave's four 8-row groups of A / B at that slice, %[oa0], %[oa1] / %[ob0],
%[ob1] the lane's byte offset within an even / odd group (row in group and swizzled chunk),
%[m0] the LDS address of the wave's first A row in the other stage.

Schedule of a slice (8 steps, step s computes tile (ni, mi) = (s >> 1, s & 1)):
  entry   read the first B fragment and the A fragment of row group 0; promote the carried
          tile-7 product of the previous slice; read the A fragment of row group 1.
  step s  wait for this step's fragments (counting only older LDS reads); the two chained
          MFMAs of tile s (v_mfma_f32_32x32x64_f8f6f4: the second accumulates on the first,
          together one 128-deep slice of a 32 x 32 tile); the global_load_lds_dwordx4 copies
          of the next slice that DMA_PLAN puts at this step (M0 = LDS destination, one wait
          state after the M0 write); fragment / scale reads for later steps; the promotion
          of tile s-1.
  exit    wait for this wave's copies, then meet the other waves at the barrier.
Every LDS read is waited for inside the block.

Hazards: a VALU read of an MFMA result needs HAZARD_WAIT_STATES wait states (instructions, or
s_nop k = k + 1) after the MFMA was issued (the figure the compiler's own hazard recognizer
uses for 16-pass XDL results on gfx950).  The generator counts the instructions between
each product's last MFMA and its first VALU read and pads only where they fall short.
Fragment registers are overwritten by LDS reads only after the MFMAs reading them were
issued (MFMAs read their A/B operands when they issue).
"""
import os

HAZARD_WAIT_STATES = 20
# copies of the next slice issued at each of the 8 steps (8 copies in all).  Two per step over the
# first half of the slice: the copies get more than half a slice to land before the end-of-slice
# wait (an L2 miss served from HBM takes longer than one step), while the address unit's queue
# still never holds more than two of them per wave.  Measured on MI355X against one copy per step:
# FWD / DGRAD 4-7% faster, WGRAD 1-4%; all eight at once is slower than two per step.
DMA_PLAN = [[0, 1], [2, 3], [4, 5], [6, 7], [], [], [], []]
STAGE_B = 32768                      # byte offset of the B tile in an LDS stage
P_EVEN, P_ODD = 128, 144
A0, A1, BF0, SB = 160, 176, 192, 208


class Emitter:
    """Collects instructions, counts wait states, and checks the LDS-read bookkeeping: every
    register an MFMA or VALU instruction reads must not be the target of an LDS read that no
    s_waitcnt has covered yet (LDS reads return in order, so lgkmcnt(n) covers all but the
    newest n)."""

    def __init__(self):
        self.lines = []
        self.ws = 0                  # wait states issued so far
        self.produced = {}           # P buffer -> wait-state count just after its last MFMA
        self.pending = []            # register sets of LDS reads not yet waited for, oldest first

    def emit(self, ln):
        self.lines.append(ln)
        self.ws += int(ln.split()[1]) + 1 if ln.startswith("s_nop") else 1

    def nops(self, n):
        while n > 0:
            k = min(n, 16)
            self.emit(f"s_nop {k - 1}")
            n -= k

    def wait_lgkm(self, n):
        self.emit(f"s_waitcnt lgkmcnt({n})")
        self.pending = self.pending[len(self.pending) - n:] if n else []

    def use(self, regs):
        for p in self.pending:
            assert not (p & regs), f"register read before its LDS read was waited for: {sorted(p & regs)[:4]}"

    def read(self, dst, addr, offset):
        regs = set(range(dst, dst + 4))
        for p in self.pending:
            assert not (p & regs), "LDS read overwrites registers of a pending read"
        self.emit(f"ds_read_b128 v[{dst}:{dst + 3}], %[{addr}] offset:{offset}")
        self.pending.append(regs)
        assert len(self.pending) <= 15, "more LDS reads in flight than lgkmcnt can count"

    def frag(self, dst, addr, offset):
        """4 LDS reads: the lane's 4 swizzled 16-byte chunks of one A / B fragment."""
        for j in range(4):
            self.read(dst + 4 * j, f"{addr}{j}", offset)

    def mfma_pair(self, p, b, a):
        self.use(set(range(b, b + 16)) | set(range(a, a + 16)))
        self.emit(f"v_mfma_f32_32x32x64_f8f6f4 v[{p}:{p + 15}], v[{b}:{b + 7}], v[{a}:{a + 7}], 0")
        self.emit(f"v_mfma_f32_32x32x64_f8f6f4 v[{p}:{p + 15}], v[{b + 8}:{b + 15}], v[{a + 8}:{a + 15}], v[{p}:{p + 15}]")
        self.produced[p] = self.ws

    def mfma_pair_mx(self, acc, b, a, sb, sa):
        """Two scaled MFMAs accumulating into acc: block byte 0 of the scale pairs, then byte 1."""
        self.use(set(range(b, b + 16)) | set(range(a, a + 16)) | {sb, sa})
        for half, sel in ((0, "op_sel:[0,0,0] op_sel_hi:[0,0,0]"), (8, "op_sel:[1,1,0] op_sel_hi:[0,0,0]")):
            self.emit(f"v_mfma_scale_f32_32x32x64_f8f6f4 v[{acc}:{acc + 15}], v[{b + half}:{b + half + 7}], "
                      f"v[{a + half}:{a + half + 7}], v[{acc}:{acc + 15}], v{sb}, v{sa} {sel}")
        self.produced[acc] = self.ws

    def read_u16(self, dst, addr, offset):
        regs = {dst}
        for p in self.pending:
            assert not (p & regs), "LDS read overwrites a register of a pending read"
        self.emit(f"ds_read_u16 v{dst}, %[{addr}] offset:{offset}")
        self.pending.append(regs)
        assert len(self.pending) <= 15, "more LDS reads in flight than lgkmcnt can count"

    def hazard(self, p):
        """Pad before the first VALU read of product buffer p (produced in this block)."""
        self.nops(HAZARD_WAIT_STATES - (self.ws - self.produced[p]))

    def dma(self, k):
        """Copy k of the next slice: group q = k >> 1, A for even k, B for odd k."""
        q = k >> 1
        if k & 1 == 0:
            self.emit(f"s_add_u32 m0, %[m0], {q * 8 * 128}")
            self.emit("s_nop 0")
            self.emit(f"global_load_lds_dwordx4 %[oa{q & 1}], %[ga{q}]")
        else:
            self.emit(f"s_add_u32 m0, %[m0], {STAGE_B + q * 8 * 128}")
            self.emit("s_nop 0")
            self.emit(f"global_load_lds_dwordx4 %[ob{q & 1}], %[gb{q}]")

    def fma_row(self, T, p, sc):
        for v in range(16):
            self.emit(f"v_fmac_f32 v{16 * T + v}, v{p + v}, %[{sc}]")

    def fma_col(self, T, p, sa):
        self.use(set(range(SB, SB + 16)))
        for v in range(16):
            self.emit(f"v_mul_f32 v{p + v}, v{p + v}, v{SB + v}")
        for v in range(16):
            self.emit(f"v_fmac_f32 v{16 * T + v}, v{p + v}, %[{sa}]")

    def sb_reads(self, ni):
        """The lane's 16 column scales of column tile ni: 4 quads (columns 8g + 4h .. +3)."""
        for g in range(4):
            self.read(SB + 4 * g, "sbj", ni * 128 + 32 * g)


def gen_rowscale():
    e = Emitter()
    e.frag(BF0, "bj", 0)                  # B, column tile 0 -> buffer 0
    e.frag(A0, "aj", 0)                   # A, row group 0
    e.nops(HAZARD_WAIT_STATES - 8)        # carried product: counted from the block start
    e.fma_row(7, P_ODD, "scp")
    e.frag(A1, "aj", 4096)                # A, row group 1
    e.wait_lgkm(4)                        # B(0), A0
    for s in range(8):
        ni, mi = s >> 1, s & 1
        if s == 1:
            e.wait_lgkm(4)                # A1 (the B fragment of tile 2 is newer)
        elif mi == 0 and ni > 0:
            e.wait_lgkm(0)                # B fragment read two steps earlier
        e.mfma_pair(P_EVEN if mi == 0 else P_ODD, BF0 + 16 * (ni & 1), A0 + 16 * mi)
        for k in DMA_PLAN[s]:
            e.dma(k)
        if mi == 0 and ni < 3:
            e.frag(BF0 + 16 * ((ni + 1) & 1), "bj", (ni + 1) * 4096)
        if s > 0:
            q = s - 1
            pq = P_EVEN if (q & 1) == 0 else P_ODD
            e.hazard(pq)
            e.fma_row(2 * (q >> 1) + (q & 1), pq, f"sc{q & 1}")
    e.emit("s_waitcnt vmcnt(0) lgkmcnt(0)")
    e.emit("s_barrier")
    return e.lines


def gen_colscale():
    e = Emitter()
    e.frag(BF0, "bj", 0)                  # B, column tile 0
    e.frag(A0, "aj", 0)                   # A, row group 0
    e.nops(HAZARD_WAIT_STATES - 8)        # carried product: counted from the block start
    e.fma_col(7, P_ODD, "sap")            # the previous slice's column-tile-3 scales
    e.frag(A1, "aj", 4096)                # A, row group 1
    e.wait_lgkm(4)                        # B(0), A0
    for s in range(8):
        ni, mi = s >> 1, s & 1
        if s == 1:
            e.wait_lgkm(4)                # A1 (the scales of column tile 0 are newer)
        elif mi == 0 and ni > 0:
            e.wait_lgkm(0)                # B(ni), read at the previous step
        e.mfma_pair(P_EVEN if mi == 0 else P_ODD, BF0, A0 + 16 * mi)
        for k in DMA_PLAN[s]:
            e.dma(k)
        if mi == 1 and ni < 3:
            e.frag(BF0, "bj", (ni + 1) * 4096)   # B(ni+1): the MFMAs reading B(ni) have issued
        if s == 0:
            e.sb_reads(0)
        if s > 0:
            q = s - 1
            pq = P_EVEN if (q & 1) == 0 else P_ODD
            if mi == 1:                   # tile (ni, 0): column tile ni's scales (older than B(ni+1))
                e.wait_lgkm(4 if ni < 3 else 0)
            e.hazard(pq)
            e.fma_col(2 * (q >> 1) + (q & 1), pq, f"sa{q & 1}")
            if mi == 0:                   # tile (ni-1, 1) was the last user of the old scales
                e.sb_reads(ni)
    e.emit("s_waitcnt vmcnt(0) lgkmcnt(0)")
    e.emit("s_barrier")
    assert not e.pending
    return e.lines


SA0, SB0 = 128, 130            # MXSCALE scale pairs: v128 + mi, v130 + ni


def gen_mxscale():
    e = Emitter()
    e.read_u16(SA0, "xaj", 0)             # row group 0
    e.read_u16(SB0, "xbj", 0)             # column tile 0
    e.frag(BF0, "bj", 0)                  # B, column tile 0 -> buffer 0
    e.frag(A0, "aj", 0)                   # A, row group 0
    e.frag(A1, "aj", 4096)                # A, row group 1
    e.wait_lgkm(4)                        # all but A1
    for s in range(8):
        ni, mi = s >> 1, s & 1
        if s == 1:
            e.wait_lgkm(7)                # A1 and the scales of row group 1 (newer: 3 scales, B(1))
        elif mi == 0 and ni > 0:
            e.wait_lgkm(0)                # B fragment and scales of column tile ni
        e.mfma_pair_mx(16 * (2 * ni + mi), BF0 + 16 * (ni & 1), A0 + 16 * mi, SB0 + ni, SA0 + mi)
        for k in DMA_PLAN[s]:
            e.dma(k)
        if s == 0:
            e.read_u16(SA0 + 1, "xaj", 128)
            for n in range(1, 4):
                e.read_u16(SB0 + n, "xbj", 128 * n)
        if mi == 0 and ni < 3:
            e.frag(BF0 + 16 * ((ni + 1) & 1), "bj", (ni + 1) * 4096)
    e.emit("s_waitcnt vmcnt(0) lgkmcnt(0)")
    e.emit("s_barrier")
    assert not e.pending
    return e.lines


def gen_tail(col):
    """After the last slice: promote the carried tile-7 product (padding kept for a block
    boundary the generator cannot see)."""
    e = Emitter()
    e.nops(HAZARD_WAIT_STATES)
    if col:
        e.fma_col(7, P_ODD, "sap")
    else:
        e.fma_row(7, P_ODD, "scp")
    return e.lines


def macro(name, lines):
    out = [f"#define {name} \\"]
    out += [f'  "{ln}\\n\\t" \\' for ln in lines]
    out.append('  ""')
    return "\n".join(out) + "\n"


def main(out_path=None):
    row, col, mxs = gen_rowscale(), gen_colscale(), gen_mxscale()
    here = os.path.dirname(os.path.abspath(__file__))
    with open(out_path or os.path.join(here, "gemm_slice_asm.inc"), "w") as f:
        f.write("// Generated by gen_slice_asm.py -- one 128-deep slice of the FP8 GEMM (see there).\n")
        f.write("// FWD / DGRAD: one promotion scale per lane and row group\n")
        f.write(macro("PURO_SLICE_ASM_ROWSCALE", row))
        f.write("// promotion of the carried product after the last slice\n")
        f.write(macro("PURO_SLICE_ASM_ROWSCALE_TAIL", gen_tail(False)))
        f.write("// WGRAD: per-column scales from LDS times one row scale per lane and row group\n")
        f.write(macro("PURO_SLICE_ASM_COLSCALE", col))
        f.write(macro("PURO_SLICE_ASM_COLSCALE_TAIL", gen_tail(True)))
        f.write("// MXFP8: E8M0 block scales applied by the scaled MFMA, no promotion\n")
        f.write(macro("PURO_SLICE_ASM_MXSCALE", mxs))
        f.write("// after the last slice: wait states between the last MFMA and the epilogue's reads\n")
        e = Emitter()
        e.nops(HAZARD_WAIT_STATES)
        f.write(macro("PURO_SLICE_ASM_MX_TAIL", e.lines))
        f.write("// VGPRs the blocks use besides the pinned accumulators and the carried product (and, for\n"
                "// COLSCALE, the carried column scales in v[208:223])\n")
        f.write("#define PURO_SLICE_ASM_CLOBBERS " + ", ".join(f'"v{r}"' for r in list(range(128, 144)) + list(range(160, 224))) + "\n")
        f.write("#define PURO_SLICE_ASM_COLSCALE_CLOBBERS " + ", ".join(f'"v{r}"' for r in list(range(128, 144)) + list(range(160, 208))) + "\n")
        f.write("#define PURO_SLICE_ASM_MX_CLOBBERS " + ", ".join(f'"v{r}"' for r in list(range(128, 134)) + list(range(160, 224))) + "\n")
    print(f"rowscale {len(row)}, colscale {len(col)}, mxscale {len(mxs)} instructions")


if __name__ == "__main__":
    main()
