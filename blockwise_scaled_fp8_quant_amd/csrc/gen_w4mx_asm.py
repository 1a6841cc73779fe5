"""Generate gemm_w4mx_asm.inc: the hand-scheduled gfx950 K loop of the MXFP8 GEMM in its four-wave
form (one wave per SIMD, a 128 x 128 output tile per wave).

    python blockwise_scaled_fp8_quant_amd/csrc/gen_w4mx_asm.py     # rewrites gemm_w4mx_asm.inc

The generated text is committed; the library build does not run this script.

MXFP8 operands carry one E8M0 scale per 32 elements of a row along the contraction, and the scaled
FP8 MFMA (v_mfma_scale_f32_16x16x128_f8f6f4) applies both operands' block scales itself, so each
slice product accumulates straight into the tile's accumulator: no promotion on the vector ALUs.
The accumulators (64 tiles of 16 x 16, 4 fp32 per lane each) then fit in the 256 AGPRs of a wave
that has a SIMD to itself, and the operand fragments and scales sit in VGPRs.

How the instruction applies the scales (measured on gfx950 with a probe: one 32-byte row piece
set to 1.0, per-lane scale bytes 2^lane): lane group g (lanes 16 g .. 16 g + 15) holds bytes
16 g .. 16 g + 15 of its row's 128-byte slice in its first four source registers and bytes
64 + 16 g .. + 15 in the last four; the scale of 32-element block b of row r is lane 16 b + r's
byte.  So lane group g is fed 16-byte chunks g and g + 4 of its row: block b then covers exactly
the data of MX block b, and each lane supplies the scale byte of its own row and block g.

Register map (per lane):
  a[0:255]    accumulators of tiles (mi, ni): a[4 (8 mi + ni) : + 3]
  v[0:63]     A fragments, row group mi: v[8 mi : + 7]
  v[64:127]   B fragments, column group ni: v[64 + 8 ni : + 7]
  v[128:135]  A scale bytes, row group mi: v[128 + mi] (row 128 wm + 16 mi + lane % 16, block lane / 16)
  v[136:143]  B scale bytes, column group ni: v[136 + ni]
  v[243:246]  copy offsets (row in 8-row group, swizzled chunk, and the K offset of the slice being
              copied) for even / odd groups of A and of B; v247, v248: prefetch offsets
Operands: %[aj0], %[aj1] / %[bj0], %[bj1]: LDS byte addresses of the lane's two 16-byte chunks in its
A / B row of stage 0; %[xaj] / %[xbj]: LDS byte addresses of the lane's A / B scale byte in stage 0
(stage and row / column group offsets are immediates); %[osa]: the lane's offset for the scale
copies; %[rA], %[rB], %[rS], %[rX]: buffer resources of the tile's A rows, B rows, A scales,
B scales; s[64:71] / s[72:79]: the byte offsets of the wave's 8-row copy groups in A / B;
%[ssa] / %[ssb]: offsets of the wave's scale rows of the slice being copied; %[ssp] / %[ssq]: the
same two slices ahead (prefetch); %[sstep] / %[sstepb]: bytes between slices of the A / B scales;
%[mw] / %[ms]: the wave's LDS base for its tile copies / scale copies.

LDS (bytes): stage s holds A rows at 32768 s + 128 r, B rows at 65536 + 32768 s + 128 r (chunk c of
row r at c ^ ((r >> 1) & 7)); A scales at 131072 + 2048 s (256 rows x 4 bytes), B scales 1024
bytes further.  Copies: each wave copies A rows 64 w .. 64 w + 63 and B rows 64 w .. + 63 of the
next slice as 8-row groups (buffer_load_dwordx4 ... lds), plus the 4 scale bytes of each of its 64
A and 64 B rows (one buffer_load_dword ... lds each), then pulls the slice after next into L2 (one
dword per row of A, B and both scale arrays, into an LDS area nothing reads).

Schedule of a slice: the entry reads the first fragments and scales; step k (k = 0 .. 63) runs the
MFMA of tile (k / 8, k % 8) once its fragments and scales have landed, then up to STEP_SLOTS slots
of the slice's other instructions (fragment and scale reads for later steps, copies), issued by a
list scheduler in order of urgency; the exit waits for the copies and meets the other waves at the
barrier.  No register an LDS read writes is read before an lgkmcnt wait covers it (reads complete
in order), never more than 15 are outstanding, and an LDS-DMA load follows an SALU write of M0 by
at least one wait state.  A fragment or scale of the next slice is read only after the last MFMA
that reads its register in this slice has issued (MFMAs read their sources at issue).
"""
import os

STEP_SLOTS = 5                 # issue slots beside each MFMA (its 8 passes leave about that many)
STAGE_BYTES = 32768
B_BASE = 65536
S_BASE = 131072
S_STAGE = 2048
MFMA_READ_WAIT = 18            # MFMA result -> first read by the code after the loop (AGPR reads)

VOFF = {"oa0": 243, "oa1": 244, "ob0": 245, "ob1": 246}
PF = {"pa": 247, "pb": 248}
PF_LDS = 135168
PF_LOADS = 4                   # prefetch loads per slice (A rows, B rows, A scales, B scales)
QA, QB = 64, 72


def acc(mi, ni):
    return 4 * (8 * mi + ni)


def frag_a(mi):
    return 8 * mi


def frag_b(ni):
    return 64 + 8 * ni


def sa_reg(mi):
    return 128 + mi


def sb_reg(ni):
    return 136 + ni


class Emitter:
    def __init__(self):
        self.lines = []
        self.ws = 0
        self.pending = []            # register sets of outstanding LDS reads, oldest first
        self.m0_at = None

    def emit(self, ln, ws=1):
        self.lines.append(ln)
        self.ws += ws

    def nops(self, n):
        while n > 0:
            k = min(n, 16)
            self.emit(f"s_nop {k - 1}", k)
            n -= k

    def ds_read(self, regs, text):
        regs = set(regs)
        for p in self.pending:
            assert not (p & regs), f"LDS read overwrites registers of a pending read: {text}"
        self.emit(text)
        self.pending.append(regs)
        assert len(self.pending) <= 15, "more than 15 LDS reads outstanding"

    def wait_for(self, regs):
        regs = set(regs)
        last = -1
        for i, p in enumerate(self.pending):
            if p & regs:
                last = i
        if last < 0:
            return
        keep = len(self.pending) - 1 - last
        self.emit(f"s_waitcnt lgkmcnt({keep})")
        self.pending = self.pending[last + 1:]

    def mfma(self, mi, ni):
        a, b, c = frag_a(mi), frag_b(ni), acc(mi, ni)
        regs = [f"v{r}" for r in range(a, a + 8)] + [f"v{r}" for r in range(b, b + 8)]
        regs += [f"v{sa_reg(mi)}", f"v{sb_reg(ni)}"]
        self.wait_for(regs)
        # operand roles swapped as in the blockwise form: the B fragment is the first source
        self.emit(f"v_mfma_scale_f32_16x16x128_f8f6f4 a[{c}:{c + 3}], v[{b}:{b + 7}], v[{a}:{a + 7}], "
                  f"a[{c}:{c + 3}], v{sb_reg(ni)}, v{sa_reg(mi)} op_sel:[0,0,0] op_sel_hi:[0,0,0]")

    def m0(self, text):
        self.emit(text)
        self.m0_at = self.ws

    def dma(self, text):
        if self.m0_at is not None and self.ws - self.m0_at < 1:
            self.nops(1)
        self.emit(text)


def copy_items(stage_next):
    """(m0 instruction, load instruction) pairs copying the next slice into stage `stage_next`, then
    the L2 prefetches of the slice after it."""
    out = []
    so = stage_next * STAGE_BYTES
    a = [(f"s_add_u32 m0, %[mw], {so + q * 1024}",
          f"buffer_load_dwordx4 v{VOFF['oa0' if q % 2 == 0 else 'oa1']}, %[rA], s{QA + q} offen lds") for q in range(8)]
    b = [(f"s_add_u32 m0, %[mw], {B_BASE + so + q * 1024}",
          f"buffer_load_dwordx4 v{VOFF['ob0' if q % 2 == 0 else 'ob1']}, %[rB], s{QB + q} offen lds") for q in range(8)]
    ss = stage_next * S_STAGE                                # %[ms] holds 131072 + 256 w
    s = [(f"s_add_u32 m0, %[ms], {ss}", "buffer_load_dword %[osa], %[rS], %[ssa] offen lds"),
         (f"s_add_u32 m0, %[ms], {ss + 1024}", "buffer_load_dword %[osa], %[rX], %[ssb] offen lds")]
    inter = []
    for q in range(8):
        inter += [a[q], b[q]]
    pf = [(f"s_mov_b32 m0, {PF_LDS}", f"buffer_load_dword v{PF['pa']}, %[rA], s{QA} offen lds"),
          (f"s_mov_b32 m0, {PF_LDS}", f"buffer_load_dword v{PF['pb']}, %[rB], s{QB} offen lds"),
          (f"s_mov_b32 m0, {PF_LDS}", "buffer_load_dword %[osa], %[rS], %[ssp] offen lds"),
          (f"s_mov_b32 m0, {PF_LDS}", "buffer_load_dword %[osa], %[rX], %[ssq] offen lds")]
    return s + inter + pf


def gen_slice(stage, copies):
    e = Emitter()
    st = stage * STAGE_BYTES
    sst = stage * S_STAGE

    def read_a(mi):
        a = frag_a(mi)
        e.ds_read({f"v{r}" for r in range(a, a + 4)}, f"ds_read_b128 v[{a}:{a + 3}], %[aj0] offset:{st + 2048 * mi}")
        e.ds_read({f"v{r}" for r in range(a + 4, a + 8)}, f"ds_read_b128 v[{a + 4}:{a + 7}], %[aj1] offset:{st + 2048 * mi}")

    def read_b(ni):
        b = frag_b(ni)
        e.ds_read({f"v{r}" for r in range(b, b + 4)}, f"ds_read_b128 v[{b}:{b + 3}], %[bj0] offset:{st + 2048 * ni}")
        e.ds_read({f"v{r}" for r in range(b + 4, b + 8)}, f"ds_read_b128 v[{b + 4}:{b + 7}], %[bj1] offset:{st + 2048 * ni}")

    def read_sa(mi):
        e.ds_read({f"v{sa_reg(mi)}"}, f"ds_read_u8 v{sa_reg(mi)}, %[xaj] offset:{sst + 64 * mi}")

    def read_sb(ni):
        e.ds_read({f"v{sb_reg(ni)}"}, f"ds_read_u8 v{sb_reg(ni)}, %[xbj] offset:{sst + 64 * ni}")

    # ---------------- entry: what the first two steps need
    read_a(0)
    read_b(0)
    read_sa(0)
    read_sb(0)
    read_b(1)
    read_sb(1)
    if copies:
        for r in list(VOFF.values()) + list(PF.values()):
            e.emit(f"v_add_u32 v{r}, 128, v{r}")
        e.emit("s_add_u32 %[ssa], %[ssa], %[sstep]")
        e.emit("s_add_u32 %[ssb], %[ssb], %[sstepb]")
        e.emit("s_add_u32 %[ssp], %[ssa], %[sstep]")
        e.emit("s_add_u32 %[ssq], %[ssb], %[sstepb]")
    dmas = copy_items(stage ^ 1) if copies else []

    # The rest of the slice's instructions, for a list scheduler: an item is ready at step `first`
    # and must be emitted by step `last` (it is needed at step last + 1 or later).
    items = []

    def item(name, first, last, size, fn):
        items.append({"name": name, "first": first, "last": last, "size": size, "fn": fn})

    for ni in range(2, 8):                       # B(ni) and its scales: first needed at step ni
        item(f"rb{ni}", 0, ni - 2, 2, lambda ni=ni: read_b(ni))
        item(f"sb{ni}", 0, ni - 1, 1, lambda ni=ni: read_sb(ni))
    for mi in range(1, 8):                       # A(mi): first needed at step 8 mi; its registers
        # were last read by the MFMAs of row group mi in the previous slice
        item(f"ra{mi}", 8 * (mi - 1), 8 * mi - 3, 2, lambda mi=mi: read_a(mi))
        item(f"sa{mi}", 8 * (mi - 1), 8 * mi - 2, 1, lambda mi=mi: read_sa(mi))
    for i, (m0, ld) in enumerate(dmas):
        item(f"dma{i}", 1 + i, 3 + 2 * i, 2, lambda m0=m0, ld=ld: (e.m0(m0), e.dma(ld)))

    def take(it):
        it["fn"]()
        items.remove(it)

    for k in range(64):
        e.mfma(k // 8, k % 8)
        room = STEP_SLOTS
        while room > 0:
            r = [it for it in sorted(items, key=lambda it: it["last"]) if it["first"] <= k and it["size"] <= room]
            if not r:
                break
            room -= r[0]["size"]
            take(r[0])
        for it in sorted(items, key=lambda it: it["last"]):
            if it["first"] <= k and it["last"] <= k:
                take(it)
    assert not items, [it["name"] for it in items]
    e.emit(f"s_waitcnt vmcnt({PF_LOADS if copies else 0}) lgkmcnt(0)")
    e.pending = []
    e.emit("s_barrier")
    return e.lines


def gen_prologue():
    """Copies (and prefetches) of the first slices; the accumulators are zeroed while they fly."""
    e = Emitter()
    e.emit("s_add_u32 %[ssp], %[ssa], %[sstep]")
    e.emit("s_add_u32 %[ssq], %[ssb], %[sstepb]")
    for m0, ld in copy_items(0):
        e.m0(m0)
        e.dma(ld)
    for r in range(256):
        e.emit(f"v_accvgpr_write_b32 a{r}, 0")
    e.emit(f"s_waitcnt vmcnt({PF_LOADS})")
    e.emit("s_barrier")
    return e.lines


def gen_tail():
    """After the last slice: every prefetch landed (its LDS area is outside the epilogue's staging
    only while the K loop runs), and wait states between the last MFMAs and the reads of their
    accumulators that follow the statement."""
    e = Emitter()
    e.emit("s_waitcnt vmcnt(0)")
    e.nops(MFMA_READ_WAIT)
    return e.lines


def macro(name, lines):
    out = [f"#define {name} \\"]
    out += [f'  "{ln}\\n\\t" \\' for ln in lines]
    out.append('  ""')
    return "\n".join(out) + "\n"


def main(out_path=None):
    here = os.path.dirname(os.path.abspath(__file__))
    blocks = {(stage, copies): gen_slice(stage, copies) for stage in (0, 1) for copies in (True, False)}
    loop = gen_prologue()
    loop += ["s_cmp_le_i32 %[pairs], 0", "s_cbranch_scc1 L_w4mx_rem%=", "L_w4mx_loop%=:"]
    loop += blocks[(0, True)] + blocks[(1, True)]
    loop += ["s_sub_i32 %[pairs], %[pairs], 1", "s_cmp_gt_i32 %[pairs], 0", "s_cbranch_scc1 L_w4mx_loop%=",
             "L_w4mx_rem%=:", "s_cmp_eq_i32 %[rem], 2", "s_cbranch_scc0 L_w4mx_one%="]
    loop += blocks[(0, True)] + blocks[(1, False)]
    loop += ["s_branch L_w4mx_tail%=", "L_w4mx_one%=:"]
    loop += blocks[(0, False)]
    loop += ["L_w4mx_tail%=:"] + gen_tail()
    with open(out_path or os.path.join(here, "gemm_w4mx_asm.inc"), "w") as f:
        f.write("// Generated by gen_w4mx_asm.py -- the K loop of the four-wave MXFP8 GEMM (see there).\n")
        f.write(macro("PURO_W4MX_MAINLOOP", loop))
        f.write("// VGPRs the slice blocks write besides their operands (fragments and scale bytes)\n")
        f.write("#define PURO_W4MX_CLOBBERS " + ", ".join(f'"v{r}"' for r in range(0, 144)) + "\n")
    n = {k: len(v) for k, v in blocks.items()}
    print("instructions per slice block:", n)


if __name__ == "__main__":
    import sys
    main(sys.argv[1] if len(sys.argv) > 1 else None)
