"""Generate gemm_w4_asm.inc: the hand-scheduled gfx950 instruction sequence of one 128-deep slice of
the blockwise-scaled FP8 GEMM in its four-wave form (one wave per SIMD, a 128 x 128 output tile per
wave, FWD and DGRAD: one promotion scale per row).

    python blockwise_scaled_fp8_quant_amd/csrc/gen_w4_asm.py     # rewrites gemm_w4_asm.inc

The generated text is committed; the library build does not run this script.

Why this shape.  With every 128-deep slice product promoted by the vector ALUs into a separate fp32
accumulator, a wave's accumulator has to live mostly in architectural VGPRs.  At two waves per SIMD a
wave has 256 registers in all, which caps its tile at 64 x 128; each slice it then reads 64 + 128 rows
of 128 bytes from LDS for 2 * 64 * 128 * 128 flops.  At one wave per SIMD a wave has 256 VGPRs plus 256
AGPRs: its operand fragments can sit in AGPRs (the FP8 MFMA reads them there), 7/8 of a 128 x 128
accumulator in VGPRs and the last 1/8 in AGPRs, so each wave reads 128 + 128 rows per slice for twice
the flops -- a third less LDS read traffic per flop for the same 256 x 256 block tile.

Per slice a wave issues 64 v_mfma_f32_16x16x128_f8f6f4 (E4M3 x E4M3 -> fp32, one 128-deep slice of a
16 x 16 output tile each, 8 passes).  Operand roles are swapped (the B fragment is the instruction's
first source), so lane l holds row l % 16 of its 16-row group and the 4 adjacent columns
4 (l / 16) .. + 3 of the 16-column group: one row scale per lane and row group, and (FWD / DGRAD) one
128 x 128 weight-block scale per wave, so the promotion of a tile is 4 FMAs: C += P * sc.

Register map (per lane):
  v[0:223]    accumulators of tiles (mi, ni), ni < 7: v[4 (7 mi + ni) : + 3]
  a[0:31]     accumulators of tiles (mi, 7): a[4 mi : + 3]  (promoted through the temporaries)
  a[32:95]    A fragments, row group mi: a[32 + 8 mi : + 7]  (32 bytes of the row's slice)
  a[96:159]   B fragments, column group ni: a[96 + 8 ni : + 7]
  v[224:235]  slice products P, three buffers: MFMA k of a slice writes buffer k % 3
  v[236:237]  promotion scales sa(row) * sw of the even / odd row group being promoted
  v[238:241]  temporaries of the AGPR-tile promotion (read, FMA, write back)
  v242        sw: this slice's weight-block scale of the wave's 128 columns
  v[243:246]  copy offsets (row in 8-row group, swizzled chunk, and the K offset of the slice
              being copied) for even / odd groups of A and of B
Operands: %[aj0], %[aj1] / %[bj0], %[bj1]: LDS byte addresses of the lane's two 16-byte chunks in its
A / B row of stage 0 (stage, row group and column group offsets are immediates); %[sj]: LDS address
of the lane's row scale in stage 0 (row group offsets are immediates); %[swj]: LDS address of the
wave's weight-block scale in stage 0; %[osa]: the lane's offset for the sa copy; %[rA], %[rB], %[rS],
%[rW]: buffer resources of the tile's A rows, B rows, row scales, weight-block scales; s[64:71] /
s[72:79]: the byte offsets of the wave's 8-row copy groups in A / B; %[ssa], %[ssw]: offsets of the
slice being copied in the row-scale and weight-scale arrays; %[sstep]: bytes between slices of the
row scales; %[mw] / %[ms]: the wave's LDS base for its tile copies / scale copies.

LDS (bytes): stage s holds A rows at 32768 s + 128 r, B rows at 65536 + 32768 s + 128 r (chunk c of
row r at c ^ ((r >> 1) & 7): the 16 rows one ds_read_b128 quarter-wave touches land in 16 distinct
4-bank groups); row scales at 131072 + 2048 s (256 floats in row order) and 64 copies of each
wave's weight-block scale at 131072 + 2048 s + 1024 + 256 w.

Copies: each wave copies A rows 64 w .. 64 w + 63 and B rows 64 w .. + 63 of the next slice as 8-row
groups (buffer_load_dwordx4 ... lds: 64 lanes x 16 bytes, M0 = LDS destination), plus 64 row scales
and its own weight-block scale.  The buffer resources clamp reads past the last valid row to 0.

The K loop (prologue, slices, tail) is a single asm statement, so the compiler keeps one register
assignment for all of it.

Schedule of a slice (after the previous slice's barrier: this slice is in LDS, every wave is done
with the other stage):
  entry    fragment reads for the first MFMAs; the weight scale and the first row scale; the
           promotions of the previous slice's last two products (tile (7, 6) in P buffer 2; tile
           (7, 7) in P buffer 0, its AGPR values in the temporaries); the copy offsets advance to
           the next slice.
  step k   (k = 0 .. 63, tile (mi, ni) = (k / 8, k % 8))  wait for its fragments; the MFMA; up to
           three slots of the slice's other instructions (fragment reads for later steps, copies,
           row-scale reads and products, AGPR reads / writes); the 4 FMAs promoting product
           k - 2.  With two products in flight the promotion is always far enough behind its
           MFMA, so a step is 8 issue slots: the 8 passes of its MFMA.
  exit     wait for this wave's copies and reads, then the barrier.
Hazards (figures from the compiler's own hazard recognizer for gfx950): a VALU read of a
v_mfma_f32_16x16x128_f8f6f4 result needs 12 wait states after the MFMA; M0 written by SALU needs
one before an LDS-DMA load; the generator counts issued instructions between producer and
consumer and pads with s_nop only where fewer separate them.  Every LDS read is waited for (in
order, lgkmcnt) before its registers are read, and never more than 15 are outstanding.
"""
import os

MFMA_VALU_WAIT = 12            # v_mfma_f32_16x16x128_f8f6f4 result -> VALU read
STEP_SLOTS = 8                 # issue slots one MFMA's 8 passes leave a single wave (4 cycles each)
STAGE_BYTES = 32768
B_BASE = 65536
S_BASE = 131072
S_STAGE = 2048

P_BUF = (224, 228, 232)
SC = (236, 237)
TMP = 238
SW = 242
VOFF = {"oa0": 243, "oa1": 244, "ob0": 245, "ob1": 246}
PF = {"pa": 247, "pb": 248}    # prefetch offsets: lane's row of A / B, two slices ahead
PF_LDS = 135168                # 256 bytes the prefetches land in (never read)
PF_LOADS = 3                   # prefetch loads per slice (A rows, B rows, row scales)
QA, QB = 64, 72                # s[64:71], s[72:79]


def acc_v(mi, ni):
    return 4 * (7 * mi + ni)


def frag_a(mi):
    return 32 + 8 * mi


def frag_b(ni):
    return 96 + 8 * ni


class Emitter:
    def __init__(self):
        self.lines = []
        self.ws = 0
        self.pending = []            # register sets of outstanding LDS reads, oldest first
        self.mfma_at = {}            # P buffer -> wait-state count right after the MFMA writing it
        self.m0_at = None

    def emit(self, ln, ws=1):
        self.lines.append(ln)
        self.ws += ws

    def nops(self, n):
        while n > 0:
            k = min(n, 16)
            self.emit(f"s_nop {k - 1}", k)
            n -= k

    # ---- LDS reads and waits
    def ds_read(self, kind, dst_regs, text):
        regs = set(dst_regs)
        for p in self.pending:
            assert not (p & regs), f"LDS read overwrites registers of a pending read: {text}"
        self.emit(text)
        self.pending.append(regs)
        assert len(self.pending) <= 15, "more than 15 LDS reads outstanding"

    def wait_for(self, regs):
        """lgkmcnt wait so that every pending read writing any of regs has completed."""
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

    def use(self, regs):
        for p in self.pending:
            assert not (p & set(regs)), f"register {sorted(p & set(regs))[:2]} read before its LDS read completed"

    # ---- MFMA and promotion
    def mfma(self, k, mi, ni):
        a, b = frag_a(mi), frag_b(ni)
        regs = [f"a{r}" for r in range(a, a + 8)] + [f"a{r}" for r in range(b, b + 8)]
        self.wait_for(regs)
        p = P_BUF[k % 3]
        self.emit(f"v_mfma_f32_16x16x128_f8f6f4 v[{p}:{p + 3}], a[{b}:{b + 7}], a[{a}:{a + 7}], 0")
        self.mfma_at[p] = self.ws

    def hazard(self, p):
        self.nops(MFMA_VALU_WAIT - (self.ws - self.mfma_at[p]))

    def promote_v(self, p, mi, ni, sc):
        self.use({f"v{sc}"})
        self.hazard(p)
        base = acc_v(mi, ni)
        for j in range(4):
            self.emit(f"v_fmac_f32 v{base + j}, v{p + j}, v{sc}")

    def promote_t(self, p, sc):
        """FMAs of an AGPR tile's product into the temporaries (which hold its accumulator)."""
        self.use({f"v{sc}"} | {f"v{TMP + j}" for j in range(4)})
        self.hazard(p)
        for j in range(4):
            self.emit(f"v_fmac_f32 v{TMP + j}, v{p + j}, v{sc}")

    def agpr_read(self, mi, j):
        self.emit(f"v_accvgpr_read_b32 v{TMP + j}, a{4 * mi + j}")

    def agpr_write(self, mi, j):
        self.emit(f"v_accvgpr_write_b32 a{4 * mi + j}, v{TMP + j}")

    # ---- copies (LDS DMA)
    def m0(self, text):
        self.emit(text)
        self.m0_at = self.ws

    def dma(self, text):
        # an LDS-DMA load reads M0 one wait state after the SALU write at the earliest
        if self.m0_at is not None and self.ws - self.m0_at < 1:
            self.nops(1)
        self.emit(text)


def copy_items(stage_next):
    """(m0 instruction, load instruction) pairs copying the next slice into stage `stage_next`."""
    out = []
    so = stage_next * STAGE_BYTES
    for q in range(8):                                       # A groups, then B groups
        out.append((f"s_add_u32 m0, %[mw], {so + q * 1024}",
                    f"buffer_load_dwordx4 v{VOFF['oa0' if q % 2 == 0 else 'oa1']}, %[rA], s{QA + q} offen lds"))
    for q in range(8):
        out.append((f"s_add_u32 m0, %[mw], {B_BASE + so + q * 1024}",
                    f"buffer_load_dwordx4 v{VOFF['ob0' if q % 2 == 0 else 'ob1']}, %[rB], s{QB + q} offen lds"))
    ss = stage_next * S_STAGE                                # %[ms] holds 131072 + 256 w
    out.append((f"s_add_u32 m0, %[ms], {ss}", "buffer_load_dword %[osa], %[rS], %[ssa] offen lds"))
    out.append((f"s_add_u32 m0, %[ms], {ss + 1024}", "buffer_load_dword off, %[rW], %[ssw] lds"))
    # interleave A and B groups so both operands arrive at the same pace
    a, b, s = out[:8], out[8:16], out[16:]
    inter = []
    for q in range(8):
        inter += [a[q], b[q]]
    return s + inter + prefetch_items()


def prefetch_items():
    """Loads that pull the slice after the one being copied into L2 (one dword per row of the wave's
    64 A rows, 64 B rows and 64 row scales, landing in an LDS area nobody reads; the per-lane A and B
    offsets the kernel sets up point each run of lanes at one row, so that the tiles resident on an
    XCD request each shared line once).  Issued after the copies: loads complete in order, so
    waiting for the copies with vmcnt(PF_LOADS) leaves them in flight."""
    return [(f"s_mov_b32 m0, {PF_LDS}", f"buffer_load_dword v{PF['pa']}, %[rA], s{QA} offen lds"),
            (f"s_mov_b32 m0, {PF_LDS}", f"buffer_load_dword v{PF['pb']}, %[rB], s{QB} offen lds"),
            (f"s_mov_b32 m0, {PF_LDS}", "buffer_load_dword %[osa], %[rS], %[ssp] offen lds")]


def gen_slice(stage, copies, carried_ws):
    """carried_ws: wait states that at least separate the previous block's last MFMA from this
    block's first instruction."""
    e = Emitter()
    e.mfma_at[P_BUF[0]] = -carried_ws          # product 63 of the previous slice
    e.mfma_at[P_BUF[2]] = -carried_ws - 8      # product 62
    st = stage * STAGE_BYTES
    sst = stage * S_STAGE

    def read_a(mi):
        a = frag_a(mi)
        e.ds_read("A", [f"a{r}" for r in range(a, a + 4)], f"ds_read_b128 a[{a}:{a + 3}], %[aj0] offset:{st + 2048 * mi}")
        e.ds_read("A", [f"a{r}" for r in range(a + 4, a + 8)], f"ds_read_b128 a[{a + 4}:{a + 7}], %[aj1] offset:{st + 2048 * mi}")

    def read_b(ni):
        b = frag_b(ni)
        e.ds_read("B", [f"a{r}" for r in range(b, b + 4)], f"ds_read_b128 a[{b}:{b + 3}], %[bj0] offset:{st + 2048 * ni}")
        e.ds_read("B", [f"a{r}" for r in range(b + 4, b + 8)], f"ds_read_b128 a[{b + 4}:{b + 7}], %[bj1] offset:{st + 2048 * ni}")

    def read_sa(mi):
        # row scale of row group mi (rows 128 wm + 16 mi + l % 16) into SC[mi % 2]
        e.ds_read("S", {f"v{SC[mi % 2]}"}, f"ds_read_b32 v{SC[mi % 2]}, %[sj] offset:{sst + 64 * mi}")

    def scale_product(mi):
        r = SC[mi % 2]
        e.wait_for({f"v{r}", f"v{SW}"})
        e.emit(f"v_mul_f32 v{r}, v{r}, v{SW}")

    # ---------------- entry
    read_a(0)
    read_b(0)
    read_b(1)
    e.ds_read("W", {f"v{SW}"}, f"ds_read_b32 v{SW}, %[swj] offset:{sst}")
    read_sa(0)
    # carried promotions of the previous slice's tiles (7, 6) and (7, 7) (scale SC[1]); (7, 7)'s
    # accumulator is in the temporaries
    e.promote_v(P_BUF[2], 7, 6, SC[1])
    e.promote_t(P_BUF[0], SC[1])
    for j in range(4):
        e.agpr_write(7, j)
    read_sa(1)                        # SC[1] is free once the carried FMAs have read it
    if copies:
        for r in list(VOFF.values()) + list(PF.values()):
            e.emit(f"v_add_u32 v{r}, 128, v{r}")
        e.emit("s_add_u32 %[ssa], %[ssa], %[sstep]")
        e.emit("s_add_u32 %[ssp], %[ssa], %[sstep]")
        e.emit("s_add_u32 %[ssw], %[ssw], 4")
    dmas = copy_items(stage ^ 1) if copies else []

    # The rest of the slice's instructions, as items for a list scheduler: an item becomes ready at
    # step `first` (after the items in `after` were emitted) and must be emitted by step `last`.
    # Each step issues its MFMA, then ready items while the promotion of the previous product is
    # not yet allowed (MFMA -> VALU distance), the promotion, then more ready items up to
    # STEP_SLOTS instructions (items whose last step has come are emitted regardless).
    items = []

    def item(name, first, last, size, fn, after=()):
        items.append({"name": name, "first": first, "last": last, "size": size, "fn": fn, "after": set(after)})

    for ni in range(2, 8):
        item(f"rb{ni}", 0, max(ni - 2, 0), 2, lambda ni=ni: read_b(ni))
    for mi in range(7):
        item(f"ra{mi + 1}", 8 * mi, 8 * mi + 5, 2, lambda mi=mi: read_a(mi + 1))
    # row mi's products are promoted at steps 8 mi + 2 .. 8 mi + 9 with SC[mi % 2]
    item("sp0", 0, 1, 2, lambda: scale_product(0))
    item("sp1", 0, 9, 2, lambda: scale_product(1))
    for mi in range(2, 8):
        # SC[mi % 2] is free once row mi - 2's last product (promoted at step 8 mi - 7) is done
        item(f"rs{mi}", 8 * mi - 6, 8 * mi - 3, 1, lambda mi=mi: read_sa(mi))
        item(f"sp{mi}", 8 * mi - 5, 8 * mi + 1, 2, lambda mi=mi: scale_product(mi), after=[f"rs{mi}"])
    for mi in range(8):
        prev = [f"aw{mi - 1}.{j}" for j in range(4)] if mi > 0 else []
        for j in range(4):
            item(f"ar{mi}.{j}", 8 * mi + 1, 8 * mi + 8, 1, lambda mi=mi, j=j: e.agpr_read(mi, j), after=prev)
        if mi < 7:
            for j in range(4):
                # after the promotion of product 8 mi + 7 (step 8 mi + 9): `first` one step later
                item(f"aw{mi}.{j}", 8 * mi + 10, 8 * mi + 15, 1, lambda mi=mi, j=j: e.agpr_write(mi, j))
    # copies of the next slice: early in the slice (an operand tile read from HBM rather than L2
    # takes the longest), at most about one per step
    for i, (m0, ld) in enumerate(dmas):
        item(f"dma{i}", 1 + i, 3 + 2 * i, 2, lambda m0=m0, ld=ld: (e.m0(m0), e.dma(ld)))

    done = set()

    def ready(k):
        return [it for it in items if it["first"] <= k and it["after"] <= done]

    def take(it):
        it["fn"]()
        done.add(it["name"])
        items.remove(it)

    # ---------------- steps
    for k in range(64):
        mi, ni = k // 8, k % 8
        start = e.ws
        e.mfma(k, mi, ni)
        prom = None
        if k >= 2:
            q = k - 2
            prom = (P_BUF[q % 3], q // 8, q % 8)
        # before the promotion: up to STEP_SLOTS - 5 slots of ready items (most urgent first); they
        # also cover the MFMA -> VALU distance, s_nop pads what they leave
        room = STEP_SLOTS - 1 - 4
        while room > 0:
            r = [it for it in sorted(ready(k), key=lambda it: it["last"]) if it["size"] <= room]
            if not r:
                break
            room -= r[0]["size"]
            take(r[0])
        if prom is not None:
            p, qm, qn = prom
            if qn == 7:
                e.promote_t(p, SC[qm % 2])
            else:
                e.promote_v(p, qm, qn, SC[qm % 2])
        # items whose last step has come go out regardless
        for it in sorted(ready(k), key=lambda it: it["last"]):
            if it["last"] <= k:
                take(it)
    assert not items, [it["name"] for it in items]
    # exit: products 62 (tile (7, 6), buffer 2) and 63 (tile (7, 7), buffer 0, its accumulator in the
    # temporaries) are carried to the next block
    e.emit(f"s_waitcnt vmcnt({PF_LOADS if copies else 0}) lgkmcnt(0)")
    e.pending = []
    e.emit("s_barrier")
    return e.lines, e.ws - e.mfma_at[P_BUF[0]]


def gen_prologue():
    """Copies of the first slice into stage 0 (the copy offsets already hold that slice); while they
    are in flight, zero the accumulators, the products and scales "carried" into the first slice
    (so its carried promotions add nothing) and the AGPR-tile temporaries."""
    e = Emitter()
    e.emit("s_add_u32 %[ssp], %[ssa], %[sstep]")
    for m0, ld in copy_items(0):
        e.m0(m0)
        e.dma(ld)
    for r in range(0, 242):
        if r not in (SW,):
            e.emit(f"v_mov_b32 v{r}, 0")
    for r in range(32):
        e.emit(f"v_accvgpr_write_b32 a{r}, 0")
    e.emit(f"s_waitcnt vmcnt({PF_LOADS})")
    e.emit("s_barrier")
    return e.lines


def gen_tail(carried_ws):
    """After the last slice: promote the carried tiles (7, 6) and (7, 7) and write (7, 7)'s
    accumulator back."""
    e = Emitter()
    e.mfma_at[P_BUF[0]] = -carried_ws
    e.mfma_at[P_BUF[2]] = -carried_ws - 8
    e.promote_v(P_BUF[2], 7, 6, SC[1])
    e.promote_t(P_BUF[0], SC[1])
    for j in range(4):
        e.agpr_write(7, j)
    return e.lines


def macro(name, lines):
    out = [f"#define {name} \\"]
    out += [f'  "{ln}\\n\\t" \\' for ln in lines]
    out.append('  ""')
    return "\n".join(out) + "\n"


def main(out_path=None):
    here = os.path.dirname(os.path.abspath(__file__))
    # the wait states every block leaves after its last MFMA bound what the next block (or the
    # tail) may assume; iterate once so the entry padding uses the blocks' own figure
    carried = 0
    for _ in range(2):
        blocks, after = {}, []
        for stage in (0, 1):
            for copies in (True, False):
                blocks[(stage, copies)], ws = gen_slice(stage, copies, carried)
                after.append(ws)
        carried = min(after)
    # The whole K loop is one asm statement (one register assignment for the compiler to honour):
    # the prologue copies the first slice; %[pairs] iterations run a stage-0 and a stage-1 slice
    # that both copy the slice after them; then the last one or two slices (%[rem]); then the tail.
    loop = gen_prologue()
    loop += ["s_cmp_le_i32 %[pairs], 0", "s_cbranch_scc1 L_w4_rem%=", "L_w4_loop%=:"]
    loop += blocks[(0, True)] + blocks[(1, True)]
    loop += ["s_sub_i32 %[pairs], %[pairs], 1", "s_cmp_gt_i32 %[pairs], 0", "s_cbranch_scc1 L_w4_loop%=",
             "L_w4_rem%=:", "s_cmp_eq_i32 %[rem], 2", "s_cbranch_scc0 L_w4_one%="]
    loop += blocks[(0, True)] + blocks[(1, False)]
    loop += ["s_branch L_w4_tail%=", "L_w4_one%=:"]
    loop += blocks[(0, False)]
    loop += ["L_w4_tail%=:"] + gen_tail(carried)
    with open(out_path or os.path.join(here, "gemm_w4_asm.inc"), "w") as f:
        f.write("// Generated by gen_w4_asm.py -- the K loop of the four-wave FP8 GEMM (see there).\n")
        f.write(macro("PURO_W4_MAINLOOP", loop))
        f.write("// AGPRs the slice blocks write besides the accumulators (operand fragments)\n")
        f.write("#define PURO_W4_CLOBBERS " + ", ".join(f'"a{r}"' for r in range(32, 160)) + "\n")
    n = {k: len(v) for k, v in blocks.items()}
    print("instructions per slice block:", n, "carried wait states", carried)


if __name__ == "__main__":
    import sys
    main(sys.argv[1] if len(sys.argv) > 1 else None)
