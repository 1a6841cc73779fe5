"""Generate gemm_slice_asm.inc: the hand-scheduled gfx950 instruction sequence for one
128-deep slice of the blockwise-scaled FP8 GEMM (FWD / DGRAD, row-scale promotion).

    python blockwise_scaled_fp8_quant_amd/csrc/gen_slice_asm.py   # rewrites gemm_slice_asm.inc

The generated text is committed; the library build does not run this script.

Register map (per lane; pinned by the asm statement's constraints and clobbers):
  v[0:127]    accumulators: output tile T = 2*ni + mi (32 x 32, 16 fp32 per lane) in v[16T:16T+15]
  v[128:143]  slice product P of even tiles (clobbered)
  v[144:159]  slice product P of odd tiles; tile 7's product is carried out of the block and
              promoted at the start of the next block (or by the tail block after the loop)
  v[160:175]  A fragment, row group mi = 0 (4 x 16-byte LDS chunks per lane)
  v[176:191]  A fragment, row group mi = 1
  v[192:207]  B fragment buffer 0 (column tiles ni = 0, 2), v[208:223] buffer 1 (ni = 1, 3)
Operands: %[aj0..3] / %[bj0..3] LDS byte addresses of this lane's 4 swizzled 16-byte chunks in
its A / B row (row group / column tile offsets are 4096-byte immediates); %[sc0], %[sc1] the
promotion scale of row group 0 / 1 for this slice; %[scp] the scale of the carried product;
for the copy of the next slice into the other LDS stage: %[ga0..3] / %[gb0..3] the
(wave-uniform) global addresses of the wave's four 8-row groups of A / B at that slice,
%[oa0], %[oa1] / %[ob0], %[ob1] the lane's byte offset within an even / odd group (row in
group and swizzled chunk), %[m0] the LDS address of the wave's first A row in the other stage.

Schedule:
  entry   read the first B fragment and the A fragment of row group 0; pad; promote the
          carried tile-7 product of the previous slice; read the A fragment of row group 1;
          wait for the first eight reads only.
  step s  (s = 0..7, tile (ni, mi) = (s >> 1, s & 1)):
          1. wait for this step's fragments (the B fragment read two steps earlier, or A of
             row group 1), counting only the older reads;
          2. the two chained MFMAs of tile s, back to back (the second accumulates on the
             first: v_mfma_f32_32x32x64_f8f6f4, one 128-deep slice of a 32 x 32 tile);
          3. one of the eight global_load_lds_dwordx4 copies of the next slice (M0 = LDS
             destination, one wait state after the M0 write): spreading the copies over the
             slice keeps the address unit's queue from stalling the wave;
          4. on mi == 0, the four LDS reads of the next column tile's B fragment (into the
             other buffer, last read by the MFMAs two instructions earlier);
          5. padding so that at least 20 wait states separate the MFMA that produced tile
             s-1's product from its first VALU read (the spacing the compiler's own hazard
             recognizer uses for 16-pass XDL results on gfx950);
          6. the 16 promotion FMAs of tile s-1:  C_acc += P * sc.
  exit    wait for this wave's copies, then meet the other waves at the barrier.
Every LDS read is waited for inside the block.
"""
import os

HAZARD_WAIT_STATES = 20


def nops(n):
    out = []
    while n > 0:
        k = min(n, 16)
        out.append(f"s_nop {k - 1}")
        n -= k
    return out


def dma(k):
    """Copy k of the next slice: group q = k >> 1, A for even k, B for odd k."""
    q = k >> 1
    if k & 1 == 0:
        return [f"s_add_u32 m0, %[m0], {q * 8 * 128}", "s_nop 0",
                f"global_load_lds_dwordx4 %[oa{q & 1}], %[ga{q}]"]
    return [f"s_add_u32 m0, %[m0], {32768 + q * 8 * 128}", "s_nop 0",
            f"global_load_lds_dwordx4 %[ob{q & 1}], %[gb{q}]"]


def reads(dst, addr, offset):
    return [f"ds_read_b128 v[{dst + 4 * j}:{dst + 4 * j + 3}], %[{addr}{j}] offset:{offset}" for j in range(4)]


def fmas(T, p, sc):
    return [f"v_fmac_f32 v{16 * T + v}, v{p + v}, %[{sc}]" for v in range(16)]


def waits(n_instr):
    """Wait states an instruction list contributes (s_nop k counts k + 1)."""
    return n_instr


def generate():
    L = []
    # entry
    L += reads(192, "bj", 0)            # B, column tile 0 -> buffer 0
    L += reads(160, "aj", 0)            # A, row group 0
    L += nops(HAZARD_WAIT_STATES - 8)   # carried product came from the previous block's last MFMA
    L += fmas(7, 144, "scp")
    L += reads(176, "aj", 4096)         # A, row group 1
    L.append("s_waitcnt lgkmcnt(4)")
    for s in range(8):
        ni, mi = s >> 1, s & 1
        bb = 192 + 16 * (ni & 1)
        ab = 160 + 16 * mi
        p = 128 + 16 * (s & 1)
        if s == 1:
            L.append("s_waitcnt lgkmcnt(4)")          # A row group 1 (B of tile 1 is newer)
        elif mi == 0 and ni > 0:
            L.append("s_waitcnt lgkmcnt(0)")          # B fragment read two steps earlier
        L.append(f"v_mfma_f32_32x32x64_f8f6f4 v[{p}:{p + 15}], v[{bb}:{bb + 7}], v[{ab}:{ab + 7}], 0")
        L.append(f"v_mfma_f32_32x32x64_f8f6f4 v[{p}:{p + 15}], v[{bb + 8}:{bb + 15}], v[{ab + 8}:{ab + 15}], v[{p}:{p + 15}]")
        ws = 2
        d = dma(s)
        L += d
        ws += 3 + 0                                    # s_add, s_nop 0 (1 wait state), load
        if mi == 0 and ni < 3:
            L += reads(192 + 16 * ((ni + 1) & 1), "bj", (ni + 1) * 4096)
            ws += 4
        if s > 0:
            L += nops(HAZARD_WAIT_STATES - ws)
            q = s - 1
            L += fmas(2 * (q >> 1) + (q & 1), 128 + 16 * (q & 1), f"sc{q & 1}")
    L.append("s_waitcnt vmcnt(0) lgkmcnt(0)")
    L.append("s_barrier")
    return L


def generate_tail():
    """After the last slice: promote the carried tile-7 product."""
    return nops(HAZARD_WAIT_STATES) + fmas(7, 144, "scp")


def main():
    lines = generate()
    here = os.path.dirname(os.path.abspath(__file__))
    with open(os.path.join(here, "gemm_slice_asm.inc"), "w") as f:
        f.write("// Generated by gen_slice_asm.py -- one 128-deep slice of the FWD/DGRAD GEMM (see there).\n")
        f.write("#define PURO_SLICE_ASM_ROWSCALE \\\n")
        for ln in lines:
            f.write(f'  "{ln}\\n\\t" \\\n')
        f.write('  ""\n')
        f.write("// promotion of the carried product after the last slice\n")
        f.write("#define PURO_SLICE_ASM_ROWSCALE_TAIL \\\n")
        for ln in generate_tail():
            f.write(f'  "{ln}\\n\\t" \\\n')
        f.write('  ""\n')
        f.write("// VGPRs the block uses besides the pinned accumulators and the carried product\n")
        f.write("#define PURO_SLICE_ASM_CLOBBERS " + ", ".join(f'"v{r}"' for r in list(range(128, 144)) + list(range(160, 224))) + "\n")
    print(f"{len(lines)} instructions")


if __name__ == "__main__":
    main()
