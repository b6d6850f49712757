"""Writes gemm_loop.inc: the main loop of the 4-wavefront 256 x 256 bf16 GEMM
kernel (gemm.hip, gemm_bf16_sched_kernel) as one inline-assembly block per
operand layout. Run from this directory: python3 gen_gemm_loop.py

Why assembly: the schedule below keeps the matrix cores fed from a single
wavefront per SIMD, which needs every LDS read issued a whole k-tile before
its MFMA and the direct-to-LDS copies spread between the MFMAs; the compiler
reorders such code into just-in-time reads.

Block: 4 wavefronts (2 x 2), each owning a 128 x 128 quarter of the output
tile as 4 x 4 MFMA 32x32x16 accumulators (256 AGPRs). Contraction tiles are 32
deep; LDS holds 4 of them (stages), each [A 256 x 32 | B 256 x 32] bf16 = 32
KB:
  - a k-contiguous operand sits as [row][32 k], 16-byte chunk c of row r at
    chunk c ^ ((r >> 2) & 3) (conflict-free for 128-bit reads);
  - an operand whose contraction index is not the contiguous one sits as
    [32 k][256 rows], chunk c of k-row k at c ^ ((k & 3) << 2), and its
    fragments come from pairs of 64-bit transpose reads (ds_read_b64_tr_b16).
Copies go global -> LDS directly (global_load_lds_dwordx4, 1 KB per wavefront
instruction, 8 per wavefront per tile); the lanes pick their source chunks so
that the fixed lane -> LDS order lands the swizzled layout.

Schedule of one k-tile t (stage t % 4), per wavefront:
  wait for the copy of tile t+1 (vmcnt) and barrier -- after it, every
  wavefront has finished reading tile t-1 and tile t+1 has landed;
  16 MFMAs on the fragments of tile t, step 0 (k 0..15), with the fragment
  reads of tile t+1 step 0 and the 8 copies of tile t+3 (into tile t-1's
  stage) between them;
  16 MFMAs on tile t step 1 (k 16..31), with the reads of tile t+1 step 1.
Fragments live in two register sets (128 VGPRs, v128..v255) that alternate
between tiles, so every read has a whole tile of MFMAs to land in. The loop
body covers 4 tiles (one per stage, so that all LDS offsets are immediates).
Copies past the last tile re-read the last tile (the source offset stops
advancing), which keeps the wait counts uniform; those stages are never used.
A contraction of KT 32-deep tiles that is not a multiple of 4 enters the body
at slot (-KT mod 4) (one prologue per entry slot), so every k-tile count ends
with the body's last slot.

Operands of the asm block (names used below):
  c00..c33   accumulators ("+a", f32x16), cIJ = A fragment I x B fragment J
  voA0..3, voB0..3  per-lane byte offsets of this wavefront's 4 copy blocks
  rem        copies left before the source stops advancing; iters: loop count
             (passes over the body, the first one entered at slot `first`)
  ta, tb     scratch SGPRs
  ldsA/ldsB  LDS byte address of this wavefront's first copy block in stage 0
  sbA/sbB    global base addresses; ksA/ksB: bytes per 32-deep k-tile
  fa0..fa7, fb0..fb7  LDS fragment base addresses (see frag_base below)
"""

import os

STAGES = 4
KT_BYTES = 32 * 2          # one 32-deep k-tile of a k-contiguous row
STAGE_BYTES = 2 * 256 * 32 * 2
B_OFFSET = 256 * 32 * 2    # operand B follows A inside a stage

pairs = [(i, j) for i in range(4) for j in range(4)]


def freg(buf, kk, op, idx):
    """fragment register tuple: buffer 0/1, step kk, operand 0 (A) / 1 (B), fragment idx"""
    b = 128 + 64 * buf + 32 * kk + 16 * op + 4 * idx
    return b


def reads(layout, op, buf, stage, kk):
    """LDS reads of one operand's 4 fragments for one 16-deep step"""
    x = "ab"[op]
    hi = 1 if stage >= 2 else 0
    so = (stage & 1) * STAGE_BYTES
    out = []
    for i in range(4):
        r = freg(buf, kk, op, i)
        if layout == "kc":
            # base per (lo/hi, kk): fragments i are 32 rows (2 KB) apart
            out.append([f"ds_read_b128 v[{r}:{r + 3}], %[f{x}{2 * hi + kk}] offset:{so + i * 2048}"])
        else:
            # base per (lo/hi, i): step kk is 16 k-rows (8 KB) further, the second
            # half of the fragment 4 k-rows (2 KB)
            out.append([f"ds_read_b64_tr_b16 v[{r}:{r + 1}], %[f{x}{4 * hi + i}] offset:{so + kk * 8192}"])
            out.append([f"ds_read_b64_tr_b16 v[{r + 2}:{r + 3}], %[f{x}{4 * hi + i}] "
                        f"offset:{so + kk * 8192 + 2048}"])
    return out


def copies(stage):
    out = []
    for q in range(4):
        for x in "AB":
            out.append([f"s_add_u32 m0, %[lds{x}], {stage * STAGE_BYTES + q * 1024}",
                        "s_nop 0",   # M0 write -> LDS DMA needs one wait state
                        f"global_load_lds_dwordx4 %[vo{x}{q}], %[sb{x}]"])
    return out


def advance():
    out = ["s_cmp_gt_i32 %[rem], 0",
           "s_cselect_b32 %[ta], %[ksA], 0",
           "s_cselect_b32 %[tb], %[ksB], 0",
           "s_sub_i32 %[rem], %[rem], 1"]
    for x, t in (("A", "ta"), ("B", "tb")):
        for q in range(4):
            out.append(f"v_add_u32 %[vo{x}{q}], %[{t}], %[vo{x}{q}]")
    return out


def mfma(buf, kk, i, j):
    a, b = freg(buf, kk, 0, i), freg(buf, kk, 1, j)
    # (B fragment, A fragment): lane l ends up with row l % 32 of the A fragment
    return f"v_mfma_f32_32x32x16_bf16 %[c{i}{j}], v[{b}:{b + 3}], v[{a}:{a + 3}], %[c{i}{j}]"


def spread(mfmas, units):
    """the 16 MFMAs with the units (instruction groups) spread evenly between them"""
    out = []
    n = len(units)
    k = 0
    for m, ins in enumerate(mfmas):
        out.append(ins)
        while k < n and k * len(mfmas) < (m + 1) * n:
            out += units[k]
            k += 1
    assert k == n
    return out


def interleave(a, b):
    out = []
    for i in range(max(len(a), len(b))):
        if i < len(a):
            out.append(a[i])
        if i < len(b):
            out.append(b[i])
    return out


ORDERS = {
    "row": [(i, j) for i in range(4) for j in range(4)],
    "col": [(i, j) for j in range(4) for i in range(4)],
    "snake": [(i, j if i % 2 == 0 else 3 - j) for i in range(4) for j in range(4)],
}


def loop(la, lb, reads_first=False, copies_step=0, early=0, order="row"):
    """the asm lines for operand layouts la, lb ("kc" / "mn"). The defaults are
    the schedule described above; reads_first issues a step's fragment reads
    right after its first MFMA instead of spreading them, copies_step = 1 moves
    the copies into the second step, early = n issues a tile's first n MFMAs
    (whose fragments are already in registers) before its copy wait and
    barrier, order picks the accumulators' MFMA order within a step
    (measurement variants)."""
    pairs = ORDERS[order]
    nread = sum(4 if l == "kc" else 8 for l in (la, lb))   # LDS reads per 16-deep step
    wait_step = f"s_waitcnt lgkmcnt({min(nread, 15)})"
    L = ["s_nop 4"]   # accumulator initialisation (VALU/AGPR writes) -> MFMA
    # k-tile 0 runs in slot `first` of the 4-slot body (first = -KT mod 4), so
    # that any number of k-tiles ends with the body's last slot: one prologue
    # per entry slot
    for f in range(1, STAGES):
        L += [f"s_cmp_eq_u32 %[first], {f}", f"s_cbranch_scc1 L%=_pro{f}"]
    for f in range(STAGES):
        if f:
            L.append(f"L%=_pro{f}:")
        for t in range(STAGES - 1):
            for u in copies((f + t) % STAGES):
                L += u
            L += advance()
        L.append(f"s_waitcnt vmcnt({8 * (STAGES - 2)})")
        L.append("s_barrier")
        for kk in range(2):
            for u in reads(la, 0, f & 1, f, kk) + reads(lb, 1, f & 1, f, kk):
                L += u
        L.append(f"s_branch L%=_slot{f}")
    L.append("L%=_ktile:")
    for u in range(STAGES):
        X, Y = u & 1, (u + 1) & 1
        nxt, dst = (u + 1) % STAGES, (u + STAGES - 1) % STAGES
        L.append(f"L%=_slot{u}:")
        if early:
            L.append(wait_step)
            L += [mfma(X, 0, i, j) for i, j in pairs[:early]]
        L.append(f"s_waitcnt vmcnt({8 * (STAGES - 3)})")
        L.append("s_barrier")
        if not early:
            L.append(wait_step)
        for kk in range(2):
            r = reads(la, 0, Y, nxt, kk) + reads(lb, 1, Y, nxt, kk)
            c = copies(dst) + [advance()] if kk == copies_step else []
            m = [mfma(X, kk, i, j) for i, j in pairs]
            if kk == 0 and early:
                m = m[early:]
            if reads_first:
                L += [m[0]] + [x for u in r for x in u] + spread(m[1:], c)
            else:
                L += spread(m, interleave(r, c[:-1]) + c[-1:] if c else r)
            if kk == 0:
                L.append(wait_step)
    L += ["s_sub_i32 %[iters], %[iters], 1", "s_cmp_gt_i32 %[iters], 0", "s_cbranch_scc1 L%=_ktile"]
    L.append("s_waitcnt vmcnt(0) lgkmcnt(0)")
    L += ["s_nop 7"] * 3   # last MFMAs -> accumulator reads by the epilogue
    return L


LAYOUTS = (("NT", "kc", "kc"), ("NN", "kc", "mn"), ("TN", "mn", "mn"))


def render():
    """the text of gemm_loop.inc"""
    out = ["// Generated by gen_gemm_loop.py (the schedule is described there); do not edit.", ""]
    for name, la, lb in LAYOUTS:
        out.append(f"#define MTB_GEMM_LOOP_{name} \\")
        for line in loop(la, lb):
            out.append(f'  "{line}\\n" \\')
        out.append("")
    regs = ", ".join(f'"v{r}"' for r in range(128, 256))
    out.append(f"#define MTB_GEMM_LOOP_CLOBBERS {regs}")
    return "\n".join(out) + "\n"


def main():
    here = os.path.dirname(os.path.abspath(__file__))
    with open(os.path.join(here, "gemm_loop.inc"), "w") as f:
        f.write(render())


if __name__ == "__main__":
    main()
