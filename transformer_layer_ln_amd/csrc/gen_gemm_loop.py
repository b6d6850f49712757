"""Writes gemm_loop.inc: the main loops of the hand-scheduled bf16 GEMM
kernels (gemm.hip, sched_tile) as one inline-assembly block per tile shape and
operand layout. Run from this directory: python3 gen_gemm_loop.py

Why assembly: the schedules below keep the matrix cores fed with every LDS
read issued well before its MFMA and the direct-to-LDS copies spread between
the MFMAs; the compiler reorders such code into just-in-time reads.

Block: 4 wavefronts (2 x 2), each owning an (FM x 32) x (FN x 32) part of the
output tile as FM x FN MFMA 32x32x16 accumulators (16 AGPRs each): block tile
BM x BN = 64 FM x 64 FN. Contraction tiles are 32 deep; LDS holds STAGES of
them, each [A BM x 32 | B BN x 32] bf16:
  - a k-contiguous operand sits as [row][32 k], 16-byte chunk c of row r at
    chunk c ^ ((r >> 2) & 3) (conflict-free for 128-bit reads);
  - an operand whose contraction index is not the contiguous one sits as
    [32 k][rows], chunk c of k-row k at c ^ ((k & 3) << 2), and its fragments
    come from pairs of 64-bit transpose reads (ds_read_b64_tr_b16).
Copies go global -> LDS directly (global_load_lds_dwordx4, 1 KB per wavefront
instruction: BM / 64 of them per wavefront and k-tile for A, BN / 64 for B);
the lanes pick their source chunks so that the fixed lane -> LDS order lands
the swizzled layout.

Schedule of one k-tile t (stage t % STAGES), per wavefront (one block per
CU, 4 stages):
  wait for the copy of tile t+1 (vmcnt) and barrier -- after it, every
  wavefront has finished reading tile t-1 and tile t+1 has landed;
  the MFMAs of tile t, step 0 (k 0..15), with the fragment reads of tile t+1
  step 0 and the copies of tile t+3 (into tile t-1's stage) between them;
  the MFMAs of tile t step 1 (k 16..31), with the reads of tile t+1 step 1.
Fragments live in two register sets that alternate between tiles, so every
read has a whole tile of MFMAs to land in. The loop body covers the slots
whose LDS offsets and register sets repeat (STAGES tiles, STAGES even), so
every LDS offset is an immediate. Copies past the last tile re-read
the last tile (the source offset stops advancing), which keeps the wait
counts uniform; those stages are never used. A contraction of KT 32-deep
tiles enters the body at slot (-KT mod SLOTS) (one prologue per entry slot),
so every k-tile count ends with the body's last slot.

Operands of the asm block (names used below):
  cIJ        accumulators ("+a", f32x16), A fragment I x B fragment J
  voA0.., voB0..  per-lane byte offsets of this wavefront's copy blocks
  rem        copies left before the source stops advancing; iters: loop count
             (passes over the body, the first one entered at slot `first`)
  ta, tb     scratch SGPRs
  ldsA/ldsB  LDS byte address of this wavefront's first copy block in stage 0
  sbA/sbB    global base addresses; ksA/ksB: bytes per 32-deep k-tile
  fa0.., fb0..  LDS fragment base addresses (see Shape.bases)
"""

import os

KT_BYTES = 32 * 2          # one 32-deep k-tile of a k-contiguous row


class Shape:
    """A block tile of 2 x 2 wavefronts with FM x FN accumulators each."""

    def __init__(self, name, fm, fn, stages, frag_top=256):
        self.name, self.fm, self.fn, self.stages = name, fm, fn, stages
        self.bm, self.bn = 64 * fm, 64 * fn
        self.a_bytes, self.b_bytes = self.bm * KT_BYTES, self.bn * KT_BYTES
        self.stage_bytes = self.a_bytes + self.b_bytes
        self.b_offset = self.a_bytes            # operand B follows A inside a stage
        self.qa, self.qb = self.bm // 64, self.bn // 64   # copy blocks per wavefront and k-tile
        self.cpt = self.qa + self.qb
        self.sets = (stages + 1) // 2           # fragment base sets: stages 2i, 2i+1 share set i
        assert 2 * self.stage_bytes <= 65536 + self.stage_bytes and self.stage_bytes <= 32768
        nbuf = 2                                # register sets alternating between tiles
        assert stages % 2 == 0
        self.slots = stages
        self.per_step = 4 * (fm + fn)
        self.per_buf = 2 * self.per_step
        self.frag_lo = frag_top - nbuf * self.per_buf   # first fragment VGPR
        self.frag_hi = frag_top

    def freg(self, buf, kk, op, idx):
        """first VGPR of a fragment: register set buf, step kk, operand 0 (A) / 1 (B), fragment idx"""
        return self.frag_lo + self.per_buf * buf + self.per_step * kk + 4 * self.fm * op + 4 * idx

    def nfrag(self, op):
        return self.fm if op == 0 else self.fn

    def rows(self, op):
        return self.bm if op == 0 else self.bn

    def nbases(self, layout, op):
        """fragment base registers of one operand: kc -> one per (set, step); mn -> one per (set, fragment)"""
        return self.sets * (2 if layout == "kc" else self.nfrag(op))

    def base_index(self, layout, op, s, kk, i):
        st = s // 2
        return 2 * st + kk if layout == "kc" else self.nfrag(op) * st + i

    def read_offset(self, layout, op, s, kk, i, half=0):
        so = (s % 2) * self.stage_bytes
        if layout == "kc":
            return so + i * 2048      # fragments i are 32 rows (2 KB) apart
        # step kk is 16 k-rows further, the second half of the fragment 4 k-rows
        rb = self.rows(op) * 2
        return so + kk * 16 * rb + half * 4 * rb


# the kernels' shapes: 256 x 256, and 256 x 192 for the 1536-wide products
# (256 tiles instead of 192 on 256 CUs)
S256 = Shape("256", 4, 4, 4)
S192 = Shape("192", 4, 3, 4)
SHAPES = (S256, S192)

# the default shape's constants (used by the host-side checks)
STAGES = S256.stages
STAGE_BYTES = S256.stage_bytes
B_OFFSET = S256.b_offset


def freg(buf, kk, op, idx):
    return S256.freg(buf, kk, op, idx)


def reads(sh, layout, op, buf, stage, kk):
    """LDS reads of one operand's fragments for one 16-deep step"""
    x = "ab"[op]
    out = []
    for i in range(sh.nfrag(op)):
        r = sh.freg(buf, kk, op, i)
        b = sh.base_index(layout, op, stage, kk, i)
        if layout == "kc":
            out.append([f"ds_read_b128 v[{r}:{r + 3}], %[f{x}{b}] offset:{sh.read_offset(layout, op, stage, kk, i)}"])
        else:
            out.append([f"ds_read_b64_tr_b16 v[{r}:{r + 1}], %[f{x}{b}] "
                        f"offset:{sh.read_offset(layout, op, stage, kk, i, 0)}"])
            out.append([f"ds_read_b64_tr_b16 v[{r + 2}:{r + 3}], %[f{x}{b}] "
                        f"offset:{sh.read_offset(layout, op, stage, kk, i, 1)}"])
    return out


def copies(sh, stage):
    out = []
    for q in range(max(sh.qa, sh.qb)):
        for x, n in (("A", sh.qa), ("B", sh.qb)):
            if q < n:
                out.append([f"s_add_u32 m0, %[lds{x}], {stage * sh.stage_bytes + q * 1024}",
                            "s_nop 0",   # M0 write -> LDS DMA needs one wait state
                            f"global_load_lds_dwordx4 %[vo{x}{q}], %[sb{x}]"])
    return out


def advance(sh):
    out = ["s_cmp_gt_i32 %[rem], 0",
           "s_cselect_b32 %[ta], %[ksA], 0",
           "s_cselect_b32 %[tb], %[ksB], 0",
           "s_sub_i32 %[rem], %[rem], 1"]
    for x, t, n in (("A", "ta", sh.qa), ("B", "tb", sh.qb)):
        for q in range(n):
            out.append(f"v_add_u32 %[vo{x}{q}], %[{t}], %[vo{x}{q}]")
    return out


def mfma(sh, buf, kk, i, j):
    a, b = sh.freg(buf, kk, 0, i), sh.freg(buf, kk, 1, j)
    # (B fragment, A fragment): lane l ends up with row l % 32 of the A fragment
    return f"v_mfma_f32_32x32x16_bf16 %[c{i}{j}], v[{b}:{b + 3}], v[{a}:{a + 3}], %[c{i}{j}]"


def spread(mfmas, units):
    """the MFMAs with the units (instruction groups) spread evenly between them"""
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


def orders(sh):
    fm, fn = sh.fm, sh.fn
    return {
        "row": [(i, j) for i in range(fm) for j in range(fn)],
        "col": [(i, j) for j in range(fn) for i in range(fm)],
        "snake": [(i, j if i % 2 == 0 else fn - 1 - j) for i in range(fm) for j in range(fn)],
    }


ORDERS = orders(S256)


def nreads(sh, la, lb):
    """LDS read instructions per 16-deep step"""
    return sum(sh.nfrag(op) * (1 if l == "kc" else 2) for op, l in ((0, la), (1, lb)))


def loop(la, lb, reads_first=False, copies_step=0, early=0, order="row", sh=S256):
    """the asm lines for operand layouts la, lb ("kc" / "mn") and shape sh. The
    defaults are the schedules described above; reads_first issues a step's
    fragment reads right after its first MFMA instead of spreading them,
    copies_step = 1 moves the copies into the second step, early = n issues a
    tile's first n MFMAs (whose fragments are already in registers) before its
    copy wait and barrier, order picks the accumulators' MFMA order within a
    step (measurement variants)."""
    pairs = orders(sh)[order]
    S = sh.stages
    wait_step = f"s_waitcnt lgkmcnt({min(nreads(sh, la, lb), 15)})"
    L = ["s_nop 4"]   # accumulator initialisation (VALU/AGPR writes) -> MFMA
    # k-tile 0 runs in slot `first` of the body (first = -KT mod SLOTS), so
    # that any number of k-tiles ends with the body's last slot: one prologue
    # per entry slot
    for f in range(1, sh.slots):
        L += [f"s_cmp_eq_u32 %[first], {f}", f"s_cbranch_scc1 L%=_pro{f}"]
    for f in range(sh.slots):
        if f:
            L.append(f"L%=_pro{f}:")
        for t in range(S - 1):
            for u in copies(sh, (f + t) % S):
                L += u
            L += advance(sh)
        L.append(f"s_waitcnt vmcnt({sh.cpt * (S - 2)})")
        L.append("s_barrier")
        for kk in range(2):
            for u in reads(sh, la, 0, f & 1, f % S, kk) + reads(sh, lb, 1, f & 1, f % S, kk):
                L += u
        L.append(f"s_branch L%=_slot{f}")
    L.append("L%=_ktile:")
    for u in range(sh.slots):
        X, Y = u & 1, (u + 1) & 1
        nxt, dst = (u + 1) % S, (u + S - 1) % S
        L.append(f"L%=_slot{u}:")
        if early:
            L.append(wait_step)
            L += [mfma(sh, X, 0, i, j) for i, j in pairs[:early]]
        L.append(f"s_waitcnt vmcnt({sh.cpt * (S - 3)})")
        L.append("s_barrier")
        if not early:
            L.append(wait_step)
        for kk in range(2):
            r = reads(sh, la, 0, Y, nxt, kk) + reads(sh, lb, 1, Y, nxt, kk)
            c = copies(sh, dst) + [advance(sh)] if kk == copies_step else []
            m = [mfma(sh, X, kk, i, j) for i, j in pairs]
            if kk == 0 and early:
                m = m[early:]
            if reads_first:
                L += [m[0]] + [x for u2 in r for x in u2] + spread(m[1:], c)
            else:
                L += spread(m, interleave(r, c[:-1]) + c[-1:] if c else r)
            if kk == 0:
                L.append(wait_step)
    L += ["s_sub_i32 %[iters], %[iters], 1", "s_cmp_gt_i32 %[iters], 0", "s_cbranch_scc1 L%=_ktile"]
    L.append("s_waitcnt vmcnt(0) lgkmcnt(0)")
    L += ["s_nop 7"] * 3   # last MFMAs -> accumulator reads by the epilogue
    return L


LAYOUTS = (("NT", "kc", "kc"), ("NN", "kc", "mn"), ("TN", "mn", "mn"))
# which layouts each shape is built for: 256 x 192 only for the 1536-wide
# forward products (both operands k-contiguous)
SHAPE_LAYOUTS = {"256": LAYOUTS, "192": LAYOUTS[:1]}


def render():
    """the text of gemm_loop.inc"""
    out = ["// Generated by gen_gemm_loop.py (the schedule is described there); do not edit.", ""]
    for sh in SHAPES:
        suffix = "" if sh is S256 else "_" + sh.name
        for name, la, lb in SHAPE_LAYOUTS[sh.name]:
            out.append(f"#define MTB_GEMM_LOOP_{name}{suffix} \\")
            for line in loop(la, lb, sh=sh):
                out.append(f'  "{line}\\n" \\')
            out.append("")
        regs = ", ".join(f'"v{r}"' for r in range(sh.frag_lo, sh.frag_hi))
        out.append(f"#define MTB_GEMM_LOOP_CLOBBERS{suffix} {regs}")
        out.append("")
    return "\n".join(out)


def main():
    here = os.path.dirname(os.path.abspath(__file__))
    with open(os.path.join(here, "gemm_loop.inc"), "w") as f:
        f.write(render())


if __name__ == "__main__":
    main()
