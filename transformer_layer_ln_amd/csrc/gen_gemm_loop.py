"""Writes gemm_loop.inc: the main loops of the hand-scheduled bf16 GEMM
kernels (gemm.hip, sched_tile) as one inline-assembly block per tile shape and
operand layout. Run from this directory: python3 gen_gemm_loop.py

Why assembly: the schedules below keep the matrix cores fed with every LDS
read issued well before its MFMA and the memory operations spread between the
MFMAs; the compiler reorders such code into just-in-time reads.

Block: 2 x (W / 2) wavefronts, each owning an (FM x 32) x (FN x 32) part of
the output tile as FM x FN MFMA 32x32x16 accumulators (16 AGPRs each): block
tile BM x BN = 64 FM x 16 W FN. Contraction tiles are 32 deep. W = 4 (one
wavefront per SIMD, 128 x 128 each) or W = 8 (two per SIMD, 128 x 64 each: 128
accumulator AGPRs and at most 128 VGPRs per wavefront, so that while one
wavefront waits on its fragment reads, copies or the barrier, the other's
MFMAs keep the SIMD's matrix core busy; it reads 1.5x the LDS bytes per MFMA
and measured 4-7 % faster on the block's GEMMs with k-contiguous operands).
The copies of a k-tile are dealt evenly over the W wavefronts.

Operands reach the MFMAs one of two ways:
  - through LDS: LDS holds STAGES 32-deep tiles of the operand ([A BM x 32 |
    B BN x 32] per stage, for the operands that go this way), copied global ->
    LDS directly (global_load_lds_dwordx4, 1 KB per wavefront instruction:
    BM / 64 of them per wavefront and k-tile for A, BN / 64 for B; the lanes
    pick their source chunks so that the fixed lane -> LDS order lands the
    swizzled layout), then read into fragment registers:
      * a k-contiguous operand sits as [row][32 k], 16-byte chunk c of row r
        at chunk c ^ ((r >> 2) & 3) (conflict-free for 128-bit reads);
      * an operand whose contraction index is not the contiguous one sits as
        [32 k][rows], chunk c of k-row k at c ^ ((k & 3) << 2), and its
        fragments come from pairs of 64-bit transpose reads
        (ds_read_b64_tr_b16);
  - direct: a k-contiguous operand's MFMA fragment is 16 contiguous bytes of
    one row per lane (lane l: row l % 32, k 8 (l / 32) .. + 7), so each
    wavefront loads its own fragments from global memory straight into
    registers (global_load_dwordx4, 1 KB per instruction: 2 F per k-tile for
    the operand's F fragments). The two wavefronts that share those rows each
    load them (the second mostly from the L1 cache), but the operand takes no
    LDS bandwidth: with both operands through LDS, LDS traffic (copies in,
    fragment reads out) is what bounds the loop.
The direct path is a measurement variant (loop(direct="auto")): a direct
fragment load touches 32 rows x 32 bytes, twice the cache lines per byte of
an LDS copy, and the L1 / texture path it saturates made the loop slower than
with both operands through LDS.

Schedule of one k-tile t (slot t % STAGES), per wavefront (one block per CU,
4 stages):
  wait for the memory operations issued two tiles back (vmcnt: the copy of
  tile t+1, the direct fragments of tile t) and barrier -- after it every
  wavefront has finished reading tile t-1 and tile t+1 has landed;
  the MFMAs of tile t, step 0 (k 0..15), with the fragment reads of tile t+1
  step 0, the copies of tile t+3 (into tile t-1's stage) and the direct loads
  of tile t+3 between them;
  the MFMAs of tile t step 1 (k 16..31), with the reads of tile t+1 step 1.
LDS fragments live in two register sets that alternate between tiles, so
every read has a whole tile of MFMAs to land in; direct fragments in STAGES
register sets, one per slot (tile t+3's loads go to the set tile t-1 used).
The loop body covers the slots whose LDS offsets and register sets repeat
(STAGES tiles, STAGES even), so every LDS offset is an immediate. Copies and
direct loads past the last tile re-read the last tile (the source offsets stop
advancing), which keeps the wait counts uniform; those stages and sets are
never used. A contraction of KT 32-deep tiles enters the body at slot
(-KT mod SLOTS) (one prologue per entry slot), so every k-tile count ends with
the body's last slot.

Operands of the asm block (names used below):
  cIJ        accumulators ("+a", f32x16), A fragment I x B fragment J
  voA0.., voB0..  per-lane byte offsets: of this wavefront's copy blocks (LDS
             operand) or of its fragments' rows at k 8 (l / 32) (direct)
  rem        k-tiles left before the source offsets stop advancing; iters:
             loop count (passes over the body, the first one entered at slot
             `first`)
  ta, tb     scratch SGPRs
  ldsA/ldsB  LDS byte address of this wavefront's first copy block in stage 0
  sbA/sbB    global base addresses; ksA/ksB: bytes per 32-deep k-tile
  fa0.., fb0..  LDS fragment base addresses (see Shape.bases)
"""

import os

KT_BYTES = 32 * 2          # one 32-deep k-tile of a k-contiguous row


def direct_for(la, lb):
    """the operand loaded straight into registers for these layouts"""
    if lb == "kc":
        return "b"
    if la == "kc":
        return "a"
    return None


class Shape:
    """A block tile of 2 x (waves / 2) wavefronts with FM x FN accumulators
    each; direct names the operand ("a", "b") whose fragments bypass LDS, or
    None. frag_top: one past the last VGPR the fragments may use (256 with one
    wavefront per SIMD; 128 with two, whose accumulators take the other 128
    of the SIMD's registers per lane)."""

    def __init__(self, name, fm, fn, stages, direct=None, frag_top=256, waves=4, per_cu=1):
        self.name, self.fm, self.fn, self.stages = name, fm, fn, stages
        self.direct = direct
        self.waves, self.frag_top, self.per_cu = waves, frag_top, per_cu
        self.bm, self.bn = 64 * fm, 32 * (waves // 2) * fn
        self.a_bytes = 0 if direct == "a" else self.bm * KT_BYTES
        self.b_bytes = 0 if direct == "b" else self.bn * KT_BYTES
        self.stage_bytes = self.a_bytes + self.b_bytes
        self.b_offset = self.a_bytes            # operand B follows A inside a stage
        # LDS copy blocks per wavefront and k-tile; direct loads per k-tile
        self.qa = 0 if direct == "a" else self.a_bytes // 1024 // waves
        self.qb = 0 if direct == "b" else self.b_bytes // 1024 // waves
        assert self.qa * 1024 * waves == self.a_bytes and self.qb * 1024 * waves == self.b_bytes
        self.ncopy = self.qa + self.qb
        self.nd = 0 if direct is None else 2 * self.nfrag("ab".index(direct))
        self.cpt = self.ncopy + self.nd         # vector memory operations per k-tile
        self.sets = (stages + 1) // 2           # fragment base sets: stages 2i, 2i+1 share set i
        assert 2 * self.stage_bytes <= 65536 + self.stage_bytes and self.stage_bytes <= 32768
        assert stages % 2 == 0
        self.slots = stages
        # fragment registers: per operand [register set][step][fragment], A's block then B's
        self.nbuf = [stages if self.is_direct(op) else 2 for op in (0, 1)]
        self.op_regs = [self.nbuf[op] * 2 * 4 * self.nfrag(op) for op in (0, 1)]
        self.frag_lo = frag_top - sum(self.op_regs)   # first fragment VGPR
        self.frag_hi = frag_top
        assert self.frag_lo >= 0

    def is_direct(self, op):
        return self.direct == "ab"[op]

    def freg(self, buf, kk, op, idx):
        """first VGPR of a fragment: register set buf, step kk, operand 0 (A) / 1 (B), fragment idx"""
        F = self.nfrag(op)
        base = self.frag_lo + (self.op_regs[0] if op == 1 else 0)
        return base + buf * 8 * F + kk * 4 * F + 4 * idx

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


# the kernels' shapes: 256 x 256, 256 x 192 for the 1536-wide products (256
# tiles instead of 192 on 256 CUs), 256 x 256 on 8 wavefronts (two per SIMD,
# 128 x 64 each), and 128 x 128 on 4 wavefronts of 64 x 64 with two blocks per
# CU (64 KB of LDS each), for products too small to fill the chip with the
# larger tiles, where one block's first copies and epilogue overlap the other
# block's loop
S256 = Shape("256", 4, 4, 4)
S192 = Shape("192", 4, 3, 4)
S256W8 = Shape("w8", 4, 2, 4, frag_top=128, waves=8)
S128 = Shape("128", 2, 2, 4, frag_top=128, per_cu=2)
SHAPES = (S256, S192, S256W8, S128)


def shape_for(sh, la, lb, direct=None):
    """the variant of sh that a loop over layouts (la, lb) runs (direct="auto":
    with the operand direct_for picks loaded straight into registers)"""
    d = direct_for(la, lb) if direct == "auto" else direct
    return Shape(sh.name, sh.fm, sh.fn, sh.stages, d, frag_top=sh.frag_top, waves=sh.waves,
                 per_cu=sh.per_cu)


def reads(sh, layout, op, buf, stage, kk):
    """LDS reads of one operand's fragments for one 16-deep step (none for a direct operand)"""
    if sh.is_direct(op):
        return []
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
    """one k-tile's memory operations: the LDS copies into `stage` and the
    direct loads into register set `stage`"""
    out = []
    for q in range(max(sh.qa, sh.qb)):
        for x, n in (("A", sh.qa), ("B", sh.qb)):
            if q < n:
                out.append([f"s_add_u32 m0, %[lds{x}], {stage * sh.stage_bytes + q * 1024}",
                            "s_nop 0",   # M0 write -> LDS DMA needs one wait state
                            f"global_load_lds_dwordx4 %[vo{x}{q}], %[sb{x}]"])
    if sh.direct:
        op = "ab".index(sh.direct)
        x = sh.direct.upper()
        for kk in range(2):
            for i in range(sh.nfrag(op)):
                r = sh.freg(stage, kk, op, i)
                out.append([f"global_load_dwordx4 v[{r}:{r + 3}], %[vo{x}{i}], %[sb{x}] offset:{32 * kk}"])
    return out


def advance(sh):
    out = ["s_cmp_gt_i32 %[rem], 0",
           "s_cselect_b32 %[ta], %[ksA], 0",
           "s_cselect_b32 %[tb], %[ksB], 0",
           "s_sub_i32 %[rem], %[rem], 1"]
    for x, t, op in (("A", "ta", 0), ("B", "tb", 1)):
        n = sh.nfrag(op) if sh.is_direct(op) else (sh.qa, sh.qb)[op]
        for q in range(n):
            out.append(f"v_add_u32 %[vo{x}{q}], %[{t}], %[vo{x}{q}]")
    return out


def mfma(sh, buf, kk, i, j, slot=0):
    ba = slot if sh.is_direct(0) else buf
    bb = slot if sh.is_direct(1) else buf
    a, b = sh.freg(ba, kk, 0, i), sh.freg(bb, kk, 1, j)
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
    return sum(sh.nfrag(op) * (1 if l == "kc" else 2) for op, l in ((0, la), (1, lb))
               if not sh.is_direct(op))


def loop(la, lb, reads_first=False, copies_step=0, early=0, order="row", sh=S256, direct=None):
    """the asm lines for operand layouts la, lb ("kc" / "mn") and shape sh. The
    defaults are the schedules described above; direct="auto" loads the
    operand direct_for picks straight into registers; reads_first issues a step's fragment reads right after its
    first MFMA instead of spreading them, copies_step = 1 moves the copies into
    the second step, early = n issues a tile's first n MFMAs (whose fragments
    are already in registers) before its copy wait and barrier, order picks the
    accumulators' MFMA order within a step (measurement variants)."""
    sh = shape_for(sh, la, lb, direct)
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
            L += [mfma(sh, X, 0, i, j, u) for i, j in pairs[:early]]
        L.append(f"s_waitcnt vmcnt({sh.cpt * (S - 3)})")
        L.append("s_barrier")
        if not early:
            L.append(wait_step)
        for kk in range(2):
            r = reads(sh, la, 0, Y, nxt, kk) + reads(sh, lb, 1, Y, nxt, kk)
            c = copies(sh, dst) + [advance(sh)] if kk == copies_step else []
            m = [mfma(sh, X, kk, i, j, u) for i, j in pairs]
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


# ---------------------------------------------------------------------------
# 64-deep k-tiles (loop64): a 32-deep tile of a k-contiguous operand is 64
# bytes of each row, so its copies (16 rows x 64 bytes per instruction) ask
# the L2 for half cache lines; a 64-deep tile copies whole 128-byte lines (8
# rows x 128 bytes per instruction) and halves the requests. Built for the
# 8-wavefront 256 x 256 tile with both operands k-contiguous (S256W8_64,
# reads one step ahead): 6-7 % faster than its 32-deep loop there, where the
# L2's request rate limits the copies; with a transposed operand (whose
# copies move whole lines in either loop) 2-8 % slower, and reading two steps
# ahead was no faster. On the 4-wavefront tiles (S256_64, S192_64, kept as
# measurement variants) it was no faster for the 8192 x 2048 x 4096 product
# and 3-12 % slower for the others: one wavefront per SIMD stalls on the
# step waits before the request rate matters. Two stages of [A BM x 64 | B BN x
# 64] (the same LDS as four 32-deep stages), four 16-deep steps per tile:
#   - a k-contiguous operand sits as [row][64 k], 16-byte chunk j of row r at
#     chunk j ^ ((r >> 1) & 7) (conflict-free for 128-bit reads: 16 rows of
#     one chunk hit 16 distinct bank groups; the same for rows 32 apart);
#   - an operand whose contraction index is not the contiguous one sits as
#     [64 k][rows], chunk c of k-row k at c ^ ((k & 3) << 2), as above.
# Schedule of tile t (stage t % 2), per wavefront:
#   steps 0..2: wait for the step's fragments (lgkmcnt(0)); the step's MFMAs
#   with the fragment reads of the next step between them;
#   step 3: wait for the step's fragments and the copy of tile t+1 (vmcnt(0),
#   lgkmcnt(0)) and barrier -- after it every wavefront has read all of tile
#   t and tile t+1 has landed; the MFMAs of step 3 with the reads of tile t+1
#   step 0 and the copies of tile t+2 (into tile t's stage) between them.
# Fragments alternate between two register sets by step. Copies get one
# 64-deep tile of lead (as the 32-deep loop's two tiles). A contraction of
# KT64 tiles enters the two-slot body at slot (-KT64 mod 2).

class Shape64:
    """The 64-deep variant of a block tile of wr x (waves / wr) wavefronts
    with FM x FN accumulators; fragment reads run ra steps ahead of their
    MFMAs (nbuf register sets)."""

    def __init__(self, name, fm, fn, ra=1, frag_top=256, waves=4, wr=2):
        self.name, self.fm, self.fn = name, fm, fn
        self.direct = None                # both operands through LDS
        self.waves, self.frag_top, self.per_cu = waves, frag_top, 1
        self.bm, self.bn = 32 * wr * fm, 32 * (waves // wr) * fn
        self.stages, self.steps, self.slots = 2, 4, 2
        self.a_bytes, self.b_bytes = self.bm * 128, self.bn * 128
        self.stage_bytes = self.a_bytes + self.b_bytes
        self.b_offset = self.a_bytes
        # copy blocks (1 KB) per wavefront and k-tile
        self.qa, self.qb = self.a_bytes // 1024 // waves, self.b_bytes // 1024 // waves
        assert self.qa * 1024 * waves == self.a_bytes and self.qb * 1024 * waves == self.b_bytes
        self.cpt = self.qa + self.qb
        assert ra in (1, 2)
        self.ra = ra
        self.nbuf = 2 if ra == 1 else 4   # divides the body's 8 steps
        self.per_step = 4 * (fm + fn)
        self.frag_lo = frag_top - self.nbuf * self.per_step
        self.frag_hi = frag_top

    def freg(self, buf, op, idx):
        """first VGPR of a fragment: register set buf, operand 0 (A) / 1 (B), fragment idx"""
        return self.frag_lo + self.per_step * buf + 4 * self.fm * op + 4 * idx

    def is_direct(self, op):
        return False

    def nfrag(self, op):
        return self.fm if op == 0 else self.fn

    def rows(self, op):
        return self.bm if op == 0 else self.bn

    def nbases(self, layout, op):
        """fragment base registers: kc -> one per (stage, step); mn -> one per (stage, fragment)"""
        return self.stages * (self.steps if layout == "kc" else self.nfrag(op))

    def base_index(self, layout, op, stage, step, i):
        return stage * self.steps + step if layout == "kc" else stage * self.nfrag(op) + i

    def read_offset(self, layout, op, step, i, half=0):
        if layout == "kc":
            return i * 32 * 128       # fragments i are 32 rows of 128 bytes apart
        rb = self.rows(op) * 2        # one k-row; step s is 16 k-rows further, a fragment's second half 4
        return step * 16 * rb + half * 4 * rb


S256_64 = Shape64("256", 4, 4, ra=2)
S192_64 = Shape64("192", 4, 3, ra=2)
S256W8_64 = Shape64("w8", 4, 2, ra=1, frag_top=128, waves=8)
# 256 x 192 on 8 wavefronts (4 x 2, 64 x 96 each): its B tile is 24 copy
# blocks of 8 rows, three per wavefront (the 32-deep tile's 12 blocks of 16
# rows do not split over 8)
S192W8_64 = Shape64("192w8", 2, 3, ra=1, frag_top=128, waves=8, wr=4)
SHAPES64 = (S256_64, S192_64, S256W8_64, S192W8_64)


def reads64(sh, layout, op, buf, stage, step):
    x = "ab"[op]
    out = []
    for i in range(sh.nfrag(op)):
        r = sh.freg(buf, op, i)
        b = sh.base_index(layout, op, stage, step, i)
        if layout == "kc":
            out.append([f"ds_read_b128 v[{r}:{r + 3}], %[f{x}{b}] offset:{sh.read_offset(layout, op, step, i)}"])
        else:
            out.append([f"ds_read_b64_tr_b16 v[{r}:{r + 1}], %[f{x}{b}] offset:{sh.read_offset(layout, op, step, i, 0)}"])
            out.append([f"ds_read_b64_tr_b16 v[{r + 2}:{r + 3}], %[f{x}{b}] "
                        f"offset:{sh.read_offset(layout, op, step, i, 1)}"])
    return out


def loop64(la, lb, sh=S256_64, order="row"):
    """the asm lines of the 64-deep loop for operand layouts la, lb and shape sh"""
    pairs = orders(sh)[order]
    ra, nb, NS = sh.ra, sh.nbuf, sh.steps

    def mfma64(buf, i, j):
        a, b = sh.freg(buf, 0, i), sh.freg(buf, 1, j)
        return f"v_mfma_f32_32x32x16_bf16 %[c{i}{j}], v[{b}:{b + 3}], v[{a}:{a + 3}], %[c{i}{j}]"

    def step_reads(buf, stage, step):
        return reads64(sh, la, 0, buf, stage, step) + reads64(sh, lb, 1, buf, stage, step)

    wait_step = f"s_waitcnt lgkmcnt({min(nreads(sh, la, lb), 15)})"
    L = ["s_nop 4"]   # accumulator initialisation (VALU/AGPR writes) -> MFMA
    L += ["s_cmp_eq_u32 %[first], 1", "s_cbranch_scc1 L%=_pro1"]
    for f in range(sh.slots):
        if f:
            L.append(f"L%=_pro{f}:")
        for t in range(sh.stages):
            for u in copies(sh, (f + t) % sh.stages):
                L += u
            L += advance(sh)
        L.append(f"s_waitcnt vmcnt({sh.cpt})")
        L.append("s_barrier")
        for s in range(ra):   # the first ra steps of tile 0
            for u in step_reads((NS * f + s) % nb, f, s):
                L += u
        L.append(f"s_branch L%=_slot{f}")
    L.append("L%=_ktile:")
    for u in range(sh.slots):
        L.append(f"L%=_slot{u}:")
        for step in range(NS):
            g = NS * u + step                  # step within the body: its register set is g % nb
            rs = step + ra                     # the step whose fragments are read now
            tile_next = rs >= NS
            if ra == 1 and step == NS - 1:
                # the step's fragments and tile t+1's copy, then every wavefront is done with tile t
                L += ["s_waitcnt vmcnt(0) lgkmcnt(0)", "s_barrier"]
                c = copies(sh, u) + [advance(sh)]
            elif ra == 2 and step == NS - 2:
                # tile t+1's copy has landed everywhere before its first reads
                L += ["s_waitcnt vmcnt(0)", wait_step, "s_barrier"]
                c = []
            elif ra == 2 and step == NS - 1:
                # the last reads of tile t retired everywhere: its stage takes tile t+2
                L += [wait_step, "s_barrier"]
                c = copies(sh, u) + [advance(sh)]
            else:
                L.append(wait_step if ra == 2 else "s_waitcnt lgkmcnt(0)")
                c = []
            r = step_reads((g + ra) % nb, 1 - u if tile_next else u, rs % NS)
            m = [mfma64(g % nb, i, j) for i, j in pairs]
            L += spread(m, interleave(r, c[:-1]) + c[-1:] if c else r)
    L += ["s_sub_i32 %[iters], %[iters], 1", "s_cmp_gt_i32 %[iters], 0", "s_cbranch_scc1 L%=_ktile"]
    L.append("s_waitcnt vmcnt(0) lgkmcnt(0)")
    L += ["s_nop 7"] * 3   # last MFMAs -> accumulator reads by the epilogue
    return L


LAYOUTS = (("NT", "kc", "kc"), ("NN", "kc", "mn"), ("TN", "mn", "mn"))
# which layouts each shape is built for: 256 x 192 only for the 1536-wide
# forward products (both operands k-contiguous)
SHAPE_LAYOUTS = {"256": LAYOUTS, "192": LAYOUTS[:1], "w8": LAYOUTS, "128": LAYOUTS, "192w8": LAYOUTS[:1]}


def render():
    """the text of gemm_loop.inc"""
    out = ["// Generated by gen_gemm_loop.py (the schedule is described there); do not edit.", ""]

    def block(name, lines, lo, hi):
        out.append(f"#define {name} \\")
        for line in lines:
            out.append(f'  "{line}\\n" \\')
        out.append("")
        regs = ", ".join(f'"v{r}"' for r in range(lo, hi))
        out.append(f"#define {name.replace('_LOOP', '_LOOP_CLOBBERS', 1)} {regs}")
        out.append("")

    for sh in SHAPES:
        suffix = "" if sh is S256 else "_" + sh.name.upper()
        for name, la, lb in SHAPE_LAYOUTS[sh.name]:
            v = shape_for(sh, la, lb)
            block(f"MTB_GEMM_LOOP_{name}{suffix}", loop(la, lb, sh=sh), v.frag_lo, v.frag_hi)
    # the 64-deep loop of the 8-wavefront 256 x 256 tile (contractions that are a
    # multiple of 64, both operands k-contiguous)
    for sh in (S256W8_64, S192W8_64):
        name, la, lb = LAYOUTS[0]
        block(f"MTB_GEMM_LOOP64_{name}_{sh.name.upper()}", loop64(la, lb, sh=sh), sh.frag_lo, sh.frag_hi)
    return "\n".join(out)


def main():
    here = os.path.dirname(os.path.abspath(__file__))
    with open(os.path.join(here, "gemm_loop.inc"), "w") as f:
        f.write(render())


if __name__ == "__main__":
    main()
