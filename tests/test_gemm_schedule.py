"""Host-side checks of the hand-scheduled GEMM main loop (the inline assembly
that csrc/gen_gemm_loop.py writes to csrc/gemm_loop.inc).

1. The committed include is what the generator produces.
2. A symbolic execution of one wavefront's instruction stream (the four
   wavefronts of a block run the same stream, so what holds for one holds for
   all) over several contraction lengths, per operand layout, checks:
   - every MFMA multiplies an A and a B fragment of the same k-tile and
     16-deep step, both landed (their LDS reads, or their direct global loads,
     retired by an s_waitcnt), and every accumulator sums each (k-tile, step)
     exactly once, in order;
   - an LDS read sees a stage only when the stage's last copy completed on
     every lane (vmcnt) before a barrier, and reads the fragment its
     destination registers are meant for;
   - a copy into a stage is issued only when every read of the stage's
     previous tile retired before a barrier (no wavefront still reads it);
   - the copies (and the direct loads, both steps of each) fetch k-tiles 0,
     1, ..., KT-1 in order and then re-fetch the last one, for any KT (the
     body is entered at slot -KT mod SLOTS); M0 is written, with a wait
     state, before every copy; direct loads write only the direct operand's
     fragment registers;
   - wait counts fit their fields, LDS read offsets fit 16 bits, copy
     destinations stay inside their operand's part of a stage.
   This for every tile shape the generator builds (256 x 256, 256 x 192),
   with the direct operand each layout takes and with both operands through
   LDS.
"""
import importlib.util
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "transformer_layer_ln_amd", "csrc")


def _gen():
    spec = importlib.util.spec_from_file_location("gen_gemm_loop", os.path.join(CSRC, "gen_gemm_loop.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


GEN = _gen()


def test_committed_include_matches_generator():
    with open(os.path.join(CSRC, "gemm_loop.inc")) as f:
        assert f.read() == GEN.render()


class ScheduleError(AssertionError):
    pass


class Wave:
    """Symbolic state of one wavefront running the loop of shape `sh` (the
    variant for these layouts, with its direct operand) for KT k-tiles."""

    def __init__(self, layouts, KT, sh=GEN.S256, direct=None):
        self.lay = layouts                 # {"a": "kc"|"mn", "b": ...}
        sh = GEN.shape_for(sh, layouts["a"], layouts["b"], direct)
        self.sh = sh
        self.KT = KT
        self.first = -KT % sh.slots       # the body slot k-tile 0 runs in
        self.iters = (KT + self.first) // sh.slots
        self.rem = KT - 1
        self.nq = {"A": sh.qa, "B": sh.qb}
        keys = [(x, q) for x in "AB" for q in range(self.nq[x])]
        if sh.direct:
            x = sh.direct.upper()
            keys += [(x, i) for i in range(sh.nfrag("AB".index(x)))]
        self.src = {k: 0 for k in keys}   # k-tile the copy / direct offset points at
        self.copied = {k: [] for k in keys}
        self.t = {"ta": None, "tb": None}
        self.scc = None
        self.m0 = None
        self.lgkm = []       # outstanding LDS reads, oldest first: (regs, content, stage)
        self.vm = []         # outstanding copies (stage, x, q) and direct loads ("direct", regs)
        self.regs = {}       # first VGPR of a 2-register half -> (content, landed)
        self.epoch = 0       # barriers passed
        S = sh.stages
        self.visible = {s: None for s in range(S)}       # k-tile readable in a stage
        self.blocks = {s: {} for s in range(S)}          # (x, q) -> [tile, complete]
        self.reads_done = {s: [] for s in range(S)}      # epochs of retired reads
        self.reads_open = {s: 0 for s in range(S)}
        self.acc = {(i, j): [] for i in range(sh.fm) for j in range(sh.fn)}
        self.prev = []       # the last two instructions (M0 hazard check)

    def fail(self, msg):
        raise ScheduleError(msg)

    # --- memory counters
    def retire_lgkm(self, n):
        while len(self.lgkm) > n:
            regs, content, stage = self.lgkm.pop(0)
            for r in regs:
                self.regs[r] = (content, True)
            self.reads_open[stage] -= 1
            self.reads_done[stage].append(self.epoch)

    def retire_vm(self, n):
        while len(self.vm) > n:
            item = self.vm.pop(0)
            if item[0] == "direct":
                for r in item[1]:
                    content, _ = self.regs[r]
                    self.regs[r] = (content, True)
            else:
                stage, x, q = item
                self.blocks[stage][(x, q)][1] = True

    def barrier(self):
        self.epoch += 1
        for s, blk in self.blocks.items():
            tiles = {t for t, _ in blk.values()}
            if len(blk) == self.sh.ncopy and len(tiles) == 1 and all(c for _, c in blk.values()):
                self.visible[s] = tiles.pop()

    # --- instructions
    def ds_read(self, kind, reg, base, off):
        sh = self.sh
        SB = sh.stage_bytes
        if off > 65535:
            self.fail(f"LDS read offset {off} does not fit 16 bits")
        x, n = base[0], int(base[1:])
        op = "ab".index(x)
        F = sh.nfrag(op)
        if self.lay[x] == "kc":
            if kind != "ds_read_b128":
                self.fail("k-contiguous operand read with " + kind)
            st, kk = n // 2, n % 2
            stage = 2 * st + off // SB
            idx, half = (off % SB) // 2048, None
            if (off % SB) % 2048:
                self.fail(f"read offset {off} is not a fragment start")
            regs = [reg, reg + 2]
        else:
            if kind != "ds_read_b64_tr_b16":
                self.fail("transposed operand read with " + kind)
            rb = sh.rows(op) * 2
            st, idx = n // F, n % F
            stage = 2 * st + off // SB
            rem = off % SB
            kk, half = rem // (16 * rb), (rem % (16 * rb)) // (4 * rb)
            if rem % (4 * rb) or kk > 1 or half > 1:
                self.fail(f"transpose read offset {off} is not a fragment half")
            regs = [reg] if half == 0 else [reg - 2]
        if stage >= sh.stages or idx >= F:
            self.fail(f"read of stage {stage} fragment {idx}: outside the tile")
        tile = self.visible[stage]
        if tile is None:
            self.fail(f"read of stage {stage} before its copy completed behind a barrier")
        r0 = regs[0]
        if sh.is_direct(op):
            self.fail(f"LDS read of the direct operand {x}")
        exp = [sh.freg(b, kk, op, idx) for b in range(2)]
        if r0 not in exp or r0 < sh.frag_lo or r0 + 4 > sh.frag_hi:
            self.fail(f"fragment (kk {kk}, op {x}, {idx}) read into v{r0}, expected one of {exp}")
        content = (tile, kk, op, idx)
        dest = regs if half is None else [reg]
        for r in dest:
            self.regs[r] = (content, False)
        self.lgkm.append((dest, content, stage))
        self.reads_open[stage] += 1

    def copy(self, x, q):
        sh = self.sh
        SB = sh.stage_bytes
        if len(self.prev) < 2 or self.prev[-1] != "s_nop" or self.prev[-2] != "m0":
            self.fail("copy not preceded by an M0 write and one wait state")
        mx, moff = self.m0
        stage, mq = moff // SB, (moff % SB) // 1024
        # the last wavefront's block ends at M0 + its 3 Q KB + 1 KB, inside the operand's region
        region = sh.a_bytes if x == "A" else sh.b_bytes
        if mx != x or mq != q or moff % 1024 or q >= self.nq[x] or stage >= sh.stages or \
                (moff % SB) + 3 * self.nq[x] * 1024 + 1024 > region:
            self.fail(f"M0 {self.m0} does not address block {q} of operand {x}")
        if self.reads_open[stage] or any(e >= self.epoch for e in self.reads_done[stage]):
            self.fail(f"copy into stage {stage} while a read of its previous tile may be in flight")
        self.reads_done[stage] = []
        tile = self.src[(x, q)]
        self.copied[(x, q)].append(tile)
        self.visible[stage] = None
        self.blocks[stage][(x, q)] = [tile, False]
        self.vm.append((stage, x, q))

    def direct_load(self, reg, x, i, off):
        sh = self.sh
        op = "AB".index(x)
        if not sh.is_direct(op) or i >= sh.nfrag(op) or off not in (0, 32):
            self.fail(f"direct load of {x}{i} offset {off}: not a direct fragment")
        kk = off // 32
        lo = sh.freg(0, 0, op, 0)
        hi = sh.freg(sh.nbuf[op] - 1, 1, op, sh.nfrag(op) - 1) + 4
        if reg < lo or reg + 4 > hi or (reg - sh.freg(0, kk, op, i)) % (8 * sh.nfrag(op)):
            self.fail(f"direct load of {x}{i} step {kk} into v{reg}: not one of its register sets")
        tile = self.src[(x, i)]
        self.copied[(x, i)].append(tile)
        content = (tile, kk, op, i)
        dest = [reg, reg + 2]
        for r in dest:
            self.regs[r] = (content, False)
        self.vm.append(("direct", dest))

    def mfma(self, i, j, rb, ra):
        ca, cb = [], []
        for r, out in ((ra, ca), (rb, cb)):
            for h in (r, r + 2):
                if h not in self.regs or not self.regs[h][1]:
                    self.fail(f"MFMA c{i}{j} reads v{h} before its LDS read or direct load retired")
                out.append(self.regs[h][0])
        if ca[0] != ca[1] or cb[0] != cb[1]:
            self.fail(f"MFMA c{i}{j}: fragment halves from different reads {ca} {cb}")
        (ta, ka, oa, ia), (tb, kb, ob, jb) = ca[0], cb[0]
        if (oa, ob, ia, jb) != (0, 1, i, j) or ta != tb or ka != kb:
            self.fail(f"MFMA c{i}{j} multiplies A {ca[0]} with B {cb[0]}")
        self.acc[(i, j)].append((ta, ka))

    def run(self, lines):
        labels = {l[:-1]: k for k, l in enumerate(lines) if l.endswith(":")}
        pc, steps = 0, 0
        while pc < len(lines):
            steps += 1
            if steps > 10 ** 6:
                self.fail("no exit from the loop")
            line = lines[pc]
            pc += 1
            tag = self.step(line)
            if tag in ("branch", "jump"):
                pc = labels[line.split()[-1]]
            self.prev = (self.prev + [tag or line.split()[0]])[-2:]

    def step(self, line):
        f = line.replace(",", " ").split()
        op = f[0]
        if line.endswith(":"):
            return "label"
        if op in ("ds_read_b128", "ds_read_b64_tr_b16"):
            reg = int(re.match(r"v\[(\d+):", f[1]).group(1))
            base = re.match(r"%\[f([ab]\d)\]", f[2]).group(1)
            self.ds_read(op, reg, base, int(f[3].split(":")[1]))
        elif op == "v_mfma_f32_32x32x16_bf16":
            i, j = int(f[1][3]), int(f[1][4])
            rb = int(re.match(r"v\[(\d+):", f[2]).group(1))
            ra = int(re.match(r"v\[(\d+):", f[3]).group(1))
            self.mfma(i, j, rb, ra)
        elif op == "s_waitcnt":
            for part in f[1:]:
                name, n = re.match(r"(\w+)\((\d+)\)", part).groups()
                n = int(n)
                if name == "lgkmcnt":
                    if n > 15:
                        self.fail("lgkmcnt field is 4 bits")
                    self.retire_lgkm(n)
                else:
                    if n > 63:
                        self.fail("vmcnt field is 6 bits")
                    self.retire_vm(n)
        elif op == "s_barrier":
            self.barrier()
        elif op == "s_add_u32" and f[1] == "m0":
            self.m0 = (re.match(r"%\[lds([AB])\]", f[2]).group(1), int(f[3]))
            return "m0"
        elif op == "s_nop":
            return "s_nop"
        elif op == "global_load_lds_dwordx4":
            x, q = re.match(r"%\[vo([AB])(\d)\]", f[1]).groups()
            self.copy(x, int(q))
        elif op == "global_load_dwordx4":
            reg = int(re.match(r"v\[(\d+):", f[1]).group(1))
            x, i = re.match(r"%\[vo([AB])(\d)\]", f[2]).groups()
            if f[3] != f"%[sb{x}]":
                self.fail("direct load from another operand's base: " + line)
            self.direct_load(reg, x, int(i), int(f[4].split(":")[1]))
        elif op == "s_cmp_gt_i32":
            self.scc = (self.rem if f[1] == "%[rem]" else self.iters) > 0
        elif op == "s_cmp_eq_u32" and f[1] == "%[first]":
            self.scc = self.first == int(f[2])
        elif op == "s_branch":
            return "jump"
        elif op == "s_cselect_b32":
            self.t[f[1][2:-1]] = 1 if self.scc else 0
        elif op == "s_sub_i32":
            if f[1] == "%[rem]":
                self.rem -= 1
            else:
                self.iters -= 1
        elif op == "v_add_u32":
            x, q = re.match(r"%\[vo([AB])(\d)\]", f[1]).groups()
            self.src[(x, int(q))] += self.t[f[2][2:-1]]
        elif op == "s_cbranch_scc1":
            return "branch" if self.scc else "fallthrough"
        else:
            self.fail("unmodelled instruction: " + line)
        return None


def _check_run(la, lb, KT, sh=GEN.S256, **variant):
    lines = GEN.loop(la, lb, sh=sh, **variant)
    assert lines[0] == "s_nop 4" and lines[-3:] == ["s_nop 7"] * 3   # accumulator hazards
    w = Wave({"a": la, "b": lb}, KT, sh, variant.get("direct"))
    w.run(lines)
    assert not w.lgkm and not w.vm, "memory operations outstanding at the end"
    want = [(t, kk) for t in range(KT) for kk in (0, 1)]
    for ij, got in w.acc.items():
        assert got == want, f"{sh.name} {variant} KT {KT} accumulator c{ij[0]}{ij[1]}"
    for key, tiles in w.copied.items():
        if w.sh.direct and key[0] == w.sh.direct.upper():
            tiles = tiles[::2]     # each tile's two steps load the same k-tile
        n = len(tiles)
        assert tiles == list(range(KT)) + [KT - 1] * (n - KT), f"copy sequence of {key}: {tiles}"
    return w


@pytest.mark.parametrize("name,la,lb", GEN.LAYOUTS)
@pytest.mark.parametrize("KT", [1, 2, 3, 4, 5, 6, 7, 8, 13, 32, 501])
def test_schedule_symbolic_execution(name, la, lb, KT):
    _check_run(la, lb, KT)


@pytest.mark.parametrize("name,la,lb", GEN.LAYOUTS[:2])
@pytest.mark.parametrize("KT", [1, 2, 3, 5, 8, 13])
def test_schedule_with_direct_operand(name, la, lb, KT):
    """The measurement variant that loads the k-contiguous operand straight
    into registers obeys the same waits and k-tile order."""
    _check_run(la, lb, KT, direct="auto")


@pytest.mark.parametrize("shape", [s.name for s in GEN.SHAPES if s is not GEN.S256])
@pytest.mark.parametrize("KT", [1, 2, 3, 4, 5, 6, 7, 8, 11, 13, 32, 128])
def test_other_shapes_symbolic_execution(shape, KT):
    """The 256 x 192, 8-wavefront 256 x 256 and 128 x 128 loops, for every layout built."""
    sh = next(s for s in GEN.SHAPES if s.name == shape)
    for name, la, lb in GEN.SHAPE_LAYOUTS[shape]:
        _check_run(la, lb, KT, sh)


def test_shapes_fit_their_registers_and_lds():
    """Fragment registers inside the clobbered range (and a quarter of the
    wavefront's VGPRs left to the compiled code around the loop: 64 of 256
    with one wavefront per SIMD, 32 of 128 with two), stages inside a CU's
    160 KB of LDS (per block, times the blocks a CU holds), copy blocks
    whole, wait counts inside their fields. The direct-operand variants
    exist for the one-wavefront-per-SIMD shapes."""
    for sh in GEN.SHAPES:
        for name, la, lb in GEN.SHAPE_LAYOUTS[sh.name]:
            for d in (None, "auto") if sh.waves * sh.per_cu == 4 else (None,):
                v = GEN.shape_for(sh, la, lb, d)
                assert v.stages * v.stage_bytes * v.per_cu <= 160 * 1024, (sh.name, name)
                assert v.a_bytes % 4096 == 0 and v.b_bytes % 4096 == 0, (sh.name, name)
                assert v.frag_top // 4 <= v.frag_lo and v.frag_hi <= v.frag_top, (sh.name, name, d)
                assert v.frag_top == 256 * 4 // (v.waves * v.per_cu), (sh.name, name, d)
                assert v.cpt * (v.stages - 2) <= 63, (sh.name, name, d)


@pytest.mark.parametrize("name,la,lb", GEN.LAYOUTS)
@pytest.mark.parametrize("variant", [dict(early=2), dict(reads_first=True), dict(copies_step=1),
                                     dict(order="col"), dict(order="snake")])
def test_measurement_variants_are_valid_schedules(name, la, lb, variant):
    """The generator's measurement variants (timed against the default in
    alternating runs) obey the same waits, barriers and k-tile order."""
    for KT in (1, 2, 3, 5, 13):
        _check_run(la, lb, KT, **variant)


def test_symbolic_execution_catches_a_short_wait():
    """The checker itself: dropping the wait before the second step's MFMAs
    (an MFMA would use fragments still in flight) must be reported."""
    la, lb = "kc", "kc"
    lines = GEN.loop(la, lb)
    waits = [k for k, l in enumerate(lines) if l.startswith("s_waitcnt lgkmcnt")]
    bad = lines[:waits[2]] + lines[waits[2] + 1:]
    with pytest.raises(ScheduleError, match="before its LDS read"):
        Wave({"a": la, "b": lb}, 8).run(bad)


@pytest.mark.parametrize("name,la,lb", GEN.LAYOUTS[:2])
def test_symbolic_execution_catches_a_short_direct_wait(name, la, lb):
    """The checker itself: a body wait that lets one more tile of memory
    operations stay in flight (the direct fragments of the tile about to run
    would not have landed) must be reported."""
    sh = GEN.shape_for(GEN.S256, la, lb, "auto")
    lines = GEN.loop(la, lb, direct="auto")
    body = lines.index("L%=_ktile:")
    good = f"s_waitcnt vmcnt({sh.cpt * (sh.stages - 3)})"
    bad = lines[:body] + [f"s_waitcnt vmcnt({sh.cpt * (sh.stages - 2)})" if l == good else l
                          for l in lines[body:]]
    with pytest.raises(ScheduleError):
        Wave({"a": la, "b": lb}, 8, direct="auto").run(bad)


def test_symbolic_execution_catches_an_early_copy():
    """Moving a barrier behind the copies of a tile (a wavefront could still
    read the stage being overwritten, or read a stage whose copy has not
    landed) must be reported."""
    la, lb = "kc", "mn"
    lines = GEN.loop(la, lb)
    loop_start = lines.index("L%=_ktile:")
    k = lines.index("s_barrier", loop_start)
    bad = lines[:k] + lines[k + 1:]
    with pytest.raises(ScheduleError):
        Wave({"a": la, "b": lb}, 8).run(bad)


class Wave64(Wave):
    """Symbolic state of one wavefront running the 64-deep loop (gen_gemm_loop.loop64)."""

    def __init__(self, layouts, KT, sh=GEN.S256_64):
        self.lay = layouts
        self.sh = sh
        self.KT = KT
        self.first = -KT % sh.slots
        self.iters = (KT + self.first) // sh.slots
        self.rem = KT - 1
        self.nq = {"A": sh.qa, "B": sh.qb}
        keys = [(x, q) for x in "AB" for q in range(self.nq[x])]
        self.src = {k: 0 for k in keys}
        self.copied = {k: [] for k in keys}
        self.t = {"ta": None, "tb": None}
        self.scc = None
        self.m0 = None
        self.lgkm = []
        self.vm = []
        self.regs = {}
        self.epoch = 0
        S = sh.stages
        self.visible = {s: None for s in range(S)}
        self.blocks = {s: {} for s in range(S)}
        self.reads_done = {s: [] for s in range(S)}
        self.reads_open = {s: 0 for s in range(S)}
        self.acc = {(i, j): [] for i in range(sh.fm) for j in range(sh.fn)}
        self.prev = []

    def barrier(self):
        self.epoch += 1
        for s, blk in self.blocks.items():
            tiles = {t for t, _ in blk.values()}
            if len(blk) == self.sh.cpt and len(tiles) == 1 and all(c for _, c in blk.values()):
                self.visible[s] = tiles.pop()

    def ds_read(self, kind, reg, base, off):
        sh = self.sh
        if off > 65535:
            self.fail(f"LDS read offset {off} does not fit 16 bits")
        x, n = base[0], int(base[1:])
        op = "ab".index(x)
        F = sh.nfrag(op)
        if self.lay[x] == "kc":
            if kind != "ds_read_b128":
                self.fail("k-contiguous operand read with " + kind)
            stage, step = n // sh.steps, n % sh.steps
            idx, half = off // 4096, None
            if off % 4096:
                self.fail(f"read offset {off} is not a fragment start")
            regs = [reg, reg + 2]
        else:
            if kind != "ds_read_b64_tr_b16":
                self.fail("transposed operand read with " + kind)
            rb = sh.rows(op) * 2
            stage, idx = n // F, n % F
            step, half = off // (16 * rb), (off % (16 * rb)) // (4 * rb)
            if off % (4 * rb) or step >= sh.steps or half > 1:
                self.fail(f"transpose read offset {off} is not a fragment half")
            regs = [reg] if half == 0 else [reg - 2]
        if stage >= sh.stages or idx >= F:
            self.fail(f"read of stage {stage} fragment {idx}: outside the tile")
        tile = self.visible[stage]
        if tile is None:
            self.fail(f"read of stage {stage} before its copy completed behind a barrier")
        r0 = regs[0]
        exp = [sh.freg(b, op, idx) for b in range(sh.nbuf)]
        if r0 not in exp:
            self.fail(f"fragment (step {step}, op {x}, {idx}) read into v{r0}, expected one of {exp}")
        content = (tile, step, op, idx)
        dest = regs if half is None else [reg]
        for r in dest:
            self.regs[r] = (content, False)
        self.lgkm.append((dest, content, stage))
        self.reads_open[stage] += 1


def _check_run64(la, lb, KT, sh=GEN.S256_64):
    """Symbolic run of loop64 (the shape's own read-ahead) for KT 64-deep tiles."""
    lines = GEN.loop64(la, lb, sh=sh)
    assert lines[0] == "s_nop 4" and lines[-3:] == ["s_nop 7"] * 3
    w = Wave64({"a": la, "b": lb}, KT, sh)
    w.run(lines)
    assert not w.lgkm and not w.vm, "memory operations outstanding at the end"
    want = [(t, s) for t in range(KT) for s in range(sh.steps)]
    for ij, got in w.acc.items():
        assert got == want, f"64-deep {sh.name} KT {KT} accumulator c{ij[0]}{ij[1]}"
    for key, tiles in w.copied.items():
        n = len(tiles)
        assert tiles == list(range(KT)) + [KT - 1] * (n - KT), f"copy sequence of {key}: {tiles}"
    return w


@pytest.mark.parametrize("name,la,lb", GEN.LAYOUTS)
@pytest.mark.parametrize("KT", [1, 2, 3, 4, 5, 8, 13, 64, 251])
def test_schedule64_symbolic_execution(name, la, lb, KT):
    """The 64-deep loop (KT 64-deep tiles) for every layout, 256 x 256."""
    _check_run64(la, lb, KT)


@pytest.mark.parametrize("KT", [1, 2, 3, 4, 7, 24])
def test_schedule64_other_shapes(KT):
    for sh in GEN.SHAPES64:
        for name, la, lb in GEN.SHAPE_LAYOUTS[sh.name]:
            _check_run64(la, lb, KT, sh)


@pytest.mark.parametrize("ra", [1, 2])
@pytest.mark.parametrize("name,la,lb", GEN.LAYOUTS)
def test_schedule64_read_ahead_variants(ra, name, la, lb):
    """Both read-ahead depths of the 64-deep loop (one step: two register
    sets; two steps: four)."""
    sh = GEN.Shape64("256", 4, 4, ra=ra)
    for KT in (1, 2, 3, 6, 11):
        _check_run64(la, lb, KT, sh)


def test_shapes64_fit():
    """Two 64-deep stages in a CU's LDS (no more than four 32-deep ones, the
    epilogue's staging area), wait counts and read offsets in their fields."""
    for sh in GEN.SHAPES64:
        assert sh.stages * sh.stage_bytes <= 160 * 1024 and sh.frag_lo >= sh.frag_top // 4
        assert sh.frag_top == 256 * 4 // sh.waves
        assert sh.cpt <= 63
        assert sh.read_offset("kc", 0, 3, sh.fm - 1) < 65536
        assert sh.read_offset("mn", 1, 3, sh.fn - 1, 1) < 65536


def test_schedule64_catches_a_missing_barrier():
    """Dropping the barrier of step 3 (copies into a stage other wavefronts may
    still read, reads of a stage whose copy has not landed everywhere) must be
    reported."""
    la, lb = "kc", "kc"
    lines = GEN.loop64(la, lb)
    k = lines.index("s_barrier", lines.index("L%=_ktile:"))
    bad = lines[:k] + lines[k + 1:]
    with pytest.raises(ScheduleError):
        Wave64({"a": la, "b": lb}, 8).run(bad)


def test_schedule64_catches_a_short_wait():
    """A step wait that leaves the step's fragment reads in flight must be reported."""
    la, lb = "kc", "mn"
    lines = GEN.loop64(la, lb)
    body = lines.index("L%=_ktile:")
    k = next(i for i in range(body, len(lines)) if lines[i].startswith("s_waitcnt lgkmcnt"))
    bad = lines[:k] + lines[k + 1:]
    with pytest.raises(ScheduleError, match="before its LDS read"):
        Wave64({"a": la, "b": lb}, 8).run(bad)
