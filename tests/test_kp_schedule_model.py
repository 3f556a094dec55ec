"""Host model of the K-phase GEMM kernel's LDS ring schedule (gemm.hip:
gemm_kp_kernel / kp_kloop / kp_issue / kp_store_tile), run on the CPU.

The kernel streams each work unit's K range through an NSLOT-deep LDS ring
with direct buffer -> LDS loads (1 KB per instruction: 64 lanes x 16 B at
M0 + 16 lane), waits for its own loads with hand-counted `s_waitcnt vmcnt(n)`
and relies on one barrier per stage for the other waves' loads.  A mistake in
the slot / window-buffer / exchange-chunk arithmetic or in a wait count would
read stale data or write LDS outside the ring.  This model replays, for every
configuration the kernel is instantiated with (the layout constants come from
the kernel's own header, compiled with g++), the exact sequence of loads,
waits, barriers, LDS reads and writes of a workgroup over a chain of units,
and checks:

  1. every load's LDS destination (M0 .. M0 + 1 KB) lies inside the ring or
     the scale-window buffers, and the waves' loads cover each slot exactly;
  2. when a stage (and its scale window) is read, every wave's loads of it
     have completed (loads complete in issue order; a wave's vmcnt counts
     its loads and the epilogue's stores);
  3. no load, exchange write or output-tile write lands on a slot or window
     buffer whose previous contents some wave may still read (a barrier
     separates the last read from the write), and none overwrites a stage
     that was loaded but not yet read (the next unit's prefetched stages);
  4. every wait is tight: the newest load it must see complete is exactly
     the oldest one it leaves outstanding minus one.

The shape of the one recorded GPU fault (grouped split-K test: 4 experts
with 70 / 0 / 5 / 33 rows, N = 513, K = 2048, 2 splits, 32-row tiles, the
first launch to reach the 4-wave 32-row kernel's steady block) is modelled
explicitly.  The faulting variant itself was never committed, so only
today's arithmetic can be replayed.
"""
import os
import re
import subprocess
import tempfile
from dataclasses import dataclass

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DUMP = os.path.join(ROOT, "tests", "kp_model", "layout_dump.cpp")
GEMM = os.path.join(ROOT, "block_scaled_fp4_nibble_amd", "csrc", "gemm.hip")
VMCNT_MAX = 63


@pytest.fixture(scope="module")
def layouts():
    tmp = tempfile.mkdtemp(prefix="kp_model_")
    exe = os.path.join(tmp, "dump")
    subprocess.run(["g++", "-std=c++17", "-O1", DUMP, "-o", exe], check=True)
    out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout
    res = {}
    for line in out.strip().splitlines():
        d = {k: int(v) for k, v in (kv.split("=") for kv in line.split())}
        res[(d["BM"], d["NSLOT"], d["KW"], d["BN"])] = d
    return res


def test_model_covers_every_instantiation(layouts):
    # the kernel configurations gemm.hip launches
    src = open(GEMM).read()
    launched = set()
    for m in re.finditer(r"NVFP4_KP\((\d+),\s*(\d+),\s*(\d+),\s*(\d+)\)", src):
        launched.add(tuple(int(v) for v in m.groups()))
    assert launched and launched == set(layouts)


@dataclass
class U:
    k_beg: int
    k_end: int

    @property
    def nch(self):
        return (self.k_end - self.k_beg + 127) // 128


class ModelError(AssertionError):
    pass


class Workgroup:
    def __init__(self, L):
        self.L = L
        self.KW = L["KW"]
        self.ops = [[] for _ in range(self.KW)]  # per wave: issued VMEM ops, in order
        self.done = [0] * self.KW                # per wave: ops[:done] have completed
        self.epoch = 0                           # barriers passed
        self.last_read = {}                      # LDS region -> epoch of its last read
        self.pending = {}                        # LDS region -> op loaded there, not yet read
        self.last_idx = [{} for _ in range(self.KW)]  # per wave: op -> index of its last load
        self.waits = 0
        self.overwait = 0

    # -- hardware --------------------------------------------------------
    def issue(self, w, op):
        if len(self.ops[w]) - self.done[w] >= VMCNT_MAX:  # issue stalls at 63 outstanding
            self.done[w] += 1
        self.last_idx[w][op] = len(self.ops[w])
        self.ops[w].append(op)

    def wait(self, w, n, need):
        """s_waitcnt vmcnt(n); `need`: ops that must be complete afterwards."""
        self.waits += 1
        if n < VMCNT_MAX:
            self.done[w] = max(self.done[w], len(self.ops[w]) - n)
        for op in need:
            if self.last_idx[w][op] >= self.done[w]:
                raise ModelError("wave %d: %r not complete after vmcnt(%d)" % (w, op, n))
        if need:
            newest = max(self.last_idx[w][op] for op in need)
            if newest != self.done[w] - 1:
                self.overwait += 1

    def barrier(self):
        self.epoch += 1

    # -- LDS regions -------------------------------------------------------
    def write(self, region, what, landing=None):
        if self.last_read.get(region, -1) >= self.epoch:
            raise ModelError("%s writes %r while a wave may still read it" % (what, region))
        if region in self.pending:
            raise ModelError("%s overwrites unread %r in %r" % (what, self.pending[region], region))
        if landing is not None:
            self.pending[region] = landing

    def read(self, region, expect):
        got = self.pending.get(region)
        if got != expect:
            raise ModelError("read %r expecting %r, holds %r" % (region, expect, got))
        self.last_read[region] = self.epoch


def dma_chunks(L, wave, kind):
    """LDS byte offsets (relative to the stage / window base) of a wave's
    1 KB loads, as kp_issue / kp_issue_scales compute them."""
    KW = L["KW"]
    if kind == "w":
        return [L["kW"] + (wave * L["kWPerWave"] + tt) * 1024 for tt in range(L["kWPerWave"])]
    if kind == "x":
        out = []
        for tt in range(L["kXPerWave"]):
            t = wave * L["kXPerWave"] + tt if L["kXInstr"] >= KW else wave % L["kXInstr"]
            out.append(L["kX"] + t * 1024)
        return out
    out = []
    for tt in range(L["kSPerWave"]):
        t = wave * L["kSPerWave"] + tt if L["kSInstr"] >= KW else wave % L["kSInstr"]
        out.append(t * 1024)
    return out


def test_load_destinations_in_bounds_and_cover_slots(layouts):
    for cfg, L in layouts.items():
        for kind, base, size in (("w", 0, L["kStage"]), ("x", 0, L["kStage"]),
                                 ("s", 0, L["kWinBytes"])):
            cover = set()
            for w in range(L["KW"]):
                for off in dma_chunks(L, w, kind):
                    assert 0 <= off and off + 1024 <= size, (cfg, kind, off)
                    cover.add(off)
            if kind == "w":
                assert cover == set(range(L["kW"], L["kX"], 1024)), cfg
            elif kind == "x":
                assert cover == set(range(L["kX"], L["kStage"], 1024)), cfg
            else:
                assert cover == set(range(0, L["kWinBytes"], 1024)), cfg
        # every slot and window buffer inside the LDS array
        for sl in range(cfg[1]):
            assert (sl + 1) * L["kStage"] <= L["kSWin"]
        assert L["kSWin"] + L["kWinBufs"] * L["kWinBytes"] == L["kTotal"]


def simulate(L, units, can_pf, epi_rb=None, wait_bias=0, read_off=0, pn_extra=0):
    """Replay gemm_kp_kernel for one workgroup over `units` (its units in
    order).  epi_rb: output tile row bytes of the LDS epilogue (None: the
    widest, BN FP32 values).  wait_bias / read_off / pn_extra plant mistakes
    (waits looser by that many loads, stage reads from a shifted slot, more
    prefetched stages than free slots) to show that the checks catch them."""
    KW, D, WS = L["KW"], L["NSLOT"], L["kWinStages"]
    LS, SPW, E = L["kLoadsPerStage"], L["kSPerWave"], L["kEpiStores"]
    CPS, NSLOT = L["kChunksPerStage"], L["NSLOT"]
    wg = Workgroup(L)
    sb0 = wb0 = pf = 0
    ex = False
    for ui, cu in enumerate(units):
        nch = cu.nch
        nwin = (nch + WS - 1) // WS
        has_next = ui + 1 < len(units)
        nx = units[ui + 1] if has_next else None
        pn = min(L["kPrefetch"] + pn_extra, nx.nch) if (has_next and can_pf and nch >= NSLOT) else 0

        def slot(c):
            return ("slot", (sb0 + c) % NSLOT)

        def wbuf(i):
            return ("win", (wb0 + i) % L["kWinBufs"])

        def st_op(u, c):
            return ("S", u, c)

        def win_op(u, i):
            return ("W", u, i)

        def issue_window(u, i, buf):
            wg.write(buf, "window %d of unit %d" % (i, u), landing=win_op(u, i))
            for w in range(KW):
                for _ in range(SPW):
                    wg.issue(w, win_op(u, i))

        def issue_stage(u, c, sl):
            wg.write(sl, "stage %d of unit %d" % (c, u), landing=st_op(u, c))
            for w in range(KW):
                for _ in range(LS):
                    wg.issue(w, st_op(u, c))

        def loads_after(lo, hi):
            n = wait_bias + (E if (ex and lo < pf) else 0)
            for i in range(1, D):
                if lo + i <= hi:
                    n += LS + (SPW if (lo + i) % WS == 0 else 0)
            return n

        win_reads = {}  # window index -> stages of it read so far

        def read_stage(c):
            sl = ("slot", (sb0 + c + read_off) % NSLOT)
            wg.read(sl, st_op(ui, c))
            wg.pending.pop(sl)
            i = c // WS
            wg.read(wbuf(i), win_op(ui, i))
            win_reads[i] = win_reads.get(i, 0) + 1
            if win_reads[i] == min(WS, nch - i * WS):
                wg.pending.pop(wbuf(i))

        def need(c):
            return [st_op(ui, c), win_op(ui, c // WS)]

        nx_ops = 0
        for st in range(pf, min(D, nch)):
            if st % WS == 0:
                issue_window(ui, st // WS, wbuf(st // WS))
            issue_stage(ui, st, slot(st))
        for w in range(KW):
            wg.wait(w, loads_after(0, min(D, nch) - 1), need(0))
        wg.barrier()
        read_stage(0)

        full_last = cu.k_end - cu.k_beg == nch * 128
        c_lim = nch - WS - D + (1 if full_last else 0)
        c = 0
        while c < c_lim:  # steady blocks: compile-time waits
            for T in range(WS):
                cc = c + T
                k_after = sum(LS + (SPW if (T + i) % WS == 0 else 0) for i in range(2, D))
                for w in range(KW):
                    wg.wait(w, wait_bias + k_after + (E if (ex and cc + 1 < pf) else 0),
                            need(cc + 1))
                wg.barrier()
                if (T + D) % WS == 0:
                    issue_window(ui, (cc + D) // WS, wbuf((cc + D) // WS))
                issue_stage(ui, cc + D, slot(cc + D))
                read_stage(cc + 1)
            c += WS
        while c < nch:  # general iterations
            for cc in (c, c + 1):
                if cc >= nch:
                    break
                if cc + 1 < nch:
                    for w in range(KW):
                        wg.wait(w, loads_after(cc + 1, min(cc + D - 1, nch - 1)) + nx_ops,
                                need(cc + 1))
                    wg.barrier()
                    if cc + D < nch:
                        if (cc + D) % WS == 0:
                            issue_window(ui, (cc + D) // WS, wbuf((cc + D) // WS))
                        issue_stage(ui, cc + D, slot(cc + D))
                    elif cc + D - nch < pn:
                        j = cc + D - nch
                        if j == 0:
                            issue_window(ui + 1, 0, ("win", (wb0 + nwin) % L["kWinBufs"]))
                            nx_ops += SPW
                        issue_stage(ui + 1, j, slot(cc + D))
                        nx_ops += LS
                    read_stage(cc + 1)
            c += 2
        assert not any(k[0] == "slot" and v[1] == ui for k, v in wg.pending.items())
        # K-half exchange in the slots the prefetch leaves free
        wg.barrier()
        xslots = {("slot", (sb0 + nch + pn + k // CPS) % NSLOT) for k in range(L["kRedChunks"])}
        for r in xslots:
            wg.write(r, "exchange of unit %d" % ui)
        wg.barrier()
        for r in xslots:
            wg.last_read[r] = wg.epoch
        wg.barrier()
        if can_pf:
            # output tile through the same slots: rows of rb bytes, RPS per slot
            rb = epi_rb or L["BN"] * 4
            rps = L["kStage"] // rb
            assert rps % 4 == 0 and (L["BM"] + rps - 1) // rps <= L["kRedSlots"]
            sl0 = (sb0 + nch + pn) % NSLOT
            tslots = {("slot", (sl0 + row // rps) % NSLOT) for row in range(L["BM"])}
            for r in tslots:
                wg.write(r, "output tile of unit %d" % ui)
            wg.barrier()
            for r in tslots:
                wg.last_read[r] = wg.epoch
            wg.barrier()
            for w in range(KW):
                for _ in range(E):
                    wg.issue(w, ("E", ui))
        sb0 = (sb0 + nch) % NSLOT
        wb0 = (wb0 + (nch + WS - 1) // WS) % L["kWinBufs"]
        pf = pn
        ex = pn > 0
    return wg


def unit_chains(rng):
    """Unit sequences a workgroup can see: whole-K units of every length,
    split-K ranges, ragged last stages, long chains."""
    chains = []
    for nch in range(1, 26):
        chains.append([U(0, 128 * nch)])
        chains.append([U(0, 128 * nch - 64)])               # ragged last stage
        chains.append([U(0, 128 * nch)] * 3)
    for _ in range(60):
        n = int(rng.integers(2, 12))
        chains.append([U(0, 64 * int(rng.integers(1, 48))) for _ in range(n)])
    # split-K ranges of one tile (K split into 1024-deep halves, 7-stage splits)
    chains.append([U(0, 1024), U(1024, 2048)])
    chains.append([U(896 * s, min(7168, 896 * (s + 1))) for s in range(8)])
    return chains


@pytest.mark.parametrize("can_pf", [True, False])
def test_schedule_model_every_configuration(layouts, can_pf):
    rng = np.random.default_rng(2024)
    chains = unit_chains(rng)
    for cfg, L in layouts.items():
        for chain in chains:
            rbs = [None] if not can_pf else [L["BN"] * 4, L["BN"] * 2, L["BN"], L["BN"] // 2 * 2]
            for rb in rbs:
                try:
                    wg = simulate(L, chain, can_pf, rb)
                except ModelError as e:
                    raise AssertionError("%s %s pf=%s: %s" % (cfg, [u.nch for u in chain],
                                                              can_pf, e))
                assert wg.overwait == 0, (cfg, [u.nch for u in chain], wg.overwait)


def test_recorded_fault_shape(layouts):
    """Grouped split-K: 4 experts (70 / 0 / 5 / 33 rows), N = 513, K = 2048,
    2 splits on the 4-wave 32-row kernel.  Every unit holds one 1024-deep K
    half (8 stages: one steady block, then the general iterations); with 60
    units and 512 resident workgroups each workgroup runs one unit, and with
    the grid capped (several units per workgroup) the chain alternates the
    two K halves.  No prefetch across units (a K split is never prefetched)."""
    L = layouts[(32, 4, 4, 128)]
    halves = [U(0, 1024), U(1024, 2048)]
    for chain in ([halves[0]], [halves[1]], halves * 4, [halves[1], halves[0]] * 3):
        wg = simulate(L, chain, can_pf=False)
        assert wg.overwait == 0
    # the same shape with 2, 5 and 12 splits (K ranges of 1024, 448 -> 512,
    # 192 -> 256 rounded to 64-multiples of the split)
    for splits in (2, 5, 12):
        ks = -(-2048 // splits)
        ks = -(-ks // 64) * 64
        ranges = [U(s * ks, min(2048, (s + 1) * ks)) for s in range(-(-2048 // ks))]
        wg = simulate(L, ranges, can_pf=False)
        assert wg.overwait == 0


def test_model_detects_planted_mistakes(layouts):
    """The model has teeth: waits one load too loose, stage reads from the
    neighbouring slot and a prefetch into the exchange slots are each caught."""
    L = layouts[(64, 4, 8, 256)]
    chain = [U(0, 128 * 12)] * 3
    simulate(L, chain, True)
    with pytest.raises(ModelError):
        simulate(L, chain, True, wait_bias=1)
    with pytest.raises(ModelError):
        simulate(L, chain, True, read_off=1)
    with pytest.raises(ModelError):
        simulate(L, chain, True, pn_extra=1)
    L32 = layouts[(32, 4, 4, 128)]
    with pytest.raises(ModelError):
        simulate(L32, [U(0, 1024), U(1024, 2048)], False, wait_bias=1)
