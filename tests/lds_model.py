"""A host-side model of the LDS schedules of the attention kernels.

The query-side, key-side and shift kernels stage operands in LDS and hand
data between the waves of a workgroup (four, or eight in the causal query
side that splits the feature steps in two halves) across barriers: the ring of
feature-step operand buffers (s_op) with the z values in the last slot of a
step, the key-feature buffers (s_kf), the operands copied global -> LDS by the
DMA path (all steps, and M' in the key-feature buffers), the V^T tile, and on
the key side the double-buffered tile state.  This module replays, wave by
wave and barrier phase by barrier phase, every LDS access these kernels make
(the same index arithmetic, the same constexpr choices of buffering, derived
here from the same formulas), and checks at byte granularity:

  * every access lies inside its array;
  * every byte read was written before and is visible to the reader: by the
    same wave earlier in program order, or by any wave in an earlier barrier
    phase (DMA copies count as written when the issuing wave waits for its
    vector-memory counter);
  * no byte written by one wave in a phase is read or written by another
    wave in the same phase.

A read of LDS that the launch never wrote would return whatever an earlier
workgroup or launch left there; this is the failure that shows on a process's
first launch and hides on later ones.  The model is checked against planted
mistakes (a barrier removed, a buffer index changed) in test_lds_schedule.py.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

WAVES = 4
LANES = np.arange(64)
C = LANES & 31
G = LANES >> 5
MAX_LDS = 160 * 1024


class Violation(AssertionError):
    pass


@dataclass
class Tracker:
    sizes: dict                                # array name -> bytes
    mutate: set = field(default_factory=set)   # planted mistakes (tests of the model itself)
    waves: int = WAVES

    def __post_init__(self):
        self.epoch = 0
        self.w_epoch = {n: np.full(s, -1, np.int64) for n, s in self.sizes.items()}
        self.w_wave = {n: np.full(s, -1, np.int64) for n, s in self.sizes.items()}
        self.r_epoch = {n: np.full(s, -1, np.int64) for n, s in self.sizes.items()}
        self.r_mask = {n: np.zeros(s, np.int64) for n, s in self.sizes.items()}
        self.pending = {w: [] for w in range(self.waves)}   # DMA copies in flight per wave
        self.total = sum(self.sizes.values())

    def _bytes(self, name, starts, width):
        idx = (np.asarray(starts, np.int64)[:, None] + np.arange(width)[None, :]).ravel()
        if idx.size and (idx.min() < 0 or idx.max() >= self.sizes[name]):
            raise Violation(f"{name}: access [{idx.min()}, {idx.max()}] outside [0, {self.sizes[name]})")
        return np.unique(idx)

    def write(self, wave, name, starts, width):
        b = self._bytes(name, starts, width)
        other_r = (self.r_epoch[name][b] == self.epoch) & ((self.r_mask[name][b] & ~(1 << wave)) != 0)
        if other_r.any():
            raise Violation(f"{name}: wave {wave} writes byte {b[other_r][0]} that another wave reads in phase "
                            f"{self.epoch}")
        other_w = (self.w_epoch[name][b] == self.epoch) & (self.w_wave[name][b] != wave) & (self.w_wave[name][b] >= 0)
        if other_w.any():
            raise Violation(f"{name}: waves {wave} and {self.w_wave[name][b][other_w][0]} write byte "
                            f"{b[other_w][0]} in phase {self.epoch}")
        self.w_epoch[name][b] = self.epoch
        self.w_wave[name][b] = wave

    def read(self, wave, name, starts, width):
        b = self._bytes(name, starts, width)
        we, ww = self.w_epoch[name][b], self.w_wave[name][b]
        never = we < 0
        if never.any():
            raise Violation(f"{name}: wave {wave} reads byte {b[never][0]} that was never written (phase {self.epoch})")
        same_phase_other = (ww != wave) & (we == self.epoch)
        if same_phase_other.any():
            raise Violation(f"{name}: wave {wave} reads byte {b[same_phase_other][0]} written by wave "
                            f"{ww[same_phase_other][0]} in the same phase {self.epoch}")
        fresh = self.r_epoch[name][b] != self.epoch
        self.r_mask[name][b[fresh]] = 0
        self.r_epoch[name][b] = self.epoch
        self.r_mask[name][b] |= 1 << wave

    def dma(self, wave, name, start, nbytes=1024):
        """One global -> LDS copy by a wave: lane l fills bytes [16 l, 16 l + 16) of the 1 KB at start
        (the first nbytes / 16 lanes when the others are idle)."""
        self._bytes(name, [start], nbytes)
        self.pending[wave].append((name, start, nbytes))

    def waitcnt(self, wave):
        """The wave waits for its vector-memory counter: its DMA copies have landed."""
        for name, start, nbytes in self.pending[wave]:
            self.write(wave, name, [start], nbytes)
        self.pending[wave] = []


def run_waves(tr: Tracker, programs):
    """programs[w] is a generator yielding at each barrier; phases advance together.
    In each round every wave still running must reach the same barrier, or all
    of them must finish (a wave that leaves early may do so only after the last
    barrier)."""
    gens = list(programs)
    alive = [True] * len(gens)
    while any(alive):
        running = sum(alive)
        hits = 0
        for w in range(len(gens)):
            if not alive[w]:
                continue
            try:
                next(gens[w])
                hits += 1
            except StopIteration:
                alive[w] = False
        if hits not in (0, running):
            raise Violation("waves reach different numbers of barriers")
        tr.epoch += 1


# ---------------------------------------------------------------------------
# shared definitions (the kernels' constants)
# ---------------------------------------------------------------------------
def fold_exponent(elem, d_h, r16):
    return elem == 2 and 2 * d_h < 3 * 16 * r16


def vblocks(dh):
    return (dh + 31) // 32


def vblocks_ones(dh):
    return (dh + 1 + 31) // 32


def vloads_per_thread(dh, tt, nt=256):
    return (tt * (dh // 8) + nt - 1) // nt


def vt_pos(t):
    return (t & ~12) | ((t & 4) << 1) | ((t & 8) >> 1)


def frag_lanes(base_elem, elem):
    """Byte starts of the 64 lanes of one 8-element operand fragment at element base_elem."""
    return (base_elem + LANES * 8) * elem


def store_vt(tr, w, name, base, dh, tt, vst, elem, nt=256):
    """store_vt: rows t0 .. t0 + TT - 1 of V into s_vt[d][vt_pos(t)] (every thread of wave w, nt threads)."""
    for p in range(vloads_per_thread(dh, tt, nt)):
        e = 64 * w + LANES + p * nt
        ok = e < tt * (dh // 8)
        e = e[ok]
        tl, d8 = e % tt, (e // tt) * 8
        pos = np.array([vt_pos(int(t)) for t in tl], np.int64)
        for i in range(8):
            tr.write(w, name, (base + (d8 + i) * vst + pos) * elem, elem)


def store_v(tr, w, name, base, dh, tt, elem, nt=256):
    """store_v (bf16): token row tid % TT, 16-byte pieces at columns 8 (tid / TT) + p (nt / TT) 8,
    in s_v[t][d] with rows dh + 16 elements apart."""
    vsn, step = dh + 16, nt // tt * 8
    tid = 64 * w + LANES
    for p in range(vloads_per_thread(dh, tt, nt)):
        col = (tid // tt) * 8 + p * step
        assert np.all(col < dh)   # the kernel asserts every piece is inside the row
        tr.write(w, name, (base + (tid % tt) * vsn + col) * elem, 16)


def v_frag_read_tr(tr, w, name, base, dh, db, tb0, k, elem, ones=False):
    """v_frag_tr (bf16): two transpose loads; each lane reads 8 bytes at its own address."""
    if (ones or dh % 32 != 0) and db * 32 >= dh:
        return
    vsn = dh + 16
    x, q = LANES & 15, LANES >> 4
    row = tb0 + 16 * k + 4 * G + (x >> 2)
    col = np.minimum(db * 32 + 16 * (q & 1) + 4 * (x & 3), dh - 4)
    for half in range(2):
        tr.read(w, name, (base + (row + 8 * half) * vsn + col) * elem, 8)


def v_frag_read(tr, w, name, base, dh, vst, db, tb0, k, elem, ones=False):
    d = db * 32 + C
    ok = ~(((ones or dh % 32 != 0)) & (d >= dh))
    starts = (base + d[ok] * vst + tb0 + 16 * k + 8 * G[ok]) * elem
    if starts.size:
        tr.read(w, name, starts, 8 * elem)


# ---------------------------------------------------------------------------
# query side (qout_kernel)
# ---------------------------------------------------------------------------
@dataclass
class QoutConfig:
    elem: int          # 2 (bf16) or 4 (fp32)
    dh: int
    r16: int
    nqb: int
    causal: bool
    allfb: int         # > 0: all steps staged by DMA (bf16, causal, FB <= allfb)
    fb: int            # feature blocks of the call
    m: int             # features (m <= 32 fb)
    kshift: bool = False

    def derived(self):
        e, dh = self.elem, self.dh
        kd, nm, db = dh // 16, (2 if e == 2 else 1), vblocks(dh)
        nb = WAVES * self.nqb
        tt = 32 * nb
        vst = tt + 8
        fold = fold_exponent(e, dh, self.r16)
        uk = kd if fold else self.r16
        nof = uk   # omega' (W') fragments per step: one part (fp16 on the bf16 path)
        nstep = nof + 2 * db + 1
        vt_elems = dh * vst if self.causal else 8
        k_base = vt_elems * e
        k_op = nstep * 512 * e
        k_kf = nb * 2 * 512 * e if self.causal else 0
        # non-causal with at most 8 operand slots per step: each wave reads them
        # from L2 itself, nothing staged
        self_read = not self.causal and self.allfb == 0 and nstep <= 8
        stage = not self_read and k_base + k_op + k_kf <= MAX_LDS
        opb = 0 if not stage else (2 if k_base + 2 * k_op + 2 * k_kf <= MAX_LDS else 1)
        kbuf = 2 if k_base + opb * k_op + 2 * k_kf <= MAX_LDS else 1
        kf_elems = kbuf * nb * 2 * 512 if self.causal else 8
        all_ = self.allfb > 0
        op_elems = self.allfb * nstep * 512 if all_ else (opb * nstep * 512 if stage else 8)
        mfrg = ((self.r16 + 1) // 2) * kd * nm
        m_lds = all_ and self.causal and mfrg * 512 <= kf_elems
        return dict(kd=kd, nm=nm, db=db, nb=nb, tt=tt, vst=vst, fold=fold, uk=uk, nof=nof, nstep=nstep,
                    zs=nstep - 1, zw=8 * e // 4, perw=(nstep + WAVES - 1) // WAVES, vt_elems=vt_elems,
                    stage=stage, opb=opb, kbuf=kbuf, kf_elems=kf_elems, all=all_, op_elems=op_elems,
                    mfrg=mfrg, m_lds=m_lds, r32=(self.r16 + 1) // 2, self_read=self_read)


def qout_model(cfg: QoutConfig, mutate=frozenset()):
    D = cfg.derived()
    e = cfg.elem
    sizes = {"s_vt": D["vt_elems"] * e, "s_kf": D["kf_elems"] * e, "s_op": D["op_elems"] * e,
             # unstaged form: z of every feature (dynamic LDS, 4 bytes each)
             "s_zall": 128 * cfg.fb if D["self_read"] else 0}
    if sum(sizes.values()) > MAX_LDS:
        raise Violation(f"LDS {sum(sizes.values())} bytes > {MAX_LDS}")
    tr = Tracker(sizes, set(mutate))
    nstep, nm, uk, zs = D["nstep"], D["nm"], D["uk"], D["zs"]

    def op_read(w, fb, buf, f):
        if D["all"]:
            tr.read(w, "s_op", frag_lanes((fb * nstep + f) * 512, e), 8 * e)
        elif D["stage"]:
            tr.read(w, "s_op", frag_lanes((buf * nstep + f) * 512, e), 8 * e)

    def zrow4(w, fb, buf, jj):
        if D["all"]:
            zb = (fb * nstep + zs) * 512 * e
        elif D["stage"]:
            zb = (buf * nstep + zs) * 512 * e
        else:
            if D["self_read"]:
                tr.read(w, "s_zall", fb * 128 + (8 * jj + 4 * G) * 4, 16)
            return
        tr.read(w, "s_op", zb + (8 * jj + 4 * G) * 4, 16)

    def exponent_reads(w, fb, buf):
        for k in range(uk):
            op_read(w, fb, buf, k)

    def store_step(w, buf):
        if D["stage"] and not D["all"]:
            for q in range(D["perw"]):
                f = w + WAVES * q
                if f < nstep:
                    tr.write(w, "s_op", frag_lanes((buf * nstep + f) * 512, e), 8 * e)

    def wave(w):
        # DMA staging of all steps and M'
        if D["all"]:
            for idx in range(w, cfg.fb * nstep, WAVES):
                tr.dma(w, "s_op", idx * 512 * e)
            if D["m_lds"]:
                for idx in range(w, D["mfrg"], WAVES):
                    tr.dma(w, "s_kf", idx * 512 * e)
            if "no_wait_before_vt" not in tr.mutate:
                tr.waitcnt(w)
        if cfg.causal:
            store_vt(tr, w, "s_vt", 0, cfg.dh, D["tt"], D["vst"], e)
        if D["m_lds"]:
            yield                                            # M' and every wave's copies visible
        # projections (key shifts and unfolded u) read M' from LDS when staged there
        if D["m_lds"]:
            nproj = cfg.nqb * (0 if D["fold"] else 1) + (cfg.nqb if cfg.causal and not cfg.kshift else 0)
            for _ in range(nproj):
                for rb in range(D["r32"]):
                    for kd in range(D["kd"]):
                        for part in range(nm):
                            tr.read(w, "s_kf", frag_lanes((((rb * D["kd"] + kd) * nm + part) * 64) * 8, e), 8 * e)
        if D["all"]:
            tr.waitcnt(w)
            yield
            exponent_reads(w, 0, 0)                          # the query shift from feature block 0
            fbs = range(cfg.fb)
        else:
            if D["self_read"]:                               # z copies: 1 KB (256 values) per wave instruction
                for i in range(w, (cfg.fb * 32 + 255) // 256, WAVES):
                    tr.dma(w, "s_zall", i * 1024, min(1024, 128 * cfg.fb - 1024 * i))
            store_step(w, 0)
            if D["self_read"] and "no_z_wait" not in tr.mutate:
                tr.waitcnt(w)
            yield
            exponent_reads(w, 0, 0)
            fbs = range(cfg.fb)
        for fb in fbs:
            buf = 0 if D["all"] else (fb & 1 if D["opb"] == 2 else 0)
            # step(fb, buf)
            if not D["fold"]:
                for k in range(uk):
                    op_read(w, fb, buf, k)
            for _j in range(cfg.nqb):
                if D["fold"]:
                    exponent_reads(w, fb, buf)
                for jj in range(4):
                    zrow4(w, fb, buf, jj)
            for db in range(D["db"]):
                for k in range(2):
                    op_read(w, fb, buf, D["nof"] + 2 * db + k)
            if cfg.causal:
                kb = (fb & 1 if D["kbuf"] == 2 else 0)
                if "kbuf_index_fixed" in tr.mutate:
                    kb = 0
                kbase = kb * D["nb"] * 2 * 512
                for j in range(cfg.nqb):
                    if D["fold"]:
                        exponent_reads(w, fb, buf)
                    for k in range(2):
                        tr.write(w, "s_kf", frag_lanes(kbase + ((w * cfg.nqb + j) * 2 + k) * 512, e), 8 * e)
                if "no_kbuf_barrier" not in tr.mutate:
                    yield
                for j in range(cfg.nqb):
                    gq = w * cfg.nqb + j
                    for kb2 in range(D["nb"]):
                        if kb2 <= gq:
                            for k in range(2):
                                tr.read(w, "s_kf", frag_lanes(kbase + (kb2 * 2 + k) * 512, e), 8 * e)
                if D["kbuf"] == 1 and "no_kbuf1_barrier" not in tr.mutate:
                    yield
            if not D["all"] and D["stage"]:
                if fb + 1 < cfg.fb:
                    if D["opb"] == 1 and "no_opb1_barrier" not in tr.mutate:
                        yield
                    nbuf = (fb + 1) & 1 if D["opb"] == 2 else 0
                    if "ring_same_buffer" in tr.mutate:
                        nbuf = buf
                    store_step(w, nbuf)
                if "no_step_barrier" not in tr.mutate:
                    yield
        # epilogue: the intra-chunk products read the V^T tile
        if cfg.causal:
            for j in range(cfg.nqb):
                gq = w * cfg.nqb + j
                for kb2 in range(D["nb"]):
                    if kb2 > gq:
                        continue
                    for k in range(2):
                        for db in range(D["db"]):
                            v_frag_read(tr, w, "s_vt", 0, cfg.dh, D["vst"], db, 32 * kb2, k, e)

    run_waves(tr, [wave(w) for w in range(WAVES)])
    return tr


# ---------------------------------------------------------------------------
# causal query side with eight waves (qout8_kernel): the feature steps in two
# halves, each half with its own pair of key-feature buffers; the halves' N and
# D meet in s_op at the end, and the output rows are staged in s_kf (or s_vt)
# ---------------------------------------------------------------------------
WAVES8 = 8


def qout8_fits(elem, dh, r16, allfb=8):
    kd, nm, db = dh // 16, (2 if elem == 2 else 1), vblocks(dh)
    uk = kd if fold_exponent(elem, dh, r16) else r16
    nstep = uk + 2 * db + 1
    vt = dh * 136 * elem
    op = allfb * nstep * 512 * elem
    kf = 2 * 2 * WAVES * 2 * 512 * elem
    xch = WAVES * (db * 16 + 1) * 64 * 4
    ost = WAVES * 32 * (dh + 8) * elem
    return elem == 2 and vt + op + kf <= MAX_LDS and xch <= op and (ost <= kf or ost <= vt)


def qout8_model(cfg: QoutConfig, mutate=frozenset()):
    e, dh = cfg.elem, cfg.dh
    kd, nm, db = dh // 16, (2 if e == 2 else 1), vblocks(dh)
    fold = fold_exponent(e, dh, cfg.r16)
    uk = kd if fold else cfg.r16
    nof = uk
    nstep = nof + 2 * db + 1
    zs = nstep - 1
    vst = 136
    kfh = 2 * WAVES * 2 * 512                  # elements: the two key-feature buffers of one half
    kf_elems, op_elems, vt_elems = 2 * kfh, cfg.allfb * nstep * 512, dh * vst
    mfrg = ((cfg.r16 + 1) // 2) * kd * nm
    m_lds = mfrg * 512 <= kf_elems
    xw = db * 16 + 1
    ost = dh + 8
    ost_kf = WAVES * 32 * ost <= kf_elems
    sizes = {"s_vt": vt_elems * e, "s_kf": kf_elems * e, "s_op": op_elems * e}
    if sum(sizes.values()) > MAX_LDS:
        raise Violation(f"LDS {sum(sizes.values())} bytes > {MAX_LDS}")
    tr = Tracker(sizes, set(mutate), waves=WAVES8)
    op_read = lambda w, fb, f: tr.read(w, "s_op", frag_lanes((fb * nstep + f) * 512, e), 8 * e)  # noqa: E731

    def exponent_reads(w, fb):
        for k in range(uk):
            op_read(w, fb, k)

    # each half's first step (0 and nit) is copied by DMA at the start; the
    # other steps' slots are requested into registers, PL per wave, and
    # written to LDS in the first step, before its barrier
    nit = (cfg.fb + 1) // 2
    early = [0] + ([nit] if cfg.fb > 1 else [])
    n_late = (cfg.fb - len(early)) * nstep
    pl = ((cfg.allfb - 2) * nstep + WAVES8 - 1) // WAVES8

    def late_slot(l):
        j, f = divmod(l, nstep)
        return (1 + j if j < nit - 1 else nit + 1 + (j - (nit - 1))), f

    def wave(w):
        half = w // WAVES
        qb = w % WAVES if half == 0 else WAVES - 1 - w % WAVES   # reversed in the second half
        if m_lds:
            for idx in range(w, mfrg, WAVES8):
                tr.dma(w, "s_kf", idx * 512 * e)
        for idx in range(w, len(early) * nstep, WAVES8):
            fb_e, f = early[idx // nstep], idx % nstep
            tr.dma(w, "s_op", (fb_e * nstep + f) * 512 * e)
        if "no_wait8" not in tr.mutate:
            tr.waitcnt(w)
        store_vt(tr, w, "s_vt", 0, dh, 128, vst, e, nt=64 * WAVES8)
        yield                                            # M', V^T and every copy visible
        if m_lds:
            nproj = (0 if fold else 1) + (0 if (fold and cfg.kshift) else 1)
            for _ in range(nproj):
                for rb in range((cfg.r16 + 1) // 2):
                    for kd_ in range(kd):
                        for part in range(nm):
                            tr.read(w, "s_kf", frag_lanes(((rb * kd + kd_) * nm + part) * 512, e), 8 * e)
        exponent_reads(w, 0)                             # the query shift
        if m_lds and "no_m_barrier8" not in tr.mutate:
            yield                                        # M' no longer read
        for it in range(nit):
            fb = half * nit + it
            live = fb < cfg.fb
            kbase = half * kfh + ((it & 1) if "kbuf8_index_fixed" not in tr.mutate else 0) * WAVES * 2 * 512
            if live:
                exponent_reads(w, fb)                    # queries (unfolded: the step's omega' read once)
                for jj in range(4):
                    tr.read(w, "s_op", (fb * nstep + zs) * 512 * e + (8 * jj + 4 * G) * 4, 16)
                for d in range(db):
                    for k in range(2):
                        op_read(w, fb, nof + 2 * d + k)
                if fold:
                    exponent_reads(w, fb)                # keys
                for k in range(2):
                    tr.write(w, "s_kf", frag_lanes(kbase + (qb * 2 + k) * 512, e), 8 * e)
            if it == 0 and "late8_after_barrier" not in tr.mutate:
                for p_ in range(pl):
                    l = w + WAVES8 * p_
                    if l < n_late:
                        fb2, f2 = late_slot(l)
                        tr.write(w, "s_op", frag_lanes((fb2 * nstep + f2) * 512, e), 8 * e)
            if "no_kbuf8_barrier" not in tr.mutate:
                yield
            if it == 0 and "late8_after_barrier" in tr.mutate:   # planted: the late slots written too late
                for p_ in range(pl):
                    l = w + WAVES8 * p_
                    if l < n_late:
                        fb2, f2 = late_slot(l)
                        tr.write(w, "s_op", frag_lanes((fb2 * nstep + f2) * 512, e), 8 * e)
            if live:
                for kb2 in range(qb + 1):
                    for k in range(2):
                        tr.read(w, "s_kf", frag_lanes(kbase + (kb2 * 2 + k) * 512, e), 8 * e)
        for kb2 in range(qb + 1):                        # this half's scores times V
            for k in range(2):
                for d in range(db):
                    v_frag_read(tr, w, "s_vt", 0, dh, vst, d, 32 * kb2, k, e)
        xbase = qb * xw * 64 * 4
        xbytes = xbase + (np.arange(xw)[:, None] * 64 + LANES[None, :]).ravel() * 4
        if half == 1:
            tr.write(w, "s_op", xbytes, 4)
        if "no_exchange_barrier" not in tr.mutate:
            yield                                        # the hand-over is in
        if half == 1:
            return
        tr.read(w, "s_op", xbytes, 4)
        buf = "s_kf" if ost_kf else "s_vt"
        base = qb * 32 * ost
        for i in range(16):
            row = 8 * (i >> 2) + 4 * G + (i & 3)
            for d in range(db):
                dd = d * 32 + C
                ok = dd < dh
                tr.write(w, buf, (base + row[ok] * ost + dd[ok]) * e, e)
        cpr = dh // 8
        for q0 in range(0, 32 * cpr, 64):
            q = q0 + LANES
            q = q[q < 32 * cpr]
            row, col = q // cpr, (q % cpr) * 8
            tr.read(w, buf, (base + row * ost + col) * e, 16)

    run_waves(tr, [wave(w) for w in range(WAVES8)])
    return tr


def qout8_cases():
    """The eight-wave query side: bf16, causal, m a multiple of 32; every step
    count from 1 to 8 (each splits differently into early and late steps)."""
    out = []
    for dh in HEAD_DIMS:
        for r16 in RANK_BLOCKS:
            if not (qout_all_fits(2, dh, r16) and qout8_fits(2, dh, r16)):
                continue
            fold = fold_exponent(2, dh, r16)
            for fb in range(1, 9):
                fbw = 2 if dh <= 64 else 1
                nf = -(-fb // (4 * fbw))
                kshift = fold and (nf > 1 or dh >= 128)
                out.append((QoutConfig(2, dh, r16, 1, True, 8, fb, 32 * fb, kshift), f"q8 d{dh} r{r16} fb{fb}"))
    return out


# ---------------------------------------------------------------------------
# key side (kstate_kernel, the tiled form)
# ---------------------------------------------------------------------------
@dataclass
class KstateConfig:
    elem: int
    dh: int
    r16: int
    fbw: int
    tiles: int         # tiles of 128 tokens in the unit
    kshift: bool = False

    def derived(self):
        e, dh = self.elem, self.dh
        kd, nm = dh // 16, (2 if e == 2 else 1)
        tt = 128
        vst = tt + 8
        fold = fold_exponent(e, dh, self.r16)
        uk = kd if fold else self.r16
        up = 1 if fold else nm
        zmma = (not fold) or dh % 32 != 0
        dbk = vblocks_ones(dh) if zmma else vblocks(dh)
        mfr = ((self.r16 + 1) // 2) * kd * nm
        m_lds = mfr * 512 * e <= 32 * 1024
        vtr = e == 2                    # bf16: V in its row layout, read by transpose loads
        v_elems = tt * (dh + 16) if vtr else dh * vst
        tile_state = (WAVES * up * uk * 512 + v_elems) * e + tt * 4
        nbuf = 2 if 2 * tile_state + (mfr * 512 * e if m_lds else 0) <= MAX_LDS else 1
        return dict(kd=kd, nm=nm, tt=tt, vst=vst, fold=fold, uk=uk, up=up, zmma=zmma, dbk=dbk, mfr=mfr,
                    m_lds=m_lds, nbuf=nbuf, r32=(self.r16 + 1) // 2, vhold=dbk <= 4, vtr=vtr, v_elems=v_elems)


def kstate_tile_lds_bytes(elem, dh, r16):
    fold = fold_exponent(elem, dh, r16)
    uk = dh // 16 if fold else r16
    up = 1 if fold else (2 if elem == 2 else 1)
    mbytes = ((r16 + 1) // 2) * (dh // 16) * (2 if elem == 2 else 1) * 512 * elem
    v_elems = 128 * (dh + 16) if elem == 2 else dh * 136
    return (WAVES * up * uk * 512 + v_elems) * elem + 128 * 4 + (mbytes if mbytes <= 32 * 1024 else 16)


def kstate_model(cfg: KstateConfig, mutate=frozenset()):
    D = cfg.derived()
    e = cfg.elem
    nb, up, uk = D["nbuf"], D["up"], D["uk"]
    u_slot = lambda buf, w, part, k: ((((buf * WAVES + w) * up + part) * uk + k) * 512)  # noqa: E731
    sizes = {"s_u": nb * WAVES * up * uk * 512 * e, "s_init": nb * 128 * 4, "s_vt": nb * D["v_elems"] * e,
             "s_m": (D["mfr"] * 512 if D["m_lds"] else 8) * e}
    if sum(sizes.values()) > MAX_LDS:
        raise Violation(f"LDS {sum(sizes.values())} bytes > {MAX_LDS}")
    tr = Tracker(sizes, set(mutate))

    def project_tile(w, buf):
        if D["m_lds"] and (not D["fold"] or not cfg.kshift):
            for rb in range(D["r32"]):
                for kd in range(D["kd"]):
                    for part in range(D["nm"]):
                        tr.read(w, "s_m", frag_lanes(((rb * D["kd"] + kd) * D["nm"] + part) * 512, e), 8 * e)
        if D["fold"]:
            for k in range(uk):
                tr.write(w, "s_u", frag_lanes(u_slot(buf, w, 0, k), e), 8 * e)
        else:
            # u as one fp16 fragment per K-step (bf16 path) or one fp32 fragment
            for k in range(cfg.r16):
                tr.write(w, "s_u", frag_lanes(u_slot(buf, w, 0, k), e), 8 * e)
        tr.write(w, "s_init", (buf * 128 + 32 * w + C[G == 0]) * 4, 4)
        if D["vtr"]:
            store_v(tr, w, "s_vt", buf * D["v_elems"], cfg.dh, 128, e)
        else:
            store_vt(tr, w, "s_vt", buf * cfg.dh * D["vst"], cfg.dh, 128, D["vst"], e)

    def vread(w, buf, db, tb0, k):
        if D["vtr"]:
            v_frag_read_tr(tr, w, "s_vt", buf * D["v_elems"], cfg.dh, db, tb0, k, e, ones=D["zmma"])
        else:
            v_frag_read(tr, w, "s_vt", buf * cfg.dh * D["vst"], cfg.dh, D["vst"], db, tb0, k, e, ones=D["zmma"])

    def compute_tile(w, buf):
        for tb in range(WAVES):
            for jj in range(4):
                tr.read(w, "s_init", (buf * 128 + 32 * tb + 8 * jj + 4 * G) * 4, 16)
            if D["vhold"]:
                for db in range(D["dbk"]):
                    for k in range(2):
                        vread(w, buf, db, 32 * tb, k)
            for _f in range(cfg.fbw):
                for k in range(uk):
                    tr.read(w, "s_u", frag_lanes(u_slot(buf, tb, 0, k), e), 8 * e)
                    if not D["fold"] and e == 4:   # fp32: the exponent's lo read is part 0 again
                        tr.read(w, "s_u", frag_lanes(u_slot(buf, tb, up - 1, k), e), 8 * e)
                if not D["vhold"]:
                    for db in range(D["dbk"]):
                        for k in range(2):
                            vread(w, buf, db, 32 * tb, k)

    def wave(w):
        if D["m_lds"]:   # M' by the DMA path, 1 KB per wave instruction, then vmcnt(0)
            for i in range(w, D["mfr"] * 512 * e // 1024, WAVES):
                tr.dma(w, "s_m", i * 1024)
            if "no_m_wait" not in tr.mutate:
                tr.waitcnt(w)
        if nb == 2:
            yield                                   # M' in LDS
            project_tile(w, 0)
            yield
            for it in range(cfg.tiles):
                more = it + 1 < cfg.tiles
                compute_tile(w, it & 1)
                if more:
                    project_tile(w, (it + 1) & 1 if "tile_same_buffer" not in tr.mutate else it & 1)
                yield
        else:
            yield
            for _ in range(cfg.tiles):
                project_tile(w, 0)
                yield
                compute_tile(w, 0)
                if "no_tile_end_barrier" not in tr.mutate:
                    yield

    run_waves(tr, [wave(w) for w in range(WAVES)])
    return tr


# ---------------------------------------------------------------------------
# key shifts (shift_kernel): M' slices double-buffered through LDS
# ---------------------------------------------------------------------------
def shift_model(elem, dh, r16, mutate=frozenset()):
    kd, nm = dh // 16, (2 if elem == 2 else 1)
    sl = kd * nm
    ps = (sl * 64 + 255) // 256
    r32 = (r16 + 1) // 2
    tr = Tracker({"s_m": 2 * sl * 512 * elem}, set(mutate))

    def put(w, buf):
        for p in range(ps):
            idx = 64 * w + LANES + p * 256
            ok = idx < sl * 64
            tr.write(w, "s_m", (buf * sl * 512 + idx[ok] * 8) * elem, 8 * elem)

    def wave(w):
        put(w, 0)
        yield
        for rb in range(r32):
            for kd_ in range(kd):
                for part in range(nm):
                    tr.read(w, "s_m", frag_lanes((rb & 1) * sl * 512 + ((kd_ * nm + part) * 64) * 8, elem), 8 * elem)
            if rb + 1 < r32:
                put(w, (rb + 1) & 1 if "shift_same_buffer" not in tr.mutate else rb & 1)
            yield

    run_waves(tr, [wave(w) for w in range(WAVES)])
    return tr


# ---------------------------------------------------------------------------
# every instantiation the library builds, with the launch choices of the host
# ---------------------------------------------------------------------------
DTYPES = (2, 4)
HEAD_DIMS = (16, 32, 64, 128, 256)
RANK_BLOCKS = (1, 2, 4, 8, 16)


def qout_all_fits(elem, dh, r16, allfb=8):
    kd, nm, db = dh // 16, (2 if elem == 2 else 1), vblocks(dh)
    uk = kd if fold_exponent(elem, dh, r16) else r16
    nstep = uk + 2 * db + 1
    vt = dh * (128 + 8) * elem
    return elem == 2 and vt + allfb * nstep * 512 * elem + 2 * 4 * 2 * 512 * elem <= MAX_LDS


def qout_cases():
    """(QoutConfig, label) for every launched query-side variant and a few feature counts."""
    out = []
    for elem in DTYPES:
        for dh in HEAD_DIMS:
            for r16 in RANK_BLOCKS:
                fold = fold_exponent(elem, dh, r16)
                for fb in (1, 2, 3, 9):
                    m = 32 * fb - (16 if fb > 1 else 0)
                    # non-causal: one or two query blocks per wave (two only for d_h <= 128)
                    for nqb in ((1, 2) if dh <= 128 else (1,)):
                        out.append((QoutConfig(elem, dh, r16, nqb, False, 0, fb, m), f"nc e{elem} d{dh} r{r16} "
                                    f"nqb{nqb} fb{fb}"))
                    # causal: one query block per wave, all-step staging when it fits and FB <= 8
                    if (dh * (128 + 8) + 4 * 2 * 512) * elem <= MAX_LDS:
                        allfb = 8 if (qout_all_fits(elem, dh, r16) and fb <= 8) else 0
                        fbw = 2 if dh <= 64 else 1
                        nf = -(-fb // (4 * fbw))
                        kshift = fold and (nf > 1 or dh >= 128)
                        out.append((QoutConfig(elem, dh, r16, 1, True, allfb, fb, m, kshift),
                                    f"c e{elem} d{dh} r{r16} fb{fb} all{allfb}"))
    return out


def kstate_cases():
    out = []
    for elem in DTYPES:
        for dh in HEAD_DIMS:
            for r16 in RANK_BLOCKS:
                if kstate_tile_lds_bytes(elem, dh, r16) > MAX_LDS:
                    continue   # the one-block-at-a-time key side runs instead
                fbw = 2 if dh <= 64 else 1
                fold = fold_exponent(elem, dh, r16)
                for tiles in (1, 3):
                    for kshift in ((False, True) if fold else (False,)):
                        out.append((KstateConfig(elem, dh, r16, fbw, tiles, kshift=kshift),
                                    f"e{elem} d{dh} r{r16} t{tiles} kshift{int(kshift)}"))
    return out
