"""A host model of what happens inside one workgroup of the decode kernels
(`simulate`: batch 1; `simulate_batched`: the MFMA kernel for 2 to 8
sequences): the ordering between its 3 loader waves, its sync wave and its 8
compute waves, through the LDS words they share, over a real queue of the
library's schedule (mk_plan_units), under random schedules with long random
stalls of single waves.  The description below is the batch-1 kernel's;
`simulate_batched` says how the batched one differs.

What it models, wave by wave (the kernel's LDS protocol, not its
arithmetic):

* loader wave lw streams the queue's weight pages n with n % 3 == lw into
  ring slot n % P once every compute wave has released page n - P, keeps at
  most 3 of its pages in flight, and each page lands (data, then its
  sentinel) some time later, in issue order per wave;
* the sync wave, before each unit, waits until the unit that used the same
  result slot (four units earlier) has finished its epilogue; O and DOWN
  units then get their residual rows and QKV units their RoPE values staged
  in that slot; each activation piece goes to activation slot seq % 2 once
  every compute wave has released the piece two before it, and is published
  by raising the ready count;
* compute wave cw passes the unit's first piece, reads its own pieces
  (rows cw, cw + 8, ...) from the pages in stream order, releasing pages as
  it moves on, writes its rows into the result slot, releases the
  activation slot, and counts itself done; the last wave to do so runs the
  epilogue and frees the slot.

With `attn` (the positions of the step and the query heads per KV head),
attention units of paged plans stream their K/V rows through the same ring
(pages counted from the unit's split and the position), and their compute
waves follow the paged attention body: the first wave of each head writes
the head's q into the unit's activation slot and counts itself on a
cumulative LDS counter that the head's other waves wait on; each wave reads
pages rp, rp + WPH, ... of the unit (WPH waves per head); the other waves
leave their partial (m, l, o) in the slot and count themselves on a second
cumulative counter, which the first wave waits on before merging.

Checks: no deadlock; a page is read only from the slot it landed in and is
not replaced before the wave's read ends; an activation piece read is the
one for that unit and piece; a result slot is written only by its own unit
and only after the previous unit's epilogue; every unit's epilogue runs once
with all eight waves counted.  `knobs` plant protocol errors (a loader that
reuses a slot one page early, an activation slot reused one piece early, a
sync wave without the result-slot wait and with four activation slots) so
that tests can show the model catches each."""
from __future__ import annotations

import random

OP_QKV, OP_ATTN, OP_RED, OP_O, OP_FFN, OP_DOWN, OP_LM = 1, 2, 3, 4, 5, 6, 7
GEMV = (OP_QKV, OP_O, OP_FFN, OP_DOWN, OP_LM)
NCW, NLW, ACC = 8, 3, 4


class ProtocolError(AssertionError):
    pass


def attn_geom(u, p: int):
    """(K/V pages, whether the split holds any row) of a paged attention
    unit at position p: rows [lo, min(lo + split_len, p + 1)) of which those
    before p come from the cache, ppp rows per page."""
    lo = u.aux1 * u.split_len
    hi = min(lo + u.split_len, p + 1)
    nr = max(0, min(hi, p) - lo)
    return (nr + u.ppp - 1) // u.ppp, lo < hi


def paged(u, attn) -> bool:
    return attn is not None and u.op == OP_ATTN and u.ppp > 0


class _Attn:
    """LDS state of the paged attention body shared by a workgroup's
    compute waves: the two cumulative counters, which unit's q (per head)
    and partials (per head and wave) each activation slot holds."""

    def __init__(self, group: int, knobs):
        self.G = group
        self.WPH = NCW // group
        self.aq = 0
        self.am = 0
        self.q = {}      # (slot, head) -> unit
        self.mg = {}     # (slot, head, rp) -> unit
        self.tgt = [[0, 0] for _ in range(NCW)]   # each wave's running targets
        self.no_aq_wait = "no_aq_wait" in knobs
        self.no_am_wait = "no_am_wait" in knobs

    def clobber(self, slot, by):
        """Another unit's activation piece is written into the slot."""
        for k in [k for k in self.q if k[0] == slot]:
            self.q[k] = ("overwritten by", by)
        for k in [k for k in self.mg if k[0] == slot]:
            self.mg[k] = ("overwritten by", by)

    def wave(self, sim, cw, vq, u, n, seq, np_, rows, nxs):
        """Compute wave cw through a paged attention unit whose pages start
        at stream index n (a generator, like the waves)."""
        G, WPH = self.G, self.WPH
        h, rp = cw % G, cw // G
        self.tgt[cw][0] += G
        self.tgt[cw][1] += G * (WPH - 1)
        while not sim.st["xready"] > seq:
            yield 0
        slot = seq % nxs
        if rp == 0:
            if rows:
                self.q[(slot, h)] = vq
                yield 1
            self.aq += 1
        elif not self.no_aq_wait:
            while not self.aq >= self.tgt[cw][0]:
                yield 0
        rel = n
        for jp in range(rp, np_, WPH):
            pg = n + jp
            if pg > rel:
                sim.cons[cw] = pg
                rel = pg
            while sim.sent[pg % sim.P] != pg:
                yield 0
            if self.q.get((slot, h)) != vq:
                sim.err(f"wave {cw} reads q of head {h} for unit {vq} from slot {slot} holding "
                        f"{self.q.get((slot, h))}")
            sim.read_page(pg, cw)
            yield 1
            sim.read_page(pg, cw)
        if WPH > 1:
            if rp > 0:
                self.mg[(slot, h, rp)] = vq
                yield 1
                self.am += 1
            else:
                if not self.no_am_wait:
                    while not self.am >= self.tgt[cw][1]:
                        yield 0
                for r in range(1, WPH):
                    got = self.mg.get((slot, h, r))
                    if got != vq:
                        sim.err(f"wave {cw} merges partial {r} of head {h} for unit {vq} "
                                f"from slot {slot} holding {got}")
                yield 1
        sim.cons[cw] = n + np_


class _Sim:
    """What the attention body needs of a model's state."""

    def __init__(self, **kw):
        self.__dict__.update(kw)


def simulate(units, seed: int, ring_pages: int = 8, nxs: int = 2, depth: int = 3,
             stall_p: float = 0.01, max_stall: int = 2000, knobs=(), budget: int = 20_000_000,
             attn=None):
    """Run one workgroup's queue (a list of mk_unit_info) once; raises
    ProtocolError on a violated check.  Returns the number of scheduler
    steps taken.  attn = (positions, query heads per KV head) models the
    K/V pages of paged attention units (None: they carry no pages)."""
    rng = random.Random(seed)
    P = ring_pages
    early_slot = "early_slot" in knobs
    early_xs = "early_xs" in knobs
    no_guard = "no_guard" in knobs
    cons = [0] * NCW
    xcons = [0] * NCW
    st = {"xready": 0, "epi": 0}
    done = [0] * ACC
    ring = [None] * P
    sent = [None] * P
    inflight = []          # [land_time, slot, page, wave]
    xs = [None] * nxs      # (vq, k)
    acc = [None] * ACC     # owning unit
    epis = [0] * len(units)
    now = [0]
    geo = [attn_geom(u, attn[0][u.b]) if paged(u, attn) else (0, False) for u in units]
    att = _Attn(attn[1], knobs) if attn is not None else None

    def err(msg):
        raise ProtocolError(msg)

    def nx_of(u):
        return u.nk if u.op in GEMV else 1

    def pages_of(vq):
        u = units[vq]
        return u.pages if u.op in GEMV else geo[vq][0]

    def read_page(pg, cw):
        if ring[pg % P] != pg:
            err(f"page {pg} read from slot {pg % P} holding {ring[pg % P]}")

    sim = _Sim(st=None, cons=cons, sent=sent, P=P, err=err, read_page=read_page)

    def loader(lw):
        n = 0
        for vq, u in enumerate(units):
            yield 1
            for _ in range(pages_of(vq)):
                if n % NLW == lw:
                    lag = P + 1 if early_slot else P
                    while not (n < P or min(cons) >= n - lag + 1):
                        yield 0
                    while sum(1 for x in inflight if x[3] == lw) >= depth:
                        yield 0
                    ring[n % P] = ("loading", n)
                    t = now[0] + rng.randint(1, 40)
                    mine = [x[0] for x in inflight if x[3] == lw]
                    if mine:
                        t = max(t, max(mine) + 1)
                    inflight.append([t, n % P, n, lw])
                n += 1

    def sync():
        seq = 0
        for vq, u in enumerate(units):
            yield 1
            if vq >= ACC and not no_guard:
                while not st["epi"] + ACC > vq:
                    yield 0
            # the unit's counter waits (other workgroups): some delay
            for _ in range(rng.randint(0, 3)):
                yield 1
            if u.op in (OP_O, OP_DOWN, OP_QKV):
                a = vq % ACC
                if acc[a] not in (None, vq):
                    err(f"sync stages unit {vq} into result slot {a} held by unit {acc[a]}")
                acc[a] = vq
            for k in range(nx_of(u)):
                s = seq + k
                need = s - nxs + (0 if early_xs else 1)
                while not (s < nxs or min(xcons) >= need):
                    yield 0
                if u.op in GEMV:     # (an attention unit's slot is its compute waves')
                    xs[s % nxs] = (vq, k)
                    if att:
                        att.clobber(s % nxs, vq)
                    yield 1
                st["xready"] = s + 1
            seq += nx_of(u)

    def compute(cw):
        n = 0
        seq = 0
        for vq, u in enumerate(units):
            yield 1
            a = vq % ACC
            if paged(u, attn):
                yield from att.wave(sim, cw, vq, u, n, seq, geo[vq][0], geo[vq][1], nxs)
            while not st["xready"] > seq:
                yield 0
            if u.op in GEMV:
                per = u.n_items * u.ipw
                rel = n
                for k in range(u.nk):
                    if k > 0:
                        xcons[cw] = seq + k
                    if cw >= per and k > 0:
                        continue
                    while not st["xready"] > seq + k:
                        yield 0
                    if cw >= per:
                        continue
                    got = xs[(seq + k) % nxs]
                    if got != (vq, k):
                        err(f"wave {cw} reads activation piece {got} for unit {vq} piece {k}")
                    yield 1
                    for r in range(cw, per, NCW):
                        t = k * per + r
                        pg = n + t // u.ppp
                        if pg > rel:
                            cons[cw] = pg
                            rel = pg
                        while sent[pg % P] != pg:
                            yield 0
                        read_page(pg, cw)
                        yield 1
                        if ring[pg % P] != pg:
                            err(f"page {pg} replaced in slot {pg % P} during its read")
                        if acc[a] not in (None, vq):
                            err(f"wave {cw} writes unit {vq} into result slot {a} held by unit {acc[a]}")
                        acc[a] = vq
                cons[cw] = n + pages_of(vq)
            n += pages_of(vq)
            seq += nx_of(u)
            xcons[cw] = seq
            yield 1
            done[a] += 1
            if done[a] == NCW:
                for _ in range(rng.randint(1, 20)):   # the epilogue's stores and signals
                    yield 1
                if acc[a] not in (None, vq):
                    err(f"epilogue of unit {vq} finds result slot {a} held by unit {acc[a]}")
                epis[vq] += 1
                acc[a] = None
                done[a] = 0
                st["epi"] = vq + 1

    sim.st = st
    waves = [loader(i) for i in range(NLW)] + [sync()] + [compute(i) for i in range(NCW)]
    alive = list(range(len(waves)))
    asleep = [0] * len(waves)
    last = 0   # last step at which a wave moved on
    while alive:
        now[0] += 1
        if now[0] > budget:
            err("no progress within the step budget")
        if (now[0] - last > 20000 and not inflight and all(asleep[i] <= now[0] for i in alive)):
            err("deadlock: every wave waits and nothing is in flight")
        for x in [x for x in inflight if x[0] <= now[0]]:
            ring[x[1]] = x[2]
            sent[x[1]] = x[2]
            inflight.remove(x)
        awake = [i for i in alive if asleep[i] <= now[0]]
        if not awake:
            continue
        i = rng.choice(awake)
        if rng.random() < stall_p:
            asleep[i] = now[0] + rng.randint(1, max_stall)
            continue
        try:
            if next(waves[i]):
                last = now[0]
        except StopIteration:
            alive.remove(i)
            last = now[0]
    bad = [vq for vq, c in enumerate(epis) if c != 1]
    if bad:
        err(f"units whose epilogue ran {epis[bad[0]]} times: {bad[:5]}")
    return now[0]


def simulate_batched(units, seed: int, ring_pages: int = 6, nxs: int = 4, inflight_pieces: int = 3,
                     depth: int = 3, stall_p: float = 0.01, max_stall: int = 2000, knobs=(),
                     budget: int = 20_000_000, attn=None):
    """The same for the batched (MFMA) kernel.  Its protocol differs in the
    sync wave, which keeps up to three activation pieces of a unit in
    flight (each waits for its slot of four, lands in order and is then
    published); in the weight pages each compute wave reads (16 weight rows
    x 32 elements per MFMA step: two 1 KB blocks, tile t = cw mod T and K
    steps kg, kg + nwt, ...; wide LM units: whole tiles cw, cw + 8, ...);
    and in the partial-tile buffer of each unit (two, alternating), which
    its waves fill after their K steps once the unit two before has run its
    epilogue, and which that epilogue sums.  Paged attention (`attn`) as in
    `simulate`, each sequence at its own position.  Knobs as `simulate`,
    plus "no_part_guard" (waves fill the partial-tile buffer without
    waiting)."""
    rng = random.Random(seed)
    P = ring_pages
    early_slot = "early_slot" in knobs
    early_xs = "early_xs" in knobs
    no_guard = "no_guard" in knobs
    no_part_guard = "no_part_guard" in knobs
    cons = [0] * NCW
    xcons = [0] * NCW
    st = {"xready": 0, "epi": 0}
    done = [0] * ACC
    ring = [None] * P
    sent = [None] * P
    inflight = []          # weight pages: [land_time, slot, page, wave]
    pieces = []            # activation pieces in flight: [land_time, slot, (vq, k)]
    xs = [None] * nxs
    acc = [None] * ACC
    part = [None] * 2
    epis = [0] * len(units)
    now = [0]
    geo = [attn_geom(u, attn[0][u.b]) if paged(u, attn) else (0, False) for u in units]
    att = _Attn(attn[1], knobs) if attn is not None else None

    def err(msg):
        raise ProtocolError(msg)

    def gv(u):
        return u.op in GEMV

    def nx_of(u):
        return u.nk if gv(u) else 1

    def pages_of(vq):
        u = units[vq]
        return u.pages if gv(u) else geo[vq][0]

    def wide(u):
        return gv(u) and (u.ppp + 1) // 2 > NCW

    def take_acc(vq, who):
        a = vq % ACC
        if acc[a] not in (None, vq):
            err(f"{who} writes unit {vq} into result slot {a} held by unit {acc[a]}")
        acc[a] = vq

    def loader(lw):
        n = 0
        for vq, u in enumerate(units):
            yield 1
            for _ in range(pages_of(vq)):
                if n % NLW == lw:
                    lag = P + 1 if early_slot else P
                    while not (n < P or min(cons) >= n - lag + 1):
                        yield 0
                    while sum(1 for x in inflight if x[3] == lw) >= depth:
                        yield 0
                    ring[n % P] = ("loading", n)
                    t = now[0] + rng.randint(1, 40)
                    mine = [x[0] for x in inflight if x[3] == lw]
                    if mine:
                        t = max(t, max(mine) + 1)
                    inflight.append([t, n % P, n, lw])
                n += 1

    def sync():
        seq = 0
        for vq, u in enumerate(units):
            yield 1
            if vq >= ACC and not no_guard:
                while not st["epi"] + ACC > vq:
                    yield 0
            if u.op == OP_QKV:
                take_acc(vq, "sync (RoPE values)")
            for _ in range(rng.randint(0, 3)):   # the unit's counter waits
                yield 1
            if not gv(u):
                need = seq - nxs + (0 if early_xs else 1)
                while not (seq < nxs or min(xcons) >= need):
                    yield 0
                st["xready"] = seq + 1
                seq += 1
                continue
            issued = landed = 0
            while landed < u.nk:
                if issued < u.nk and issued - landed < inflight_pieces:
                    s = seq + issued
                    need = s - nxs + (0 if early_xs else 1)
                    while not (s < nxs or min(xcons) >= need):
                        yield 0
                    xs[s % nxs] = ("loading", vq, issued)
                    if att:
                        att.clobber(s % nxs, vq)
                    if issued == 0 and u.op in (OP_O, OP_DOWN):
                        take_acc(vq, "sync (residual rows)")
                    t = now[0] + rng.randint(1, 40)
                    if pieces:
                        t = max(t, max(p[0] for p in pieces) + 1)
                    pieces.append([t, s % nxs, (vq, issued)])
                    issued += 1
                    yield 1
                else:
                    while any(p[2] == (vq, landed) for p in pieces):
                        yield 0
                    if landed + 1 == u.nk and u.op in (OP_QKV, OP_FFN, OP_LM):
                        take_acc(vq, "sync (1/rms)")
                    yield 1
                    st["xready"] = seq + landed + 1
                    landed += 1
            seq += u.nk

    def read_page(pg, cw):
        if ring[pg % P] != pg:
            err(f"wave {cw} reads page {pg} from slot {pg % P} holding {ring[pg % P]}")

    sim = _Sim(st=st, cons=cons, sent=sent, P=P, err=err, read_page=read_page)

    def read_piece(vq, k, seq, cw):
        got = xs[(seq + k) % nxs]
        if got != (vq, k):
            err(f"wave {cw} reads activation piece {got} for unit {vq} piece {k}")

    def compute(cw):
        n = 0
        seq = 0
        for vq, u in enumerate(units):
            yield 1
            if paged(u, attn):
                yield from att.wave(sim, cw, vq, u, n, seq, geo[vq][0], geo[vq][1], nxs)
            elif not gv(u):
                while not st["xready"] > seq:
                    yield 0
            else:
                nrb = u.ppp
                T = (nrb + 1) // 2
                rel = n
                if wide(u):
                    if vq >= 2 and not no_part_guard:
                        while not st["epi"] + 1 >= vq:
                            yield 0
                    if part[vq % 2] not in (None, vq):
                        err(f"wave {cw} takes the candidate area of unit {part[vq % 2]} for unit {vq}")
                    part[vq % 2] = vq
                    ntw = (T - cw + NCW - 1) // NCW
                    have = set()
                    for k in range(u.nk):
                        if k > 0:
                            xcons[cw] = seq + k
                        while not st["xready"] > seq + k:
                            yield 0
                        for kb in range(4):
                            read_piece(vq, k, seq, cw)
                            yield 1
                            for r in range(min(ntw, 4)):
                                t = cw + NCW * r
                                lo = (k * 4 + kb) * nrb + 2 * t
                                hi = (k * 4 + kb) * nrb + min(2 * t + 1, nrb - 1)
                                pa, pb = n + lo // 16, n + hi // 16
                                if pa > rel:
                                    cons[cw] = pa
                                    rel = pa
                                for pg in range(pa, pb + 1):
                                    while sent[pg % P] != pg:
                                        yield 0
                                read_page(pa, cw)
                                read_page(pb, cw)
                                yield 1
                                read_page(pa, cw)
                                read_page(pb, cw)
                else:
                    t = cw % T
                    nwt = (NCW - 1 - t) // T + 1
                    kg = cw // T
                    lo_rb, hi_rb = 2 * t, min(2 * t + 1, nrb - 1)
                    kcur = None
                    for j in range(kg, u.nk * 8, nwt):
                        k, ks = j >> 3, j & 7
                        if k != kcur:
                            if k > 0:
                                xcons[cw] = seq + k
                            while not st["xready"] > seq + k:
                                yield 0
                            kcur = k
                        l0 = (k * nrb + lo_rb) * 4 + (ks >> 1)
                        l1 = (k * nrb + hi_rb) * 4 + (ks >> 1)
                        p0, p1 = n + l0 // 16, n + l1 // 16
                        if p0 > rel:
                            cons[cw] = p0
                            rel = p0
                        for pg in (p0, p1):
                            while sent[pg % P] != pg:
                                yield 0
                        read_piece(vq, k, seq, cw)
                        read_page(p0, cw)
                        read_page(p1, cw)
                        yield 1
                        read_page(p0, cw)
                        read_page(p1, cw)
                    if vq >= 2 and not no_part_guard:
                        while not st["epi"] + 1 >= vq:
                            yield 0
                    if part[vq % 2] not in (None, vq):
                        err(f"wave {cw} writes its partial tile of unit {vq} over unit {part[vq % 2]}")
                    part[vq % 2] = vq
                cons[cw] = n + pages_of(vq)
            n += pages_of(vq)
            seq += nx_of(u)
            xcons[cw] = seq
            yield 1
            a = vq % ACC
            done[a] += 1
            if done[a] == NCW:
                for _ in range(rng.randint(1, 20)):   # the epilogue reads both buffers
                    yield 1
                if acc[a] not in (None, vq):
                    err(f"epilogue of unit {vq} finds result slot {a} held by unit {acc[a]}")
                if gv(u) and part[vq % 2] != vq:
                    err(f"epilogue of unit {vq} finds partial tiles of unit {part[vq % 2]}")
                epis[vq] += 1
                acc[a] = None
                if gv(u):
                    part[vq % 2] = None
                done[a] = 0
                st["epi"] = vq + 1

    waves = [loader(i) for i in range(NLW)] + [sync()] + [compute(i) for i in range(NCW)]
    alive = list(range(len(waves)))
    asleep = [0] * len(waves)
    last = 0
    while alive:
        now[0] += 1
        if now[0] > budget:
            err("no progress within the step budget")
        if (now[0] - last > 20000 and not inflight and not pieces
                and all(asleep[i] <= now[0] for i in alive)):
            err("deadlock: every wave waits and nothing is in flight")
        for x in [x for x in inflight if x[0] <= now[0]]:
            ring[x[1]] = x[2]
            sent[x[1]] = x[2]
            inflight.remove(x)
        for p in [p for p in pieces if p[0] <= now[0]]:
            xs[p[1]] = p[2]
            pieces.remove(p)
        awake = [i for i in alive if asleep[i] <= now[0]]
        if not awake:
            continue
        i = rng.choice(awake)
        if rng.random() < stall_p:
            asleep[i] = now[0] + rng.randint(1, max_stall)
            continue
        try:
            if next(waves[i]):
                last = now[0]
        except StopIteration:
            alive.remove(i)
            last = now[0]
    bad = [vq for vq, c in enumerate(epis) if c != 1]
    if bad:
        err(f"units whose epilogue ran {epis[bad[0]]} times: {bad[:5]}")
    return now[0]
